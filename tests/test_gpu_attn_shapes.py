"""GPU parity of the draft chain for every attention kernel the library
builds (head dim x query heads per KV head x KV dtype), against the oracle.

Small drafters (d 256, one block, V 4096) over ragged contexts, so that the
split-K partition has a ragged last split and the cross-attention runs every
instantiation of the bf16 matrix-core kernel and of the fp32 vector kernel.
Two sequences take the several-sequence GEMV and head paths, one sequence the
one-sequence paths.
"""
import pytest

import mtp_synth as syn
from tests.gpu_harness import GpuDrafter, compare_draft, log

pytestmark = pytest.mark.gpu

# (kv dtype, weight dtype, head_dim, n_head_q, n_head_kv): G = n_head_q / n_head_kv
CASES = [
    (syn.BF16, syn.BF16, 256, 4, 1),
    (syn.BF16, syn.BF16, 256, 4, 2),
    (syn.BF16, syn.BF16, 256, 4, 4),
    (syn.BF16, syn.BF16, 256, 8, 1),
    (syn.BF16, syn.BF16, 128, 8, 1),
    (syn.BF16, syn.BF16, 128, 8, 2),
    (syn.BF16, syn.BF16, 128, 8, 4),
    (syn.BF16, syn.BF16, 128, 8, 8),
    (syn.F32, syn.F32, 64, 4, 1),
    (syn.F32, syn.F32, 64, 8, 1),
    (syn.F32, syn.F32, 64, 4, 2),
    (syn.F32, syn.F32, 64, 4, 4),
    (syn.F32, syn.F32, 128, 4, 1),
    (syn.F32, syn.F32, 256, 4, 1),
]


@pytest.mark.parametrize("kv,wd,hd,hq,hkv", CASES,
                         ids=[f"{'bf16' if c[0] == syn.BF16 else 'f32'}-hd{c[2]}-hq{c[3]}-hkv{c[4]}" for c in CASES])
@pytest.mark.parametrize("n_seq", [1, 2], ids=["S1", "S2"])
def test_attention_instantiations_match_oracle(orc, kv, wd, hd, hq, hkv, n_seq):
    name = f"kv={'bf16' if kv == syn.BF16 else 'f32'} hd={hd} Hq={hq} Hkv={hkv} S={n_seq}"
    log(f"case attention shapes: {name}")
    m = syn.make_model(11 + hd + 7 * hq + hkv, d_model=256, d_hprev=256, n_blocks=1, n_head_q=hq, n_head_kv=hkv,
                       head_dim=hd, d_ff=512, n_vocab=4096, w_dtype=wd, head_dtype=wd, kv_dtype=kv)
    # 1000 cells: 16 splits of 64, the last one 40 cells long; 333: 6, the last 13
    ctx = [1000, 333][:n_seq]
    dr = syn.make_draft_inputs(5 + hd, m, ctx, 3)
    gpu = GpuDrafter(m, n_seq, 3).run(dr)
    c = compare_draft(m, gpu, orc.draft_block(m, dr))
    log(f"  {name}: steps={c.compared_steps} near_ties={c.near_ties} max_logit_err={c.max_logit_err:.3g} "
        f"max_h_err={c.max_h_err:.3g}")
    assert c.near_ties <= 1


@pytest.mark.parametrize("kv,wd,hd,hq,hkv", [
    (syn.BF16, syn.BF16, 256, 4, 1),
    (syn.F32, syn.F32, 64, 4, 1),
], ids=["bf16-hd256", "f32-hd64"])
def test_degenerate_and_boundary_contexts_match_oracle(orc, kv, wd, hd, hq, hkv):
    """One visible cell (attention is then that cell's V), one and two tiles,
    both sides of a 64-cell split, 2047 cells (32 splits of 64) and 2049
    (in a batch, 17 splits of 128, the last holding one cell; alone, 33 of
    64), and 8193 cells (129 splits of 64 would exceed the 128 partial slots,
    so the split doubles to 128 cells and the last split holds one cell), in
    one batch and the 1-, 2049- and 8193-cell ones alone."""
    name = f"kv={'bf16' if kv == syn.BF16 else 'f32'} hd={hd}"
    ctx = [1, 2, 16, 17, 64, 65, 2047, 2049, 8193]
    log(f"case boundary contexts {name}: ctx {ctx}")
    m = syn.make_model(41 + hd, d_model=256, d_hprev=256, n_blocks=1, n_head_q=hq, n_head_kv=hkv, head_dim=hd,
                       d_ff=512, n_vocab=4096, w_dtype=wd, head_dtype=wd, kv_dtype=kv)
    dr = syn.make_draft_inputs(9 + hd, m, ctx, 3)
    g = GpuDrafter(m, len(ctx), 3)
    c = compare_draft(m, g.run(dr), orc.draft_block(m, dr))
    log(f"  batch: steps={c.compared_steps} near_ties={c.near_ties} max_logit_err={c.max_logit_err:.3g}")
    assert c.near_ties <= 1
    for s in (0, 7, 8):
        one = g.run(dr, seq_idx=[s])
        c1 = compare_draft(m, one, orc.draft_block(m, dr, seq_idx=[s]), [0])
        assert c1.near_ties == 0


# bf16 shapes whose long-context sequences run two kv heads per workgroup
WIDE_CASES = [c for c in CASES if c[0] == syn.BF16 and c[4] % 2 == 0 and not (c[2] == 256 and c[3] // c[4] == 8)]


@pytest.mark.parametrize("kv,wd,hd,hq,hkv", WIDE_CASES,
                         ids=[f"bf16-hd{c[2]}-hq{c[3]}-hkv{c[4]}" for c in WIDE_CASES])
def test_two_heads_per_workgroup_long_context_matches_oracle(orc, kv, wd, hd, hq, hkv):
    """From 65536 visible cells a sequence's attention workgroups serve two
    kv heads each, over at most 64 splits: 70001 cells split into 35 splits
    of 2048, the last holding 369 cells.  Alone (one-sequence grid), and in a
    batch beside a 3000-cell sequence that keeps one head per workgroup in
    the same launch."""
    name = f"hd={hd} Hq={hq} Hkv={hkv}"
    log(f"case two kv heads per workgroup: {name}, ctx 70001 alone and with 3000")
    m = syn.make_model(61 + hd + 7 * hq + hkv, d_model=256, d_hprev=256, n_blocks=1, n_head_q=hq, n_head_kv=hkv,
                       head_dim=hd, d_ff=512, n_vocab=4096, w_dtype=wd, head_dtype=wd, kv_dtype=kv)
    dr = syn.make_draft_inputs(13 + hd, m, [70001, 3000], 3)
    g = GpuDrafter(m, 2, 3)
    c = compare_draft(m, g.run(dr), orc.draft_block(m, dr))
    log(f"  batch: steps={c.compared_steps} near_ties={c.near_ties} max_logit_err={c.max_logit_err:.3g} "
        f"max_h_err={c.max_h_err:.3g}")
    assert c.near_ties <= 1
    one = g.run(dr, seq_idx=[0])
    c1 = compare_draft(m, one, orc.draft_block(m, dr, seq_idx=[0]), [0])
    log(f"  alone: near_ties={c1.near_ties} max_logit_err={c1.max_logit_err:.3g}")
    assert c1.near_ties <= 1
    g.close()


def test_two_heads_per_workgroup_over_a_wrapping_swa_ring_matches_oracle(orc):
    """A sliding window of 70000 cells over a ring of the same capacity, with
    attn_pos past the capacity: the window wraps around the ring inside one
    of its 2048-cell splits, and the sequence's workgroups serve both kv
    heads.  Beside a 3000-cell sequence, whose window (all of its positions)
    keeps one head per workgroup, and alone."""
    log("case two kv heads per workgroup over a wrapping 70000-cell SWA ring")
    m = syn.make_model(67, d_model=256, d_hprev=256, n_blocks=2, n_head_q=8, n_head_kv=2, head_dim=256, d_ff=512,
                       n_vocab=4096, w_dtype=syn.BF16, head_dtype=syn.BF16, kv_dtype=syn.BF16, swa_window=70000,
                       block_src=[syn.KV_SWA, syn.KV_FULL])
    dr = syn.make_draft_inputs(69, m, [100001, 3000], 3)
    g = GpuDrafter(m, 2, 3)
    c = compare_draft(m, g.run(dr), orc.draft_block(m, dr))
    log(f"  batch: steps={c.compared_steps} near_ties={c.near_ties} max_logit_err={c.max_logit_err:.3g} "
        f"max_h_err={c.max_h_err:.3g}")
    assert c.near_ties <= 1
    one = g.run(dr, seq_idx=[0])
    c1 = compare_draft(m, one, orc.draft_block(m, dr, seq_idx=[0]), [0])
    log(f"  alone: near_ties={c1.near_ties} max_logit_err={c1.max_logit_err:.3g}")
    assert c1.near_ties <= 1
    g.close()
