"""GPU parity of the draft chain exactly as a serving loop runs it: no logit
rows requested, so every LM-head kernel takes its argmax-only form ("Gemma 4
MTP" s.4: the full row is kept only for diagnostics; "Fused NextN draft
graph", the readback contract: the drafts and the next hidden state only),
launched through the captured chain on the first call and replayed after.

Also: the longest contexts (131072 cells, where the split-K attention runs
1024-cell splits and the two-tile steady-state loop of every wave several
times) and the captured-chain cache past its capacity.

Rule (as in the other draft tests): ids bit-exact, h_last within the
tolerance, a differing id allowed only at an oracle near tie (top-2 margin
under the tolerance), counted and reported.
"""
import numpy as np
import pytest

import mtp_synth as syn
from tests.gpu_harness import GpuDrafter, compare_draft, log, record

pytestmark = pytest.mark.gpu


def _check(name, m, gpu, orc_out, idx=None, max_near=1):
    c = compare_draft(m, gpu, orc_out, idx)
    log(f"  {name}: steps={c.compared_steps} near_ties={c.near_ties} max_logit_err={c.max_logit_err:.3g} "
        f"max_h_err={c.max_h_err:.3g}")
    record(name, compared_steps=c.compared_steps, near_ties=c.near_ties, max_logit_err=c.max_logit_err,
           max_h_err=c.max_h_err)
    assert c.near_ties <= max_near
    return c


def _replayed_without_logits(g, dr, seq_idx=None):
    """Two calls without logit rows (capture, then replay): both give the
    same bits."""
    a = g.run(dr, want_logits=False, seq_idx=seq_idx)
    b = g.run(dr, want_logits=False, seq_idx=seq_idx)
    assert np.array_equal(a["drafts"], b["drafts"]) and np.array_equal(a["h_last"], b["h_last"])
    assert a["logits"] is None
    return a


def test_c2_full_size_without_logits_matches_oracle(orc):
    """One sequence: the one-sequence LM head in its argmax-only form."""
    log("case c2 full, no logits: bf16, V=262144, ctx=8192, S=1 N=3")
    w = syn.c2_gemma_bf16()
    g = GpuDrafter(w.model, 1, 3)
    gpu = _replayed_without_logits(g, w.draft)
    o = orc.draft_block(w.model, w.draft)
    _check("c2 no logits", w.model, gpu, o)
    # the same chain with logit rows gives the same ids and h (the logit
    # stores are the only difference between the two head forms)
    full = g.run(w.draft)
    assert np.array_equal(full["drafts"], gpu["drafts"]) and np.array_equal(full["h_last"], gpu["h_last"])
    g.close()


def test_c3_full_size_without_logits_sampled_sequences(orc):
    """16 sequences: the matrix-core bf16 LM head in its argmax-only form."""
    log("case c3 full, no logits: 16 seqs, ctx U[4096, 32768]; oracle on 4 sampled sequences")
    w = syn.c3_interleaved()
    g = GpuDrafter(w.model, 16, 3)
    gpu = _replayed_without_logits(g, w.draft)
    idx = [1, 6, 11, 14]
    _check("c3 no logits", w.model, gpu, orc.draft_block(w.model, w.draft, seq_idx=idx), idx)
    g.close()


def test_c4_full_size_131072_cells_sampled_sequences(orc):
    """The long-context workload at its real size: 8 sequences x 131072
    cells, Q8_0 head, N=4 (the matrix-core Q8_0 head in its argmax-only
    form, and with logit rows), oracle on 2 sampled sequences."""
    log("case c4 full: 8 seqs x 131072 cells, Q8_0 head, N=4; oracle on sequences 2 and 7")
    w = syn.c4_longctx_q8()
    g = GpuDrafter(w.model, 8, 4)
    gpu = _replayed_without_logits(g, w.draft)
    log("  GPU done (no logits); running the oracle")
    idx = [2, 7]
    o = orc.draft_block(w.model, w.draft, seq_idx=idx)
    _check("c4 full no logits", w.model, gpu, o, idx)
    full = g.run(w.draft)
    assert np.array_equal(full["drafts"], gpu["drafts"]) and np.array_equal(full["h_last"], gpu["h_last"])
    _check("c4 full with logits", w.model, full, o, idx)
    g.close()


def test_long_ragged_context_alone_and_in_a_batch(orc):
    """100003 visible cells split into 2048-cell splits (49 splits, the last
    1699 cells) whose workgroups serve both kv heads: each wave of a full
    split walks 64 tiles, the steady-state loop many times, and the last
    split is ragged.  Alone (one-sequence paths) and beside a 131072-cell
    and a 5000-cell sequence (batch paths; the 5000-cell one keeps one kv
    head per workgroup in the same launch)."""
    log("case long ragged context: 100003 cells alone and with 131072 / 5000")
    m = syn.make_model(57, d_model=256, d_hprev=256, n_blocks=1, n_head_q=8, n_head_kv=2, head_dim=256, d_ff=512,
                       n_vocab=4096, w_dtype=syn.BF16, head_dtype=syn.BF16, kv_dtype=syn.BF16)
    dr = syn.make_draft_inputs(59, m, [100003, 131072, 5000], 3)
    g = GpuDrafter(m, 3, 3)
    o = orc.draft_block(m, dr)
    _check("ctx 100003 in a batch of 3", m, g.run(dr), o)
    _check("ctx 100003 in a batch of 3, no logits", m, g.run(dr, want_logits=False), o)
    one = g.run(dr, seq_idx=[0])
    _check("ctx 100003 alone", m, one, orc.draft_block(m, dr, seq_idx=[0]), [0])
    g.close()


def test_short_sequences_same_bits_beside_a_long_one():
    """A sequence's attention arithmetic depends on that sequence alone:
    short sequences give the same bits in a batch whose launches also run a
    long (two kv heads per workgroup) sequence as in a batch without it."""
    log("case short sequences beside a long one: same bits")
    m = syn.make_model(63, d_model=256, d_hprev=256, n_blocks=2, n_head_q=8, n_head_kv=2, head_dim=256, d_ff=512,
                       n_vocab=4096, w_dtype=syn.BF16, head_dtype=syn.BF16, kv_dtype=syn.BF16)
    dr = syn.make_draft_inputs(65, m, [3000, 131072, 5000], 3)
    g = GpuDrafter(m, 3, 3)
    full = g.run(dr)
    short = g.run(dr, seq_idx=[0, 2])
    for k, s in enumerate((0, 2)):
        for key in ("drafts", "logits", "h_last"):
            assert np.array_equal(short[key][k], full[key][s]), (s, key)
    g.close()


def test_graph_cache_past_capacity_stays_exact(orc):
    """More launch shapes than the context keeps captured chains (16): the
    least recently used chain is evicted while earlier launches are still
    queued (all 24 calls are enqueued before the one wait), and a shape seen
    again is captured anew.  Every call's ids match the oracle bit for bit."""
    import torch
    import mtp_draft_verify_amd as mtp
    from mtp_synth.device import upload_seqs
    log("case captured-chain cache: 20 launch shapes, then the first 4 again, one wait at the end")
    m = syn.make_model(61, d_model=256, d_hprev=256, n_blocks=1, n_head_q=4, n_head_kv=1, head_dim=64, d_ff=512,
                       n_vocab=4096, w_dtype=syn.F32, head_dtype=syn.F32, kv_dtype=syn.F32)
    dr = syn.make_draft_inputs(63, m, [700, 300, 1200, 90, 2500], 5)
    g = GpuDrafter(m, 5, 5)
    up = {S: upload_seqs(m, dr, "cuda", list(range(S))) for S in (1, 2, 3, 4, 5)}
    shapes = [(S, N) for S in (1, 2, 3, 4, 5) for N in (1, 2, 3, 5)]       # 20 shapes
    calls = []
    for S, N in shapes + shapes[:4]:
        seqs, lt, hp, _ = up[S]
        out = torch.full((S, N), -7, dtype=torch.int32, device="cuda")
        g.ctx.draft_block(mtp.make_seqs(seqs), lt, hp, N, out)
        calls.append((S, N, out))
    torch.cuda.synchronize()
    ref = {S: orc.draft_block(m, dr, seq_idx=list(range(S)), n_steps=5) for S in (1, 2, 3, 4, 5)}
    near = 0
    for S, N, out in calls:
        o = ref[S]
        sub = dict(drafts=o["drafts"][:, :N], h_last=None, logits=o["logits"][:, :N], margin=o["margin"][:, :N])
        c = compare_draft(m, dict(drafts=out.cpu().numpy(), h_last=None, logits=None), sub)
        near += c.near_ties
    record("graph cache 24 calls", near_ties=near)
    assert near <= 1
    g.close()
