"""GPU parity of the draft chain (through the C ABI) against the CPU oracle."""
import numpy as np
import pytest

import mtp_synth as syn
from tests.gpu_harness import GpuDrafter, compare_draft, log, record

pytestmark = pytest.mark.gpu


def _check(w, gpu_out, orc_out, idx=None, max_near=1):
    c = compare_draft(w.model, gpu_out, orc_out, idx)
    log(f"  {w.name}: steps={c.compared_steps} near_ties={c.near_ties} max_logit_err={c.max_logit_err:.3g} "
        f"max_h_err={c.max_h_err:.3g}")
    record(w.name, compared_steps=c.compared_steps, near_ties=c.near_ties, max_logit_err=c.max_logit_err,
           max_h_err=c.max_h_err)
    assert c.near_ties <= max_near
    return c


def test_c1_tiny_fp32_matches_oracle(orc):
    log("case c1 tiny fp32: S=1 N=3 ctx=512")
    w = syn.c1_tiny()
    g = GpuDrafter(w.model, 1, 3)
    _check(w, g.run(w.draft), orc.draft_block(w.model, w.draft))


def test_c1_shapes_ragged_multi_seq(orc):
    log("case c1 shapes: S=3 N=5 ctx=300 (ragged split tail)")
    w = syn.c1_tiny(n_seq=3, n_steps=5, ctx=300)
    g = GpuDrafter(w.model, 4, 6)
    _check(w, g.run(w.draft), orc.draft_block(w.model, w.draft))


def test_c2_gemma_bf16_full_size_matches_oracle(orc):
    log("case c2 full: bf16, V=262144, ctx=8192, S=1 N=3")
    w = syn.c2_gemma_bf16()
    g = GpuDrafter(w.model, 1, 3)
    _check(w, g.run(w.draft), orc.draft_block(w.model, w.draft))


def test_c2_shapes_ragged_vocab_and_context(orc):
    log("case c2 shapes: V=262144-123, ctx=1000, S=3 N=2")
    w = syn.c2_gemma_bf16(n_vocab=262144 - 123, ctx=1000, n_seq=3, n_steps=2)
    g = GpuDrafter(w.model, 3, 2)
    _check(w, g.run(w.draft), orc.draft_block(w.model, w.draft))


def test_c3_interleaved_swa_full_small_contexts(orc):
    log("case c3 small: 16 seqs, ctx U[700, 5000], SWA window 1024 ring")
    w = syn.c3_interleaved(ctx_range=(700, 5000), full_cap=5000)
    g = GpuDrafter(w.model, 16, 3)
    _check(w, g.run(w.draft), orc.draft_block(w.model, w.draft), max_near=2)


def test_c3_full_size_sampled_sequences(orc):
    log("case c3 full: 16 seqs, ctx U[4096, 32768]; oracle on 4 sampled sequences")
    w = syn.c3_interleaved()
    g = GpuDrafter(w.model, 16, 3)
    gpu = g.run(w.draft)
    idx = [0, 5, 10, 15]
    _check(w, gpu, orc.draft_block(w.model, w.draft, seq_idx=idx), idx)


def test_c4_q8_head_small_context(orc):
    log("case c4 small: Q8_0 head, 8 seqs, ctx 3000, N=4")
    w = syn.c4_longctx_q8(ctx=3000)
    g = GpuDrafter(w.model, 8, 4)
    _check(w, g.run(w.draft), orc.draft_block(w.model, w.draft))


def _rows(out, idx):
    return {k: (v[idx] if isinstance(v, np.ndarray) else v) for k, v in out.items()}


def test_q8_head_ragged_vocab_packed_unpacked_and_one_sequence(orc):
    """The several-sequence Q8_0 head streams the head's unit-order copy,
    whose last 16-row tile is padded with zero rows when V % 16 != 0.  Up
    to 8 sequences share each MFMA between the activations' hi and lo
    halves (packed), 9 to 16 take one MFMA per half (unpacked), and one
    sequence runs the row-major one-sequence head.  All three against the
    oracle on the same sequences."""
    log("case q8 ragged: V=262144-123, ctx=1500, N=3; S=12 (unpacked), 5 (packed), 1")
    w = syn.c4_longctx_q8(n_vocab=262144 - 123, ctx=1500, n_seq=12, n_steps=3)
    ref = orc.draft_block(w.model, w.draft)
    g = GpuDrafter(w.model, 12, 3)
    _check(w, g.run(w.draft), ref)
    few = [3, 7, 0, 11, 5]
    _check(w, g.run(w.draft, seq_idx=few), _rows(ref, few))
    _check(w, g.run(w.draft, seq_idx=[6]), _rows(ref, [6]))


@pytest.mark.parametrize("d_model,n_seq", [(256, 5), (256, 12), (512, 7), (512, 11), (288, 6)])
def test_q8_head_widths(orc, d_model, n_seq):
    """The several-sequence Q8_0 head at one and two 256-column units per
    tile (d = 256, 512; packed at <= 8 sequences, unpacked above), and at a
    width that is not a multiple of 256 (d = 288: no unit-order copy, the
    row-major head instead), on a ragged vocabulary."""
    log(f"case q8 width: d={d_model}, S={n_seq}, V=30011, ctx=700, N=3")
    w = syn.c4_longctx_q8(d_model=d_model, n_vocab=30011, ctx=700, n_seq=n_seq, n_steps=3)
    g = GpuDrafter(w.model, n_seq, 3)
    _check(w, g.run(w.draft), orc.draft_block(w.model, w.draft))


def test_chained_equals_step_by_step_on_gpu():
    """One N-step call == N one-step calls chained through (token, h), bit for
    bit (the fused-vs-sequential check of the evaluation record)."""
    log("case chain==steps: c3 small shapes")
    w = syn.c3_interleaved(ctx_range=(700, 3000), full_cap=3000, n_seq=5)
    g = GpuDrafter(w.model, 5, 3)
    full = g.run(w.draft)
    tok, h = w.draft.last_tok.copy(), w.draft.h_prev.copy()
    for k in range(3):
        one = g.run(w.draft, n_steps=1, last_tok=tok, h_prev=h, pos0_shift=k)
        assert np.array_equal(one["drafts"][:, 0], full["drafts"][:, k])
        assert np.array_equal(one["logits"][:, 0], full["logits"][:, k])
        tok, h = one["drafts"][:, 0].copy(), one["h_last"].copy()
    assert np.array_equal(h, full["h_last"])


def test_sequence_alone_equals_sequence_in_batch():
    """Per-sequence results do not depend on the rest of the batch.  Batches
    of two or more run the GEMVs and the LM head on the matrix cores, where
    every sequence is its own output column: a pair taken out of a batch of
    6 gives the same bits.  A single sequence runs the wave-reduction path,
    whose fp32 sums are ordered differently: same ids, logits and h within
    fp32 rounding."""
    log("case alone==batch")
    w = syn.c3_interleaved(ctx_range=(700, 3000), full_cap=3000, n_seq=6)
    g = GpuDrafter(w.model, 6, 3)
    batch = g.run(w.draft)
    pair = g.run(w.draft, seq_idx=[4, 1])
    for k, s in enumerate((4, 1)):
        for key in ("drafts", "logits", "h_last"):
            assert np.array_equal(pair[key][k], batch[key][s]), key
    for s in (0, 4):
        one = g.run(w.draft, seq_idx=[s])
        assert np.array_equal(one["drafts"][0], batch["drafts"][s])
        np.testing.assert_allclose(one["logits"][0], batch["logits"][s], rtol=0, atol=1e-4)
        np.testing.assert_allclose(one["h_last"][0], batch["h_last"][s], rtol=0, atol=1e-4)


def test_kv_is_read_only_and_unseen_cells_are_never_read():
    """The drafter never writes the target KV, and cells outside the visible
    range (past attn_pos, outside the SWA window) can hold NaN without any
    effect ("Gemma 4 MTP" s.5; the audit page's no-invalid-read check)."""
    import torch
    from mtp_synth.device import upload_seqs
    log("case kv read-only + poisoned cells")
    w = syn.c3_interleaved(ctx_range=(1500, 2500), full_cap=4096, n_seq=4)
    g = GpuDrafter(w.model, 4, 3)
    ref = g.run(w.draft)
    # poison: full cells > attn_pos; SWA ring cells are all visible when ctx >= W,
    # so rebuild each ring with extra capacity and poison the unused cells
    for s in w.draft.seqs:
        full, swa = s.src[syn.KV_FULL], s.src[syn.KV_SWA]
        k, v = full.k.copy(), full.v.copy()
        k[s.attn_pos + 1:] = 0x7FC0
        v[s.attn_pos + 1:] = 0x7FC0
        C = swa.n_cells + 77
        k2 = np.full((C,) + swa.k.shape[1:], 0x7FC0, np.uint16)
        v2 = np.full((C,) + swa.v.shape[1:], 0x7FC0, np.uint16)
        W = w.model.swa_window
        for p in range(s.attn_pos - W + 1, s.attn_pos + 1):
            k2[p % C], v2[p % C] = swa.k[p % swa.n_cells], swa.v[p % swa.n_cells]
        s.src = [syn.KVSource(k, v), syn.KVSource(k2, v2), None]
    seqs, lt, hp, keep = upload_seqs(w.model, w.draft, "cuda")
    before = [torch.cat([t.view(torch.int16).flatten().to(torch.int64) for t in keep]).sum().item()]
    import mtp_draft_verify_amd as mtp
    drafts = torch.zeros((4, 3), dtype=torch.int32, device="cuda")
    h = torch.zeros((4, w.model.d_hprev), device="cuda")
    logits = torch.zeros((4, 3, w.model.n_vocab), device="cuda")
    g.ctx.draft_block(seqs, lt, hp, 3, drafts, h, logits)
    torch.cuda.synchronize()
    after = torch.cat([t.view(torch.int16).flatten().to(torch.int64) for t in keep]).sum().item()
    assert before[0] == after
    assert np.array_equal(drafts.cpu().numpy(), ref["drafts"])
    assert np.array_equal(logits.cpu().numpy(), ref["logits"])
    assert np.array_equal(h.cpu().numpy(), ref["h_last"])


def test_repeated_calls_are_deterministic():
    log("case determinism")
    w = syn.c2_gemma_bf16(ctx=2000, n_vocab=65536)
    g = GpuDrafter(w.model, 1, 3)
    a = g.run(w.draft)
    b = g.run(w.draft)
    for k in a:
        assert np.array_equal(a[k], b[k])


def test_captured_chain_replays_match_direct_launches():
    """The chain captured once per launch shape and replayed with new
    per-call parameters (other context lengths in the same split bucket,
    other tokens and hidden states) gives the same bits as individually
    launched kernels (a stale-parameter replay would not)."""
    import mtp_draft_verify_amd as mtp
    log("case graph replay == direct launches")
    w = syn.c3_interleaved(ctx_range=(2100, 2600), full_cap=3000, n_seq=3)
    g = GpuDrafter(w.model, 3, 3)
    outs = []
    for shift in (0, 7, 19):
        for s in w.draft.seqs:
            s.attn_pos += shift
            s.pos0 += shift
        g.ctx.profile(0)
        replay = g.run(w.draft, last_tok=(w.draft.last_tok + shift) % w.model.n_vocab,
                       h_prev=w.draft.h_prev * (1 + 0.1 * shift))
        g.ctx.profile(1 << mtp.MTP_PROF_GEMV)     # kernel timing launches kernel by kernel
        direct = g.run(w.draft, last_tok=(w.draft.last_tok + shift) % w.model.n_vocab,
                       h_prev=w.draft.h_prev * (1 + 0.1 * shift))
        g.ctx.profile(0)
        for k in replay:
            assert np.array_equal(replay[k], direct[k]), (shift, k)
        outs.append(replay["drafts"])
    assert not all(np.array_equal(outs[0], o) for o in outs[1:])


def test_centroid_head_full_size_matches_oracle(orc):
    log("case c6: centroid head, 2048 centroids x 128 ids, top 32; bf16 c2 drafter, ctx 8192, S=1 N=3")
    w = syn.c6_centroid()
    g = GpuDrafter(w.model, 1, 3)
    gpu = g.run(w.draft)
    o = orc.draft_block(w.model, w.draft)
    _check(w, gpu, o)
    # the full logit row: -1e30 outside the candidates, as the verifier expects
    assert (gpu["logits"] == np.float32(-1e30)).sum() == (o["logits"] == np.float32(-1e30)).sum()


def test_centroid_head_several_sequences_with_confidence(orc):
    log("case c6 small: centroid head, S=3, N=2, ctx 1000 (+confidence)")
    w = syn.c6_centroid(n_seq=3, n_steps=2, ctx=1000)
    g = GpuDrafter(w.model, 3, 2)
    gpu = g.run(w.draft, conf=True)
    o = orc.draft_block(w.model, w.draft)
    _check(w, gpu, o)
    np.testing.assert_allclose(gpu["conf"], o["conf"], rtol=1e-3)
