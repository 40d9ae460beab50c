"""GPU test of mtp_verify_greedy_noalloc (through the C ABI): the greedy
verify for callers that cannot allocate must give exactly what the
context-owning mtp_verify_greedy gives, and what the oracle gives, on two
calls in a row, the second smaller than the first (the static scratch keeps
the first call's contents and must not leak them into the second); a call
beyond the scratch's rows is refused with nothing enqueued."""
import numpy as np
import pytest

import mtp_synth as syn
from tests.gpu_harness import log, record

pytestmark = pytest.mark.gpu


def _ctx_verify(logits, drafts):
    import torch
    import mtp_draft_verify_amd as mtp
    S, R, V = logits.shape
    desc = mtp.make_desc(d_model=32, d_hprev=8, n_blocks=1, n_head_q=1, n_head_kv=1, head_dim=64, d_ff=8,
                         n_vocab=V, w_dtype=0, head_dtype=0, kv_dtype=0, max_seqs=S, max_steps=max(R - 1, 1))
    ctx = mtp.Context(desc, None)
    toks = torch.full((S, R), -9, dtype=torch.int32, device="cuda")
    na = torch.full((S,), -9, dtype=torch.int32, device="cuda")
    ctx.verify_greedy(logits, drafts, toks, na)
    torch.cuda.synchronize()
    ctx.close()
    return toks.cpu().numpy(), na.cpu().numpy()


def _noalloc_verify(logits, drafts, stream=None):
    import torch
    import mtp_draft_verify_amd as mtp
    S, R, V = logits.shape
    toks = torch.full((S, R), -9, dtype=torch.int32, device="cuda")
    na = torch.full((S,), -9, dtype=torch.int32, device="cuda")
    mtp.mtp_verify_greedy_noalloc(stream, logits, drafts, toks, na)
    torch.cuda.synchronize()
    return toks.cpu().numpy(), na.cpu().numpy()


def test_noalloc_greedy_verify_matches_the_context_verify_twice(orc):
    import torch
    import mtp_draft_verify_amd as mtp
    cases = [(19, 8, 4, 262144, 0.7), (23, 3, 2, 50000 - 3, 0.8)]     # second call: fewer rows, ragged vocab
    for seed, S, N, V, p in cases:
        log(f"case no-alloc greedy verify: S={S} N={N} V={V}")
        gv = syn.make_greedy_verify(seed, S, N, V, p, "max5")
        logits = torch.from_numpy(gv.logits).cuda()
        drafts = torch.from_numpy(gv.drafts).cuda()
        t_n, n_n = _noalloc_verify(logits, drafts)
        t_c, n_c = _ctx_verify(logits, drafts)
        t_o, n_o = orc.verify_greedy(gv.logits, gv.drafts)
        assert np.array_equal(t_n, t_c) and np.array_equal(n_n, n_c)
        assert np.array_equal(t_n, t_o) and np.array_equal(n_n, n_o)
        record(f"no-alloc greedy verify S={S} N={N}", compared=S, mismatches_on_clean=0)
    # the same rows again on a side stream of the same device
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        t_s, n_s = _noalloc_verify(logits, drafts, stream=side)
    assert np.array_equal(t_s, t_o) and np.array_equal(n_s, n_o)


def test_noalloc_greedy_verify_refuses_more_rows_than_its_scratch():
    import torch
    import mtp_draft_verify_amd as mtp
    S, N = mtp.NOALLOC_MAX_ROWS // 4 + 1, 3                 # 4 * S rows > the maximum
    logits = torch.zeros((S, N + 1, 2), dtype=torch.float32, device="cuda")
    drafts = torch.zeros((S, N), dtype=torch.int32, device="cuda")
    toks = torch.full((S, N + 1), -9, dtype=torch.int32, device="cuda")
    na = torch.full((S,), -9, dtype=torch.int32, device="cuda")
    with pytest.raises(mtp.MTPError) as ei:
        mtp.mtp_verify_greedy_noalloc(None, logits, drafts, toks, na)
    assert ei.value.code == mtp.MTP_E_SHAPE
    assert "static scratch" in mtp.mtp_last_error()
    torch.cuda.synchronize()
    assert (toks.cpu().numpy() == -9).all() and (na.cpu().numpy() == -9).all()
