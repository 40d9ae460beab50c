"""GPU parity of the greedy verify from hidden states (through the C ABI)
against the oracle: the target's final RMSNorm, its LM head over the 1 + N
verify rows of every sequence and the argmax, fused ("MTP decoding", why a
wider decode can be faster).

Tokens and accept lengths must match bit for bit, except after a row whose
oracle top-2 margin is below the bf16 logit tolerance (a near tie, counted and
reported separately).
"""
import numpy as np
import pytest

import mtp_synth as syn
from tests.gpu_harness import log

pytestmark = pytest.mark.gpu

NEAR = 2e-2      # bf16 logit tolerance: margins below it are near ties


def _run(ctx, hv, reps=1):
    import torch
    import mtp_draft_verify_amd as mtp
    dev = "cuda"
    w = torch.from_numpy(hv.head.view(np.int16)).to(dev)
    g = torch.from_numpy(hv.g).to(dev) if hv.g is not None else None
    head = mtp.make_lm_head(w, g, hv.d, hv.n_vocab, mtp.MTP_BF16, hv.eps)
    hidden = torch.from_numpy(hv.hidden).to(dev)
    drafts = torch.from_numpy(hv.drafts).to(dev)
    S, R = hv.hidden.shape[:2]
    outs = []
    for _ in range(reps):
        tok = torch.full((S, R), -7, dtype=torch.int32, device=dev)
        na = torch.full((S,), -7, dtype=torch.int32, device=dev)
        ctx.verify_greedy_hidden(head, hidden, drafts, tok, na)
        torch.cuda.synchronize()
        outs.append((tok.cpu().numpy(), na.cpu().numpy()))
    return outs


def _ctx(max_seqs, max_steps):
    import mtp_draft_verify_amd as mtp
    desc = mtp.make_desc(d_model=256, d_hprev=256, n_blocks=1, n_head_q=4, n_head_kv=1, head_dim=64, d_ff=1024,
                         n_vocab=4096, w_dtype=mtp.MTP_F32, head_dtype=mtp.MTP_F32, kv_dtype=mtp.MTP_F32,
                         max_seqs=max_seqs, max_steps=max_steps)
    return mtp.Context(desc, None)


def _compare(hv, tok, na, orc, idx):
    """Bit-exact on every sequence whose rows before the decision have no
    near tie; returns the number of near-tie sequences."""
    sub = syn.HiddenVerifyInputs(hv.d, hv.n_vocab, hv.head_dtype, hv.head, hv.g, hv.eps, hv.hidden[idx],
                                 hv.drafts[idx], hv.planted[idx])
    ot, on, margin = orc.verify_greedy_hidden(sub.hidden, sub.head, sub.head_dtype, sub.n_vocab, sub.g, sub.eps,
                                              sub.drafts)
    near = 0
    for j, s in enumerate(idx):
        a = on[j]
        if (margin[j, :a + 1] < NEAR).any():
            near += 1
            continue
        assert na[s] == a, (s, na[s], a)
        assert tok[s].tolist() == ot[j].tolist(), (s, tok[s], ot[j])
    return near


def test_hidden_verify_full_size_sampled_sequences(orc):
    log("case c8 full: d 2816, V 262144 bf16 head + final-norm gain, 16 seqs x 4 rows (64 rows, one pass); "
        "oracle on 4 sampled sequences")
    w = syn.c8_hidden_verify()
    hv = w.hidden
    ctx = _ctx(16, 3)
    (tok, na), (tok2, na2) = _run(ctx, hv, reps=2)
    assert np.array_equal(tok, tok2) and np.array_equal(na, na2)      # keys are cleared between calls
    near = _compare(hv, tok, na, orc, [0, 5, 10, 15])
    log(f"  accept lengths {na.tolist()}, near-tie sequences {near}")
    assert near <= 1
    # planted rows with a matching draft prefix are accepted as planted
    assert (na >= 0).all() and (na <= 3).all() and na.sum() > 0
    ctx.close()


@pytest.mark.parametrize("S,N,d,V,gain", [
    (3, 2, 256, 20000 - 123, True),      # 9 rows (one row group, ragged), one chunk, ragged vocabulary
    (5, 4, 512, 20000, False),           # 25 rows (two row groups), two chunks, no norm
    (8, 4, 768, 16387, True),            # 40 rows (three row groups)
    (16, 4, 512, 9000, True),            # 80 rows: a 64-row pass and a 16-row pass
    (6, 0, 256, 5000, True),             # no drafts: only the free token
])
def test_hidden_verify_shapes(orc, S, N, d, V, gain):
    log(f"case hidden verify shapes: S={S} N={N} d={d} V={V} gain={gain}")
    hv = syn.make_hidden_verify(17, S, N, d, V, gain=gain, p_accept=0.7)
    ctx = _ctx(16, 4)
    (tok, na), = _run(ctx, hv)
    near = _compare(hv, tok, na, orc, list(range(S)))
    log(f"  accept lengths {na.tolist()}, near-tie sequences {near}")
    assert near <= 1
    ctx.close()


def test_hidden_verify_scratch_grows_with_the_head_width(orc):
    """One context, a narrow head then a wider one (the staging buffer is
    reallocated) then the narrow one again: every call matches the oracle."""
    log("case hidden verify scratch regrowth: d 256 -> 1024 -> 256")
    ctx = _ctx(4, 3)
    for d in (256, 1024, 256):
        hv = syn.make_hidden_verify(5 + d, 4, 3, d, 6000)
        (tok, na), = _run(ctx, hv)
        assert _compare(hv, tok, na, orc, list(range(4))) <= 1
    ctx.close()
