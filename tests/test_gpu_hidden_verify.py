"""GPU parity of the verifies from hidden states (through the C ABI) against
the oracle: the target's final RMSNorm and its LM head over the 1 + N verify
rows of every sequence in one pass over the weights ("MTP decoding", why a
wider decode can be faster), then the greedy argmax, or the exact sampling
verify on the logit rows.

Greedy: tokens and accept lengths must match bit for bit, except after a row
whose oracle top-2 margin is below the bf16 logit tolerance (a near tie,
counted and reported separately).  Sampling: sequences whose oracle run
flagged no near-boundary decision must match bit for bit.
"""
import math

import numpy as np
import pytest

import mtp_synth as syn
from tests.gpu_harness import log, record

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


def _ctx(max_seqs, max_steps, n_vocab=4096, d_max=2816, sample=True):
    import mtp_draft_verify_amd as mtp
    desc = mtp.make_desc(d_model=256, d_hprev=256, n_blocks=1, n_head_q=4, n_head_kv=1, head_dim=64, d_ff=1024,
                         n_vocab=n_vocab, w_dtype=mtp.MTP_F32, head_dtype=mtp.MTP_F32, kv_dtype=mtp.MTP_F32,
                         max_seqs=max_seqs, max_steps=max_steps, hidden_d_max=((d_max + 255) // 256) * 256,
                         hidden_sample=int(sample))
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
    record("hidden greedy verify", compared=len(idx) - near, near_ties=near)
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


def test_hidden_verify_scratch_sized_at_create_serves_every_width(orc):
    """One context sized for heads up to 1024 wide: a narrow head, the widest
    one, then the narrow one again all match the oracle (the staging scratch
    is allocated once at create).  A wider head, more sequences or rows than
    the context was sized for, and a sampling call on a context created
    without its logit rows are refused before anything is enqueued: the
    outputs keep their fill."""
    import torch
    import mtp_draft_verify_amd as mtp
    log("case hidden verify scratch sized at create: d 256 -> 1024 -> 256, then refusals")
    ctx = _ctx(4, 3, 6000, d_max=1024, sample=False)
    for d in (256, 1024, 256):
        hv = syn.make_hidden_verify(5 + d, 4, 3, d, 6000)
        (tok, na), = _run(ctx, hv)
        assert _compare(hv, tok, na, orc, list(range(4))) <= 1
    dev = "cuda"
    sp = mtp.make_sampler(temp=0.8, top_p=0.95, min_p=0.05, rep_penalty=1.0, presence_penalty=0.0,
                          penalty_last_n=0, seed=1)
    for d, S, N, sample in ((1280, 4, 3, False), (256, 5, 3, False), (256, 4, 4, False), (256, 4, 3, True)):
        hv = syn.make_hidden_verify(3, S, N, d, 6000)
        w = torch.from_numpy(hv.head.view(np.int16)).to(dev)
        head = mtp.make_lm_head(w, torch.from_numpy(hv.g).to(dev), d, 6000, mtp.MTP_BF16, hv.eps)
        hidden, drafts = torch.from_numpy(hv.hidden).to(dev), torch.from_numpy(hv.drafts).to(dev)
        tok = torch.full((S, N + 1), -7, dtype=torch.int32, device=dev)
        na = torch.full((S,), -7, dtype=torch.int32, device=dev)
        with pytest.raises(mtp.MTPError) as ei:
            if sample:
                ctx.verify_sample_hidden(head, hidden, None, drafts, None, None, sp, 0, tok, na)
            else:
                ctx.verify_greedy_hidden(head, hidden, drafts, tok, na)
        assert ei.value.code == mtp.MTP_E_SHAPE, (d, S, N, sample)
        torch.cuda.synchronize()
        assert (tok.cpu().numpy() == -7).all() and (na.cpu().numpy() == -7).all()
    ctx.close()


# ------------------------------------------------- sampling verify from hidden rows
def _run_sample(ctx, hv, q, history, history_len, sp, round_):
    import torch
    import mtp_draft_verify_amd as mtp
    dev = "cuda"
    w = torch.from_numpy(hv.head.view(np.int16)).to(dev)
    g = torch.from_numpy(hv.g).to(dev) if hv.g is not None else None
    head = mtp.make_lm_head(w, g, hv.d, hv.n_vocab, mtp.MTP_BF16, hv.eps)
    hidden = torch.from_numpy(hv.hidden).to(dev)
    drafts = torch.from_numpy(hv.drafts).to(dev)
    qt = torch.from_numpy(q).to(dev) if q is not None else None
    ht = torch.from_numpy(history).to(dev)
    hl = torch.from_numpy(history_len).to(dev)
    S, R = hv.hidden.shape[:2]
    tok = torch.full((S, R), -7, dtype=torch.int32, device=dev)
    na = torch.full((S,), -7, dtype=torch.int32, device=dev)
    s = mtp.make_sampler(temp=sp.temp, top_p=sp.top_p, min_p=sp.min_p, rep_penalty=sp.rep_penalty,
                         presence_penalty=sp.presence_penalty, freq_penalty=sp.freq_penalty, top_k=sp.top_k,
                         penalty_last_n=sp.penalty_last_n, seed=sp.seed)
    ctx.verify_sample_hidden(head, hidden, qt, drafts, ht, hl, s, round_, tok, na)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), na.cpu().numpy()


def _sample_case(seed, S, N, d, V, gain, one_hot):
    """Target rows with a moderately planted token (beta 0.25), drafts mostly
    the planted tokens, q rows N(0, 6) (or one-hot), 40-token histories of
    varied length.  (Broader rows put the top-p cut deep in the tail, where
    the oracle flags a near-boundary decision for a large share of the
    sequences; the candidate forms of broad rows are covered by the logit-row
    sampling tests.)"""
    hv = syn.make_hidden_verify(seed, S, N, d, V, gain=gain, beta=0.25, p_accept=0.7)
    r = np.random.default_rng(seed)
    q = None if one_hot else (math.sqrt(6.0) * r.standard_normal((S, N, V))).astype(np.float32)
    history = r.integers(0, V, (S, 40)).astype(np.int32)
    history_len = r.integers(0, 41, S).astype(np.int32)
    return hv, q, history, history_len


SAMPLER = syn.Sampler(temp=0.8, top_p=0.95, min_p=0.05, rep_penalty=1.05, presence_penalty=0.2, freq_penalty=0.0,
                      top_k=0, penalty_last_n=32, seed=7)


def _compare_sample(orc, ctx, hv, q, history, history_len, sp, round_):
    """Unflagged sequences (no near-boundary decision in the oracle run) must
    match bit for bit, and at most 10% may be flagged; the logits differ from
    the oracle's by fp32 rounding, far inside the flags' 1e-5 windows.
    Returns the flagged count."""
    t_o, n_o, fl = orc.verify_sample_hidden(hv.hidden, hv.head, hv.head_dtype, hv.n_vocab, hv.g, hv.eps, q,
                                            hv.drafts, history, history_len, sp, round_)
    t_g, n_g = _run_sample(ctx, hv, q, history, history_len, sp, round_)
    clean = fl == 0
    bad = np.nonzero(clean & ((n_g != n_o) | np.any(t_g != t_o, axis=1)))[0]
    log(f"  S={len(fl)} flagged={int((~clean).sum())} accept_mean={n_o.mean():.3f} mismatches_on_clean={len(bad)}")
    record(f"hidden sampling verify round {round_}", compared=int(clean.sum()), flagged=int((~clean).sum()),
           mismatches_on_clean=len(bad))
    assert len(bad) == 0, (bad[:5], t_g[bad[:3]], t_o[bad[:3]], n_g[bad[:3]], n_o[bad[:3]])
    assert (t_g[:, 0] >= 0).all() and (n_g >= 0).all()
    assert (~clean).mean() <= 0.1
    return int((~clean).sum())


@pytest.mark.parametrize("S,N,d,V,gain,one_hot", [
    (6, 3, 256, 20000 - 123, True, False),      # 24 rows, ragged vocabulary, q rows
    (8, 4, 512, 9000, False, True),             # 40 rows, no norm, one-hot drafts
    (16, 4, 768, 16387, True, False),           # 80 rows: a 64-row pass and a 16-row pass
    (5, 0, 256, 5000, True, True),              # no drafts: only the bonus token
])
def test_hidden_sampling_verify_shapes(orc, S, N, d, V, gain, one_hot):
    log(f"case hidden sampling verify: S={S} N={N} d={d} V={V} gain={gain} one_hot={one_hot}")
    hv, q, history, history_len = _sample_case(31 + d, S, N, d, V, gain, one_hot)
    ctx = _ctx(16, 4, V)
    for rd in (0, 5):
        _compare_sample(orc, ctx, hv, q, history, history_len, SAMPLER, rd)
    ctx.close()


def test_hidden_sampling_verify_full_width(orc):
    """The c8 head shape (d 2816, V 262144, bf16, gain) on 4 sequences x 4 rows."""
    log("case hidden sampling verify full width: d 2816, V 262144, 4 seqs x 4 rows")
    hv, q, history, history_len = _sample_case(77, 4, 3, 2816, 262144, True, False)
    ctx = _ctx(4, 3, 262144)
    _compare_sample(orc, ctx, hv, q, history, history_len, SAMPLER, 2)
    ctx.close()


def test_hidden_sampling_then_greedy_reuses_the_context(orc):
    """A sampling verify from hidden rows leaves no state behind: a greedy one
    on the same context right after still matches the oracle."""
    log("case hidden sampling then greedy on one context")
    ctx = _ctx(8, 3, 7000)
    hv, q, history, history_len = _sample_case(5, 8, 3, 512, 7000, True, False)
    _compare_sample(orc, ctx, hv, q, history, history_len, SAMPLER, 0)
    hv2 = syn.make_hidden_verify(9, 8, 3, 512, 7000, p_accept=0.7)
    (tok, na), = _run(ctx, hv2)
    assert _compare(hv2, tok, na, orc, list(range(8))) <= 1
    ctx.close()
