"""GPU parity of the per-step draft confidence and the p_min trim
(mtp_draft_block_conf, through the C ABI) against the oracle.

conf[s, k] is the largest softmax probability of step k's logits.  Both
sides compute it from fp32 logits that agree to the chain's logit tolerance,
so the GPU value must match to a relative 1e-3 (the largest logit error seen
is ~1e-5, which moves conf by that relative amount).  The trim must then give
the same kept prefix and the same -1 tail bit for bit, except for sequences
whose confidence sits within that tolerance of p_min (reported separately).
"""
import numpy as np
import pytest

import mtp_synth as syn
from tests.gpu_harness import GpuDrafter, compare_draft, log

pytestmark = pytest.mark.gpu

CONF_RTOL = 1e-3


def _pick_p_min(conf):
    """Just under the median first-step confidence: at least half of the
    sequences keep their first draft, and later steps (whose confidences
    spread around it) stop at different depths."""
    v = np.sort(conf[:, 0])
    return float(v[len(v) // 2] * 0.99)


def _case(orc, w, max_seqs, max_steps, idx=None):
    g = GpuDrafter(w.model, max_seqs, max_steps)
    o = orc.draft_block(w.model, w.draft, seq_idx=idx)
    plain = g.run(w.draft, seq_idx=idx)
    full = g.run(w.draft, seq_idx=idx, conf=True, p_min=0.0)
    # confidence on or off: identical drafts, logits and h
    for key in ("drafts", "logits", "h_last"):
        assert np.array_equal(plain[key], full[key]), key
    assert (full["n_keep"] == w.draft.n_steps).all()
    c = compare_draft(w.model, full, o)
    S = o["drafts"].shape[0]
    rel = np.abs(full["conf"].astype(np.float64) - o["conf"]) / o["conf"]
    # compare confidence only along each sequence's agreeing prefix
    ok = np.zeros_like(rel, dtype=bool)
    for s in range(S):
        for k in range(o["drafts"].shape[1]):
            ok[s, k] = True
            if full["drafts"][s, k] != o["drafts"][s, k]:
                break
    max_rel = float(rel[ok].max())
    log(f"  {w.name}: conf range [{o['conf'].min():.3g}, {o['conf'].max():.3g}], max rel err {max_rel:.3g}, "
        f"near ties {c.near_ties}")
    assert max_rel <= CONF_RTOL

    p_min = _pick_p_min(o["conf"])
    trimmed = g.run(w.draft, seq_idx=idx, conf=True, p_min=p_min)
    od, keep, near = orc.pmin_trim(o["drafts"], o["conf"], p_min, tol=CONF_RTOL * p_min)
    clean = (near == 0) & np.all(ok, axis=1)
    bad = np.nonzero(clean & ((trimmed["n_keep"] != keep) | np.any(trimmed["drafts"] != od, axis=1)))[0]
    log(f"  p_min {p_min:.3g}: n_keep {trimmed['n_keep'].tolist()}, near-threshold {int((near != 0).sum())}")
    assert len(bad) == 0, (bad, trimmed["n_keep"][bad], keep[bad])
    assert keep.sum() > 0

    none = g.run(w.draft, seq_idx=idx, conf=True, p_min=1.01)
    assert (none["n_keep"] == 0).all() and (none["drafts"] == -1).all()
    g.close()


def test_confidence_tiny_fp32_one_and_several_sequences(orc):
    log("case conf c1: fp32, S=1 and S=3 (wave-reduction head)")
    _case(orc, syn.c1_tiny(), 1, 3)
    _case(orc, syn.c1_tiny(n_seq=3, n_steps=5, ctx=300), 4, 6)


def test_confidence_bf16_full_vocab_one_sequence(orc):
    log("case conf c2: bf16, V=262144, S=1 (wave-reduction head)")
    _case(orc, syn.c2_gemma_bf16(), 1, 3)


def test_confidence_bf16_matrix_core_head(orc):
    log("case conf c3 small: bf16, 16 seqs (matrix-core head)")
    _case(orc, syn.c3_interleaved(ctx_range=(700, 3000), full_cap=3000, n_seq=6), 6, 3)


def test_confidence_q8_0_matrix_core_head(orc):
    log("case conf c4 small: Q8_0 head, 3 seqs, ctx 1500")
    _case(orc, syn.c4_longctx_q8(n_seq=3, ctx=1500), 3, 4)
