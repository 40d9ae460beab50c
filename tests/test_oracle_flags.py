"""Pins of the oracle's near-boundary flags in the exact sampling verify
("opus-mtp-turbo: Track 1 report" s.4: the sampling chain and the accept /
resample rule).

Every integer decision of the sampling verify (a min-p keep, the top-p cut,
the accept test, the Gumbel-max draw, the top-k cut) is taken in fp32 on the
GPU and in fp64-then-fp32 by the oracle.  Where the two could round to
different sides, the oracle flags the sequence and the parity tests compare
it separately.  A flag that fired too broadly would hollow those tests out; one
that fired too narrowly would let a rounding difference fail them.  So each
flag is pinned here with hand-built rows that put its decision just inside
(half the window) and just outside (twice the window) its window, on both
sides of the threshold, with operands chosen so that a wrong threshold or a
wrong operand (the token's probability instead of its ratio to the row
maximum, p instead of max(p, q), the wrong Gumbel error terms) changes the
outcome of at least one case.

Windows (the oracle's own definitions):
  min-p   |pi_t / pi_max - min_p| <= 1e-5 * min_p
  top-p   |cum - top_p| <= 1e-5 at the crossing token, or the same for the
          cumulative sum just before it
  accept  |u * q(d) - p(d)| < 1e-5 * max(p(d), q(d))
  Gumbel  best key - second key <= err_best + err_second, with
          err_t = 4e-6 * (e_t / w_t) + 4e-6 * (1 + |g_t| + |ln w_t|),
          g_t = -ln(-ln U_t), w the draw's weights and e their error scale
          (e = 2p for a draw from p)
  top-k   the k-th and (k+1)-th raw logits are equal
"""
import math

import numpy as np
import pytest

import mtp_synth as syn

NEAR_MINP, NEAR_TOPP, NEAR_ACCEPT, NEAR_GUMBEL, NEAR_TOPK = 1, 2, 4, 8, 16
STREAM_ACCEPT, STREAM_RESIDUAL, STREAM_BONUS = 0, 1, 2


def _sp(**kw):
    base = dict(temp=1.0, top_p=1.0, min_p=0.0, rep_penalty=1.0, presence_penalty=0.0, freq_penalty=0.0, top_k=0,
                penalty_last_n=0, seed=1)
    base.update(kw)
    return syn.Sampler(**base)


def _f32(x):
    return np.asarray(x, np.float64).astype(np.float32)


# half / twice the window, and 0.9 / 1.1 of it (a threshold or a term off by
# more than about 10% fails one of the tight pairs); placements through fp32
# logits are exact to about 1% of a window
FRACS = [(0.5, True), (-0.5, True), (2.0, False), (-2.0, False), (0.9, True), (-0.9, True), (1.1, False),
         (-1.1, False)]


@pytest.mark.parametrize("frac,flagged", FRACS)
def test_min_p_flag_window(orc, frac, flagged):
    """Token 2's ratio to the row maximum (token 1) sits at
    min_p * (1 + delta).  Three tokens, so that its probability (about
    0.026) is far from its ratio (0.05): a flag computed on the probability
    would never fire here."""
    min_p = 0.05
    delta = frac * 1e-5
    z = _f32([math.log(0.3), 0.0, math.log(min_p * (1 + delta))])
    ratio = math.exp(float(z[2]) - float(z[1]))
    assert abs((ratio / min_p - 1) / 1e-5 - frac) < 0.02          # fp32 logits keep the placement
    p, fl = orc.sample_dist(z, [], _sp(min_p=min_p))
    assert bool(fl & NEAR_MINP) == flagged, (delta, fl)
    assert fl & ~NEAR_MINP == 0
    assert (p[2] > 0) == (delta > 0)                                # the keep decision itself


def _two_token_row(a):
    """fp32 logits of the distribution (a, 1 - a) and the probability of
    token 0 they realise."""
    z = _f32([math.log(a), math.log(1 - a)])
    e = np.exp(z.astype(np.float64) - z.max())
    return z, float(e[0] / e.sum())


@pytest.mark.parametrize("frac,flagged", FRACS)
def test_top_p_flag_window(orc, frac, flagged):
    """top_p = a - frac * 1e-5: for frac > 0 the crossing is token 0 with
    cum = a just above top_p (one token kept); for frac < 0 it is token 1,
    with the sum before it (a) just below top_p (both kept)."""
    z, a = _two_token_row(0.7)
    top_p = a - frac * 1e-5
    kept = 1 if frac > 0 else 2
    p, fl = orc.sample_dist(z, [], _sp(top_p=top_p))
    assert bool(fl & NEAR_TOPP) == flagged, (frac, fl)
    assert fl & ~NEAR_TOPP == 0
    assert int((p > 0).sum()) == kept


def _accept_case(orc, pf_target, q_row=None, seed=11):
    """One sequence, one draft (token 0), V = 2: returns (flags, n_accept)
    of the exact verify whose p row gives the draft probability pf_target."""
    z, pf = _two_token_row(pf_target)
    p_logits = np.stack([z, _f32([0.0, 0.0])])[None]              # [1, 2, 2]: draft row, bonus row
    q = None if q_row is None else q_row[None, None].astype(np.float32)
    t, n, fl = orc.verify_sample(p_logits, q, np.zeros((1, 1), np.int32), np.zeros((1, 0), np.int32),
                                 np.zeros(1, np.int32), _sp(seed=seed), 0)
    return int(fl[0]), int(n[0]), pf


def _seed_with_uniform_in(orc, lo, hi):
    for seed in range(1, 1000):
        u = orc.uniform(seed, 0, 0, 0, STREAM_ACCEPT, 0)
        if lo < u < hi:
            return seed, u
    raise AssertionError("no seed")


@pytest.mark.parametrize("k,flagged", FRACS)
def test_accept_flag_window_one_hot(orc, k, flagged):
    """q one-hot at the draft: the test is u < p(d); the window is 1e-5 *
    max(p, 1) = 1e-5 around u."""
    seed, u = _seed_with_uniform_in(orc, 0.3, 0.7)
    fl, n, pf = _accept_case(orc, u + k * 1e-5, seed=seed)
    assert abs((pf - u) / 1e-5 - k) < 0.02
    assert bool(fl & NEAR_ACCEPT) == flagged, (k, fl)
    assert n == (1 if k > 0 else 0)


@pytest.mark.parametrize("k,flagged", FRACS)
def test_accept_flag_window_uses_the_larger_of_p_and_q(orc, k, flagged):
    """A general q with q(d) = b = 0.9 and p(d) = u * b + k * 1e-5 * b: the
    window is 1e-5 * max(p, q) = 1e-5 * b.  With u below 0.3 the distance
    |u q - p| = |k| 1e-5 b lies outside a window taken on p alone
    (1e-5 * p < 0.3e-5 b) in the k = +-0.5 cases, which must still flag."""
    seed, u = _seed_with_uniform_in(orc, 0.15, 0.3)
    b = 0.9
    q_row = _f32([math.log(b), math.log(1 - b)])
    qb = float(np.exp(q_row[0]) / np.exp(q_row.astype(np.float64)).sum())
    target = u * qb + k * 1e-5 * qb
    fl, n, pf = _accept_case(orc, target, q_row=q_row, seed=seed)
    assert abs((pf - u * qb) / (1e-5 * qb) - k) < 0.02
    assert pf < 0.3 * qb + 1e-4                       # p(d) < 0.3 q(d): the max is q's
    assert bool(fl & NEAR_ACCEPT) == flagged, (k, fl)
    assert n == (1 if k > 0 else 0)


def _gumbel_bound(p, g):
    """err_0 + err_1 of the oracle's Gumbel draw from w = p, e = 2p."""
    return sum(4e-6 * 2.0 + 4e-6 * (1.0 + abs(g[t]) + abs(math.log(p[t]))) for t in range(2))


@pytest.mark.parametrize("frac,flagged", FRACS)
def test_gumbel_flag_window(orc, frac, flagged):
    """Bonus draw (no drafts) from p = (a, 1 - a): keys ln p_t + g_t with
    g_t = -ln(-ln U(seed, 0, 0, 0, bonus, t)).  a is solved so that key 0 -
    key 1 = frac * (err_0 + err_1); the draw is flagged iff |gap| is within
    the bound, and token 0 wins iff the gap is positive."""
    seed = 5
    g = [-math.log(-math.log(orc.uniform(seed, 0, 0, 0, STREAM_BONUS, t))) for t in range(2)]
    a = 0.5
    for _ in range(8):                       # the bound depends (weakly) on a
        bound = _gumbel_bound([a, 1 - a], g)
        x = frac * bound + g[1] - g[0]       # ln a - ln(1 - a)
        a = 1.0 / (1.0 + math.exp(-x))
    z, a_real = _two_token_row(a)
    gap = (math.log(a_real) + g[0]) - (math.log(1 - a_real) + g[1])
    bound = _gumbel_bound([a_real, 1 - a_real], g)
    assert abs(gap / bound - frac) < 0.02, (gap, bound)
    t, n, fl = orc.verify_sample(z[None, None], None, np.zeros((1, 0), np.int32), np.zeros((1, 0), np.int32),
                                 np.zeros(1, np.int32), _sp(seed=seed), 0)
    assert bool(fl[0] & NEAR_GUMBEL) == flagged, (frac, fl)
    assert t[0, 0] == (0 if frac > 0 else 1)


@pytest.mark.parametrize("z,flagged", [([3.0, 2.0, 2.0, 1.0], True), ([3.0, 2.0, 1.99999, 1.0], False),
                                       ([2.0, 3.0, 1.0, 2.0], True), ([3.0, 3.0, 3.0, 1.0], True)])
def test_top_k_flag_fires_on_a_tie_at_the_cut(orc, z, flagged):
    """top_k = 2: flagged exactly when the 2nd and 3rd largest raw logits
    are equal (the cut then depends on the tie order)."""
    p, fl = orc.sample_dist(_f32(z), [], _sp(top_k=2))
    assert bool(fl & NEAR_TOPK) == flagged, (z, fl)
    assert int((p > 0).sum()) == 2


def test_well_separated_rows_raise_no_flag(orc):
    """Rows whose every decision is far from its threshold raise no flag at
    all, through the whole verify (penalties, min-p, top-p, accept test,
    residual draw)."""
    V = 8
    z = _f32([4.0, 1.0, 0.0, -1.0, -3.0, 2.0, 0.5, -2.0])
    p_logits = np.tile(z, (3, 3, 1)).astype(np.float32)
    drafts = np.array([[0, 5], [5, 0], [7, 7]], np.int32)
    hist = np.array([[1, 2], [3, 3], [6, 1]], np.int32)
    sp = _sp(temp=0.8, min_p=0.01, top_p=0.9, rep_penalty=1.1, presence_penalty=0.3, penalty_last_n=4, seed=3)
    t, n, fl = orc.verify_sample(p_logits, None, drafts, hist, np.full(3, 2, np.int32), sp, 0)
    assert (fl == 0).all(), fl
    assert (t[:, 0] >= 0).all() and (t[:, 0] < V).all()
