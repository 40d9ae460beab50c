"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against a closed form, a special case with a
textbook answer, a published test vector, or an invariant the pages state --
never against a second copy of the oracle's own formula.  Together they make
a dropped term, a wrong sign, a wrong index or a transposed operand in any
oracle function fail somewhere.
"""
import math
from pathlib import Path

import numpy as np
import pytest

import mtp_synth as syn
from tests import toys

GOLDEN = Path(__file__).resolve().parent / "golden"


# ---------------------------------------------------------------- RNG ------
def test_splitmix64_reference_outputs(orc):
    """SplitMix64 (Steele, Lea & Flood 2014): published reference outputs."""
    for line in (GOLDEN / "splitmix64.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        vals = [int(v) for v in line.split()]
        state, n, expect = vals[0], vals[1], vals[2:]
        assert orc.splitmix64_stream(state, n) == expect


def test_uniform_is_open_unit_interval_fp32_exact_and_uniform(orc):
    us = np.array([orc.uniform(7, s, 3, 1, 0, t) for s in range(40) for t in range(500)], np.float64)
    assert us.min() > 0.0 and us.max() < 1.0
    # (k + 1/2) / 2^23 is exact in fp32
    k = us * 2 ** 23 - 0.5
    assert np.all(k == np.round(k))
    # chi-square over 20 equal bins, 20000 draws: 99.99th percentile of chi2(19) ~ 50
    counts, _ = np.histogram(us, bins=20, range=(0, 1))
    exp = us.size / 20
    assert ((counts - exp) ** 2 / exp).sum() < 50
    # every coordinate matters
    base = orc.rng_u64(1, 2, 3, 4, 5, 6)
    for alt in [(9, 2, 3, 4, 5, 6), (1, 9, 3, 4, 5, 6), (1, 2, 9, 4, 5, 6), (1, 2, 3, 9, 5, 6), (1, 2, 3, 4, 9, 6),
                (1, 2, 3, 4, 5, 9)]:
        assert orc.rng_u64(*alt) != base


# ------------------------------------------------------- storage formats ---
def test_load_bf16_f32_and_q8_0_blocks(orc):
    bf = np.array([0x3F80, 0xC000, 0x3E20, 0x0000], np.uint16)     # 1, -2, 0.15625, 0
    assert [orc.load(bf, syn.BF16, 0, c, 4) for c in range(4)] == [1.0, -2.0, 0.15625, 0.0]
    f = np.array([[1.5, -3.25], [7.0, 0.5]], np.float32)
    assert orc.load(f, syn.F32, 1, 0, 2) == 7.0
    # Q8_0: fp16 scale 0.5 (0x3800, little endian) then 32 int8 values
    q = np.zeros(32, np.int8)
    q[:5] = [1, -1, 127, -127, 3]
    blk1 = np.concatenate([np.array([0x00, 0x38], np.uint8), q.view(np.uint8)])
    blk2 = np.concatenate([np.array([0x00, 0x3C], np.uint8), np.arange(32, dtype=np.int8).view(np.uint8)])  # scale 1
    row = np.concatenate([blk1, blk2])          # one row of 64 values
    vals = [orc.load(row, syn.Q8_0, 0, c, 64) for c in range(64)]
    assert vals[:5] == [0.5, -0.5, 63.5, -63.5, 1.5]
    assert vals[32:] == list(map(float, range(32)))


def test_q8_0_gemv_error_matches_published_magnitude(orc):
    """Q8_0 GEMV rel-RMSE on Gaussian x is a fraction of a percent (the audit
    page measures 0.58-1.18% on heavier-tailed real tensors; Gaussian weights
    give about 0.47%: step max|x|/127, uniform rounding error)."""
    rows, cols = 48, 1024
    w = syn.normal(11, "q8test", (rows, cols), 1 / 32)
    blocks = syn.q8_0_blocks(w)
    deq = np.array([[orc.load(blocks, syn.Q8_0, r, c, cols) for c in range(cols)] for r in range(rows)])
    x = syn.normal(12, "q8x", (cols, 16)).astype(np.float64)
    y, yq = w.astype(np.float64) @ x, deq @ x
    rel = math.sqrt(np.mean((yq - y) ** 2) / np.mean(y ** 2))
    assert 0.003 < rel < 0.007, rel


# ------------------------------------------------------- building blocks --
def test_rmsnorm_closed_forms(orc):
    eps = 1e-6
    g = np.array([1.0, 2.0], np.float32)
    y = orc.rmsnorm([3.0, 4.0], g, eps)         # mean(x^2) = 12.5
    np.testing.assert_allclose(y, np.array([3.0, 8.0]) / math.sqrt(12.5 + eps), rtol=1e-15)
    c = -0.01
    y = orc.rmsnorm(np.full(5, c), np.ones(5, np.float32), 1e-4)
    np.testing.assert_allclose(y, np.full(5, -1.0 / math.sqrt(1 + 1e-4 / c ** 2)), rtol=1e-15)


def test_rope_closed_forms(orc):
    x = np.array([0.3, -1.2, 0.7, 2.0])
    np.testing.assert_array_equal(orc.rope(x, 0), x)                   # position 0 = identity
    # hd = 2: one pair rotated by pos * theta^0 = pos radians
    y = orc.rope([1.0, 0.0], 1)
    np.testing.assert_allclose(y, [math.cos(1.0), math.sin(1.0)], rtol=1e-15)
    # hd = 4, theta = 10000: pairs (0,2) at 1 rad/pos and (1,3) at 10000^-1/2 = 0.01 rad/pos
    y = orc.rope([1.0, 1.0, 0.0, 0.0], 5)
    np.testing.assert_allclose(y, [math.cos(5), math.cos(0.05), math.sin(5), math.sin(0.05)], rtol=1e-14)
    # rotation: norm kept; scores depend on relative position only
    r = np.random.default_rng(0)
    q, k = r.standard_normal(8), r.standard_normal(8)
    assert abs(np.linalg.norm(orc.rope(q, 12345)) - np.linalg.norm(q)) < 1e-12
    a = orc.rope(q, 100) @ orc.rope(k, 90)
    b = orc.rope(q, 1010) @ orc.rope(k, 1000)
    assert abs(a - b) < 1e-11


def _attn_model(Hq=4, Hkv=2, hd=4, swa=0):
    return toys.blank_model(Hq=Hq, Hkv=Hkv, hd=hd, swa_window=swa)


def _seq(m, k, v, attn_pos, src=syn.KV_FULL, run_lo=0):
    kv = syn.KVSource(np.ascontiguousarray(k, np.float32), np.ascontiguousarray(v, np.float32))
    srcs = [None, None, None]
    srcs[src] = kv
    return syn.Seq(srcs, attn_pos=attn_pos, pos0=attn_pos + 1, run_lo=run_lo)


def test_attention_one_visible_cell_returns_its_value_row(orc):
    m = _attn_model()
    r = np.random.default_rng(1)
    k, v = r.standard_normal((6, 2, 4)), r.standard_normal((6, 2, 4))
    k[1:], v[1:] = np.nan, np.nan                 # cells past attn_pos are never read
    o = orc.attend_group(m, _seq(m, k, v, 0), syn.KV_FULL, 1, r.standard_normal((2, 4)))
    np.testing.assert_array_equal(o, np.tile(v[0, 1].astype(np.float32), (2, 1)))


def test_attention_equal_keys_or_zero_query_average_the_values(orc):
    m = _attn_model()
    r = np.random.default_rng(2)
    n = 37
    k = np.tile(r.standard_normal((1, 2, 4)), (n, 1, 1))
    v = r.standard_normal((n, 2, 4)).astype(np.float32)
    o = orc.attend_group(m, _seq(m, k, v, n - 1), syn.KV_FULL, 0, r.standard_normal((2, 4)))
    np.testing.assert_allclose(o, np.tile(v[:, 0].astype(np.float64).mean(0), (2, 1)), rtol=1e-12)
    k = r.standard_normal((n, 2, 4))
    o = orc.attend_group(m, _seq(m, k, v, 20), syn.KV_FULL, 1, np.zeros((2, 4)))
    np.testing.assert_allclose(o[0], v[:21, 1].astype(np.float64).mean(0), rtol=1e-12)


def test_sink_window_visible_cells_hand_cases(orc):
    """Sink + window source ("opus-mtp-turbo" report s.2): the draft attends to
    [0 .. min(sink, first) - 1] ++ [first .. attn_pos] with first moved up to
    the valid run's start; short contexts give one contiguous run, no cell
    twice."""
    m = _attn_model()
    m.sw_window, m.sw_sink = 256, 64
    k = np.zeros((1200, 2, 4))
    def cells(attn_pos, run_lo=0, sink=64):
        m.sw_sink = sink
        return orc.visible_cells(m, _seq(m, k, k, attn_pos, syn.KV_SINK_WINDOW, run_lo), syn.KV_SINK_WINDOW).tolist()
    assert cells(1000) == list(range(64)) + list(range(745, 1001))
    assert cells(1000, run_lo=900) == list(range(64)) + list(range(900, 1001))
    assert cells(1000, run_lo=10) == list(range(64)) + list(range(745, 1001))
    assert cells(100) == list(range(101))
    assert cells(300) == list(range(301))
    assert cells(1000, sink=0) == list(range(745, 1001))
    assert cells(1000, run_lo=20, sink=64) == list(range(64)) + list(range(745, 1001))
    assert cells(200, run_lo=150) == list(range(64)) + list(range(150, 201))
    # the page's own list: window [cell0 - 256, cell0] (W = 257 cells) and
    # sink 64 give at most 64 + 257 = 321 cells
    m.sw_window = 257
    assert cells(1000) == list(range(64)) + list(range(744, 1001))
    assert len(cells(1000)) == 321


def test_sink_window_equal_keys_average_exactly_the_visible_values(orc):
    """Equal keys give uniform weights: the output is the mean of the value
    rows of the sink and the window, and stale cells (NaN) are never read."""
    m = _attn_model()
    m.sw_window, m.sw_sink = 16, 4
    r = np.random.default_rng(9)
    n = 64
    k = np.tile(r.standard_normal((1, 2, 4)), (n, 1, 1))
    v = r.standard_normal((n, 2, 4)).astype(np.float32)
    k[4:40], v[4:40] = np.nan, np.nan           # between the sink and the valid run: stale
    k[51:], v[51:] = np.nan, np.nan             # past attn_pos
    o = orc.attend_group(m, _seq(m, k, v, 50, syn.KV_SINK_WINDOW, run_lo=40), syn.KV_SINK_WINDOW, 1,
                         r.standard_normal((2, 4)))
    want = np.concatenate([v[0:4, 1], v[40:51, 1]]).astype(np.float64).mean(0)
    np.testing.assert_allclose(o, np.tile(want, (2, 1)), rtol=1e-12)


def test_sink_window_without_sink_equals_a_sliding_window_ring(orc):
    """With no sink and no stale cells, a sink + window block over a full cache
    attends to the same positions as an SWA block over a ring of capacity W
    holding them (cell p mod W): the chains agree bit for bit."""
    W, ctx = 8, 21
    m = toys.blank_model(d=8, dh=8, V=16, swa_window=W, block_src=[syn.KV_SWA])
    m.sw_window, m.sw_sink = W, 0
    r = np.random.default_rng(4)
    k = r.standard_normal((ctx, m.n_head_kv, m.head_dim)).astype(np.float32)
    v = r.standard_normal((ctx, m.n_head_kv, m.head_dim)).astype(np.float32)
    ring_k, ring_v = np.zeros((W,) + k.shape[1:], np.float32), np.zeros((W,) + v.shape[1:], np.float32)
    for p in range(ctx):
        ring_k[p % W], ring_v[p % W] = k[p], v[p]
    lt, hp = np.array([3], np.int32), r.standard_normal((1, 8)).astype(np.float32)
    swa = syn.DraftInputs([syn.Seq([None, syn.KVSource(ring_k, ring_v), None], ctx - 1, ctx)], lt, hp, 3)
    a = orc.draft_block(m, swa)
    m.block_src = [syn.KV_SINK_WINDOW]
    sw = syn.DraftInputs([syn.Seq([None, None, syn.KVSource(k, v)], ctx - 1, ctx)], lt, hp, 3)
    b = orc.draft_block(m, sw)
    for key in ("drafts", "logits", "h_last"):
        assert np.array_equal(a[key], b[key]), key


def test_attention_two_cells_logistic_weights_and_scale(orc):
    """o = sigma(delta) v1 + (1-sigma(delta)) v0, delta = scale * q.(k1-k0)."""
    m = _attn_model(Hq=1, Hkv=1, hd=4)
    k = np.array([[[1.0, 0, 0, 0]], [[0, 2.0, 0, 0]]], np.float32)
    v = np.array([[[1.0, 0, 0, 0]], [[0, 0, 0, 3.0]]], np.float32)
    q = np.array([[0.5, 1.5, 0, 0]])
    delta = (1.5 * 2.0 - 0.5 * 1.0) * (1 / math.sqrt(4))
    w1 = 1 / (1 + math.exp(-delta))
    o = orc.attend_group(m, _seq(m, k, v, 1), syn.KV_FULL, 0, q)
    np.testing.assert_allclose(o[0], [1 - w1, 0, 0, 3 * w1], rtol=1e-14)


def test_attention_gqa_head_to_kv_head_mapping(orc):
    """query head h reads kv head h // (Hq/Hkv): with Hq=4, Hkv=2 heads 2,3
    read kv head 1 (one cell, so the output is that head's V row)."""
    m = _attn_model(Hq=4, Hkv=2, hd=4)
    k = np.zeros((1, 2, 4), np.float32)
    v = np.array([[[1, 1, 1, 1], [7, 7, 7, 7]]], np.float32)
    seq = _seq(m, k, v, 0)
    q = np.ones((2, 4))
    assert np.all(orc.attend_group(m, seq, syn.KV_FULL, 0, q) == 1.0)
    assert np.all(orc.attend_group(m, seq, syn.KV_FULL, 1, q) == 7.0)


def test_attention_swa_ring_reads_exactly_the_window(orc):
    """SWA source: position p lives at ring cell p mod C, visible positions
    are the last W up to attn_pos.  Poisoning every other cell changes
    nothing, and the result equals a full source holding the same window."""
    W, C = 5, 8
    m = _attn_model(Hq=2, Hkv=1, hd=4, swa=W)
    r = np.random.default_rng(3)
    attn_pos = 21                                   # window positions 17..21
    k = np.full((C, 1, 4), np.nan, np.float32)
    v = np.full((C, 1, 4), np.nan, np.float32)
    dense_k = r.standard_normal((W, 1, 4)).astype(np.float32)
    dense_v = r.standard_normal((W, 1, 4)).astype(np.float32)
    for j, p in enumerate(range(attn_pos - W + 1, attn_pos + 1)):
        k[p % C], v[p % C] = dense_k[j], dense_v[j]
    q = r.standard_normal((2, 4))
    o_swa = orc.attend_group(m, _seq(m, k, v, attn_pos, syn.KV_SWA), syn.KV_SWA, 0, q)
    o_full = orc.attend_group(m, _seq(m, dense_k, dense_v, W - 1), syn.KV_FULL, 0, q)
    assert np.all(np.isfinite(o_swa))
    np.testing.assert_allclose(o_swa, o_full, rtol=1e-13)
    # early in the sequence the window is clipped at position 0
    k2, v2 = np.full((C, 1, 4), np.nan, np.float32), np.full((C, 1, 4), np.nan, np.float32)
    k2[:3], v2[:3] = dense_k[:3], dense_v[:3]
    o = orc.attend_group(m, _seq(m, k2, v2, 2, syn.KV_SWA), syn.KV_SWA, 0, np.zeros((2, 4)))
    np.testing.assert_allclose(o[0], dense_v[:3, 0].astype(np.float64).mean(0), rtol=1e-13)


def test_argmax_ties_and_margin(orc):
    assert orc.argmax_f32([1.0, 3.0, 3.0, 2.0]) == (1, 0.0)
    assert orc.argmax_f32([-5.0]) [0] == 0
    r = np.random.default_rng(4)
    for _ in range(50):
        z = r.standard_normal(257).astype(np.float32)
        i, mg = orc.argmax_f32(z)
        order = sorted(range(z.size), key=lambda t: (-z[t], t))      # brute force full sort
        assert i == order[0]
        assert mg == pytest.approx(float(z[order[0]]) - float(z[order[1]]), abs=0)


# ------------------------------------------------- whole-chain closed forms -
def test_chain_embedding_path_follows_a_permutation(orc):
    """W_pre = [P | 0], tied head E = a*I, blocks silent: step k's input is
    embed_scale * E[tok] (the target's token embedding scaled by sqrt(d), Gemma 4
    MTP doc s.4), the pre-projection maps e_t to e_P(t), and the in-graph
    argmax feeds the next step.  Drafts = P(t), P^2(t), P^3(t); logits have a
    closed form."""
    d = V = dh = 8
    m = toys.blank_model(d=d, dh=dh, V=V)
    toys.zero_blocks(m)
    perm = [3, 6, 0, 7, 1, 2, 5, 4]                 # no fixed points, not an involution
    a = 0.5
    m.weights["head"] = (a * np.eye(V, d)).astype(np.float32)
    m.weights["w_pre"] = np.concatenate([toys.perm_matrix(perm), np.zeros((d, dh), np.float32)], 1)
    m.weights["w_post"] = np.eye(dh, d, dtype=np.float32)
    g = m.weights["g_final"]
    dr = toys.one_seq_inputs(m, 4, 3, last_tok=2, h_prev=np.ones(dh), n_steps=3)
    out = orc.draft_block(m, dr)
    t, exp_drafts = 2, []
    for k in range(3):
        t = perm[t]
        exp_drafts.append(t)
        xval = math.sqrt(d) * a                     # x = sqrt(d) * a * e_t
        fval = xval * toys.rms_scale(np.eye(d)[t] * xval, m.rms_eps) * g[t]
        z = np.zeros(V)
        z[t] = a * fval
        np.testing.assert_allclose(out["logits"][0, k], z.astype(np.float32), rtol=2e-7, atol=0)
    assert out["drafts"][0].tolist() == exp_drafts
    np.testing.assert_allclose(out["h_last"][0], np.eye(d)[t] * fval, rtol=2e-7)


def test_draft_confidence_closed_forms(orc):
    """The draft confidence is the largest softmax probability of the step's
    logit row ("MTP decoding", stopping early when the head is unsure):
    three tokens with weights 1:2:3 give 3/6; a flat row gives 1/V; two
    tokens a gap g apart give the logistic 1/(1 + e^-g)."""
    z = np.log(np.array([1.0, 2.0, 3.0])).astype(np.float32)
    assert abs(orc.confidence(z) - 0.5) < 1e-7
    for V in (1, 7, 262144):
        assert orc.confidence(np.full(V, -3.25, np.float32)) == 1.0 / V
    for g in (0.0, 0.5, 4.0, 30.0):
        z = np.array([1.0, 1.0 + g], np.float32)
        assert abs(orc.confidence(z) - 1.0 / (1.0 + math.exp(-g))) < 1e-7
    # shift invariance: adding a constant to every logit changes nothing
    r = np.random.default_rng(5).standard_normal(1000).astype(np.float32)
    assert abs(orc.confidence(r) - orc.confidence(r + np.float32(8.0))) < 1e-6


def test_pmin_trim_hand_cases(orc):
    """Drafting stops at the first step whose confidence is below p_min and
    that step is not proposed; p_min = 0 never stops; p_min above 1 keeps
    nothing."""
    d = np.array([[11, 12, 13], [21, 22, 23], [31, 32, 33]], np.int32)
    c = np.array([[0.9, 0.5, 0.95], [0.7, 0.8, 0.9], [0.2, 0.99, 0.99]])
    t, keep, _ = orc.pmin_trim(d, c, 0.6)
    assert keep.tolist() == [1, 3, 0]
    assert t.tolist() == [[11, -1, -1], [21, 22, 23], [-1, -1, -1]]
    t, keep, _ = orc.pmin_trim(d, c, 0.0)
    assert keep.tolist() == [3, 3, 3] and np.array_equal(t, d)
    t, keep, _ = orc.pmin_trim(d, c, 1.01)
    assert keep.tolist() == [0, 0, 0] and (t == -1).all()
    # equality keeps the step (stops only strictly below)
    _, keep, near = orc.pmin_trim(d, c, 0.7, tol=1e-9)
    assert keep.tolist() == [1, 3, 0] and near.tolist() == [0, 1, 0]


def test_chain_confidence_of_a_one_hot_logit_row(orc):
    """Permutation drafter of the embedding-path pin: every step's logits are
    a single value z* at the draft token and 0 elsewhere, so the confidence
    is 1 / (1 + (V-1) e^-z*); a zero head gives 1/V at every step."""
    d = V = dh = 8
    m = toys.blank_model(d=d, dh=dh, V=V)
    toys.zero_blocks(m)
    perm = [3, 6, 0, 7, 1, 2, 5, 4]
    a = 0.5
    m.weights["head"] = (a * np.eye(V, d)).astype(np.float32)
    m.weights["w_pre"] = np.concatenate([toys.perm_matrix(perm), np.zeros((d, dh), np.float32)], 1)
    m.weights["w_post"] = np.eye(dh, d, dtype=np.float32)
    g = m.weights["g_final"]
    dr = toys.one_seq_inputs(m, 4, 3, last_tok=2, h_prev=np.ones(dh), n_steps=3)
    out = orc.draft_block(m, dr)
    t = 2
    for k in range(3):
        t = perm[t]
        xval = math.sqrt(d) * a
        zstar = float(np.float32(a * xval * toys.rms_scale(np.eye(d)[t] * xval, m.rms_eps) * g[t]))
        assert abs(out["conf"][0, k] - 1.0 / (1.0 + (V - 1) * math.exp(-zstar))) < 1e-7
    m.weights["head"] = np.zeros((V, d), np.float32)
    out = orc.draft_block(m, dr)
    assert (out["conf"] == 1.0 / V).all() and (out["drafts"] == 0).all()


def test_centroid_head_hand_case(orc):
    """Centroid head ("Gemma 4 MTP" s.3): V=8 tokens in 4 centroid lists of 2
    (ordering [5,1 | 0,7 | 2,6 | 3,4]), top-2 centroids.  With f = e_0 the
    centroid logits are column 0 of C = [0.3, -1, 2, 0.3]: centroid 2 wins,
    then the tie 0.3 / 0.3 goes to the lower id 0.  Candidates {2, 6, 5, 1}
    get E[t] . f = E[t, 0]; every other token reads -1e30; the boundary
    margin is 0.3 - 0.3 = 0."""
    m = toys.blank_model(d=4, dh=4, V=8)
    m.n_centroids, m.centroid_top_k = 4, 2
    m.weights["centroids"] = np.array([[0.3, 1, 0, 0], [-1, 0, 0, 0], [2, 0, 0, 0], [0.3, 0, 5, 0]], np.float32)
    m.weights["token_ordering"] = np.array([5, 1, 0, 7, 2, 6, 3, 4], np.int32)
    E = np.arange(32, dtype=np.float32).reshape(8, 4) / 8 - 1
    m.weights["head"] = E
    z, margin = orc.centroid_logits(m, np.array([1.0, 0, 0, 0]))
    want = np.full(8, -1e30, np.float32)
    for t in (2, 6, 5, 1):
        want[t] = E[t, 0]
    assert np.array_equal(z, want) and margin == 0.0
    # shifting f towards feature 2 promotes centroid 3 past centroid 0
    z, margin = orc.centroid_logits(m, np.array([1.0, 0, 0.1, 0]))
    assert sorted(np.nonzero(z > -1e29)[0].tolist()) == [2, 3, 4, 6]
    assert abs(margin - (0.8 - 0.3)) < 1e-7


def test_centroid_head_with_one_list_equals_the_dense_head(orc):
    """One centroid holding the whole (permuted) vocabulary, top-1: the
    candidate set is every token, so the chain is the dense tied head's
    chain bit for bit."""
    w = syn.c1_tiny()
    dense = orc.draft_block(w.model, w.draft)
    m = w.model
    m.n_centroids, m.centroid_top_k = 1, 1
    m.weights["centroids"] = np.ones((1, m.d_model), np.float32)
    m.weights["token_ordering"] = np.random.default_rng(1).permutation(m.n_vocab).astype(np.int32)
    cent = orc.draft_block(m, w.draft)
    for k in ("drafts", "logits", "h_last", "conf"):
        assert np.array_equal(dense[k], cent[k]), k


def test_chain_hidden_path_follows_the_post_projection(orc):
    """W_pre = [0 | I]: x = h.  W_post = P: next h = P f.  The drafts walk the
    permutation through h alone, and h_last = P f of the last step (handed
    over in fp32)."""
    d = V = dh = 8
    m = toys.blank_model(d=d, dh=dh, V=V)
    toys.zero_blocks(m)
    perm = [5, 0, 6, 1, 7, 2, 4, 3]
    m.weights["head"] = np.eye(V, d, dtype=np.float32)
    m.weights["w_pre"] = np.concatenate([np.zeros((d, d), np.float32), np.eye(d, dh, dtype=np.float32)], 1)
    m.weights["w_post"] = toys.perm_matrix(perm)
    g = m.weights["g_final"]
    h0 = np.zeros(dh, np.float32)
    h0[4] = 0.3
    dr = toys.one_seq_inputs(m, 4, 3, last_tok=0, h_prev=h0, n_steps=3)
    out = orc.draft_block(m, dr)
    j, beta = 4, np.float32(0.3)
    drafts = []
    for k in range(3):
        drafts.append(j)
        f = float(beta) * toys.rms_scale(np.eye(d)[j] * float(beta), m.rms_eps) * float(g[j])
        j, beta = perm[j], np.float32(f)
    assert out["drafts"][0].tolist() == drafts
    np.testing.assert_allclose(out["h_last"][0], np.eye(dh)[j] * float(beta), rtol=2e-7)


def test_chain_attention_output_enters_through_w_o_with_gqa(orc):
    """One visible cell: every query head's attention output is its kv head's
    V row.  W_o routes (q head 2, dim 1) -- fed by kv head 1 -- to x[5]; the
    draft is 5 at every step and z[5] has a closed form."""
    d = V = dh = 8
    m = toys.blank_model(d=d, dh=dh, V=V, Hq=4, Hkv=2, hd=4)
    toys.zero_blocks(m)
    nm = m.block_names(0)
    a, gamma = 0.5, 50.0
    m.weights["head"] = (a * np.eye(V, d)).astype(np.float32)
    m.weights["w_pre"] = np.concatenate([np.eye(d, dtype=np.float32), np.zeros((d, dh), np.float32)], 1)
    wo = np.zeros((d, 16), np.float32)
    wo[5, 2 * 4 + 1] = gamma
    m.weights[nm["w_o"]] = wo
    k = np.zeros((3, 2, 4), np.float32)
    v = np.zeros((3, 2, 4), np.float32)
    v[0, 0] = [1, 0, 0, 0]
    v[0, 1] = [0, 1, 0, 0]
    dr = toys.one_seq_inputs(m, 3, 0, last_tok=1, h_prev=np.zeros(dh), n_steps=2, kv=(k, v))
    out = orc.draft_block(m, dr)
    assert out["drafts"][0].tolist() == [5, 5]
    g = m.weights["g_final"]
    x = np.zeros(d)
    x[1] = math.sqrt(d) * a                       # embedding of token 1 (step 0)
    x[5] += gamma
    np.testing.assert_allclose(out["logits"][0, 0, 5], a * x[5] * toys.rms_scale(x, m.rms_eps) * g[5], rtol=2e-7)


def test_chain_mlp_adds_down_silu_up(orc):
    """x = sqrt(d) a e_t; W_up row 0 = ones so u_0 = rmsnorm(x; g_mlp)_t;
    W_down[6, 0] = beta adds beta * silu(u_0) e_6.  silu(u) = u / (1 + e^-u)."""
    d = V = dh = 8
    m = toys.blank_model(d=d, dh=dh, V=V, F=4)
    toys.zero_blocks(m)
    nm = m.block_names(0)
    a, beta = 0.5, 10.0
    m.weights["head"] = (a * np.eye(V, d)).astype(np.float32)
    m.weights["w_pre"] = np.concatenate([np.eye(d, dtype=np.float32), np.zeros((d, dh), np.float32)], 1)
    up = np.zeros((4, d), np.float32)
    up[0] = 1.0
    down = np.zeros((d, 4), np.float32)
    down[6, 0] = beta
    m.weights[nm["w_up"]], m.weights[nm["w_down"]] = up, down
    dr = toys.one_seq_inputs(m, 2, 1, last_tok=3, h_prev=np.zeros(dh), n_steps=1)
    out = orc.draft_block(m, dr)
    x = np.zeros(d)
    x[3] = math.sqrt(d) * a
    u0 = x[3] * toys.rms_scale(x, m.rms_eps) * m.weights[nm["g_mlp"]][3]
    x[6] = beta * u0 / (1 + math.exp(-u0))
    assert out["drafts"][0, 0] == 6
    zexp = a * x * toys.rms_scale(x, m.rms_eps) * m.weights["g_final"]
    np.testing.assert_allclose(out["logits"][0, 0], zexp.astype(np.float32), rtol=2e-7, atol=1e-30)


def test_chain_query_norm_rope_position_and_scale(orc):
    """Two visible cells, hd = 2, theta irrelevant (one pair at 1 rad/pos).
    q = W_q a is head-normed, rotated to pos0 + k and scored against K with
    scale 1/sqrt(hd); o = sum softmax * V is routed to x[7].  z[7] at each
    step is a closed form of the step position."""
    d = V = dh = 8
    m = toys.blank_model(d=d, dh=dh, V=V, Hq=1, Hkv=1, hd=2)
    toys.zero_blocks(m)
    nm = m.block_names(0)
    a = 0.5
    m.weights["head"] = (a * np.eye(V, d)).astype(np.float32)
    m.weights["w_pre"] = np.concatenate([np.zeros((d, d), np.float32), np.eye(d, dh, dtype=np.float32)], 1)
    m.weights["w_post"] = np.zeros((dh, d), np.float32)   # h stays 0 after step 0
    wq = np.zeros((2, d), np.float32)
    wq[0, 0], wq[1, 1] = 1.0, 2.0
    m.weights[nm["w_q"]] = wq
    wo = np.zeros((d, 2), np.float32)
    wo[7, 0] = 1.0
    m.weights[nm["w_o"]] = wo
    k = np.array([[[3.0, 0.0]], [[0.0, 3.0]]], np.float32)
    v = np.array([[[1.0, 0.0]], [[-1.0, 0.0]]], np.float32)
    h0 = np.zeros(dh, np.float32)
    h0[0], h0[1] = 1.0, 0.5
    pos0 = 40
    dr = toys.one_seq_inputs(m, 2, 1, last_tok=0, h_prev=h0, n_steps=2, kv=(k, v), pos0=pos0)
    out = orc.draft_block(m, dr)
    ga, gq, g = m.weights[nm["g_attn"]], m.weights[nm["g_q"]], m.weights["g_final"]
    hk = h0.astype(np.float64)
    for step in range(2):
        x = hk.copy()
        an = x * toys.rms_scale(x, m.rms_eps) * ga
        q = np.array([an[0] * 1.0, an[1] * 2.0])
        qn = q * toys.rms_scale(q, m.rms_eps) * gq
        ang = pos0 + step
        qr = np.array([qn[0] * math.cos(ang) - qn[1] * math.sin(ang), qn[0] * math.sin(ang) + qn[1] * math.cos(ang)])
        s0, s1 = qr @ k[0, 0] / math.sqrt(2), qr @ k[1, 0] / math.sqrt(2)
        w0 = 1 / (1 + math.exp(s1 - s0))
        x[7] += w0 * 1.0 + (1 - w0) * -1.0
        z = a * x * toys.rms_scale(x, m.rms_eps) * g
        np.testing.assert_allclose(out["logits"][0, step], z.astype(np.float32), rtol=5e-7, atol=1e-7)
        hk = np.zeros(dh)                            # W_post = 0


def test_chain_equals_step_by_step(orc):
    """One N-step call equals N one-step calls chained through (token, h) with
    the step position advanced and attn_pos fixed (fused == per-step drafting,
    "Fused NextN draft graph" and the evaluation record's fused-vs-sequential
    check)."""
    w = syn.c1_tiny(n_seq=2)
    full = orc.draft_block(w.model, w.draft)
    tok, h = w.draft.last_tok.copy(), w.draft.h_prev.copy()
    for k in range(w.draft.n_steps):
        one = orc.draft_block(w.model, w.draft, n_steps=1, last_tok=tok, h_prev=h, pos0_shift=k)
        assert np.array_equal(one["drafts"][:, 0], full["drafts"][:, k])
        assert np.array_equal(one["logits"][:, 0], full["logits"][:, k])
        tok, h = one["drafts"][:, 0].copy(), one["h_last"].copy()
    assert np.array_equal(h, full["h_last"])


def test_chain_does_not_see_earlier_drafts_or_later_cells(orc):
    """No draft KV (Gemma 4 MTP doc s.1, s.5): cells past attn_pos (where the
    target appends during verify) are never read -- poisoning them changes
    nothing."""
    w = syn.c1_tiny()
    ref = orc.draft_block(w.model, w.draft)
    src = w.draft.seqs[0].src[0]
    seq = w.draft.seqs[0]
    k, v = src.k.copy(), src.v.copy()
    w.draft.seqs[0] = syn.Seq([syn.KVSource(np.concatenate([k, np.full((64,) + k.shape[1:], np.nan, np.float32)]),
                                            np.concatenate([v, np.full((64,) + v.shape[1:], np.nan, np.float32)])),
                               None], seq.attn_pos, seq.pos0)
    out = orc.draft_block(w.model, w.draft)
    assert np.array_equal(out["drafts"], ref["drafts"])
    assert np.array_equal(out["logits"], ref["logits"])


# ------------------------------------------------------------ verify greedy -
def test_verify_greedy_hand_cases(orc):
    """Accept the longest prefix of drafts equal to the row argmaxes; the
    first unverified row supplies the free token ("MTP decoding (--mtp)",
    How it is wired)."""
    L = np.array([[[0.1, 0.9, 0.3, 0.2],      # argmax 1
                   [0.5, 0.5, 0.1, 0.0],      # tie -> 0
                   [0.0, 0.0, 0.0, 1.0]]], np.float32)   # 3
    cases = {(1, 0): ([1, 0, 3], 2), (1, 1): ([1, 0, -1], 1), (2, 0): ([1, -1, -1], 0), (0, 0): ([1, -1, -1], 0)}
    for dr, (toks, na) in cases.items():
        t, n = orc.verify_greedy(L, np.array([dr], np.int32))
        assert t[0].tolist() == toks and n[0] == na


def test_verify_greedy_is_lossless_and_acceptance_follows_closed_form(orc):
    """Emitted tokens are exactly the target argmax sequence (lossless); with
    row i planted to win w.p. p, E[tokens/round] = (1 - a^(N+1)) / (1 - a),
    a = p + (1-p)/V (an unplanted random draft matches the argmax w.p. 1/V)."""
    S, N, V, p = 20000, 3, 256, 0.8
    gv = syn.make_greedy_verify(5, S, N, V, p, "max5")
    toks, na = orc.verify_greedy(gv.logits, gv.drafts)
    am = gv.logits.argmax(axis=2)
    for s in range(0, S, 997):
        a = na[s]
        assert toks[s, :a + 1].tolist() == am[s, :a + 1].tolist()
        assert toks[s, :a].tolist() == gv.drafts[s, :a].tolist()
        assert a == N or gv.drafts[s, a] != am[s, a]
    alpha = p + (1 - p) / V
    mean = (1 - alpha ** (N + 1)) / (1 - alpha)
    sd = np.std(na + 1) / math.sqrt(S)
    assert abs(np.mean(na + 1) - mean) < 4 * sd, (np.mean(na + 1), mean)


# ------------------------------------------------------- hidden-state verify
def test_hidden_verify_identity_head_hand_case(orc):
    """Head [I; -I] without a norm: row i's logits are (h, -h), so its token is
    the coordinate of largest magnitude, offset by d when it is negative; the
    acceptance is then read off by hand ("MTP decoding", How it is wired)."""
    d = 8
    head = np.concatenate([np.eye(d), -np.eye(d)]).astype(np.float32)
    h = np.zeros((2, 3, d), np.float32)
    h[0, 0, 2] = 1.5            # token 2
    h[0, 1, 5] = -2.0           # token 8 + 5 = 13
    h[0, 2, 0] = 0.5            # token 0
    h[1, 0, 7] = -0.25          # token 15
    h[1, 1, 1] = 3.0            # token 1
    h[1, 2, 4] = -1.0           # token 12
    h += np.float32(0.01) * np.arange(d, dtype=np.float32)    # small, the favourites stay
    drafts = np.array([[2, 13], [15, 4]], np.int32)
    t, n, margin = orc.verify_greedy_hidden(h, head, syn.F32, 2 * d, None, 1e-6, drafts)
    assert t.tolist() == [[2, 13, 0], [15, 1, -1]]
    assert n.tolist() == [2, 1]
    # row (0, 1): -h[5] = 2 - 0.05 leads, the runner-up is h[7] = 0.07
    assert abs(margin[0, 1] - (1.95 - 0.07)) < 1e-6


def test_hidden_verify_norm_scale_invariance_and_margin_scale(orc):
    """rmsnorm makes the tokens independent of a row's scale, and with unit gain
    it divides the logits (hence the top-2 margin) by sqrt(mean(h^2) + eps)."""
    S, N, d, V = 3, 2, 64, 300
    r = np.random.default_rng(7)
    head = syn.f32_to_bf16_bits(r.standard_normal((V, d)).astype(np.float32) / 8)
    h = r.standard_normal((S, N + 1, d)).astype(np.float32)
    drafts = r.integers(0, V, (S, N)).astype(np.int32)
    ones = np.ones(d, np.float32)
    t0, n0, m0 = orc.verify_greedy_hidden(h, head, syn.BF16, V, None, 1e-6, drafts)
    t1, n1, m1 = orc.verify_greedy_hidden(h, head, syn.BF16, V, ones, 1e-6, drafts)
    t2, n2, _ = orc.verify_greedy_hidden(h * np.float32(1024), head, syn.BF16, V, ones, 1e-6, drafts)
    assert (t0 == t1).all() and (t1 == t2).all() and (n0 == n1).all() and (n1 == n2).all()
    rms = np.sqrt((h.astype(np.float64) ** 2).mean(axis=2) + 1e-6)
    np.testing.assert_allclose(m1, m0 / rms, rtol=1e-5)


@pytest.mark.parametrize("dtype", [syn.BF16, syn.Q8_0])
def test_hidden_verify_equals_logit_verify_of_a_library_matmul(orc, dtype):
    """Tokens equal the logit-row verify applied to numpy's fp64 matmul of the
    normed rows with the head decoded in numpy; only fp32-level near ties may
    differ (none at this size)."""
    S, N, d, V = 4, 3, 96, 2000
    r = np.random.default_rng(11)
    wf = r.standard_normal((V, d)).astype(np.float32) / np.float32(math.sqrt(d))
    head = syn.store(wf, dtype)
    if dtype == syn.BF16:
        W = syn.bf16_bits_to_f32(head).astype(np.float64)
    else:
        blk = head.reshape(V, d // 32, 34)
        scale = blk[:, :, 0:2].copy().view(np.float16).astype(np.float64)      # [V, d/32, 1]
        W = (scale * blk[:, :, 2:].view(np.int8).astype(np.float64)).reshape(V, d)
    g = (1 + 0.1 * r.standard_normal(d)).astype(np.float32)
    h = r.standard_normal((S, N + 1, d)).astype(np.float32)
    drafts = r.integers(0, V, (S, N)).astype(np.int32)
    x = h.astype(np.float64)
    f = x / np.sqrt((x ** 2).mean(axis=2, keepdims=True) + 1e-6) * g.astype(np.float64)
    z = (f @ W.T).astype(np.float32)
    am = z.argmax(axis=2)
    drafts[:, 0] = am[:, 0]                   # some accepted prefixes
    drafts[0, 1] = am[0, 1]
    t, n, margin = orc.verify_greedy_hidden(h, head, dtype, V, g, 1e-6, drafts)
    t_ref, n_ref = orc.verify_greedy(z, drafts)
    assert margin.min() > 1e-4
    assert (t == t_ref).all() and (n == n_ref).all()
    assert n.tolist()[0] >= 2


def test_hidden_verify_recovers_planted_rows(orc):
    """Rows built around a token (beta * sqrt(d) * W_head[t] on top of unit
    noise) verify to that token, and the accepted prefix is the run of drafts
    equal to the planted tokens."""
    hv = syn.make_hidden_verify(3, 6, 3, 256, 4096, p_accept=0.7)
    t, n, margin = orc.verify_greedy_hidden(hv.hidden, hv.head, hv.head_dtype, hv.n_vocab, hv.g, hv.eps, hv.drafts)
    planted = hv.planted >= 0
    assert planted.sum() >= 18
    for s in range(6):
        for i in range(4):
            if planted[s, i] and t[s, i] >= 0:
                assert t[s, i] == hv.planted[s, i]
        a = 0
        while a < 3 and planted[s, a] and hv.drafts[s, a] == hv.planted[s, a]:
            a += 1
        assert n[s] == a
    assert 0 < n.sum() < 18


def test_sample_hidden_with_signed_identity_head_is_the_logit_row_sampling_verify(orc):
    """Head [I; -I] without a norm makes row i's logits exactly (h_i, -h_i), so
    the hidden-state sampling verify must return what the logit-row sampling
    verify returns on those rows: same tokens, accept lengths and near-boundary
    flags, with q rows, history penalties, min-p and top-p in play."""
    S, N, d = 8, 3, 64
    V = 2 * d
    r = np.random.default_rng(23)
    head = np.concatenate([np.eye(d), -np.eye(d)]).astype(np.float32)
    h = (1.5 * r.standard_normal((S, N + 1, d))).astype(np.float32)
    z = np.concatenate([h, -h], axis=2)
    q = (z[:, :N] + r.standard_normal((S, N, V))).astype(np.float32)
    drafts = np.stack([[r.choice(V, p=np.exp(q[s, i]) / np.exp(q[s, i]).sum()) for i in range(N)]
                       for s in range(S)]).astype(np.int32)
    drafts[:, 0] = z[:, 0].argmax(axis=1)        # some accepted first drafts
    history = r.integers(0, V, (S, 16)).astype(np.int32)
    history_len = np.full(S, 16, np.int32)
    sp = _sp(temp=0.7, top_p=0.9, min_p=0.02, rep_penalty=1.1, presence_penalty=0.2, penalty_last_n=8, seed=5)
    for q_rows in (q, None):
        t_h, n_h, f_h = orc.verify_sample_hidden(h, head, syn.F32, V, None, 1e-6, q_rows, drafts, history,
                                                 history_len, sp, 3)
        t_z, n_z, f_z = orc.verify_sample(z, q_rows, drafts, history, history_len, sp, 3)
        assert (t_h == t_z).all() and (n_h == n_z).all() and (f_h == f_z).all()
        assert (t_h[:, 0] >= 0).all()


# ------------------------------------------------------------ sampling chain
def _sp(**kw):
    base = dict(temp=1.0, top_p=1.0, min_p=0.0, rep_penalty=1.0, presence_penalty=0.0, freq_penalty=0.0, top_k=0,
                penalty_last_n=64, seed=1)
    base.update(kw)
    return syn.Sampler(**base)


def test_sample_dist_plain_softmax_and_temperature(orc):
    from scipy.special import softmax
    z = np.array([0.3, -1.0, 2.0, 0.0, 1.1], np.float32)
    p, fl = orc.sample_dist(z, [], _sp())
    np.testing.assert_allclose(p, softmax(z.astype(np.float64)), rtol=1e-14)
    p, _ = orc.sample_dist(z, [], _sp(temp=0.5))
    np.testing.assert_allclose(p, softmax(2.0 * z.astype(np.float64)), rtol=1e-14)


def test_sample_dist_penalties_hand_case(orc):
    """z = [2, -1, 0.5], ctx = [0, 1, 1]; rep 2, presence 0.5, freq 0.25:
    z0 = 2/2 - 0.5 - 0.25 = 0.25; z1 = -1*2 - 0.5 - 0.5 = -3; z2 unchanged."""
    z = np.array([2.0, -1.0, 0.5], np.float32)
    p, _ = orc.sample_dist(z, [0, 1, 1], _sp(rep_penalty=2.0, presence_penalty=0.5, freq_penalty=0.25))
    e = np.exp([0.25, -3.0, 0.5])
    np.testing.assert_allclose(p, e / e.sum(), rtol=1e-14)


def test_sample_dist_min_p_and_top_p_hand_cases(orc):
    z = np.log(np.array([1.0, 0.5, 0.04, 0.2], np.float64)).astype(np.float32)
    p, _ = orc.sample_dist(z, [], _sp(min_p=0.05))
    e = np.exp(z.astype(np.float64))
    e[2] = 0
    np.testing.assert_allclose(p, e / e.sum(), rtol=1e-14)
    # probabilities 0.5, 0.3, 0.15, 0.05: top-p 0.75 keeps {0, 1} (crossing token included)
    z = np.log(np.array([0.15, 0.5, 0.05, 0.3])).astype(np.float32)
    p, _ = orc.sample_dist(z, [], _sp(top_p=0.75))
    e = np.exp(z.astype(np.float64))
    e[[0, 2]] = 0
    np.testing.assert_allclose(p, e / e.sum(), rtol=1e-14)
    p, _ = orc.sample_dist(z, [], _sp(top_p=0.5))          # reaches 0.5 with one token
    assert p[1] == 1.0 and p.sum() == 1.0
    # top-k 2 keeps the two largest logits
    p, _ = orc.sample_dist(z, [], _sp(top_k=2))
    e = np.exp(z.astype(np.float64))
    e[[0, 2]] = 0
    np.testing.assert_allclose(p, e / e.sum(), rtol=1e-14)


def test_penalty_window_covers_history_tail_and_earlier_drafts(orc):
    """Row i's penalties see the last penalty_last_n tokens of history ++
    drafts[0..i) (the audit's fix: the bonus token must see the window's
    tokens)."""
    S = 4000
    # row 0 strongly prefers token 0 (the draft); row 1 would too, unless the
    # accepted draft 0 is in its penalty window
    p = np.zeros((S, 2, 4), np.float32)
    p[:, 0, 0] = 12.0
    p[:, 1] = [6.0, 5.9, 5.9, 5.9]
    drafts = np.zeros((S, 1), np.int32)
    hist = np.tile(np.array([[1, 2, 3, 3, 3]], np.int32), (S, 1))
    sp = _sp(presence_penalty=100.0, penalty_last_n=3)
    toks, na, _ = orc.verify_sample(p, None, drafts, hist, np.full(S, 5, np.int32), sp)
    assert np.all(na == 1)
    bonus = toks[:, 1]
    # window for row 1 = last 3 of [1,2,3,3,3,0] = [3,3,0]: tokens 0 and 3 banned
    assert set(np.unique(bonus)) == {1, 2}


def test_exact_rule_one_hot_q_accepts_with_probability_p_and_resamples_residual(orc):
    """Deterministic drafts (q one-hot): accept w.p. p(d); on rejection the
    token follows p with d removed, renormalised (audit page s.4)."""
    S = 60000
    z = np.array([1.0, 0.2, -0.5, 0.7, 0.0, -1.2], np.float32)
    P = np.exp(z.astype(np.float64))
    P /= P.sum()
    d = 3
    p_logits = np.tile(z, (S, 2, 1))
    toks, na, _ = orc.verify_sample(p_logits, None, np.full((S, 1), d, np.int32), np.zeros((S, 0), np.int32),
                                    np.zeros(S, np.int32), _sp())
    acc = np.mean(na == 1)
    assert abs(acc - P[d]) < 4 * math.sqrt(P[d] * (1 - P[d]) / S)
    rej = toks[na == 0, 0]
    assert d not in set(rej.tolist())
    R = P.copy()
    R[d] = 0
    R /= R.sum()
    counts = np.bincount(rej, minlength=6)
    exp = R * rej.size
    m = exp > 0
    chi2 = ((counts[m] - exp[m]) ** 2 / exp[m]).sum()
    assert chi2 < 25          # chi2(4) 99.99th percentile ~ 23.5


def test_exact_rule_general_q_acceptance_and_first_token_law(orc):
    """Leviathan et al. s.2.3: acceptance probability sum_x min(p, q); the
    first emitted token is distributed as p whatever q is."""
    S = 80000
    r = np.random.default_rng(9)
    zp = r.standard_normal(6).astype(np.float32)
    zq = (zp + r.standard_normal(6)).astype(np.float32)
    sp = _sp()
    P, _ = orc.sample_dist(zp, [], sp)
    Q, _ = orc.sample_dist(zq, [], sp)
    drafts = r.choice(6, size=(S, 1), p=Q).astype(np.int32)
    toks, na, _ = orc.verify_sample(np.tile(zp, (S, 2, 1)), np.tile(zq, (S, 1, 1)), drafts,
                                    np.zeros((S, 0), np.int32), np.zeros(S, np.int32), sp)
    alpha = np.minimum(P, Q).sum()
    assert abs(np.mean(na == 1) - alpha) < 4 * math.sqrt(alpha * (1 - alpha) / S)
    counts = np.bincount(toks[:, 0], minlength=6)
    exp = P * S
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 28          # chi2(5) 99.99th percentile ~ 25.7


# ------------------------------------------- Monte-Carlo total variation ---
def _toy_rows(toy, hist_tokens, hist_len):
    """logits of the toy LM for each row's context (last token + membership)."""
    n = hist_tokens.shape[0]
    last = hist_tokens[np.arange(n), hist_len - 1]
    member = np.zeros((n, 6), bool)
    for j in range(hist_tokens.shape[1]):
        live = j < hist_len
        member[np.arange(n)[live], hist_tokens[live, j]] = True
    return toy.logits(last, member)


def _run_speculative(orc, toy, drafter, sp, n_trials, n_draft, hist0, rule, seed):
    """Generate 3-token continuations by repeated draft + verify rounds."""
    T = 3
    H0 = len(hist0)
    hist = np.zeros((n_trials, H0 + T + n_draft), np.int32)
    hist[:, :H0] = hist0
    hlen = np.full(n_trials, H0, np.int32)
    out = np.full((n_trials, T), -1, np.int32)
    n_out = np.zeros(n_trials, np.int32)
    rng = np.random.default_rng(seed)
    qcache = {}
    rnd = 0
    while True:
        act = np.nonzero(n_out < T)[0]
        if act.size == 0:
            break
        S = act.size
        ctx = hist[act].copy()
        clen = hlen[act].copy()
        drafts = np.zeros((S, n_draft), np.int32)
        p_log = np.zeros((S, n_draft + 1, 6), np.float32)
        q_log = np.zeros((S, n_draft, 6), np.float32)
        for i in range(n_draft + 1):
            p_log[:, i] = _toy_rows(toy, ctx, clen)
            if i == n_draft:
                break
            if isinstance(drafter, str):
                dtok = p_log[:, i].argmax(axis=1).astype(np.int32)
            else:
                q_log[:, i] = p_log[:, i] + drafter
                dtok = np.zeros(S, np.int32)
                idx = {}
                for s in range(S):
                    idx.setdefault(ctx[s, :clen[s]].tobytes(), []).append(s)
                for key, rows in idx.items():
                    if key not in qcache:
                        c = ctx[rows[0], :clen[rows[0]]].tolist()
                        qcache[key] = orc.sample_dist(q_log[rows[0], i], c[-sp.penalty_last_n:], sp)[0]
                    dtok[rows] = rng.choice(6, size=len(rows), p=qcache[key])
            drafts[:, i] = dtok
            ctx[np.arange(S), clen] = dtok
            clen += 1
        if rule == "exact":
            toks, na, _ = orc.verify_sample(p_log, None if isinstance(drafter, str) else q_log, drafts, hist[act],
                                            hlen[act], sp, rnd)
        else:
            toks, na = orc.verify_greedy_match(p_log, drafts, hist[act], hlen[act], sp, rnd)
        for j in range(n_draft + 1):
            emit = (j <= na) & (n_out[act] < T)
            rows = act[emit]
            out[rows, n_out[rows]] = toks[emit, j]
            hist[rows, hlen[rows]] = toks[emit, j]
            hlen[rows] += 1
            n_out[rows] += 1
        rnd += 1
    return out


def _exact_law(orc, toy, sp, hist0):
    P = {}
    def rows(ctx):
        c = np.array([ctx], np.int32)
        return _toy_rows(toy, c, np.array([len(ctx)], np.int32))[0]
    p1, _ = orc.sample_dist(rows(hist0), hist0, sp)
    for x1 in range(6):
        if p1[x1] == 0:
            continue
        c1 = hist0 + [x1]
        p2, _ = orc.sample_dist(rows(c1), c1, sp)
        for x2 in range(6):
            if p2[x2] == 0:
                continue
            c2 = c1 + [x2]
            p3, _ = orc.sample_dist(rows(c2), c2, sp)
            for x3 in range(6):
                if p3[x3] > 0:
                    P[(x1, x2, x3)] = p1[x1] * p2[x2] * p3[x3]
    return P


def _tv(P, out):
    keys, counts = np.unique(out, axis=0, return_counts=True)
    emp = {tuple(k.tolist()): c / out.shape[0] for k, c in zip(keys, counts)}
    support = set(P) | set(emp)
    return 0.5 * sum(abs(P.get(x, 0.0) - emp.get(x, 0.0)) for x in support)


@pytest.mark.slow
def test_monte_carlo_total_variation_exact_vs_greedy_match(orc):
    """The audit page's check: 400k 3-token continuations of a 6-token toy LM
    with history-dependent logits, temp 0.6 / top-p 0.95 / min-p 0.05 /
    rep 1.08 / presence 0.4.  The exact rule's TV to the one-at-a-time law
    stays at the Monte-Carlo noise floor (page: 0.0029 vs 0.0027); the old
    greedy-match rule with a greedy drafter is far off (page: 0.79)."""
    toy = syn.make_toy(21)
    sp = syn.Sampler(temp=0.6, top_p=0.95, min_p=0.05, rep_penalty=1.08, presence_penalty=0.4, freq_penalty=0.0,
                     top_k=0, penalty_last_n=64, seed=77)
    hist0 = [2, 4]
    n = 400_000
    P = _exact_law(orc, toy, sp, hist0)
    floor = sum(math.sqrt(p * (1 - p) / (2 * math.pi * n)) for p in P.values())
    drafter = (0.8 * np.random.default_rng(3).standard_normal(6)).astype(np.float32)
    tv_exact_q = _tv(P, _run_speculative(orc, toy, drafter, sp, n, 2, hist0, "exact", 1))
    tv_exact_greedy = _tv(P, _run_speculative(orc, toy, "greedy", sp, n, 2, hist0, "exact", 2))
    tv_gm = _tv(P, _run_speculative(orc, toy, "greedy", sp, n, 2, hist0, "greedy_match", 3))
    assert tv_exact_q < 2 * floor, (tv_exact_q, floor)
    assert tv_exact_greedy < 2 * floor, (tv_exact_greedy, floor)
    assert tv_gm > 10 * floor, (tv_gm, floor)


def test_empty_distribution_rows_reject_and_draw_nothing(orc):
    """A row none of whose tokens survives the chain (every logit -inf, so no
    finite maximum) has an empty distribution: its draft is rejected (the
    accept test compares against p(d) = 0) and a draw from it yields -1.
    Sequence 0: row 0 empty (one-hot q) -> rejected at 0, token -1.
    Sequence 1: row 1 empty, general q -> draft 0 accepted (p(d) ~ 1), draft
    1 rejected, residual draw empty.  Sequence 2: both drafts accepted, the
    bonus row empty -> -1 at position 2, n_accept 2."""
    V = 50
    sp = _sp(min_p=0.05, top_p=0.95, penalty_last_n=0)
    p = np.zeros((3, 3, V), np.float32)
    drafts = np.array([[4, 5], [7, 8], [9, 10]], np.int32)
    for s in range(3):
        for i in range(2):
            p[s, i, drafts[s, i]] = 60.0          # p(d) = 1 up to exp(-60)
    p[0, 0] = -np.inf
    p[1, 1] = -np.inf
    p[2, 2] = -np.inf
    t, n, fl = orc.verify_sample(p, None, drafts, np.zeros((3, 0), np.int32), np.zeros(3, np.int32), sp, 0)
    assert n.tolist() == [0, 1, 2]
    assert t.tolist() == [[-1, -1, -1], [7, -1, -1], [9, 10, -1]]
    q = np.zeros((3, 2, V), np.float32)           # uniform q: p(d) = 1 > u q(d) accepts the planted drafts
    t2, n2, _ = orc.verify_sample(p, q, drafts, np.zeros((3, 0), np.int32), np.zeros(3, np.int32), sp, 0)
    assert n2.tolist() == [0, 1, 2]
    assert t2[0, 0] == -1 and t2[1].tolist() == [7, -1, -1] and t2[2].tolist() == [9, 10, -1]
    pe, _ = orc.sample_dist(p[0, 0], [], sp)
    assert (pe == 0).all()
