"""Seeded synthetic inputs for the MTP draft-chain / verify path.

This module only *draws numbers* and lays them out in the storage formats the
library consumes (fp32, bf16 bit patterns, Q8_0 blocks).  It holds none of the
method's arithmetic: no normalisation, attention, projection, argmax or
sampling rule lives here.  Both the CPU oracle and the GPU tests/bench take
their inputs from here, so the two sides see identical bytes.

Shapes follow the workloads on the pages: a Gemma-4-assistant-like drafter
("Gemma 4 MTP" design doc, section 3 and 4: 4 blocks, pre/post backbone
projections, a tied LM head over a 262144-token vocabulary) cross-attending
into a target KV cache; verify inputs are target logits over 1+N positions
("MTP decoding (--mtp)", section "How it is wired").  Every tensor comes from
its own PCG64 sub-stream keyed by (seed, tensor name), so shrinking one
dimension for a quick test never changes the draws of another tensor.

Storage conventions (shared with the C ABI, documented in include/mtp.h):
  * matrices are row-major [out, in];
  * bf16 tensors are uint16 arrays of bf16 bit patterns (round-to-nearest-even
    from fp32 draws);
  * the Q8_0 head is uint8 bytes [V, d/32, 34]: per 32 weights one fp16 scale
    (little endian) followed by 32 int8 values;
  * a KV source is K and V arrays [n_cells, Hkv, hd] per sequence.
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

F32, BF16, Q8_0 = 0, 1, 2
KV_FULL, KV_SWA, KV_SINK_WINDOW = 0, 1, 2
DTYPE_NAMES = {F32: "f32", BF16: "bf16", Q8_0: "q8_0"}


# ----------------------------------------------------------------------------
# random streams and storage formats
# ----------------------------------------------------------------------------
def rng_for(seed: int, name: str) -> np.random.Generator:
    """Independent PCG64 stream for one named tensor."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, zlib.crc32(name.encode())])))


def normal(seed: int, name: str, shape, std: float = 1.0) -> np.ndarray:
    a = rng_for(seed, name).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    out = np.empty(b.shape, dtype=np.uint16)
    chunk = 1 << 24
    flat_b, flat_o = b.reshape(-1), out.reshape(-1)
    for i in range(0, flat_b.size, chunk):
        x = flat_b[i:i + chunk]
        flat_o[i:i + chunk] = ((x + (np.uint32(0x7FFF) + ((x >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (used only to describe inputs)."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def q8_0_blocks(a: np.ndarray) -> np.ndarray:
    """Q8_0 storage of an fp32 matrix [rows, cols] (cols % 32 == 0).

    Per block of 32 values: d = max|x| / 127 in fp32, stored as fp16 (RNE);
    q = x / d rounded half away from zero and clamped to [-127, 127];
    an all-zero block stores d = 0, q = 0.  This only *builds* the input bytes;
    readers dequantise as fp16(d) * q.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    rows, cols = a.shape
    assert cols % 32 == 0
    out = np.empty((rows, cols // 32, 34), dtype=np.uint8)
    chunk = max(1, (1 << 22) // cols)
    for r0 in range(0, rows, chunk):
        x = a[r0:r0 + chunk].reshape(-1, cols // 32, 32)
        amax = np.abs(x).max(axis=2)
        d = (amax / np.float32(127.0)).astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            v = np.where(d[..., None] > 0, x / d[..., None], np.float32(0.0))
        q = np.sign(v) * np.floor(np.abs(v) + np.float32(0.5))
        q = np.clip(q, -127, 127).astype(np.int8)
        out[r0:r0 + chunk, :, 0:2] = d.astype(np.float16)[..., None].view(np.uint8).reshape(d.shape + (2,))
        out[r0:r0 + chunk, :, 2:] = q.view(np.uint8)
    return out


def store(a: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F32:
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(a)
    if dtype == Q8_0:
        return q8_0_blocks(a)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# drafter description + weights
# ----------------------------------------------------------------------------
@dataclass
class Model:
    d_model: int
    d_hprev: int
    n_blocks: int
    n_head_q: int
    n_head_kv: int
    head_dim: int
    d_ff: int
    n_vocab: int
    w_dtype: int
    head_dtype: int
    kv_dtype: int
    swa_window: int
    block_src: List[int]
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    attn_scale: float = 0.0      # 0 -> 1/sqrt(head_dim)
    embed_scale: float = 0.0     # 0 -> sqrt(d_model)
    n_centroids: int = 0         # centroid LM head: 0 = dense tied head
    centroid_top_k: int = 0
    sw_window: int = 0           # sink + window source: window length
    sw_sink: int = 0             #   and sink cells
    weights: Dict[str, np.ndarray] = field(default_factory=dict)

    def __post_init__(self):
        if self.attn_scale == 0.0:
            self.attn_scale = 1.0 / math.sqrt(self.head_dim)
        if self.embed_scale == 0.0:
            self.embed_scale = math.sqrt(self.d_model)

    def block_names(self, l: int):
        return {k: f"blk{l}.{k}" for k in ("g_attn", "w_q", "g_q", "w_o", "g_mlp", "w_up", "w_down")}


def make_model(seed: int, *, d_model, d_hprev, n_blocks, n_head_q, n_head_kv, head_dim, d_ff, n_vocab,
               w_dtype=BF16, head_dtype=BF16, kv_dtype=BF16, swa_window=0, block_src=None,
               head_std: Optional[float] = None, n_centroids: int = 0, centroid_top_k: int = 0) -> Model:
    """Random drafter: matrices ~ N(0, 1/fan_in), norm gains = 1 + 0.1 N(0,1).

    With n_centroids > 0 the LM head is a centroid head: token_ordering is a
    random permutation of the vocabulary cut into n_centroids lists of
    V/n_centroids ids, and centroid c is the mean of its list's embedding
    rows rescaled to unit RMS per entry (so the top centroids tend to hold
    the top tokens, as a trained head's clusters do)."""
    m = Model(d_model, d_hprev, n_blocks, n_head_q, n_head_kv, head_dim, d_ff, n_vocab, w_dtype, head_dtype,
              kv_dtype, swa_window, list(block_src if block_src is not None else [KV_FULL] * n_blocks))
    d, dh, qd = d_model, d_hprev, n_head_q * head_dim
    W = m.weights

    def mat(name, rows, cols, std=None, dt=w_dtype):
        W[name] = store(normal(seed, name, (rows, cols), std if std is not None else 1.0 / math.sqrt(cols)), dt)

    def gain(name, n):
        W[name] = (1.0 + 0.1 * normal(seed, name, (n,))).astype(np.float32)

    mat("w_pre", d, d + dh)
    mat("w_post", dh, d)
    mat("head", n_vocab, d, std=head_std if head_std is not None else 1.0 / math.sqrt(d), dt=head_dtype)
    gain("g_final", d)
    if n_centroids:
        assert n_vocab % n_centroids == 0 and 1 <= centroid_top_k <= n_centroids and head_dtype != Q8_0
        m.n_centroids, m.centroid_top_k = n_centroids, centroid_top_k
        vsc = n_vocab // n_centroids
        order = rng_for(seed, "token_ordering").permutation(n_vocab).astype(np.int32)
        E = W["head"] if head_dtype == F32 else (W["head"].astype(np.uint32) << 16).view(np.float32)
        C = E[order].reshape(n_centroids, vsc, d).astype(np.float64).mean(axis=1)
        C /= np.sqrt((C ** 2).mean(axis=1, keepdims=True)) * math.sqrt(d)
        W["centroids"] = store(C.astype(np.float32), w_dtype)
        W["token_ordering"] = order
    for l in range(n_blocks):
        nm = m.block_names(l)
        gain(nm["g_attn"], d)
        mat(nm["w_q"], qd, d)
        gain(nm["g_q"], head_dim)
        mat(nm["w_o"], d, qd)
        gain(nm["g_mlp"], d)
        mat(nm["w_up"], d_ff, d)
        mat(nm["w_down"], d, d_ff)
    return m


# ----------------------------------------------------------------------------
# per-sequence draft inputs
# ----------------------------------------------------------------------------
@dataclass
class KVSource:
    k: np.ndarray            # [n_cells, Hkv, hd] f32 or bf16 bits
    v: np.ndarray

    @property
    def n_cells(self) -> int:
        return int(self.k.shape[0])


@dataclass
class Seq:
    src: List[Optional[KVSource]]   # [full, swa, sink + window]
    attn_pos: int
    pos0: int
    run_lo: int = 0                 # first valid cell of the sink + window source


@dataclass
class DraftInputs:
    seqs: List[Seq]
    last_tok: np.ndarray     # int32 [S]
    h_prev: np.ndarray       # f32 [S, dh]
    n_steps: int


def make_kv(seed: int, name: str, n_cells: int, m: Model, fill_cells: Optional[int] = None) -> KVSource:
    shape = (n_cells, m.n_head_kv, m.head_dim)
    k = normal(seed, name + ".k", shape)
    v = normal(seed, name + ".v", shape)
    return KVSource(store(k, m.kv_dtype), store(v, m.kv_dtype))


def make_draft_inputs(seed: int, m: Model, ctx_lens, n_steps: int, *, full_cap=None, swa_cells=None,
                      share_kv: bool = False, run_lo=None) -> DraftInputs:
    """Sequences with context lengths ctx_lens (attn_pos = ctx-1, pos0 = ctx).

    full_cap: cells in each sequence's full-attention source (default max ctx).
    swa_cells: ring capacity of the sliding-window source (default swa_window);
    only built when some block reads the SWA source.
    """
    S = len(ctx_lens)
    need_swa = KV_SWA in m.block_src[:m.n_blocks]
    need_sw = KV_SINK_WINDOW in m.block_src[:m.n_blocks]
    full_cap = full_cap or max(ctx_lens)
    seqs = []
    shared = make_kv(seed, "kv.full", full_cap, m) if share_kv else None
    for s, ctx in enumerate(ctx_lens):
        full = shared if share_kv else make_kv(seed, f"kv.full.{s}", full_cap, m)
        swa = make_kv(seed, f"kv.swa.{s}", swa_cells or m.swa_window, m) if need_swa else None
        sw = make_kv(seed, f"kv.sw.{s}", full_cap, m) if need_sw else None
        seqs.append(Seq([full, swa, sw], attn_pos=int(ctx) - 1, pos0=int(ctx),
                        run_lo=int(run_lo[s]) if run_lo is not None else 0))
    last_tok = rng_for(seed, "last_tok").integers(0, m.n_vocab, size=S, dtype=np.int64).astype(np.int32)
    h_prev = normal(seed, "h_prev", (S, m.d_hprev))
    return DraftInputs(seqs, last_tok, h_prev, n_steps)


# ----------------------------------------------------------------------------
# verify inputs
# ----------------------------------------------------------------------------
def plant_accepts(logits: np.ndarray, drafts: np.ndarray, p: float, seed: int, name: str, mode: str) -> None:
    """Make row i favour draft i with probability p (rows 0..N-1), in place.

    mode "add5": z[i][d_i] += 5 (the tiny config's literal wording);
    mode "max5": z[i][d_i] = max(z[i]) + 5 (a certain win when planted).
    """
    S, R, V = logits.shape
    N = drafts.shape[1]
    hit = rng_for(seed, name).random((S, N)) < p
    for s in range(S):
        for i in range(N):
            if hit[s, i]:
                t = int(drafts[s, i])
                if mode == "add5":
                    logits[s, i, t] += np.float32(5.0)
                else:
                    logits[s, i, t] = logits[s, i].max() + np.float32(5.0)


@dataclass
class GreedyVerifyInputs:
    logits: np.ndarray   # f32 [S, N+1, V]
    drafts: np.ndarray   # int32 [S, N]


def make_greedy_verify(seed: int, S: int, N: int, V: int, p_accept: float, mode: str,
                       drafts: Optional[np.ndarray] = None) -> GreedyVerifyInputs:
    logits = normal(seed, "verify.logits", (S, N + 1, V))
    if drafts is None:
        drafts = rng_for(seed, "verify.drafts").integers(0, V, size=(S, N), dtype=np.int64).astype(np.int32)
    plant_accepts(logits, drafts, p_accept, seed, "verify.plant", mode)
    return GreedyVerifyInputs(logits, np.ascontiguousarray(drafts, dtype=np.int32))


@dataclass
class Sampler:
    temp: float = 0.6
    top_p: float = 0.95
    min_p: float = 0.05
    rep_penalty: float = 1.08
    presence_penalty: float = 0.4
    freq_penalty: float = 0.0
    top_k: int = 0
    penalty_last_n: int = 64
    seed: int = 0x5EED


@dataclass
class SampleVerifyInputs:
    p_logits: np.ndarray         # f32 [S, N+1, V]
    q_logits: Optional[np.ndarray]  # f32 [S, N, V] or None (one-hot drafts)
    drafts: np.ndarray           # int32 [S, N]
    history: np.ndarray          # int32 [S, H]
    history_len: np.ndarray      # int32 [S]
    sampler: Sampler


def make_sample_verify(seed: int, S: int, N: int, V: int, *, logit_var: float = 3.0, hist: int = 64,
                       one_hot: bool = False, sampler: Optional[Sampler] = None,
                       draft_mode: str = "sample") -> SampleVerifyInputs:
    """Temperature>0 verify inputs shaped like the exact-sampling workload.

    p logits ~ N(0, var logit_var); q logits = p[:, :N] + N(0,1) (an
    independently perturbed copy).  History: 3/4 uniform ids plus 1/4 drawn
    without replacement from the 32 highest row-0 logits, shuffled, so the
    penalties act on likely tokens.  Drafts are drawn from softmax(q / temp)
    by the Gumbel trick on this module's own stream (a stand-in drafter; the
    verify rule is exact for whatever drafts it is given only when the drafts
    follow the processed q, which the statistical tests arrange separately).
    draft_mode "argmax": each draft is instead the highest raw logit of its q
    row (of its p row when one_hot), as a greedy drafter would propose.
    """
    sampler = sampler or Sampler()
    p = normal(seed, "sample.p", (S, N + 1, V), std=math.sqrt(logit_var))
    q = None
    if not one_hot:
        q = p[:, :N] + normal(seed, "sample.q_noise", (S, N, V))
    n_top = min(hist // 4, 32)
    r = rng_for(seed, "sample.history")
    history = np.empty((S, hist), dtype=np.int32)
    for s in range(S):
        top32 = np.argsort(-p[s, 0], kind="stable")[:32]
        hs = np.concatenate([r.integers(0, V, size=hist - n_top), r.choice(top32, size=n_top, replace=False)])
        r.shuffle(hs)
        history[s] = hs
    history_len = np.full(S, hist, dtype=np.int32)
    src = q if q is not None else p[:, :N]
    if draft_mode == "argmax":
        drafts = np.argmax(src, axis=2).astype(np.int32)
    else:
        g = rng_for(seed, "sample.drafts").gumbel(size=(S, N, V)).astype(np.float32)
        drafts = np.argmax(src / np.float32(sampler.temp) + g, axis=2).astype(np.int32)
    return SampleVerifyInputs(p, q, drafts, history, history_len, sampler)


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------
C2_SHAPE = dict(d_model=1024, d_hprev=2816, n_blocks=4, n_head_q=8, n_head_kv=2, head_dim=256, d_ff=4096,
                n_vocab=262144)


@dataclass
class HiddenVerifyInputs:
    """The target's final hidden rows for a verify from hidden states."""
    d: int
    n_vocab: int
    head_dtype: int
    head: np.ndarray             # the target's LM head [V, d] in its storage format
    g: Optional[np.ndarray]      # fp32 [d] final-norm gain, or None (rows already normed)
    eps: float
    hidden: np.ndarray           # fp32 [S, N+1, d]
    drafts: np.ndarray           # int32 [S, N]
    planted: np.ndarray          # int32 [S, N+1]: token a row was built around, -1 for a pure-noise row


def make_hidden_verify(seed: int, S: int, N: int, d: int, V: int, *, head_dtype: int = BF16, p_accept: float = 0.8,
                       plant_frac: float = 0.9, beta: float = 1.0, gain: bool = True,
                       eps: float = 1e-6) -> HiddenVerifyInputs:
    """Head ~ N(0, 1/d); gain 1 + 0.1 N(0,1); hidden rows N(0,1), and with
    probability plant_frac a row also gets beta * sqrt(d) * W_head[t] added for
    a random token t (a clear favourite, as a trained target's rows have);
    draft i equals row i's planted token with probability p_accept, else it is
    another random token."""
    head_f = normal(seed, "hv.head", (V, d), std=1.0 / math.sqrt(d))
    head = store(head_f, head_dtype)
    g = (1.0 + 0.1 * normal(seed, "hv.gain", (d,))).astype(np.float32) if gain else None
    r = rng_for(seed, "hv.plant")
    tok = r.integers(0, V, size=(S, N + 1)).astype(np.int32)
    is_planted = r.random((S, N + 1)) < plant_frac
    hidden = normal(seed, "hv.hidden", (S, N + 1, d))
    for s in range(S):
        for i in range(N + 1):
            if is_planted[s, i]:
                hidden[s, i] += np.float32(beta * math.sqrt(d)) * head_f[tok[s, i]]
    planted = np.where(is_planted, tok, -1).astype(np.int32)
    other = r.integers(0, V - 1, size=(S, N)).astype(np.int32)
    hit = r.random((S, N)) < p_accept
    drafts = np.where(hit & (planted[:, :N] >= 0), planted[:, :N],
                      np.where(other >= tok[:, :N], other + 1, other)).astype(np.int32)
    del head_f
    return HiddenVerifyInputs(d, V, head_dtype, head, g, eps, hidden, drafts, planted)


@dataclass
class Workload:
    name: str
    model: Optional[Model]
    draft: Optional[DraftInputs]
    greedy: Optional[GreedyVerifyInputs] = None
    sample: Optional[SampleVerifyInputs] = None
    hidden: Optional[HiddenVerifyInputs] = None
    p_accept: float = 0.0
    plant_mode: str = "max5"


def c1_tiny(seed: int = 0, **over) -> Workload:
    """Tiny fp32: d=256, 1 block, 4/1 heads of 64, 512 KV cells, V=4096, N=3."""
    shape = dict(d_model=256, d_hprev=256, n_blocks=1, n_head_q=4, n_head_kv=1, head_dim=64, d_ff=1024,
                 n_vocab=4096)
    shape.update({k: v for k, v in over.items() if k in shape})
    m = make_model(seed, **shape, w_dtype=F32, head_dtype=F32, kv_dtype=F32)
    ctx = over.get("ctx", 512)
    S = over.get("n_seq", 1)
    N = over.get("n_steps", 3)
    dr = make_draft_inputs(seed, m, [ctx] * S, N)
    gv = make_greedy_verify(seed, S, N, m.n_vocab, 0.8, "add5")
    return Workload("c1_tiny_fp32", m, dr, gv, p_accept=0.8, plant_mode="add5")


def c2_gemma_bf16(seed: int = 1, **over) -> Workload:
    """Gemma-4-26B-like assistant, bf16: 4 blocks, full KV 8192, V=262144, S=1, N=3."""
    shape = dict(C2_SHAPE)
    shape.update({k: v for k, v in over.items() if k in shape})
    m = make_model(seed, **shape, w_dtype=BF16, head_dtype=BF16, kv_dtype=BF16, head_std=1.0 / math.sqrt(1024))
    ctx = over.get("ctx", 8192)
    S = over.get("n_seq", 1)
    N = over.get("n_steps", 3)
    dr = make_draft_inputs(seed, m, [ctx] * S, N)
    gv = make_greedy_verify(seed, S, N, m.n_vocab, 0.8, "max5")
    return Workload("c2_gemma26b_like_bf16", m, dr, gv, p_accept=0.8)


def c3_interleaved(seed: int = 1, data_seed: int = 2, **over) -> Workload:
    """Same drafter as c2; blocks 0-2 read a 1024-window SWA ring, block 3 the
    full 32768-cell KV; 16 sequences with ctx ~ U{4096..32768}, N=3."""
    shape = dict(C2_SHAPE)
    shape.update({k: v for k, v in over.items() if k in shape})
    m = make_model(seed, **shape, w_dtype=BF16, head_dtype=BF16, kv_dtype=BF16, swa_window=over.get("swa_window", 1024),
                   block_src=[KV_SWA, KV_SWA, KV_SWA, KV_FULL][:shape["n_blocks"]], head_std=1.0 / math.sqrt(1024))
    S = over.get("n_seq", 16)
    lo, hi = over.get("ctx_range", (4096, 32768))
    ctx = rng_for(data_seed, "c3.ctx").integers(lo, hi + 1, size=S)
    N = over.get("n_steps", 3)
    dr = make_draft_inputs(data_seed, m, list(ctx), N, full_cap=over.get("full_cap", hi))
    gv = make_greedy_verify(data_seed, S, N, m.n_vocab, 0.8, "max5")
    return Workload("c3_interleaved_swa_full", m, dr, gv, p_accept=0.8)


def c4_longctx_q8(seed: int = 3, **over) -> Workload:
    """Full KV 131072 (bf16), Q8_0 tied head V=262144, 8 sequences, N=4."""
    shape = dict(C2_SHAPE)
    shape.update({k: v for k, v in over.items() if k in shape})
    m = make_model(seed, **shape, w_dtype=BF16, head_dtype=Q8_0, kv_dtype=BF16, head_std=1.0 / math.sqrt(1024))
    S = over.get("n_seq", 8)
    ctx = over.get("ctx", 131072)
    N = over.get("n_steps", 4)
    dr = make_draft_inputs(seed, m, [ctx] * S, N)
    gv = make_greedy_verify(seed, S, N, m.n_vocab, 0.7, "max5")
    return Workload("c4_longctx_q8_0_head", m, dr, gv, p_accept=0.7)


def c5_sample(seed: int = 4, **over) -> Workload:
    """Verify only: V=248320, 32 sequences x 4 drafts, temperature 0.6."""
    S = over.get("n_seq", 32)
    N = over.get("n_draft", 4)
    V = over.get("n_vocab", 248320)
    sv = make_sample_verify(seed, S, N, V, one_hot=over.get("one_hot", False),
                            draft_mode=over.get("draft_mode", "sample"))
    return Workload("c5_exact_sampling_verify", None, None, sample=sv)


def c6_centroid(seed: int = 1, **over) -> Workload:
    """The c2 drafter shape with a centroid LM head instead of the dense tied
    head: 2048 centroids of 128 token ids each, top 32 centroids (4096
    candidate rows) per step; full KV 8192, S=1, N=3."""
    shape = dict(C2_SHAPE)
    shape.update({k: v for k, v in over.items() if k in shape})
    m = make_model(seed, **shape, w_dtype=BF16, head_dtype=BF16, kv_dtype=BF16, head_std=1.0 / math.sqrt(1024),
                   n_centroids=over.get("n_centroids", 2048), centroid_top_k=over.get("centroid_top_k", 32))
    ctx = over.get("ctx", 8192)
    S = over.get("n_seq", 1)
    N = over.get("n_steps", 3)
    dr = make_draft_inputs(seed, m, [ctx] * S, N)
    gv = make_greedy_verify(seed, S, N, m.n_vocab, 0.8, "max5")
    return Workload("c6_centroid_head_bf16", m, dr, gv, p_accept=0.8)


def c7_sink_window(seed: int = 1, data_seed: int = 5, **over) -> Workload:
    """The c2 drafter with every block reading a sink + window source: 64 sink
    cells plus a 257-cell window [attn_pos - 256, attn_pos] over a 12000-cell
    cache (at most 321 cells, the report's count); 8 sequences
    with ctx ~ U{2000..12000}, half of them with a valid run that starts
    inside the window (a recent prefill of fewer rows than the window), B=4."""
    shape = dict(C2_SHAPE)
    shape.update({k: v for k, v in over.items() if k in shape})
    m = make_model(seed, **shape, w_dtype=BF16, head_dtype=BF16, kv_dtype=BF16, swa_window=over.get("swa_window", 0),
                   block_src=over.get("block_src", [KV_SINK_WINDOW] * shape["n_blocks"]),
                   head_std=1.0 / math.sqrt(1024))
    m.sw_window, m.sw_sink = over.get("sw_window", 257), over.get("sw_sink", 64)
    S = over.get("n_seq", 8)
    lo, hi = over.get("ctx_range", (2000, 12000))
    r = rng_for(data_seed, "c7.ctx")
    ctx = r.integers(lo, hi + 1, size=S)
    run = [int(c) - int(r.integers(1, m.sw_window)) if s % 2 else 0 for s, c in enumerate(ctx)]
    N = over.get("n_steps", 3)
    dr = make_draft_inputs(data_seed, m, list(ctx), N, full_cap=over.get("full_cap", hi), run_lo=run)
    gv = make_greedy_verify(data_seed, S, N, m.n_vocab, 0.8, "max5")
    return Workload("c7_sink_window", m, dr, gv, p_accept=0.8)


def c8_hidden_verify(seed: int = 6, **over) -> Workload:
    """Verify from the target's hidden rows: Gemma-4-26B-like backbone width
    2816, bf16 LM head V=262144 with its final-norm gain; 16 sequences x
    (1 + 3) rows."""
    hv = make_hidden_verify(seed, over.get("n_seq", 16), over.get("n_draft", 3), over.get("d", 2816),
                            over.get("n_vocab", 262144), head_dtype=over.get("head_dtype", BF16),
                            p_accept=over.get("p_accept", 0.8), gain=over.get("gain", True))
    return Workload("c8_hidden_state_verify", None, None, hidden=hv, p_accept=0.8)


CONFIGS = {"c1": c1_tiny, "c2": c2_gemma_bf16, "c3": c3_interleaved, "c4": c4_longctx_q8, "c5": c5_sample,
           "c6": c6_centroid, "c7": c7_sink_window, "c8": c8_hidden_verify}


# ----------------------------------------------------------------------------
# toy model for the temperature>0 Monte-Carlo check (V = 6)
# ----------------------------------------------------------------------------
@dataclass
class ToyLM:
    """z(ctx)[t] = a[t] + B[last(ctx)][t] + c * [t in ctx]: history-dependent
    logits over 6 tokens (the shape of the pages' toy check)."""
    a: np.ndarray
    B: np.ndarray
    c: float

    def logits(self, ctx_last: np.ndarray, ctx_member: np.ndarray) -> np.ndarray:
        """ctx_last: int [n]; ctx_member: bool [n, 6] -> f32 [n, 6]."""
        return (self.a[None, :] + self.B[ctx_last] + self.c * ctx_member).astype(np.float32)


def make_toy(seed: int, scale: float = 0.6, c: float = 0.5) -> ToyLM:
    r = rng_for(seed, "toy")
    return ToyLM(a=(scale * r.standard_normal(6)).astype(np.float32),
                 B=(scale * r.standard_normal((6, 6))).astype(np.float32), c=c)
