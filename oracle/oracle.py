"""ctypes front end of the CPU oracle (libmtp_oracle.so).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the bench's
cpu_baseline leg, never by the product path.  It marshals mtp_synth inputs
into the oracle's own structs; all arithmetic lives in mtp_oracle.c.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from pathlib import Path
from typing import Optional

import numpy as np

import mtp_synth as syn

HERE = Path(__file__).resolve().parent
# MTP_ORACLE_LIB names another build of the same sources (the sanitizer
# build of oracle/sanitize_check.py); by default the optimised one below
LIB_PATH = Path(os.environ.get("MTP_ORACLE_LIB", str(HERE / "libmtp_oracle.so")))
SOURCES = [HERE / "mtp_oracle.c", HERE / "mtp_oracle.h"]
MAXB = 8


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math, no FMA contraction)."""
    if "MTP_ORACLE_LIB" in os.environ:
        return LIB_PATH         # an externally built variant: used as it is
    if force or not LIB_PATH.exists() or any(s.stat().st_mtime > LIB_PATH.stat().st_mtime for s in SOURCES):
        tmp = LIB_PATH.with_suffix(".so.tmp")
        cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-Wall", "-Wno-unknown-pragmas", "-o", str(tmp), str(HERE / "mtp_oracle.c"), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class OrcModel(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("d_model", "d_hprev", "n_blocks", "n_head_q", "n_head_kv", "head_dim",
                                          "d_ff", "n_vocab", "w_dtype", "head_dtype", "kv_dtype", "swa_window")] + \
               [("block_src", C.c_int32 * MAXB)] + \
               [(n, C.c_double) for n in ("rms_eps", "rope_theta", "attn_scale", "embed_scale")] + \
               [("n_centroids", C.c_int32), ("centroid_top_k", C.c_int32), ("sw_window", C.c_int32),
                ("sw_sink", C.c_int32)]


class OrcWeights(C.Structure):
    _fields_ = [("w_pre", C.c_void_p), ("w_post", C.c_void_p), ("head", C.c_void_p), ("g_final", C.c_void_p)] + \
               [(n, C.c_void_p * MAXB) for n in ("g_attn", "w_q", "g_q", "w_o", "g_mlp", "w_up", "w_down")] + \
               [("centroids", C.c_void_p), ("token_ordering", C.c_void_p)]


class OrcKV(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("n_cells", C.c_int64), ("cell_stride", C.c_int64)]


class OrcSeq(C.Structure):
    _fields_ = [("src", OrcKV * 3), ("attn_pos", C.c_int32), ("pos0", C.c_int32), ("run_lo", C.c_int32)]


class OrcSampler(C.Structure):
    _fields_ = [(n, C.c_double) for n in ("temp", "top_p", "min_p", "rep_penalty", "presence_penalty",
                                           "freq_penalty")] + \
               [("top_k", C.c_int32), ("penalty_last_n", C.c_int32), ("seed", C.c_uint64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            build(force=False)
        L = C.CDLL(str(LIB_PATH))
        P = C.c_void_p
        L.orc_load.restype = C.c_double
        L.orc_load.argtypes = [P, C.c_int32, C.c_int64, C.c_int64, C.c_int64]
        L.orc_rmsnorm.argtypes = [C.c_int32, P, P, C.c_double, P]
        L.orc_rope.argtypes = [C.c_int32, C.c_int64, C.c_double, P, P]
        L.orc_attend_group.argtypes = [C.POINTER(OrcModel), C.POINTER(OrcSeq), C.c_int32, C.c_int32, P, P]
        L.orc_argmax_f32.restype = C.c_int32
        L.orc_argmax_f32.argtypes = [C.c_int64, P, P]
        L.orc_splitmix64_next.restype = C.c_uint64
        L.orc_splitmix64_next.argtypes = [C.POINTER(C.c_uint64)]
        L.orc_rng_u64.restype = C.c_uint64
        L.orc_rng_u64.argtypes = [C.c_uint64] * 6
        L.orc_uniform.restype = C.c_float
        L.orc_uniform.argtypes = [C.c_uint64] * 6
        L.orc_draft_block.argtypes = [C.POINTER(OrcModel), C.POINTER(OrcWeights), C.c_int32, P, P, P, C.c_int32,
                                      P, P, P, P, P]
        L.orc_visible_cells.restype = C.c_int64
        L.orc_visible_cells.argtypes = [C.POINTER(OrcModel), P, C.c_int32, P, C.c_int64]
        L.orc_centroid_logits.restype = C.c_double
        L.orc_centroid_logits.argtypes = [C.POINTER(OrcModel), C.POINTER(OrcWeights), P, P]
        L.orc_confidence.restype = C.c_double
        L.orc_confidence.argtypes = [C.c_int64, P]
        L.orc_pmin_trim.argtypes = [C.c_int32, C.c_int32, P, C.c_double, C.c_double, P, P, P]
        L.orc_verify_greedy.argtypes = [C.c_int32, C.c_int32, C.c_int32, P, P, P, P]
        L.orc_verify_greedy_hidden.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_int32, P, P, C.c_int32, P,
                                               C.c_double, P, P, P, P]
        L.orc_sample_dist.argtypes = [C.c_int32, P, P, C.c_int32, C.POINTER(OrcSampler), P, P]
        L.orc_verify_sample.argtypes = [C.c_int32, C.c_int32, C.c_int32, P, P, P, P, C.c_int32, P,
                                        C.POINTER(OrcSampler), C.c_uint64, P, P, P]
        L.orc_verify_sample_hidden.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_int32, P, P, C.c_int32, P,
                                               C.c_double, P, P, P, C.c_int32, P, C.POINTER(OrcSampler),
                                               C.c_uint64, P, P, P]
        L.orc_verify_greedy_match.argtypes = [C.c_int32, C.c_int32, C.c_int32, P, P, P, C.c_int32, P,
                                              C.POINTER(OrcSampler), C.c_uint64, P, P]
        L.orc_sample_row.restype = C.c_int32
        L.orc_sample_row.argtypes = [C.c_int32, P, P, C.c_int32, C.POINTER(OrcSampler), C.c_uint64, C.c_uint64,
                                     C.c_uint64, C.c_uint64]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def orc_model(m: syn.Model) -> OrcModel:
    om = OrcModel()
    for n in ("d_model", "d_hprev", "n_blocks", "n_head_q", "n_head_kv", "head_dim", "d_ff", "n_vocab", "w_dtype",
              "head_dtype", "kv_dtype", "swa_window"):
        setattr(om, n, int(getattr(m, n)))
    for l in range(MAXB):
        om.block_src[l] = m.block_src[l] if l < len(m.block_src) else 0
    om.rms_eps, om.rope_theta, om.attn_scale, om.embed_scale = m.rms_eps, m.rope_theta, m.attn_scale, m.embed_scale
    om.n_centroids, om.centroid_top_k = m.n_centroids, m.centroid_top_k
    om.sw_window, om.sw_sink = m.sw_window, m.sw_sink
    return om


def orc_weights(m: syn.Model) -> OrcWeights:
    W = m.weights
    ow = OrcWeights()
    ow.w_pre, ow.w_post, ow.head, ow.g_final = (_p(W[k]) for k in ("w_pre", "w_post", "head", "g_final"))
    for l in range(m.n_blocks):
        nm = m.block_names(l)
        for k in ("g_attn", "w_q", "g_q", "w_o", "g_mlp", "w_up", "w_down"):
            getattr(ow, k)[l] = _p(W[nm[k]])
    if m.n_centroids:
        ow.centroids, ow.token_ordering = _p(W["centroids"]), _p(W["token_ordering"])
    return ow


def orc_seqs(m: syn.Model, seqs) -> C.Array:
    arr = (OrcSeq * len(seqs))()
    for i, s in enumerate(seqs):
        for j, src in enumerate(s.src):
            if src is not None:
                arr[i].src[j].k, arr[i].src[j].v = _p(src.k), _p(src.v)
                arr[i].src[j].n_cells = src.n_cells
                arr[i].src[j].cell_stride = m.n_head_kv * m.head_dim
        arr[i].attn_pos, arr[i].pos0, arr[i].run_lo = s.attn_pos, s.pos0, s.run_lo
    return arr


def draft_block(m: syn.Model, dr: syn.DraftInputs, seq_idx=None, want_logits: bool = True, n_steps=None,
                last_tok=None, h_prev=None, pos0_shift: int = 0):
    """Run the oracle chain; returns dict(drafts, h_last, logits, margin)."""
    idx = list(range(len(dr.seqs))) if seq_idx is None else list(seq_idx)
    seqs = [dr.seqs[i] for i in idx]
    S = len(seqs)
    N = n_steps or dr.n_steps
    om, ow = orc_model(m), orc_weights(m)
    sa = orc_seqs(m, seqs)
    for i in range(S):
        sa[i].pos0 = seqs[i].pos0 + pos0_shift
    lt = np.ascontiguousarray(dr.last_tok[idx] if last_tok is None else last_tok, dtype=np.int32)
    hp = np.ascontiguousarray(dr.h_prev[idx] if h_prev is None else h_prev, dtype=np.float32)
    drafts = np.zeros((S, N), np.int32)
    h_last = np.zeros((S, m.d_hprev), np.float32)
    logits = np.zeros((S, N, m.n_vocab), np.float32) if want_logits else None
    margin = np.zeros((S, N), np.float64)
    conf = np.zeros((S, N), np.float64)
    rc = lib().orc_draft_block(C.byref(om), C.byref(ow), S, C.cast(sa, C.c_void_p), _p(lt), _p(hp), N, _p(drafts),
                               _p(h_last), _p(logits), _p(margin), _p(conf))
    if rc != 0:
        raise RuntimeError(f"orc_draft_block failed: {rc}")
    return dict(drafts=drafts, h_last=h_last, logits=logits, margin=margin, conf=conf)


def centroid_logits(m: syn.Model, f: np.ndarray):
    """Centroid head of one final-normed vector f -> (full fp32 row, top-k boundary margin)."""
    om, ow = orc_model(m), orc_weights(m)
    f = np.ascontiguousarray(f, dtype=np.float64)
    z = np.zeros(m.n_vocab, np.float32)
    margin = lib().orc_centroid_logits(C.byref(om), C.byref(ow), _p(f), _p(z))
    return z, margin


def visible_cells(m: syn.Model, seq, src: int) -> np.ndarray:
    om = orc_model(m)
    sa = orc_seqs(m, [seq])
    cap = seq.attn_pos + 1
    cells = np.zeros(max(cap, 1), np.int64)
    n = lib().orc_visible_cells(C.byref(om), C.cast(sa, C.c_void_p), src, _p(cells), cap)
    if n < 0:
        raise RuntimeError(f"orc_visible_cells failed: {n}")
    return cells[:n]


def confidence(z: np.ndarray) -> float:
    z = np.ascontiguousarray(z, dtype=np.float32)
    return float(lib().orc_confidence(len(z), _p(z)))


def pmin_trim(drafts: np.ndarray, conf: np.ndarray, p_min: float, tol: float = 0.0):
    """-> (trimmed drafts, n_keep, near flags)"""
    d = np.ascontiguousarray(drafts, dtype=np.int32).copy()
    c = np.ascontiguousarray(conf, dtype=np.float64)
    S, N = d.shape
    keep = np.zeros(S, np.int32)
    near = np.zeros(S, np.int32)
    rc = lib().orc_pmin_trim(S, N, _p(c), C.c_double(p_min), C.c_double(tol), _p(d), _p(keep), _p(near))
    if rc != 0:
        raise RuntimeError(f"orc_pmin_trim failed: {rc}")
    return d, keep, near


def verify_greedy(logits: np.ndarray, drafts: np.ndarray):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    drafts = np.ascontiguousarray(drafts, dtype=np.int32)
    S, R, V = logits.shape
    tokens = np.zeros((S, R), np.int32)
    n_acc = np.zeros(S, np.int32)
    rc = lib().orc_verify_greedy(S, R - 1, V, _p(logits), _p(drafts), _p(tokens), _p(n_acc))
    if rc != 0:
        raise RuntimeError(f"orc_verify_greedy failed: {rc}")
    return tokens, n_acc


def verify_greedy_hidden(hidden: np.ndarray, head: np.ndarray, head_dtype: int, n_vocab: int, g, eps: float,
                         drafts: np.ndarray):
    """hidden fp32 [S, N+1, d]; head in its storage format (f32 / bf16 bits
    [V, d], or Q8_0 blocks); g fp32 [d] or None.  -> (tokens, n_accept,
    margins [S, N+1])"""
    hidden = np.ascontiguousarray(hidden, dtype=np.float32)
    drafts = np.ascontiguousarray(drafts, dtype=np.int32)
    head = np.ascontiguousarray(head)
    S, R, d = hidden.shape
    gp = None if g is None else np.ascontiguousarray(g, dtype=np.float32)
    tokens = np.zeros((S, R), np.int32)
    n_acc = np.zeros(S, np.int32)
    margin = np.zeros((S, R), np.float64)
    rc = lib().orc_verify_greedy_hidden(S, R - 1, int(n_vocab), d, _p(hidden), _p(head), int(head_dtype),
                                        _p(gp) if gp is not None else None, float(eps), _p(drafts), _p(tokens),
                                        _p(n_acc), _p(margin))
    if rc != 0:
        raise RuntimeError(f"orc_verify_greedy_hidden failed: {rc}")
    return tokens, n_acc, margin


def sampler_struct(sp: syn.Sampler) -> OrcSampler:
    o = OrcSampler()
    o.temp, o.top_p, o.min_p = sp.temp, sp.top_p, sp.min_p
    o.rep_penalty, o.presence_penalty, o.freq_penalty = sp.rep_penalty, sp.presence_penalty, sp.freq_penalty
    o.top_k, o.penalty_last_n, o.seed = sp.top_k, sp.penalty_last_n, sp.seed
    return o


def sample_dist(z: np.ndarray, ctx, sp: syn.Sampler):
    z = np.ascontiguousarray(z, dtype=np.float32)
    ctx = np.ascontiguousarray(np.asarray(ctx, dtype=np.int32))
    p = np.zeros(z.size, np.float64)
    fl = C.c_int32(0)
    o = sampler_struct(sp)
    n = lib().orc_sample_dist(z.size, _p(z), _p(ctx) if ctx.size else None, ctx.size, C.byref(o), _p(p), C.byref(fl))
    if n < 0:
        raise RuntimeError(f"orc_sample_dist failed: {n}")
    return p, fl.value


def verify_sample(p_logits, q_logits, drafts, history, history_len, sp: syn.Sampler, round_: int = 0):
    p_logits = np.ascontiguousarray(p_logits, dtype=np.float32)
    q_logits = None if q_logits is None else np.ascontiguousarray(q_logits, dtype=np.float32)
    drafts = np.ascontiguousarray(drafts, dtype=np.int32)
    history = np.ascontiguousarray(history, dtype=np.int32)
    history_len = np.ascontiguousarray(history_len, dtype=np.int32)
    S, R, V = p_logits.shape
    tokens = np.zeros((S, R), np.int32)
    n_acc = np.zeros(S, np.int32)
    flags = np.zeros(S, np.int32)
    o = sampler_struct(sp)
    rc = lib().orc_verify_sample(S, R - 1, V, _p(p_logits), _p(q_logits), _p(drafts) if drafts.size else None,
                                 _p(history) if history.size else None, history.shape[1] if history.ndim == 2 else 0,
                                 _p(history_len), C.byref(o), round_, _p(tokens), _p(n_acc), _p(flags))
    if rc != 0:
        raise RuntimeError(f"orc_verify_sample failed: {rc}")
    return tokens, n_acc, flags


def verify_sample_hidden(hidden: np.ndarray, head: np.ndarray, head_dtype: int, n_vocab: int, g, eps: float,
                         q_logits, drafts, history, history_len, sp: syn.Sampler, round_: int = 0):
    """hidden fp32 [S, N+1, d] and the head as for verify_greedy_hidden; the
    rest as for verify_sample.  -> (tokens, n_accept, flags)"""
    hidden = np.ascontiguousarray(hidden, dtype=np.float32)
    head = np.ascontiguousarray(head)
    q_logits = None if q_logits is None else np.ascontiguousarray(q_logits, dtype=np.float32)
    drafts = np.ascontiguousarray(drafts, dtype=np.int32)
    history = np.ascontiguousarray(history, dtype=np.int32)
    history_len = np.ascontiguousarray(history_len, dtype=np.int32)
    gp = None if g is None else np.ascontiguousarray(g, dtype=np.float32)
    S, R, d = hidden.shape
    tokens = np.zeros((S, R), np.int32)
    n_acc = np.zeros(S, np.int32)
    flags = np.zeros(S, np.int32)
    o = sampler_struct(sp)
    rc = lib().orc_verify_sample_hidden(S, R - 1, int(n_vocab), d, _p(hidden), _p(head), int(head_dtype),
                                        _p(gp) if gp is not None else None, float(eps), _p(q_logits),
                                        _p(drafts) if drafts.size else None, _p(history) if history.size else None,
                                        history.shape[1] if history.ndim == 2 else 0, _p(history_len), C.byref(o),
                                        round_, _p(tokens), _p(n_acc), _p(flags))
    if rc != 0:
        raise RuntimeError(f"orc_verify_sample_hidden failed: {rc}")
    return tokens, n_acc, flags


def verify_greedy_match(p_logits, drafts, history, history_len, sp: syn.Sampler, round_: int = 0):
    p_logits = np.ascontiguousarray(p_logits, dtype=np.float32)
    drafts = np.ascontiguousarray(drafts, dtype=np.int32)
    history = np.ascontiguousarray(history, dtype=np.int32)
    history_len = np.ascontiguousarray(history_len, dtype=np.int32)
    S, R, V = p_logits.shape
    tokens = np.zeros((S, R), np.int32)
    n_acc = np.zeros(S, np.int32)
    o = sampler_struct(sp)
    rc = lib().orc_verify_greedy_match(S, R - 1, V, _p(p_logits), _p(drafts), _p(history), history.shape[1],
                                       _p(history_len), C.byref(o), round_, _p(tokens), _p(n_acc))
    if rc != 0:
        raise RuntimeError(f"orc_verify_greedy_match failed: {rc}")
    return tokens, n_acc


def sample_row(z, ctx, sp: syn.Sampler, s: int, round_: int, i: int, stream: int) -> int:
    z = np.ascontiguousarray(z, dtype=np.float32)
    ctx = np.ascontiguousarray(np.asarray(ctx, dtype=np.int32))
    o = sampler_struct(sp)
    return int(lib().orc_sample_row(z.size, _p(z), _p(ctx) if ctx.size else None, ctx.size, C.byref(o), s, round_, i,
                                    stream))


def uniform(seed, s, round_, i, stream, t) -> float:
    return float(lib().orc_uniform(seed, s, round_, i, stream, t))


def rng_u64(seed, s, round_, i, stream, t) -> int:
    return int(lib().orc_rng_u64(seed, s, round_, i, stream, t))


def splitmix64_stream(state: int, n: int):
    st = C.c_uint64(state)
    return [int(lib().orc_splitmix64_next(C.byref(st))) for _ in range(n)]


def rmsnorm(x, g, eps):
    x = np.ascontiguousarray(x, dtype=np.float64)
    g = np.ascontiguousarray(g, dtype=np.float32)
    y = np.zeros_like(x)
    lib().orc_rmsnorm(x.size, _p(x), _p(g), eps, _p(y))
    return y


def rope(x, pos, theta=10000.0):
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.zeros_like(x)
    lib().orc_rope(x.size, pos, theta, _p(x), _p(y))
    return y


def attend_group(m: syn.Model, seq: syn.Seq, src: int, kvh: int, q_group: np.ndarray):
    g = m.n_head_q // m.n_head_kv
    q_group = np.ascontiguousarray(q_group, dtype=np.float64).reshape(-1)
    o = np.zeros(g * m.head_dim, np.float64)
    om = orc_model(m)
    sa = orc_seqs(m, [seq])
    rc = lib().orc_attend_group(C.byref(om), C.byref(sa[0]), src, kvh, _p(q_group), _p(o))
    if rc != 0:
        raise RuntimeError(f"orc_attend_group failed: {rc}")
    return o.reshape(g, m.head_dim)


def argmax_f32(z):
    z = np.ascontiguousarray(z, dtype=np.float32)
    mg = C.c_double(0)
    i = lib().orc_argmax_f32(z.size, _p(z), C.byref(mg))
    return int(i), mg.value


def load(arr: np.ndarray, dtype: int, row: int, col: int, ncols: int) -> float:
    return float(lib().orc_load(_p(arr), dtype, row, col, ncols))
