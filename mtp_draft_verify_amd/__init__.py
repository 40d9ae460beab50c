"""Python binding of libmtp.so (include/mtp.h): argument marshalling only.

Every step of the draft chain and the verify runs in the library's HIP kernels;
this module only builds the C structs from torch tensors (device memory and
the current HIP stream) and raises on a non-zero status.  It fails loudly when
the library is missing: there is no fallback path.

The module-level functions carry the C names (mtp_ctx_create, mtp_draft_block, mtp_draft_block_conf,
mtp_verify_greedy, mtp_verify_sample, mtp_verify_sample_hidden, mtp_ctx_destroy, mtp_strerror,
mtp_check_desc); `Context` is a small owner around them.
"""
from __future__ import annotations

import ctypes as C
from pathlib import Path
from typing import Dict, Optional, Sequence

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libmtp.so"

MTP_OK, MTP_E_INVAL, MTP_E_SHAPE, MTP_E_DTYPE, MTP_E_NOMEM, MTP_E_DEVICE, MTP_E_NOWEIGHTS, MTP_E_BUSY = \
    0, -1, -2, -3, -4, -5, -6, -7
MTP_F32, MTP_BF16, MTP_Q8_0 = 0, 1, 2
MTP_SRC_FULL, MTP_SRC_SWA, MTP_SRC_SINK_WINDOW = 0, 1, 2
MAX_BLOCKS = 8
MAX_SPLITS = 128
EXPORTS = ("mtp_ctx_create", "mtp_ctx_destroy", "mtp_draft_block", "mtp_draft_block_conf", "mtp_verify_greedy",
           "mtp_verify_greedy_hidden", "mtp_verify_sample", "mtp_verify_sample_hidden", "mtp_strerror", "mtp_check_desc", "mtp_profile_enable", "mtp_profile_read",
           "mtp_last_error", "mtp_verify_greedy_noalloc")
NOALLOC_MAX_ROWS = 16384
MTP_PROF_HEAD, MTP_PROF_ATTN, MTP_PROF_GEMV, MTP_PROF_VERIFY, MTP_PROF_MERGE, MTP_PROF_N = 0, 1, 2, 3, 4, 5


class MTPError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        detail = mtp_last_error() if code == MTP_E_DEVICE or code == MTP_E_NOMEM else ""
        super().__init__(f"{where}: {mtp_strerror(code)} ({code})" + (f" [{detail}]" if detail else ""))


class ModelDesc(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("d_model", "d_hprev", "n_blocks", "n_head_q", "n_head_kv", "head_dim",
                                          "d_ff", "n_vocab", "w_dtype", "head_dtype", "kv_dtype", "swa_window")] + \
               [("block_src", C.c_int32 * MAX_BLOCKS)] + \
               [(n, C.c_float) for n in ("rms_eps", "rope_theta", "attn_scale", "embed_scale")] + \
               [("max_seqs", C.c_int32), ("max_steps", C.c_int32), ("n_centroids", C.c_int32),
                ("centroid_top_k", C.c_int32), ("sw_window", C.c_int32), ("sw_sink", C.c_int32),
                ("hidden_d_max", C.c_int32), ("hidden_sample", C.c_int32)]


class Weights(C.Structure):
    _fields_ = [("w_pre", C.c_void_p), ("w_post", C.c_void_p), ("head", C.c_void_p), ("g_final", C.c_void_p)] + \
               [(n, C.c_void_p * MAX_BLOCKS) for n in ("g_attn", "w_q", "g_q", "w_o", "g_mlp", "w_up", "w_down")] + \
               [("centroids", C.c_void_p), ("token_ordering", C.c_void_p)]


class KVView(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("n_cells", C.c_int64), ("cell_stride", C.c_int64)]


N_SRC = 3     # full, SWA ring, sink + window


class LmHead(C.Structure):
    _fields_ = [("w", C.c_void_p), ("g_final", C.c_void_p), ("d", C.c_int32), ("n_vocab", C.c_int32),
                ("dtype", C.c_int32), ("rms_eps", C.c_float)]


class Seq(C.Structure):
    _fields_ = [("src", KVView * N_SRC), ("attn_pos", C.c_int32), ("pos0", C.c_int32), ("run_lo", C.c_int32),
                ("pad", C.c_int32)]


class Sampler(C.Structure):
    _fields_ = [(n, C.c_float) for n in ("temp", "top_p", "min_p", "rep_penalty", "presence_penalty",
                                          "freq_penalty")] + \
               [("top_k", C.c_int32), ("penalty_last_n", C.c_int32), ("seed", C.c_uint64)]


_lib = None


def lib() -> C.CDLL:
    """Load libmtp.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with mtp_draft_verify_amd/build.py "
                               "(or __graft_entry__.build()); there is no fallback path")
        # torch first: libmtp.so then binds to the HIP runtime torch already
        # loaded (same soname), so device pointers and streams from torch and
        # the library's kernels live in one runtime.  Loading the library
        # first would bring a second HIP/HSA runtime into the process.
        import torch  # noqa: F401
        L = C.CDLL(str(LIB_PATH))
        P = C.c_void_p
        L.mtp_ctx_create.argtypes = [C.POINTER(ModelDesc), C.POINTER(Weights), P, C.POINTER(P)]
        L.mtp_ctx_create.restype = C.c_int
        L.mtp_ctx_destroy.argtypes = [P]
        L.mtp_ctx_destroy.restype = None
        L.mtp_draft_block.argtypes = [P, C.c_int32, C.POINTER(Seq), P, P, C.c_int32, P, P, P]
        L.mtp_draft_block.restype = C.c_int
        L.mtp_draft_block_conf.argtypes = [P, C.c_int32, C.POINTER(Seq), P, P, C.c_int32, P, P, P, P, C.c_float, P]
        L.mtp_draft_block_conf.restype = C.c_int
        L.mtp_verify_greedy.argtypes = [P, C.c_int32, C.c_int32, C.c_int32, P, P, P, P]
        L.mtp_verify_greedy.restype = C.c_int
        L.mtp_verify_greedy_noalloc.argtypes = [P, C.c_int32, C.c_int32, C.c_int32, P, P, P, P]
        L.mtp_verify_greedy_noalloc.restype = C.c_int
        L.mtp_verify_greedy_hidden.argtypes = [P, C.c_int32, C.c_int32, C.POINTER(LmHead), P, P, P, P]
        L.mtp_verify_greedy_hidden.restype = C.c_int
        L.mtp_verify_sample.argtypes = [P, C.c_int32, C.c_int32, C.c_int32, P, P, P, P, C.c_int32, P,
                                        C.POINTER(Sampler), C.c_uint64, P, P]
        L.mtp_verify_sample.restype = C.c_int
        L.mtp_verify_sample_hidden.argtypes = [P, C.c_int32, C.c_int32, C.POINTER(LmHead), P, P, P, P, C.c_int32, P,
                                               C.POINTER(Sampler), C.c_uint64, P, P]
        L.mtp_verify_sample_hidden.restype = C.c_int
        L.mtp_strerror.argtypes = [C.c_int]
        L.mtp_strerror.restype = C.c_char_p
        L.mtp_last_error.argtypes = []
        L.mtp_last_error.restype = C.c_char_p
        L.mtp_check_desc.argtypes = [C.POINTER(ModelDesc)]
        L.mtp_check_desc.restype = C.c_int
        L.mtp_profile_enable.argtypes = [P, C.c_int]
        L.mtp_profile_enable.restype = C.c_int
        L.mtp_profile_read.argtypes = [P, C.c_int, C.POINTER(C.c_double), C.POINTER(C.c_int64)]
        L.mtp_profile_read.restype = C.c_int
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# --------------------------------------------------------------------------- C names
def mtp_strerror(code: int) -> str:
    return lib().mtp_strerror(code).decode()


def mtp_last_error() -> str:
    return lib().mtp_last_error().decode()


def mtp_check_desc(desc: ModelDesc) -> int:
    return lib().mtp_check_desc(C.byref(desc))


def mtp_ctx_create(desc: ModelDesc, weights: Optional[Weights], stream=None) -> int:
    out = C.c_void_p()
    rc = lib().mtp_ctx_create(C.byref(desc), C.byref(weights) if weights is not None else None,
                              _stream_handle(stream), C.byref(out))
    if rc != MTP_OK:
        raise MTPError(rc, "mtp_ctx_create")
    return out.value


def mtp_ctx_destroy(ctx: int) -> None:
    lib().mtp_ctx_destroy(ctx)


def mtp_draft_block(ctx: int, seqs, last_tok, h_prev, n_steps: int, out_drafts, out_h_last=None,
                    out_logits=None) -> None:
    arr = seqs if isinstance(seqs, C.Array) else make_seqs(seqs)
    rc = lib().mtp_draft_block(ctx, len(arr), arr, _ptr(last_tok), _ptr(h_prev), n_steps, _ptr(out_drafts),
                               _ptr(out_h_last), _ptr(out_logits))
    if rc != MTP_OK:
        raise MTPError(rc, "mtp_draft_block")


def mtp_draft_block_conf(ctx: int, seqs, last_tok, h_prev, n_steps: int, out_drafts, out_h_last=None,
                         out_logits=None, out_conf=None, p_min: float = 0.0, out_n_keep=None) -> None:
    arr = seqs if isinstance(seqs, C.Array) else make_seqs(seqs)
    rc = lib().mtp_draft_block_conf(ctx, len(arr), arr, _ptr(last_tok), _ptr(h_prev), n_steps, _ptr(out_drafts),
                                    _ptr(out_h_last), _ptr(out_logits), _ptr(out_conf), float(p_min),
                                    _ptr(out_n_keep))
    if rc != MTP_OK:
        raise MTPError(rc, "mtp_draft_block_conf")


def mtp_verify_greedy(ctx: int, n_seq: int, n_draft: int, n_vocab: int, logits, drafts, out_tokens,
                      out_n_accept) -> None:
    rc = lib().mtp_verify_greedy(ctx, n_seq, n_draft, n_vocab, _ptr(logits), _ptr(drafts), _ptr(out_tokens),
                                 _ptr(out_n_accept))
    if rc != MTP_OK:
        raise MTPError(rc, "mtp_verify_greedy")


def make_lm_head(w, g_final, d: int, n_vocab: int, dtype: int = MTP_BF16, rms_eps: float = 1e-6) -> LmHead:
    h = LmHead()
    h.w, h.g_final = _ptr(w), _ptr(g_final)
    h.d, h.n_vocab, h.dtype, h.rms_eps = int(d), int(n_vocab), int(dtype), float(rms_eps)
    return h


def mtp_verify_greedy_noalloc(stream, logits, drafts, out_tokens, out_n_accept) -> None:
    """The greedy verify without a context (static scratch, no allocation);
    stream: a torch stream, a raw handle, or None (torch's current stream)."""
    S, R, V = logits.shape
    rc = lib().mtp_verify_greedy_noalloc(_stream_handle(stream), S, R - 1, V, _ptr(logits), _ptr(drafts),
                                         _ptr(out_tokens), _ptr(out_n_accept))
    if rc != MTP_OK:
        raise MTPError(rc, "mtp_verify_greedy_noalloc")


def mtp_verify_greedy_hidden(ctx: int, n_seq: int, n_draft: int, head: LmHead, hidden, drafts, out_tokens,
                             out_n_accept) -> None:
    rc = lib().mtp_verify_greedy_hidden(ctx, n_seq, n_draft, C.byref(head), _ptr(hidden), _ptr(drafts),
                                        _ptr(out_tokens), _ptr(out_n_accept))
    if rc != MTP_OK:
        raise MTPError(rc, "mtp_verify_greedy_hidden")


def mtp_verify_sample(ctx: int, n_seq: int, n_draft: int, n_vocab: int, p_logits, q_logits, drafts, history,
                      history_stride: int, history_len, sampler: Sampler, round_: int, out_tokens,
                      out_n_accept) -> None:
    rc = lib().mtp_verify_sample(ctx, n_seq, n_draft, n_vocab, _ptr(p_logits), _ptr(q_logits), _ptr(drafts),
                                 _ptr(history), history_stride, _ptr(history_len), C.byref(sampler), round_,
                                 _ptr(out_tokens), _ptr(out_n_accept))
    if rc != MTP_OK:
        raise MTPError(rc, "mtp_verify_sample")


def mtp_verify_sample_hidden(ctx: int, n_seq: int, n_draft: int, head: LmHead, hidden, q_logits, drafts, history,
                             history_stride: int, history_len, sampler: Sampler, round_: int, out_tokens,
                             out_n_accept) -> None:
    rc = lib().mtp_verify_sample_hidden(ctx, n_seq, n_draft, C.byref(head), _ptr(hidden), _ptr(q_logits),
                                        _ptr(drafts), _ptr(history), history_stride, _ptr(history_len),
                                        C.byref(sampler), round_, _ptr(out_tokens), _ptr(out_n_accept))
    if rc != MTP_OK:
        raise MTPError(rc, "mtp_verify_sample_hidden")


def mtp_profile_enable(ctx: int, mask: int) -> None:
    """mask: bit (1 << class) enables event timing of that kernel class; 0 disables."""
    rc = lib().mtp_profile_enable(ctx, int(mask))
    if rc != MTP_OK:
        raise MTPError(rc, "mtp_profile_enable")


def mtp_profile_read(ctx: int, cls: int):
    """(total_ms, count) of one kernel class since the last enable/read."""
    t, n = C.c_double(), C.c_int64()
    rc = lib().mtp_profile_read(ctx, cls, C.byref(t), C.byref(n))
    if rc != MTP_OK:
        raise MTPError(rc, "mtp_profile_read")
    return t.value, n.value


# --------------------------------------------------------------------------- struct builders
def make_desc(*, d_model, d_hprev, n_blocks, n_head_q, n_head_kv, head_dim, d_ff, n_vocab, w_dtype, head_dtype,
              kv_dtype, swa_window=0, block_src=(), rms_eps=1e-6, rope_theta=10000.0, attn_scale=None,
              embed_scale=None, max_seqs=1, max_steps=4, n_centroids=0, centroid_top_k=0, sw_window=0,
              sw_sink=0, hidden_d_max=0, hidden_sample=0) -> ModelDesc:
    d = ModelDesc()
    for k, v in dict(d_model=d_model, d_hprev=d_hprev, n_blocks=n_blocks, n_head_q=n_head_q, n_head_kv=n_head_kv,
                     head_dim=head_dim, d_ff=d_ff, n_vocab=n_vocab, w_dtype=w_dtype, head_dtype=head_dtype,
                     kv_dtype=kv_dtype, swa_window=swa_window, max_seqs=max_seqs, max_steps=max_steps,
                     n_centroids=n_centroids, centroid_top_k=centroid_top_k, sw_window=sw_window,
                     sw_sink=sw_sink, hidden_d_max=hidden_d_max, hidden_sample=hidden_sample).items():
        setattr(d, k, int(v))
    for i in range(MAX_BLOCKS):
        d.block_src[i] = int(block_src[i]) if i < len(block_src) else 0
    d.rms_eps, d.rope_theta = rms_eps, rope_theta
    d.attn_scale = attn_scale if attn_scale is not None else head_dim ** -0.5
    d.embed_scale = embed_scale if embed_scale is not None else d_model ** 0.5
    return d


def make_weights(t: Dict[str, object], n_blocks: int) -> Weights:
    """t maps 'w_pre', 'w_post', 'head', 'g_final' and 'blk{l}.<name>' to device tensors
    (plus 'centroids' and 'token_ordering' for a centroid head)."""
    w = Weights()
    w.w_pre, w.w_post, w.head, w.g_final = (_ptr(t[k]) for k in ("w_pre", "w_post", "head", "g_final"))
    for l in range(n_blocks):
        for k in ("g_attn", "w_q", "g_q", "w_o", "g_mlp", "w_up", "w_down"):
            getattr(w, k)[l] = _ptr(t[f"blk{l}.{k}"])
    if "centroids" in t:
        w.centroids, w.token_ordering = _ptr(t["centroids"]), _ptr(t["token_ordering"])
    return w


def make_seqs(seqs: Sequence[dict]) -> C.Array:
    """seqs: dicts with attn_pos, pos0, optional run_lo, and per source (0 full,
    1 SWA ring, 2 sink + window) a tuple (k_tensor, v_tensor, n_cells,
    cell_stride) or None."""
    arr = (Seq * len(seqs))()
    for i, s in enumerate(seqs):
        srcs = tuple(s.get("src", ()))
        if len(srcs) > N_SRC:
            raise ValueError(f"at most {N_SRC} KV sources per sequence")
        for j, src in enumerate(srcs):
            if src is not None:
                k, v, n_cells, stride = src
                arr[i].src[j].k, arr[i].src[j].v = _ptr(k), _ptr(v)
                arr[i].src[j].n_cells, arr[i].src[j].cell_stride = int(n_cells), int(stride)
        arr[i].attn_pos, arr[i].pos0 = int(s["attn_pos"]), int(s["pos0"])
        arr[i].run_lo = int(s.get("run_lo", 0))
    return arr


def make_sampler(*, temp, top_p, min_p, rep_penalty, presence_penalty, freq_penalty=0.0, top_k=0,
                 penalty_last_n=64, seed=0) -> Sampler:
    sp = Sampler()
    sp.temp, sp.top_p, sp.min_p = temp, top_p, min_p
    sp.rep_penalty, sp.presence_penalty, sp.freq_penalty = rep_penalty, presence_penalty, freq_penalty
    sp.top_k, sp.penalty_last_n, sp.seed = top_k, penalty_last_n, seed
    return sp


class Context:
    """Owns one mtp_ctx (scratch sized at creation) bound to a HIP stream."""

    def __init__(self, desc: ModelDesc, weights: Optional[Weights] = None, stream=None, keepalive=None):
        self.desc = desc
        self._keep = keepalive          # device tensors the context borrows
        self.handle = mtp_ctx_create(desc, weights, stream)

    def draft_block(self, seqs, last_tok, h_prev, n_steps, out_drafts, out_h_last=None, out_logits=None):
        mtp_draft_block(self.handle, seqs, last_tok, h_prev, n_steps, out_drafts, out_h_last, out_logits)

    def draft_block_conf(self, seqs, last_tok, h_prev, n_steps, out_drafts, out_h_last=None, out_logits=None,
                         out_conf=None, p_min=0.0, out_n_keep=None):
        mtp_draft_block_conf(self.handle, seqs, last_tok, h_prev, n_steps, out_drafts, out_h_last, out_logits,
                             out_conf, p_min, out_n_keep)

    def verify_greedy(self, logits, drafts, out_tokens, out_n_accept):
        S, R, V = logits.shape
        mtp_verify_greedy(self.handle, S, R - 1, V, logits, drafts, out_tokens, out_n_accept)

    def verify_greedy_hidden(self, head: LmHead, hidden, drafts, out_tokens, out_n_accept):
        S, R, _ = hidden.shape
        mtp_verify_greedy_hidden(self.handle, S, R - 1, head, hidden, drafts, out_tokens, out_n_accept)

    def verify_sample(self, p_logits, q_logits, drafts, history, history_len, sampler, round_, out_tokens,
                      out_n_accept):
        S, R, V = p_logits.shape
        hs = history.shape[1] if history is not None and history.dim() == 2 else 0
        mtp_verify_sample(self.handle, S, R - 1, V, p_logits, q_logits, drafts, history, hs, history_len, sampler,
                          round_, out_tokens, out_n_accept)

    def verify_sample_hidden(self, head: LmHead, hidden, q_logits, drafts, history, history_len, sampler, round_,
                             out_tokens, out_n_accept):
        S, R, _ = hidden.shape
        hs = history.shape[1] if history is not None and history.dim() == 2 else 0
        mtp_verify_sample_hidden(self.handle, S, R - 1, head, hidden, q_logits, drafts, history, hs, history_len,
                                 sampler, round_, out_tokens, out_n_accept)

    def profile(self, mask: int):
        mtp_profile_enable(self.handle, mask)

    def profile_read(self, cls: int):
        return mtp_profile_read(self.handle, cls)

    def close(self):
        if self.handle:
            mtp_ctx_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
