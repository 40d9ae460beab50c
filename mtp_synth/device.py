"""Move synthetic inputs into device memory and describe them to the library.

Marshalling only: numpy arrays become torch device tensors with the same
bytes, and the ctypes structs of the binding point at them.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np

import mtp_synth as syn


def to_dev(a: np.ndarray, device):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def upload_model(m: syn.Model, device, max_seqs: int, max_steps: int):
    """Returns (desc, weights_struct, tensors)."""
    import mtp_draft_verify_amd as mtp
    t: Dict[str, object] = {k: to_dev(v, device) for k, v in m.weights.items()}
    desc = mtp.make_desc(d_model=m.d_model, d_hprev=m.d_hprev, n_blocks=m.n_blocks, n_head_q=m.n_head_q,
                         n_head_kv=m.n_head_kv, head_dim=m.head_dim, d_ff=m.d_ff, n_vocab=m.n_vocab,
                         w_dtype=m.w_dtype, head_dtype=m.head_dtype, kv_dtype=m.kv_dtype, swa_window=m.swa_window,
                         block_src=m.block_src, rms_eps=m.rms_eps, rope_theta=m.rope_theta,
                         attn_scale=m.attn_scale, embed_scale=m.embed_scale, max_seqs=max_seqs, max_steps=max_steps,
                         n_centroids=m.n_centroids, centroid_top_k=m.centroid_top_k, sw_window=m.sw_window,
                         sw_sink=m.sw_sink)
    w = mtp.make_weights(t, m.n_blocks)
    return desc, w, t


def upload_seqs(m: syn.Model, dr: syn.DraftInputs, device, seq_idx=None):
    """Returns (seq dicts for mtp.make_seqs, last_tok, h_prev, kept tensors)."""
    idx = list(range(len(dr.seqs))) if seq_idx is None else list(seq_idx)
    keep: List[object] = []
    cache = {}
    seqs = []
    stride = m.n_head_kv * m.head_dim
    for i in idx:
        s = dr.seqs[i]
        srcs = []
        for src in s.src:
            if src is None:
                srcs.append(None)
                continue
            key = id(src)
            if key not in cache:
                cache[key] = (to_dev(src.k, device), to_dev(src.v, device))
                keep.extend(cache[key])
            k, v = cache[key]
            srcs.append((k, v, src.n_cells, stride))
        seqs.append(dict(src=srcs, attn_pos=s.attn_pos, pos0=s.pos0, run_lo=s.run_lo))
    last_tok = to_dev(dr.last_tok[idx].astype(np.int32), device)
    h_prev = to_dev(dr.h_prev[idx].astype(np.float32), device)
    return seqs, last_tok, h_prev, keep
