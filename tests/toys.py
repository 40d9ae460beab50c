"""Hand-built drafters whose draft tokens and logits have closed forms.

Input construction only (weights, caches); the expected values are derived in
the tests from the definitions the pages give, never from either
implementation.
"""
from __future__ import annotations

import math

import numpy as np

import mtp_synth as syn


def blank_model(d=8, dh=8, V=8, Hq=2, Hkv=1, hd=4, F=8, L=1, swa_window=0, block_src=None, seed=0):
    """fp32 toy drafter with random weights, then caller overwrites."""
    m = syn.make_model(seed, d_model=d, d_hprev=dh, n_blocks=L, n_head_q=Hq, n_head_kv=Hkv, head_dim=hd, d_ff=F,
                       n_vocab=V, w_dtype=syn.F32, head_dtype=syn.F32, kv_dtype=syn.F32, swa_window=swa_window,
                       block_src=block_src)
    # positive gains keep signs (and therefore argmaxes) predictable
    for k, v in list(m.weights.items()):
        if k.startswith("g_") or ".g_" in k:
            m.weights[k] = (1.0 + np.abs(v - 1.0)).astype(np.float32)
    return m


def zero_blocks(m):
    for l in range(m.n_blocks):
        nm = m.block_names(l)
        m.weights[nm["w_o"]] = np.zeros_like(m.weights[nm["w_o"]])
        m.weights[nm["w_down"]] = np.zeros_like(m.weights[nm["w_down"]])


def perm_matrix(perm):
    n = len(perm)
    P = np.zeros((n, n), np.float32)
    for j, pj in enumerate(perm):
        P[pj, j] = 1.0          # P e_j = e_{perm[j]}
    return P


def one_seq_inputs(m, n_cells, attn_pos, last_tok, h_prev, n_steps, kv=None, pos0=None):
    if kv is None:
        k = np.zeros((n_cells, m.n_head_kv, m.head_dim), np.float32)
        v = np.zeros_like(k)
    else:
        k, v = kv
    src = syn.KVSource(k, v)
    seq = syn.Seq([src, None], attn_pos=attn_pos, pos0=attn_pos + 1 if pos0 is None else pos0)
    return syn.DraftInputs([seq], np.array([last_tok], np.int32), np.asarray(h_prev, np.float32).reshape(1, -1),
                           n_steps)


def rms_scale(x, eps):
    """1/sqrt(mean(x^2)+eps) -- the RMSNorm definition."""
    return 1.0 / math.sqrt(float(np.mean(np.asarray(x, np.float64) ** 2)) + eps)
