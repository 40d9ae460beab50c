#!/usr/bin/env python3
"""Throughput of the fused MTP draft chain + greedy verify on one MI355X.

One step = one round of the hot path.  The default (headline) workload is the
largest configuration: 8 sequences, each with a full-attention bf16 KV of
131072 positions, a draft block of B-1 = 4 chained steps (embed +
pre-projection; 4 blocks of RMSNorm/Q/split-K GQA cross-attention/O/SiLU MLP;
final norm + 262144-row Q8_0 LM head + argmax; post-projection), then the
greedy verify over the target's [8, 5, 262144] fp32 logits.  Inputs are
synthetic, seeded, and resident in HBM before timing starts; --workload
selects the other configurations (extra measurements).

Prints one JSON line: draft tokens/s (= S * N / time per round), the
whole-round algorithmic HBM GB/s, the roofline of the round's dominant kernel
(algorithmic bytes per launch / its average launch time, measured with HIP
events on the library's stream after the timed region; the other of the two
large kernels in roofline_other) and the CPU oracle's throughput on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, AMD published
METRIC = "draft tokens/s of fused MTP chain (B-1 steps) + verify; HBM GB/s vs peak"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def weight_bytes(m, S=1):
    """Algorithmic bytes of the drafter weights read once per draft step
    (a centroid head reads its centroid matrix plus each sequence's
    candidate embedding rows)."""
    import mtp_synth as syn
    es = 4 if m.w_dtype == syn.F32 else 2
    d, dh, qd, F, V = m.d_model, m.d_hprev, m.n_head_q * m.head_dim, m.d_ff, m.n_vocab
    mats = d * (d + dh) + dh * d + m.n_blocks * (2 * qd * d + 2 * F * d)
    hes = 4 if m.head_dtype == syn.F32 else 2
    if m.n_centroids:
        head = m.n_centroids * d * es + S * m.centroid_top_k * (V // m.n_centroids) * d * hes
    elif m.head_dtype == syn.Q8_0:
        head = V * (d // 32) * 34
    else:
        head = V * d * hes
    gains = 4 * ((2 * m.n_blocks + 1) * d + m.n_blocks * m.head_dim)
    return mats * es, head, gains


def kv_bytes(m, seqs):
    import mtp_synth as syn
    es = 4 if m.kv_dtype == syn.F32 else 2
    tot = 0
    for s in seqs:
        for l in range(m.n_blocks):
            if m.block_src[l] == syn.KV_FULL:
                n_vis = s.attn_pos + 1
            elif m.block_src[l] == syn.KV_SWA:
                n_vis = s.attn_pos - max(0, s.attn_pos - m.swa_window + 1) + 1
            else:   # sink + window: [0, min(sink, first)) ++ [first, attn_pos]
                first = max(s.attn_pos - m.sw_window + 1, s.run_lo, 0)
                n_vis = min(m.sw_sink, first) + s.attn_pos - first + 1
            tot += n_vis * m.n_head_kv * m.head_dim * 2 * es
    return tot


HEAD_SOURCES = ["head_kernels.hip", "widen.h", "dev_common.h", "mtp_internal.h"]
COUNTERS_FILE = ROOT / "profiles" / "head_kernel_c2_hbm_counters.txt"
HV_SOURCES = ["hv_kernels.hip", "widen.h", "dev_common.h", "mtp_internal.h"]
HV_COUNTERS_FILE = ROOT / "profiles" / "hv_head_kernel_c8_hbm_counters.txt"


def head_traffic_from_counters(path=COUNTERS_FILE, sources=HEAD_SOURCES):
    """HBM bytes per launch of a kernel from its committed rocprofv3 counter
    summary, or None when the kernel's sources changed since it was taken."""
    import hashlib
    if not path.exists():
        return None
    h = hashlib.sha256()
    for f in sources:
        h.update((ROOT / "mtp_draft_verify_amd" / "csrc" / f).read_bytes())
    fields = dict(l.split(":", 1) for l in path.read_text().splitlines() if ":" in l)
    if fields.get("kernel_source_sha256_16", "").strip() != h.hexdigest()[:16]:
        return None
    return float(fields["traffic_bytes_per_launch"])


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, reps=3):
    """The oracle as it stands (plain fp64 C, OpenMP across sequences and kv
    heads) on a bounded sample of the same workload: one draft step over all
    sequences (1 warm-up, then the median of `reps` timed runs) and one
    greedy verify over all sequences' rows, scaled to a whole round as
    N * t_step + t_verify (every step reads the same weights and KV, so each
    costs the same); then the same for one sequence on one thread."""
    import ctypes
    import statistics
    import mtp_synth as syn
    from oracle import oracle as orc
    orc.build(force=False)
    S, N, V = len(w.draft.seqs), w.draft.n_steps, w.model.n_vocab
    # verify rows from the input generator alone (the oracle's verify costs
    # the same whatever the drafts are)
    gv = syn.make_greedy_verify(7, S, N, V, w.p_accept, "max5")
    gomp = ctypes.CDLL("libgomp.so.1")
    threads = int(gomp.omp_get_max_threads())

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0
    step_all = lambda: orc.draft_block(w.model, w.draft, want_logits=False, n_steps=1)
    timed(step_all)
    t_step = statistics.median(timed(step_all) for _ in range(reps))
    t_ver = timed(lambda: orc.verify_greedy(gv.logits, gv.drafts))
    value = S * N / (N * t_step + t_ver)
    # one sequence on one thread
    gomp.omp_set_num_threads(1)
    try:
        t1 = timed(lambda: orc.draft_block(w.model, w.draft, want_logits=False, n_steps=1, seq_idx=[0]))
        t1v = timed(lambda: orc.verify_greedy(gv.logits[:1], gv.drafts[:1]))
    finally:
        gomp.omp_set_num_threads(threads)
    single = N / (N * t1 + t1v)
    return {"value": value, "unit": "draft tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"one draft step over all {S} sequence(s) (1 warm-up + median of {reps} timed runs: "
                      f"{t_step:.2f} s) and one greedy verify over all {S}x{N + 1} rows ({t_ver:.2f} s), scaled to "
                      f"a round of {N} steps as {N}*t_step + t_verify; {threads} OpenMP threads on "
                      f"'{_cpu_model()}' ({os.cpu_count()} logical CPUs visible)",
            "single_thread": {"value": single, "unit": "draft tokens/s",
                              "sample": f"one draft step of sequence 0 ({t1:.2f} s) + its verify rows ({t1v:.3f} s) "
                                        f"on one thread, scaled to {N} steps"}}


WORKLOADS = {
    "c2": ("c2_gemma_bf16", "Gemma-4-26B-like assistant drafter, bf16 weights/KV, fp32 arithmetic: 4 blocks "
           "d_model 1024, h_prev 2816, 8 q / 2 kv heads of 256, MLP 4096, full KV 8192, tied head V=262144; "
           "1 sequence, B=4 (3 draft steps) + greedy verify"),
    "c3": ("c3_interleaved", "same drafter; blocks 0-2 read a 1024-position SWA ring, block 3 a full KV of "
           "ctx ~ U{4096..32768}; 16 sequences, B=4 + greedy verify"),
    "c4": ("c4_longctx_q8", "same drafter with a Q8_0 tied head; full KV of 131072 positions; 8 sequences, "
           "B=5 (4 draft steps) + greedy verify"),
    "c5": ("c5_sample", "exact temperature>0 verify only: V=248320, 32 sequences x 4 drafts, q = perturbed copy, "
           "temp 0.6, top-p 0.95, min-p 0.05, repetition 1.08, presence 0.4 over the last 64 tokens"),
    "c6": ("c6_centroid", "the c2 drafter with a centroid LM head: 2048 centroids x 128 token ids, top 32 "
           "centroids (4096 candidate rows) per step; full KV 8192; 1 sequence, B=4 + greedy verify"),
    "c8": ("c8_hidden_verify", "greedy verify from the target's final hidden rows: Gemma-4-26B-like width 2816, "
           "bf16 LM head V=262144 with its final-norm gain, 16 sequences x (1 + 3) rows"),
    "c7": ("c7_sink_window", "the c2 drafter with every block reading a sink + window source (64 sink cells + "
           "a 257-cell window ending at attn_pos over a 12000-cell cache, half the sequences with a valid run starting inside "
           "the window); 8 sequences, B=4 + greedy verify"),
}


def bench_sample(args, dev):
    """Extra measurement: the temperature>0 verify on its own."""
    import torch
    import mtp_draft_verify_amd as mtp
    import mtp_synth as syn
    from mtp_synth.device import to_dev
    w = syn.c5_sample()
    sv = w.sample
    S, R, V = sv.p_logits.shape
    desc = mtp.make_desc(d_model=32, d_hprev=8, n_blocks=1, n_head_q=1, n_head_kv=1, head_dim=64, d_ff=8,
                         n_vocab=V, w_dtype=0, head_dtype=0, kv_dtype=0, max_seqs=S, max_steps=R - 1)
    ctx = mtp.Context(desc, None, stream=torch.cuda.current_stream())
    p, q = to_dev(sv.p_logits, dev), to_dev(sv.q_logits, dev)
    dr, hist, hl = to_dev(sv.drafts, dev), to_dev(sv.history, dev), to_dev(sv.history_len, dev)
    sp = sv.sampler
    smp = mtp.make_sampler(temp=sp.temp, top_p=sp.top_p, min_p=sp.min_p, rep_penalty=sp.rep_penalty,
                           presence_penalty=sp.presence_penalty, freq_penalty=sp.freq_penalty, top_k=sp.top_k,
                           penalty_last_n=sp.penalty_last_n, seed=sp.seed)
    toks = torch.zeros((S, R), dtype=torch.int32, device=dev)
    na = torch.zeros((S,), dtype=torch.int32, device=dev)
    rnd = [0]

    def step():
        ctx.verify_sample(p, q, dr, hist, hl, smp, rnd[0], toks, na)
        rnd[0] += 1
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # algorithmic bytes: the p and q logit rows, each read once per call
    bytes_step = (p.numel() + q.numel()) * 4
    n_diag = min(args.steps, 50)
    ctx.profile(1 << mtp.MTP_PROF_VERIFY)
    for _ in range(n_diag):
        step()
    v_ms, v_n = ctx.profile_read(mtp.MTP_PROF_VERIFY)
    ctx.profile(0)
    avg_ms = v_ms / n_diag                  # the call's kernels, summed
    achieved = bytes_step / (avg_ms * 1e-3) / 1e9
    out = {"metric": "verified draft tokens/s of exact temperature>0 verify", "value": S * (R - 1) / (ms * 1e-3),
           "unit": "draft tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": WORKLOADS["c5"][1], "n_seq": S, "n_draft": R - 1, "n_vocab": V},
           "hbm_gbps_step": bytes_step / (ms * 1e-3) / 1e9, "accepted_per_round": float(na.float().mean()),
           "roofline": {"bound": "hbm", "kernel": "sample_chunk_kernel + sample_row_kernel + sample_seq_kernel "
                                                 "(one mtp_verify_sample call)",
                        "timing": f"start/stop HIP events of each kernel launch, summed per call, over {n_diag} calls after the timed region",
                        "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                        "traffic": None, "bytes_per_launch": bytes_step, "avg_launch_ms": avg_ms, "launches": v_n}}
    ctx.close()
    print(json.dumps(out), flush=True)


def bench_hidden(args, dev):
    """Extra measurement: the greedy verify from the target's hidden rows on
    its own (final norm + LM head over the 1 + N rows + argmax + acceptance)."""
    import numpy as np
    import torch
    import mtp_draft_verify_amd as mtp
    import mtp_synth as syn
    from mtp_synth.device import to_dev
    w = syn.c8_hidden_verify()
    hv = w.hidden
    S, R, d = hv.hidden.shape
    V = hv.n_vocab
    desc = mtp.make_desc(d_model=32, d_hprev=8, n_blocks=1, n_head_q=1, n_head_kv=1, head_dim=64, d_ff=8,
                         n_vocab=V, w_dtype=0, head_dtype=0, kv_dtype=0, max_seqs=S, max_steps=R - 1,
                         hidden_d_max=d, hidden_sample=1)
    ctx = mtp.Context(desc, None, stream=torch.cuda.current_stream())
    wt = torch.from_numpy(hv.head.view(np.int16)).to(dev)
    g = to_dev(hv.g, dev)
    head = mtp.make_lm_head(wt, g, d, V, mtp.MTP_BF16, hv.eps)
    hidden, drafts = to_dev(hv.hidden, dev), to_dev(hv.drafts, dev)
    toks = torch.zeros((S, R), dtype=torch.int32, device=dev)
    na = torch.zeros((S,), dtype=torch.int32, device=dev)

    def step():
        ctx.verify_greedy_hidden(head, hidden, drafts, toks, na)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # HIP events around each call on the context's stream, after the timed region
    n_diag = min(args.steps, 50)
    ctx.profile(1 << mtp.MTP_PROF_VERIFY)
    for _ in range(n_diag):
        step()
    v_ms, v_n = ctx.profile_read(mtp.MTP_PROF_VERIFY)
    ctx.profile(0)
    avg_ms = v_ms / n_diag                  # the call's kernels, summed
    alg_bytes = V * d * 2 + S * R * d * 4         # the head once + the hidden rows
    achieved = alg_bytes / (avg_ms * 1e-3) / 1e9
    out = {"metric": "verified rows/s of greedy verify from hidden states (fused target head + argmax)",
           "value": S * R / (ms * 1e-3), "unit": "rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic",
           "config": {"workload": WORKLOADS["c8"][1], "n_seq": S, "rows_per_seq": R, "d": d, "n_vocab": V},
           "roofline": {"bound": "hbm", "kernel": "hv_prep_kernel + hv_head_kernel + verify_prefix_kernel "
                                                 "(one entry-point call)",
                        "timing": f"start/stop HIP events of each kernel launch, summed per call, over {n_diag} calls after the timed region",
                        "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                        "frac": achieved / PEAK_HBM_GBPS,
                        "traffic": head_traffic_from_counters(HV_COUNTERS_FILE, HV_SOURCES),
                        "traffic_kernel": "hv_head_kernel", "bytes_per_launch": alg_bytes,
                        "avg_launch_ms": avg_ms, "launches": v_n,
                        "mfma_tflops": 2.0 * S * R * V * d / (avg_ms * 1e-3) / 1e12},
           "accepted_per_round": float(na.float().mean())}
    # the same rows through the exact sampling verify (logit rows to context
    # scratch, then the sampling chain): one-hot drafts, no penalties
    sp = mtp.make_sampler(temp=0.8, top_p=0.95, min_p=0.05, rep_penalty=1.0, presence_penalty=0.0,
                          penalty_last_n=0, seed=11)
    hist = torch.zeros((S, 1), dtype=torch.int32, device=dev)
    hlen = torch.zeros((S,), dtype=torch.int32, device=dev)

    def sample_step(k):
        ctx.verify_sample_hidden(head, hidden, None, drafts, hist, hlen, sp, k, toks, na)
    for k in range(args.warmup):
        sample_step(k)
    torch.cuda.synchronize()
    n_s = min(args.steps, 50)
    t0 = time.perf_counter()
    for k in range(n_s):
        sample_step(k)
    torch.cuda.synchronize()
    s_ms = (time.perf_counter() - t0) * 1e3 / n_s
    out["sample_hidden"] = {"what": "mtp_verify_sample_hidden on the same rows (temp 0.8, top-p 0.95, min-p 0.05, "
                                    "one-hot drafts)", "ms_per_call": s_ms, "rows_per_s": S * R / (s_ms * 1e-3),
                            "calls": n_s, "accepted_per_round": float(na.float().mean())}
    if not args.no_cpu_baseline:
        from oracle import oracle as orc
        orc.build(force=False)
        rows, t1 = 0, time.perf_counter()
        while time.perf_counter() - t1 < args.cpu_budget and rows < 50 * S * R:
            s = (rows // R) % S
            orc.verify_greedy_hidden(hv.hidden[s:s + 1], hv.head, hv.head_dtype, V, hv.g, hv.eps, hv.drafts[s:s + 1])
            rows += R
        el = time.perf_counter() - t1
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
        out["cpu_baseline"] = {"value": rows / el, "unit": "rows/s", "cores": threads, "kind": "oracle",
                               "sample": f"{rows // R} sequence(s) x {R} rows of the same workload through the "
                                         f"oracle, {el:.1f} s wall, OpenMP threads={threads}"}
    ctx.close()
    print(json.dumps(out), flush=True)


ATTN_SOURCES = ["attn_kernels.hip", "dev_common.h", "mtp_internal.h"]
MM_SOURCES = ["mfma_kernels.hip", "widen.h", "dev_common.h", "mtp_internal.h"]


def counters_file(kernel, workload):
    return ROOT / "profiles" / f"{kernel}_{workload}_hbm_counters.txt"


def bench_draft(args, dev):
    """The headline line: rounds of draft block + greedy verify."""
    import torch
    import mtp_draft_verify_amd as mtp
    import mtp_synth as syn
    from mtp_synth.device import to_dev, upload_model, upload_seqs
    log(f"bench: generating workload {args.workload}")
    w = getattr(syn, WORKLOADS[args.workload][0])()
    m, dr = w.model, w.draft
    S, N, V = len(dr.seqs), dr.n_steps, m.n_vocab
    desc, wts, keep_w = upload_model(m, dev, S, N)
    seqs, last_tok, h_prev, keep_kv = upload_seqs(m, dr, dev)
    stream = torch.cuda.current_stream()
    ctx = mtp.Context(desc, wts, stream=stream, keepalive=keep_w)
    seq_arr = mtp.make_seqs(seqs)
    drafts = torch.zeros((S, N), dtype=torch.int32, device=dev)
    h_last = torch.zeros((S, m.d_hprev), dtype=torch.float32, device=dev)
    toks = torch.zeros((S, N + 1), dtype=torch.int32, device=dev)
    n_acc = torch.zeros((S,), dtype=torch.int32, device=dev)

    # target logits with the drafter's own drafts planted (p_accept of the
    # workload), so that the verify accepts what a real target would
    ctx.draft_block(seq_arr, last_tok, h_prev, N, drafts, h_last)
    torch.cuda.synchronize()
    gv = syn.make_greedy_verify(1, S, N, V, w.p_accept, "max5", drafts=drafts.cpu().numpy())
    logits = to_dev(gv.logits, dev)

    def step():
        ctx.draft_block(seq_arr, last_tok, h_prev, N, drafts, h_last)
        ctx.verify_greedy(logits, drafts, toks, n_acc)

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # Kernel timing: the same steps again, each launch of one kernel class
    # carrying start/stop HIP events that the runtime sets when the kernel
    # starts and finishes running on the library's stream (timing makes the
    # library launch the chain kernel by kernel instead of replaying its
    # captured graph; the kernels themselves are the same).
    def class_time(cls, n):
        ctx.profile(1 << cls)
        for _ in range(n):
            step()
        t, k = ctx.profile_read(cls)
        ctx.profile(0)
        return t, k
    head_ms, head_n = class_time(mtp.MTP_PROF_HEAD, args.steps)
    attn_ms, attn_n = class_time(mtp.MTP_PROF_ATTN, args.steps)

    # per-class breakdown over a separately profiled pass (diagnostic)
    ctx.profile((1 << mtp.MTP_PROF_N) - 1)
    n_diag = min(args.steps, 20)
    for _ in range(n_diag):
        step()
    torch.cuda.synchronize()
    breakdown = {}
    for name, cls in (("head", mtp.MTP_PROF_HEAD), ("attn", mtp.MTP_PROF_ATTN), ("merge", mtp.MTP_PROF_MERGE),
                      ("gemv", mtp.MTP_PROF_GEMV), ("verify", mtp.MTP_PROF_VERIFY)):
        t, n = ctx.profile_read(cls)
        breakdown[name] = {"ms_per_step": t / n_diag, "launches_per_step": n / n_diag}
    ctx.profile(0)
    log(f"bench: breakdown {breakdown}")

    wb, hb, gb = weight_bytes(m, S)
    kvb = kv_bytes(m, dr.seqs)
    step_bytes = wb + hb + gb + kvb + S * m.d_model * 2
    round_bytes = N * step_bytes + S * (N + 1) * V * 4
    head_launch_bytes = hb + m.d_hprev * m.d_model * 2 + 2 * S * m.d_model * 4
    if m.n_centroids:   # the head class times only the candidate-row kernel
        head_launch_bytes -= m.n_centroids * m.d_model * (4 if m.w_dtype == syn.F32 else 2)
    if m.n_centroids:
        head_name = "cand_head_kernel (centroid head candidate rows + argmax + post-proj)"
    elif S >= 2 and m.head_dtype == syn.Q8_0:
        head_name = "mm_q8_head_kernel (final RMSNorm + matrix-core Q8_0 LM head + argmax + post-proj)"
    elif S >= 2 and m.head_dtype != syn.F32:
        head_name = "mm_head_kernel (final RMSNorm + matrix-core LM head + argmax + post-proj)"
    else:
        head_name = "head_kernel (final RMSNorm + LM head GEMV + argmax + post-proj)"
    attn_name = "attn_mm_kernel (split-K GQA cross-attention, partials per split)" if m.kv_dtype != syn.F32 \
        else "attn_kernel (split-K GQA cross-attention, partials per split)"

    def roofline(name, key, total_ms, n, bytes_per_launch, sources):
        avg = total_ms / max(n, 1)
        ach = bytes_per_launch / (avg * 1e-3) / 1e9
        cf = counters_file(key, args.workload)
        return {"bound": "hbm", "kernel": name, "timing": f"start/stop HIP events of each launch over {args.steps} "
                "steps after the timed region, on the library's stream",
                "achieved": ach, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBPS,
                "traffic": head_traffic_from_counters(cf, sources), "traffic_source": cf.name,
                "bytes_per_launch": bytes_per_launch, "avg_launch_ms": avg, "launches": n}
    head_key = head_name.split()[0]
    r_head = roofline(head_name, head_key, head_ms, head_n, head_launch_bytes,
                      MM_SOURCES if head_key in ("mm_head_kernel", "mm_q8_head_kernel") else HEAD_SOURCES)
    # one attention launch reads one block's visible K and V of every sequence
    r_attn = roofline(attn_name, attn_name.split()[0], attn_ms, attn_n, kvb // m.n_blocks, ATTN_SOURCES)
    if attn_ms > head_ms:
        dominant, other = r_attn, r_head
    else:
        dominant, other = r_head, r_attn
    value = S * N / (ms_per_step * 1e-3)
    acc = n_acc.cpu().numpy()
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload][1],
                   "n_seq": S, "draft_steps": N, "n_vocab": V,
                   "kv_positions": [s_.attn_pos + 1 for s_ in dr.seqs][:16]},
        "hbm_gbps_round": round_bytes / (ms_per_step * 1e-3) / 1e9,
        "hbm_frac_round": round_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "bytes_per_round": round_bytes,
        "roofline": dominant,
        "roofline_other": other,
        "breakdown": breakdown,
        "accepted_per_round": float(acc.mean()),
    }
    ctx.close()
    del keep_kv, keep_w
    if not args.no_cpu_baseline:
        log(f"bench: cpu baseline (oracle, {args.cpu_reps} timed runs of one draft step)")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_reps)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-reps", type=int, default=3, help="timed oracle runs (median) for cpu_baseline")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time (c8 cpu_baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only copy a buffer of this many MiB 3 times (calibrates rocprofv3 byte counters)")
    ap.add_argument("--workload", default="c4", choices=sorted(WORKLOADS),
                    help="c4 (default, the headline line: the largest configuration); the others are extra "
                         "measurements")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no multi-GPU form (sequences would shard across GPUs "
              "with no exchange, each GPU running this same path on its own sequences). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mtp_draft_verify_amd as mtp
    import mtp_synth as syn
    from mtp_synth.device import to_dev, upload_model, upload_seqs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 18                   # float32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n * 4}), flush=True)
        return
    if args.workload == "c5":
        bench_sample(args, dev)
        return
    if args.workload == "c8":
        bench_hidden(args, dev)
        return
    bench_draft(args, dev)


if __name__ == "__main__":
    main()
