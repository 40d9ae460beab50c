"""Shared plumbing of the GPU tests: run the library and the oracle on the
same synthetic inputs and compare them under the stated tolerances.

Tolerances (fixed by the task's parity bar): token ids and accept lengths
bit-exact; logits within 1e-4 relative (per row, against the row's largest
|logit|) for fp32 drafters, 2e-2 absolute for bf16 / Q8_0 drafters.  A draft
id may differ only where the oracle's top-2 margin is below that tolerance (a
near-tie); such a sequence is counted and no longer compared after that step,
because the two chains then continue from different tokens.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np

import mtp_synth as syn


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


# Per-case parity counts (near ties, flagged sequences, errors), printed as
# one JSON line per case at the end of the session by tests/conftest.py, so
# that they reach the end of the pytest output whatever its verbosity.
RECORDS = []


def record(case: str, **counts) -> None:
    import os
    r = {"case": case}
    for k, v in counts.items():
        r[k] = float(v) if isinstance(v, (float, np.floating)) else int(v)
    r["test"] = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    RECORDS.append(r)


def tol_for(m: syn.Model):
    if m.w_dtype == syn.F32 and m.head_dtype == syn.F32 and m.kv_dtype == syn.F32:
        return "rel", 1e-4
    return "abs", 2e-2


@dataclass
class DraftCompare:
    near_ties: int
    compared_steps: int
    max_logit_err: float
    max_h_err: float


def compare_draft(m: syn.Model, gpu: dict, orc: dict, idx=None) -> DraftCompare:
    kind, tol = tol_for(m)
    gd, od = gpu["drafts"], orc["drafts"]
    S, N = od.shape
    idx = list(range(S)) if idx is None else list(idx)
    near, steps, max_le, max_he = 0, 0, 0.0, 0.0
    for si, s in enumerate(idx):
        diverged = False
        for k in range(N):
            if gpu.get("logits") is not None and orc.get("logits") is not None:
                g, o = gpu["logits"][s, k].astype(np.float64), orc["logits"][si, k].astype(np.float64)
                err = np.abs(g - o).max()
                lim = tol * np.abs(o).max() if kind == "rel" else tol
                max_le = max(max_le, err / (np.abs(o).max() if kind == "rel" else 1.0))
                assert err <= lim, f"seq {s} step {k}: logit error {err} > {lim}"
            steps += 1
            if gd[s, k] != od[si, k]:
                margin = orc["margin"][si, k]
                lim = tol * np.abs(orc["logits"][si, k]).max() if (kind == "rel" and orc.get("logits") is not None) else tol
                assert margin < lim, f"seq {s} step {k}: draft {gd[s, k]} != {od[si, k]} with margin {margin}"
                near += 1
                diverged = True
                break
        if not diverged and gpu.get("h_last") is not None:
            g, o = gpu["h_last"][s].astype(np.float64), orc["h_last"][si].astype(np.float64)
            err = np.abs(g - o).max()
            lim = tol * max(1.0, np.abs(o).max()) if kind == "rel" else tol
            max_he = max(max_he, err)
            assert err <= lim, f"seq {s}: h_last error {err} > {lim}"
    return DraftCompare(near, steps, max_le, max_he)


class GpuDrafter:
    """A context plus the device copies of one synthetic drafter."""

    def __init__(self, m: syn.Model, max_seqs: int, max_steps: int, device="cuda"):
        import mtp_draft_verify_amd as mtp
        from mtp_synth.device import upload_model
        self.m = m
        self.device = device
        self.desc, self.w, self.tensors = upload_model(m, device, max_seqs, max_steps)
        self.ctx = mtp.Context(self.desc, self.w, keepalive=self.tensors)

    def run(self, dr: syn.DraftInputs, n_steps=None, want_logits=True, seq_idx=None, last_tok=None, h_prev=None,
            pos0_shift=0, conf=False, p_min=0.0):
        import torch
        from mtp_synth.device import upload_seqs
        seqs, lt, hp, keep = upload_seqs(self.m, dr, self.device, seq_idx)
        for s in seqs:
            s["pos0"] += pos0_shift
        if last_tok is not None:
            lt = torch.as_tensor(np.asarray(last_tok, np.int32), device=self.device)
        if h_prev is not None:
            hp = torch.as_tensor(np.asarray(h_prev, np.float32), device=self.device)
        S, N = len(seqs), n_steps or dr.n_steps
        drafts = torch.full((S, N), -7, dtype=torch.int32, device=self.device)
        h_last = torch.zeros((S, self.m.d_hprev), dtype=torch.float32, device=self.device)
        logits = torch.zeros((S, N, self.m.n_vocab), dtype=torch.float32, device=self.device) if want_logits else None
        if conf:
            cf = torch.full((S, N), -7.0, dtype=torch.float32, device=self.device)
            nk = torch.full((S,), -7, dtype=torch.int32, device=self.device)
            self.ctx.draft_block_conf(seqs, lt, hp, N, drafts, h_last, logits, cf, p_min, nk)
        else:
            self.ctx.draft_block(seqs, lt, hp, N, drafts, h_last, logits)
        torch.cuda.synchronize()
        out = dict(drafts=drafts.cpu().numpy(), h_last=h_last.cpu().numpy(),
                   logits=logits.cpu().numpy() if logits is not None else None)
        if conf:
            out["conf"], out["n_keep"] = cf.cpu().numpy(), nk.cpu().numpy()
        del keep
        return out

    def close(self):
        self.ctx.close()
