"""GPU parity of the greedy verify (through the C ABI) against the oracle:
tokens and accept lengths bit-exact (argmax over fp32 is exact)."""
import numpy as np
import pytest

import mtp_synth as syn
from tests.gpu_harness import log

pytestmark = pytest.mark.gpu


def _gpu_verify(logits, drafts, max_seqs=None):
    import torch
    import mtp_draft_verify_amd as mtp
    S, R, V = logits.shape
    desc = mtp.make_desc(d_model=32, d_hprev=8, n_blocks=1, n_head_q=1, n_head_kv=1, head_dim=64, d_ff=8, n_vocab=V,
                         w_dtype=0, head_dtype=0, kv_dtype=0, max_seqs=max_seqs or S, max_steps=max(R - 1, 1))
    with mtp.Context(desc, None) as ctx:
        lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
        dr = torch.from_numpy(np.ascontiguousarray(drafts, np.int32).reshape(S, R - 1)).cuda()
        toks = torch.full((S, R), -9, dtype=torch.int32, device="cuda")
        na = torch.full((S,), -9, dtype=torch.int32, device="cuda")
        ctx.verify_greedy(lg, dr, toks, na)
        ctx.verify_greedy(lg, dr, toks, na)      # keys are cleared between calls
        torch.cuda.synchronize()
        return toks.cpu().numpy(), na.cpu().numpy()


@pytest.mark.parametrize("S,N,V,p,mode", [
    (1, 3, 4096, 0.8, "add5"),          # tiny config
    (1, 3, 262144, 0.8, "max5"),        # Gemma-like, one sequence
    (16, 3, 262144, 0.8, "max5"),       # interleaved config batch
    (8, 4, 262144, 0.7, "max5"),        # long-context batch
    (5, 2, 8193, 0.6, "max5"),          # ragged last chunk
    (7, 3, 5, 0.5, "max5"),             # V not a multiple of 4, smaller than a chunk
])
def test_verify_greedy_matches_oracle(orc, S, N, V, p, mode):
    log(f"case verify_greedy S={S} N={N} V={V}")
    gv = syn.make_greedy_verify(31 + S + V, S, N, V, p, mode)
    t_g, n_g = _gpu_verify(gv.logits, gv.drafts)
    t_o, n_o = orc.verify_greedy(gv.logits, gv.drafts)
    assert np.array_equal(n_g, n_o)
    assert np.array_equal(t_g, t_o)


def test_verify_greedy_edge_cases(orc):
    log("case verify_greedy edges")
    # ties (all equal -> id 0), signed zeros tie, no drafts, out-of-range drafts
    L = np.zeros((4, 3, 6), np.float32)
    L[1, :, 3] = -0.0
    L[1, :, :3] = -1.0
    L[1, :, 4:] = -1.0
    L[1, :, 5] = 0.0                     # +0 and -0 tie -> lowest id 3
    L[2] = np.arange(6, dtype=np.float32)[None, :]
    dr = np.array([[0, 0], [3, 3], [5, 4], [-1, 99]], np.int32)
    t_g, n_g = _gpu_verify(L, dr)
    t_o, n_o = orc.verify_greedy(L, dr)
    assert np.array_equal(t_g, t_o) and np.array_equal(n_g, n_o)
    assert n_g.tolist() == [2, 2, 1, 0]
    # n_draft = 0: just the argmax of the one row
    L0 = np.random.default_rng(0).standard_normal((3, 1, 1000)).astype(np.float32)
    t_g, n_g = _gpu_verify(L0, np.zeros((3, 0), np.int32))
    assert np.array_equal(t_g[:, 0], L0[:, 0].argmax(1)) and np.all(n_g == 0)
