"""GPU parity of the sink + window KV source (through the C ABI) against the
oracle: the draft attention reads cells [0, min(sink, first)) ++
[first, attn_pos], first = max(attn_pos - W + 1, run_lo, 0)
("opus-mtp-turbo: Track 1 report", findings item 2)."""
import numpy as np
import pytest

import mtp_synth as syn
from tests.gpu_harness import GpuDrafter, compare_draft, log

pytestmark = pytest.mark.gpu

BF16_NAN = 0x7FC0


def _check(w, gpu_out, orc_out, idx=None, max_near=1):
    c = compare_draft(w.model, gpu_out, orc_out, idx)
    log(f"  {w.name}: steps={c.compared_steps} near_ties={c.near_ties} max_logit_err={c.max_logit_err:.3g} "
        f"max_h_err={c.max_h_err:.3g}")
    assert c.near_ties <= max_near
    return c


def _edge_workload(**over):
    """Four sequences whose visible lists take every shape: a context shorter
    than the sink, one where sink and window touch, a stale run that starts
    past the sink (the window shrinks to two cells), and a valid run that
    starts after the window's own start."""
    w = syn.c7_sink_window(n_seq=4, ctx_range=(300, 900), full_cap=1000, n_vocab=32768, **over)
    plan = [(39, 0), (300, 0), (700, 699), (600, 500)]     # (attn_pos, run_lo)
    for s, (ap, lo) in zip(w.draft.seqs, plan):
        s.attn_pos, s.pos0, s.run_lo = ap, ap + 1, lo
    return w


def test_sink_window_full_size_sampled_sequences(orc):
    log("case c7 full: sink 64 + window 257 over 12000 cells, 8 seqs (4 with a stale run), S=8 N=3; "
        "oracle on 4 sampled sequences")
    w = syn.c7_sink_window()
    assert any(s.run_lo > s.attn_pos - w.model.sw_window + 1 for s in w.draft.seqs)
    g = GpuDrafter(w.model, 8, 3)
    gpu = g.run(w.draft)
    idx = [0, 1, 4, 7]
    _check(w, gpu, orc.draft_block(w.model, w.draft, seq_idx=idx), idx)
    g.close()


def test_sink_window_edge_lists(orc):
    log("case c7 edges: ctx < sink, sink touching the window, 2-cell window, run inside the window; "
        "with sink 64 and with no sink")
    for sink in (64, 0):
        w = _edge_workload(sw_sink=sink)
        n_vis = [len(orc.visible_cells(w.model, s, syn.KV_SINK_WINDOW)) for s in w.draft.seqs]
        log(f"  sink {sink}: visible cells {n_vis}")
        if sink:
            assert n_vis == [40, 301, 66, 165]
        g = GpuDrafter(w.model, 4, 3)
        _check(w, g.run(w.draft), orc.draft_block(w.model, w.draft))
        g.close()


def test_sink_window_mixed_with_swa_ring_and_full_blocks(orc):
    log("case c7 mixed: blocks read sink+window, SWA ring (W=512), sink+window, full KV")
    w = _edge_workload(block_src=[syn.KV_SINK_WINDOW, syn.KV_SWA, syn.KV_SINK_WINDOW, syn.KV_FULL],
                       swa_window=512)
    g = GpuDrafter(w.model, 4, 3)
    _check(w, g.run(w.draft), orc.draft_block(w.model, w.draft))
    g.close()


def test_stale_and_unseen_cells_are_never_read():
    """Cells of the stale run [min(sink, first), first) and past attn_pos hold
    NaN: the results stay bit-identical (the drafter never reads a cell that
    its visible list leaves out)."""
    log("case c7 poisoned stale cells")
    w = _edge_workload()
    g = GpuDrafter(w.model, 4, 3)
    ref = g.run(w.draft)
    W, sink = w.model.sw_window, w.model.sw_sink
    for s in w.draft.seqs:
        src = s.src[syn.KV_SINK_WINDOW]
        first = max(s.attn_pos - W + 1, s.run_lo, 0)
        keep = np.zeros(src.n_cells, bool)
        keep[:min(sink, first)] = True
        keep[first:s.attn_pos + 1] = True
        k, v = src.k.copy(), src.v.copy()
        k[~keep] = BF16_NAN
        v[~keep] = BF16_NAN
        s.src = list(s.src)
        s.src[syn.KV_SINK_WINDOW] = syn.KVSource(k, v)
    out = g.run(w.draft)
    for key in ref:
        assert np.array_equal(ref[key], out[key]), key
    g.close()
