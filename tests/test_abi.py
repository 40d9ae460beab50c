"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, and host-only validation rejects bad descriptions and
arguments without touching a device."""
import ctypes as C
import re
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]


@pytest.fixture(scope="module")
def mtp():
    import mtp_draft_verify_amd as m
    if not m.LIB_PATH.exists():
        from mtp_draft_verify_amd import build
        build.build()
    m.lib()
    return m


def test_every_declared_symbol_is_exported(mtp):
    header = (ROOT / "include" / "mtp.h").read_text()
    declared = set(re.findall(r"^(?:int|void|const char \*)\s*\*?\s*(mtp_\w+)\s*\(", header, re.M))
    assert {"mtp_ctx_create", "mtp_draft_block", "mtp_verify_greedy", "mtp_verify_sample"} <= declared
    assert declared == set(mtp.EXPORTS)
    L = C.CDLL(str(mtp.LIB_PATH))
    for name in declared:
        assert hasattr(L, name), name


def test_strerror_names_every_status(mtp):
    for code in range(0, -8, -1):
        assert mtp.mtp_strerror(code) != "unknown status"
    assert mtp.mtp_strerror(-99) == "unknown status"


def _c2_desc(mtp, **over):
    kw = dict(d_model=1024, d_hprev=2816, n_blocks=4, n_head_q=8, n_head_kv=2, head_dim=256, d_ff=4096,
              n_vocab=262144, w_dtype=mtp.MTP_BF16, head_dtype=mtp.MTP_BF16, kv_dtype=mtp.MTP_BF16,
              max_seqs=16, max_steps=4)
    kw.update(over)
    return mtp.make_desc(**kw)


def test_check_desc_accepts_the_configs_and_rejects_bad_shapes(mtp):
    assert mtp.mtp_check_desc(_c2_desc(mtp)) == mtp.MTP_OK
    assert mtp.mtp_check_desc(_c2_desc(mtp, head_dtype=mtp.MTP_Q8_0, max_seqs=8, max_steps=4)) == mtp.MTP_OK
    assert mtp.mtp_check_desc(_c2_desc(mtp, swa_window=1024, block_src=[1, 1, 1, 0])) == mtp.MTP_OK
    assert mtp.mtp_check_desc(_c2_desc(mtp, sw_window=256, sw_sink=64, block_src=[2, 2, 2, 2])) == mtp.MTP_OK
    assert mtp.mtp_check_desc(_c2_desc(mtp, sw_window=256, sw_sink=0, block_src=[2, 1, 2, 0],
                                       swa_window=512)) == mtp.MTP_OK
    tiny = dict(d_model=256, d_hprev=256, n_blocks=1, n_head_q=4, n_head_kv=1, head_dim=64, d_ff=1024, n_vocab=4096,
                w_dtype=mtp.MTP_F32, head_dtype=mtp.MTP_F32, kv_dtype=mtp.MTP_F32, max_seqs=1, max_steps=3)
    assert mtp.mtp_check_desc(mtp.make_desc(**tiny)) == mtp.MTP_OK
    assert mtp.mtp_check_desc(_c2_desc(mtp, hidden_d_max=2816, hidden_sample=1)) == mtp.MTP_OK
    bad = [
        dict(n_head_kv=3),                        # Hq % Hkv
        dict(n_blocks=9),                         # > MTP_MAX_BLOCKS
        dict(d_model=1000),                       # not a multiple of 32
        dict(w_dtype=mtp.MTP_Q8_0),               # Q8_0 only for the head
        dict(kv_dtype=7),
        dict(max_seqs=17),                        # > 16 sequences
        dict(block_src=[1, 0, 0, 0]),             # SWA block without a window
        dict(block_src=[2, 0, 0, 0]),             # sink + window block without a window
        dict(block_src=[2, 0, 0, 0], sw_window=256, sw_sink=-1),
        dict(block_src=[3, 0, 0, 0]),             # unknown source kind
        dict(head_dim=96),                        # no attention instantiation
        dict(d_ff=8192),                          # GEMV row longer than supported
        dict(max_steps=0),
        dict(hidden_d_max=300),                   # hidden-verify width not a multiple of 256
        dict(hidden_d_max=16640),                 # wider than the hidden-verify kernels take
        dict(hidden_d_max=-256),
        dict(hidden_sample=1),                    # logit rows without a head width
    ]
    for b in bad:
        rc = mtp.mtp_check_desc(_c2_desc(mtp, **b))
        assert rc < 0, b
    assert mtp.lib().mtp_check_desc(None) == mtp.MTP_E_INVAL


def test_entry_points_reject_null_context_without_device_work(mtp):
    L = mtp.lib()
    assert L.mtp_draft_block(None, 1, None, None, None, 1, None, None, None) == mtp.MTP_E_INVAL
    assert L.mtp_draft_block_conf(None, 1, None, None, None, 1, None, None, None, None, 0.5, None) == mtp.MTP_E_INVAL
    assert L.mtp_verify_greedy(None, 1, 1, 10, None, None, None, None) == mtp.MTP_E_INVAL
    head = mtp.make_lm_head(None, None, 2816, 262144)
    assert L.mtp_verify_greedy_hidden(None, 1, 3, C.byref(head), None, None, None, None) == mtp.MTP_E_INVAL
    sp = mtp.make_sampler(temp=0.6, top_p=0.95, min_p=0.05, rep_penalty=1.08, presence_penalty=0.4)
    assert L.mtp_verify_sample(None, 1, 1, 10, None, None, None, None, 0, None, C.byref(sp), 0, None,
                               None) == mtp.MTP_E_INVAL
    assert L.mtp_verify_sample_hidden(None, 1, 3, C.byref(head), None, None, None, None, 0, None, C.byref(sp), 0,
                                      None, None) == mtp.MTP_E_INVAL
    assert L.mtp_verify_sample_hidden(None, 1, 3, C.byref(head), None, None, None, None, 0, None, None, 0,
                                      None, None) == mtp.MTP_E_INVAL
    assert L.mtp_ctx_create(None, None, None, None) == mtp.MTP_E_INVAL
    assert L.mtp_profile_enable(None, 1) == mtp.MTP_E_INVAL
    assert L.mtp_profile_read(None, 0, None, None) == mtp.MTP_E_INVAL
    L.mtp_ctx_destroy(None)


def test_ctypes_structs_match_the_c_layout(mtp, tmp_path):
    """Every field of the binding's structures sits at the offset gcc gives the
    header's declaration (a drifted field would pass garbage silently)."""
    import shutil
    import subprocess
    if not shutil.which("gcc"):
        pytest.skip("no host C compiler")
    structs = {"mtp_model_desc": mtp.ModelDesc, "mtp_weights": mtp.Weights, "mtp_kv_view": mtp.KVView,
               "mtp_seq": mtp.Seq, "mtp_sampler": mtp.Sampler, "mtp_lm_head": mtp.LmHead}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "mtp.h"', 'int main(void) {']
    for cname, py in structs.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f in py._fields_:
            lines.append(f'printf("{cname} {f[0]} %zu\\n", offsetof({cname}, {f[0]}));')
    lines += ['return 0;', '}']
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", str(ROOT / "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for cname, py in structs.items():
        assert got[(cname, "size")] == C.sizeof(py), cname
        for f in py._fields_:
            assert got[(cname, f[0])] == getattr(py, f[0]).offset, (cname, f[0])
