import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def orc():
    from oracle import oracle as O
    O.build(force=False)
    return O


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """The parity counts the GPU tests recorded (near ties, flagged
    sequences, largest errors), one JSON line per case, and their totals;
    also written to $MTP_PARITY_RECORD when that names a file."""
    import json
    import os
    try:
        from tests.gpu_harness import RECORDS
    except Exception:
        return
    if not RECORDS:
        return
    tot = {"cases": len(RECORDS)}
    for r in RECORDS:
        for k in ("near_ties", "flagged", "compared", "mismatches_on_clean"):
            if k in r:
                tot[k] = tot.get(k, 0) + r[k]
    terminalreporter.write_sep("-", "parity records")
    for r in RECORDS:
        terminalreporter.write_line("PARITY " + json.dumps(r, separators=(",", ":")))
    terminalreporter.write_line("PARITY_TOTAL " + json.dumps(tot, separators=(",", ":")))
    path = os.environ.get("MTP_PARITY_RECORD")
    if path:
        with open(path, "w") as f:
            json.dump({"total": tot, "cases": RECORDS}, f, indent=1)
