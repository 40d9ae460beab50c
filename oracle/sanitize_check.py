"""Build the oracle with AddressSanitizer and UndefinedBehaviorSanitizer
(host code, gcc) and run every oracle pin against that build.

Test infrastructure, CPU only: `python oracle/sanitize_check.py`.  The
sanitized library is written beside the optimised one
(libmtp_oracle_san.so) and loaded through MTP_ORACLE_LIB; the ASan runtime
is preloaded because the Python interpreter itself is not instrumented.
Any sanitizer report aborts the run (halt_on_error), so a zero exit status
means no out-of-bounds access, use after free or undefined behaviour was
reported.  Leak checking is off: the interpreter keeps allocations alive
at exit by design.
"""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

HERE = Path(__file__).resolve().parent
ROOT = HERE.parent
SAN_LIB = HERE / "libmtp_oracle_san.so"
PIN_FILES = ["tests/test_oracle_pins.py", "tests/test_oracle_flags.py"]


def build() -> Path:
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fPIC", "-shared",
           "-Wall", "-Wno-unknown-pragmas", "-o", str(SAN_LIB), str(HERE / "mtp_oracle.c"), "-lm"]
    subprocess.run(cmd, check=True)
    return SAN_LIB


def main() -> int:
    build()
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True, capture_output=True,
                          text=True).stdout.strip()
    env = dict(os.environ)
    env.update(MTP_ORACLE_LIB=str(SAN_LIB), LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *PIN_FILES], cwd=ROOT,
                       env=env)
    print(f"sanitizer run of the oracle pins: exit status {r.returncode}", flush=True)
    return r.returncode


if __name__ == "__main__":
    sys.exit(main())
