"""Run the CPU test suite against AddressSanitizer/UBSan builds of the host code.

    python tests/sanitize.py [extra pytest args]

Builds the host-instrumented libbasa (plan, argument checks, error paths;
device code is not instrumented) and the instrumented C oracle under
``_build/``, then runs ``pytest -m "not gpu"`` in a child process that
preloads clang's sanitizer runtime and loads those builds through
``BASA_LIBRARY`` / ``BASA_ORACLE_LIBRARY``.  Any heap or stack overflow,
use-after-free or undefined behaviour (signed overflow, bad shift, misaligned
access, out-of-bounds index on a fixed array) aborts the run with a report.

Leak detection is off: the Python interpreter and torch keep allocations
alive until exit by design, which would drown real reports.
"""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main(argv: list) -> int:
    import __graft_entry__ as entry
    from video_gen_amd import build as b

    lib = b.build(sanitize=True)
    oracle = entry._build_oracle(sanitize=True)
    for path in (lib, oracle):
        syms = subprocess.run(["nm", "-D", path], capture_output=True, text=True).stdout
        if "__asan_report" not in syms:
            raise RuntimeError(f"{path} carries no ASan instrumentation")
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": b.sanitizer_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:print_summary=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "BASA_LIBRARY": lib,
        "BASA_ORACLE_LIBRARY": oracle,
    })
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-x", "-q", "-m",
           "not gpu", "-p", "no:cacheprovider", *argv]
    print("sanitized run:", lib, oracle, flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
