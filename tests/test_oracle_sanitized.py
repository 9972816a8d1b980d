"""The oracle's CPU pins run against oracle.c built with AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU).  A stray read or write past an operand, a
signed overflow, a misaligned access or a bad shift in the decoders, the loops
or the sparse-metadata reader aborts the run; the pins themselves must pass
unchanged.  The oracle is test infrastructure: this checks the checker."""
import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = oracle_build.build_sanitized(str(tmp_path / "liboracle_san.so"))
    runtime = oracle_build.sanitizer_runtime()
    if not os.path.isabs(runtime) or not os.path.exists(runtime):
        pytest.skip("gcc's ASan runtime is not installed")
    logs = tmp_path / "san"
    env = dict(os.environ, ORACLE_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:log_path=%s" % logs,
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:log_path=%s" % logs,
               OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    reports = "".join(open(tmp_path / f).read() for f in os.listdir(tmp_path) if f.startswith("san"))
    assert r.returncode == 0 and not reports, (reports + out)[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
