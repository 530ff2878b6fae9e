"""The oracle's pins again, with the oracle built under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; any report aborts the run): out
of bounds accesses, use after free and undefined arithmetic in oracle.c fail
here even where the values happen to come out right."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_pins_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from oracle import build as ob
    lib = ob.build(sanitize=True)
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm  # the build is instrumented
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not asan or not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no ASan runtime for gcc here")
    env = dict(os.environ, LD_PRELOAD=asan, ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout
