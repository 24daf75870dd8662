"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (host code
only, gcc): a driver program compiled together with the oracle's C source runs every entry
point on small seeded inputs, edge cases and malformed indices included (masked, NaN and
empty rows, K = 0, one particle, degenerate weights, an exhausted block pool and the -1
slots it leaves, out-of-range draft tokens and ancestors, a corrupt free-stack entry),
serially and with OpenMP threads.  Any sanitizer report fails the test."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "helpers", "oracle_sanitize_driver.c")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _build(openmp: bool) -> str:
    d = tempfile.mkdtemp(prefix="orc_san_")
    exe = os.path.join(d, "driver")
    cmd = ["gcc", "-std=gnu99", "-O1", "-g"] + (["-fopenmp"] if openmp else []) + SAN + \
        [DRIVER, "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        if "asan" in r.stderr.lower() or "ubsan" in r.stderr.lower():
            pytest.skip("gcc has no sanitizer runtime here: " + r.stderr[-200:])
        raise AssertionError(r.stderr)
    return exe


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not present")
@pytest.mark.parametrize("openmp", [False, True])
def test_oracle_is_clean_under_asan_and_ubsan(openmp):
    exe = _build(openmp)
    env = dict(os.environ, OMP_NUM_THREADS="4", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.strip().endswith("ok")
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
