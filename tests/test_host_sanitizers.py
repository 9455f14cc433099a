"""Host-code sanitizers (CPU only): the oracle's and the input generators' C
code built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, no GPU
code involved) and driven over every entry point by tests/sanitize/host_driver.c.
Any out-of-bounds access, use after free, leak or undefined operation ends the
run with a sanitizer report and a non-zero status."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_and_generators_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "host_driver")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "sanitize", "host_driver.c"),
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "synth", "synth.c"),
           "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and ("libasan" in r.stderr or "libubsan" in r.stderr):
        pytest.skip("sanitizer runtimes not installed")
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout[-1000:], r.stderr[-3000:])
