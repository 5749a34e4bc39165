"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer.

Host code only: oracle/nbody_oracle.c is compiled by gcc together with a
small C driver (oracle_sanitize_driver.c) that calls every entry point on
sizes 0, 1, 2, 3, 97 and 256, with two OpenMP threads.  Any out-of-bounds
access, leak or undefined operation makes the sanitizer abort the run.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _build(tmp_path, flags):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fopenmp", *flags, os.path.join(HERE, "oracle_sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "nbody_oracle.c"), "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip(f"gcc cannot build with {flags}: {r.stderr[-400:]}")
    return exe


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("flags", [
    ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
])
def test_oracle_under_sanitizers(tmp_path, flags):
    exe = _build(tmp_path, flags)
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
    assert "runtime error" not in r.stderr
    assert "AddressSanitizer" not in r.stderr
