"""The fp64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only), driven through every entry point on small cases that
reach the edges of its index arithmetic (tests/oracle_sanitize_main.c). Any
out-of-bounds access, leak, misaligned or overflowing operation makes the
sanitizers abort the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "tests", "oracle_sanitize_main.c"),
           os.path.join(ROOT, "oracle", "lsh_oracle.c"), "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
