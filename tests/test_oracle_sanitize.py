"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
host code only) and driven through every function by tests/oracle_sanitize.c:
any out-of-bounds access, leak or undefined operation fails the run."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_sanitize")
        cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-I", os.path.join(ROOT, "oracle"), os.path.join(ROOT, "tests", "oracle_sanitize.c"),
               os.path.join(ROOT, "oracle", "csa2_oracle.c"), "-lm", "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=180)
        assert r.returncode == 0, r.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "oracle sanitize run ok" in r.stdout
        assert "runtime error" not in r.stderr
