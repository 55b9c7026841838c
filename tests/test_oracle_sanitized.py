"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a driver that calls
every oracle function on small seeded inputs (tests/sanitize/oracle_driver.c, which compiles
oracle/moe_oracle.c into itself) is built with gcc -fsanitize=address,undefined and run; any
out-of-bounds access, leak or undefined behaviour aborts it.  Host code only."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_undefined_behaviour_sanitizers():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_driver")
        # the oracle's own flags (no contraction, no fast-math) plus the sanitizers; the
        # first finding aborts the run
        cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
               "-fno-fast-math", "-fopenmp", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all", DRIVER, "-o", exe, "-lm"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "oracle driver ok" in r.stdout
