"""The CPU oracle built with the host compiler's address and undefined-
behaviour checking, driven over ragged shapes with exact-size buffers
(tests/sanitize/oracle_driver.c): any out-of-bounds access, leak or
undefined operation in the checker fails the test. Host code only."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHECKS = ["address", "undefined"]


def test_oracle_under_host_sanitizers():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_driver")
        flags = ["-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-omit-frame-pointer",
                 "-fsanitize=" + ",".join(CHECKS), "-fno-sanitize-recover=all"]
        build = subprocess.run([gcc, *flags, os.path.join(ROOT, "oracle", "rx_oracle.c"),
                                os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                                "-o", exe, "-lm"], capture_output=True, text=True)
        if build.returncode != 0 and "asan" in (build.stderr + build.stdout).lower():
            pytest.skip("host sanitizer runtime not available: " + build.stderr[-300:])
        assert build.returncode == 0, build.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
        assert run.returncode == 0, run.stderr[-3000:]
        assert run.stdout.strip() == "ok"
