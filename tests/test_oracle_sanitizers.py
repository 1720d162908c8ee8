"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a C
driver (tests/oracle_sanitize_driver.c) compiles the oracle source into one
program with gcc and calls every entry point over ragged sizes, all split
modes, storage flags, factored shapes (1 x 1 up to 64 x 300, zero
gradients, tensors without a gradient). Any out-of-bounds access, use of
freed memory, leak, or undefined arithmetic aborts the run."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", os.path.join(HERE, "oracle_sanitize_driver.c"),
           "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.strip() == "ok"
