"""The library's device blob cache (precision_state_amd/csrc/blob_cache.h)
under concurrent callers, on the host: tests/blob_cache_host_test.cpp drives
it with a fake asynchronous device and tiny limits, so that it empties itself
thousands of times while eight threads take blobs and launch on them. Built
with ThreadSanitizer; every launch must read the bytes it asked for from
memory that is still allocated."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_blob_cache_never_frees_a_blob_before_its_launch(tmp_path):
    exe = tmp_path / "blob_cache_host_test"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-pthread",
           "-I", os.path.join(ROOT, "precision_state_amd", "csrc"),
           os.path.join(ROOT, "tests", "blob_cache_host_test.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True)
    r = subprocess.run([str(exe), "8", "3000"], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, TSAN_OPTIONS="halt_on_error=1"))
    print(r.stdout, r.stderr[-4000:])
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    fields = dict(kv.split("=") for kv in r.stdout.split())
    assert int(fields["errors"]) == 0 and int(fields["launches"]) == 24000
    assert int(fields["flushes"]) >= 100
