"""Build tests/kernels/libps_probe.so with hipcc for gfx950, with the
library's arithmetic flags: test-only kernels over the library's device
helpers (probe_exact.hip) and the streaming ceiling kernels that bench.py
times next to the step (stream_ceiling.hip)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libps_probe.so")


def build(verbose=False):
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(HERE, "probe_exact.hip"), os.path.join(HERE, "stream_ceiling.hip"), "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on the probe kernels:\n{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB
