"""Build synth/libps_synth.so (host + gfx950 device fill routines) with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libps_synth.so")


def build(verbose=False):
    cmd = [
        "hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
        "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        os.path.join(HERE, "synth.hip"), "-o", LIB + ".tmp",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.DEVNULL)
    os.replace(LIB + ".tmp", LIB)
    return LIB
