"""Build precision_state_amd/libps.so from csrc/ with hipcc for gfx950.

Every source is compiled with -ffp-contract=off (fused multiply-adds only
where the code calls fma), correctly rounded fp32 division and square root
(hipcc's default), denormals kept, and packed-fp32 instructions disabled.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libps.so")
OBJ_DIR = os.path.join(HERE, "_build")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(verbose=False, jobs=8):
    os.makedirs(OBJ_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OBJ_DIR, src + ".o")
        cmd = ["hipcc", "--offload-arch=gfx950", *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        msgs = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if msgs and verbose:
            print("\n".join(msgs))
        return obj

    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, sources()))
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB
