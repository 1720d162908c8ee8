"""One HIP runtime per process. libps.so and synth's library link the
system's libamdhip64; PyTorch ships its own. Whatever the import order, the
binding and synth load torch first, so the libraries bind to torch's runtime
and a single libamdhip64 is mapped: with two, device memory and streams of one
runtime are not valid in the other (a GPU process then fails at its first
launch). Checked in fresh interpreters on the host (no GPU needed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_MAPPED = "sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l})"


@pytest.mark.parametrize("first", ["import precision_state_amd", "import synth; synth.lib()",
                                   "import oracle; import synth; synth.lib(); import precision_state_amd"])
def test_single_hip_runtime_whatever_the_import_order(first):
    pytest.importorskip("torch")
    code = f"import sys; sys.path.insert(0, {ROOT!r}); {first}; import torch; print({_MAPPED})"
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    mapped = eval(out.stdout.strip().splitlines()[-1])
    assert len(mapped) == 1, mapped
