"""The Python binding's ctypes records have the layout include/ps.h declares.

A small C program built with gcc against the header prints sizeof and every
field's offsetof; each must equal the ctypes Structure's. No GPU and no call
into libps.so: this pins the argument marshalling itself."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

RECORDS = {
    "ps_tensor": ("CTensor", ["w_hi", "w_lo", "grad", "m_code", "m_scale", "v_code", "v_scale", "row_ema",
                              "col_ema", "numel", "rows", "cols", "flags", "reserved"]),
    "ps_hparams": ("CHParams", ["algo", "split_mode", "lr", "beta1", "beta2", "eps", "weight_decay",
                                "momentum_decay", "seed"]),
    "ps_factored_hparams": ("CFHParams", ["split_mode", "reserved", "lr", "beta2", "eps1", "clip_threshold",
                                          "weight_decay", "decay_rate", "beta1", "seed"]),
    "ps_offload_group": ("COffloadGroup", ["tensors", "n_tensors"]),
    "ps_offload_options": ("COffloadOptions", ["mode", "n_cus", "reserved0", "reserved1"]),
}


@pytest.fixture(scope="module")
def ps():
    import precision_state_amd as ps
    return ps


@pytest.fixture(scope="module")
def c_layout(tmp_path_factory):
    d = tmp_path_factory.mktemp("layout")
    lines = ['#include <stdio.h>', '#include "ps.h"', "int main(void) {"]
    for rec, (_, fields) in RECORDS.items():
        lines.append(f'  printf("{rec} sizeof %zu\\n", sizeof({rec}));')
        for f in fields:
            lines.append(f'  printf("{rec} {f} %zu %zu\\n", offsetof({rec}, {f}), sizeof((({rec}*)0)->{f}));')
    lines += ["  return 0;", "}"]
    src = d / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = d / "layout"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    table = {}
    for line in out.splitlines():
        parts = line.split()
        if parts[1] == "sizeof":
            table[(parts[0], None)] = (int(parts[2]),)
        else:
            table[(parts[0], parts[1])] = (int(parts[2]), int(parts[3]))
    return table


@pytest.mark.parametrize("rec", sorted(RECORDS))
def test_ctypes_record_matches_header(ps, c_layout, rec):
    import ctypes
    cls = getattr(ps, RECORDS[rec][0])
    names = [f[0] for f in cls._fields_]
    assert names == RECORDS[rec][1], "field list differs from the header's"
    assert ctypes.sizeof(cls) == c_layout[(rec, None)][0]
    for name, ctype in cls._fields_:
        off, size = c_layout[(rec, name)]
        assert getattr(cls, name).offset == off, (rec, name)
        assert ctypes.sizeof(ctype) == size, (rec, name)
