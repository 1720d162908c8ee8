"""Exhaustive checks of two exactness claims of the fused step's device
arithmetic (precision_state_amd/csrc/dev_common.h), through the test-only
probe kernels in tests/kernels/probe_exact.hip:

- sqrt_rn_fast (hardware root plus a two-neighbour residual test) equals the
  correctly rounded IEEE square root, computed here on the CPU by numpy, on
  every fp32 v = 0 or 2^-96 <= v < inf (1.88e9 inputs);
- the fused step encodes exp_avg_sq from y = sqrt(sqrt(v) * sqrt(1/s)), not
  from x = v * (1/s) as ps_encode_moments does. For each of 256 block scales
  s, every fp32 v in [0, s] gets the standalone encoder's code (which the
  exhaustive codec test ties to the oracle for every x in [0, 1]); a sample
  of v per scale is also compared with the oracle's code of x directly.

The moment codec is the pages' scaled, biased, pow()-companded uint16 storage
(sd-scripts PR #2187, second post)."""
import ctypes
import os

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "kernels", "libps_probe.so")


def _probe():
    if not os.path.exists(PROBE):
        raise RuntimeError(f"{PROBE} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(PROBE)
    L.probe_sqrt_fast.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    L.probe_fused_vcode_diff.argtypes = [ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
    L.probe_fused_vcode.argtypes = [ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32,
                                    ctypes.c_void_p]
    return L


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def test_sqrt_rn_fast_is_correctly_rounded_on_every_input():
    L = _probe()
    chunk = 1 << 28
    out = torch.empty(chunk, dtype=torch.int32, device="cuda")
    first, end = 0x0F800000, 0x7F800000            # 2^-96 .. largest finite
    ranges = [(0, 1)] + [(a, min(chunk, end - a)) for a in range(first, end, chunk)]
    total = 0
    for a, n in ranges:
        assert L.probe_sqrt_fast(a, n, ctypes.c_void_p(out.data_ptr()), _stream()) == 0
        got = out[:n].cpu().numpy().view(np.uint32)
        v = np.arange(a, a + n, dtype=np.uint64).astype(np.uint32).view(np.float32)
        want = np.sqrt(v).view(np.uint32)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, [hex(int(a + i)) for i in bad[:8]]
        total += n
        print(f"  sqrt: {hex(a)} + {n} ok", flush=True)
    assert total == 1 + (end - first)


def _scales():
    rng = np.random.default_rng(2024)
    fixed = [1.0, 2.0, np.nextafter(np.float32(1), np.float32(2)), np.nextafter(np.float32(2), np.float32(1)),
             np.nextafter(np.float32(4), np.float32(1)), 2.0 ** -126, 1.5 * 2.0 ** -100, 3.0, 1e-8, 7.3e-12,
             2.0 ** 100, 1.9999999 * 2.0 ** 60]
    s = [np.float32(x) for x in fixed]
    expo = rng.uniform(-125.0, 20.0, 256 - len(s))
    mant = rng.uniform(1.0, 2.0, 256 - len(s))
    s += [np.float32(m * 2.0 ** np.floor(e)) for m, e in zip(mant, expo)]
    return s


def test_fused_exp_avg_sq_code_equals_the_encoder_for_every_v():
    L = _probe()
    counters = torch.zeros(17, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(7)
    n_sample = 1 << 16
    vbuf = torch.empty(n_sample, dtype=torch.float32, device="cuda")
    obuf = torch.empty(n_sample, dtype=torch.int32, device="cuda")
    checked = 0
    for k, s in enumerate(_scales()):
        counters.zero_()
        assert L.probe_fused_vcode_diff(ctypes.c_float(s), ctypes.c_void_p(counters.data_ptr()), _stream()) == 0
        c = counters.cpu().numpy().view(np.uint32)
        assert c[0] == 0, (float(s), int(c[0]), [hex(int(x)) for x in c[1:1 + min(16, int(c[0]))]])
        checked += int(np.float32(s).view(np.uint32)) + 1
        # direct comparison with the oracle on a sample (v = s and v = 0 included)
        bits = rng.integers(0, int(np.float32(s).view(np.uint32)) + 1, n_sample, dtype=np.uint64).astype(np.uint32)
        bits[:2] = [0, np.float32(s).view(np.uint32)]
        v = bits.view(np.float32)
        vbuf.copy_(torch.from_numpy(v))
        assert L.probe_fused_vcode(ctypes.c_float(s), ctypes.c_void_p(vbuf.data_ptr()),
                                   ctypes.c_void_p(obuf.data_ptr()), n_sample, _stream()) == 0
        got = obuf.cpu().numpy().view(np.uint32)
        inv = np.float32(1) / np.float32(s)
        want = oracle.code_mag(v * inv, oracle.UNSIGNED)
        assert np.array_equal(got, want), (float(s), int(np.count_nonzero(got != want)))
        if k % 32 == 0:
            print(f"  scale {k}: {float(s):.6g} ok", flush=True)
    print(f"  {checked} (v, s) pairs", flush=True)
