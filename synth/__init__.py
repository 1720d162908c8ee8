"""Seeded synthetic inputs (host and device), shared by the oracle's tests,
the HIP library's tests and the benchmark. See synth.h for the generator."""
import ctypes
import os

import numpy as np

from .workloads import (STREAM_GRAD, STREAM_HI, STREAM_LO, SIGMA_G, SIGMA_W,  # noqa: F401
                        Shape, WORKLOADS, total_params)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libps_synth.so")
_lib = None

_i64, _u64, _f64, _vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
        try:   # torch's HIP runtime first, so that the library binds to it (one runtime per process)
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(_LIB_PATH)
        L.syn_host_fill_bf16_normal.argtypes = [_vp, _i64, _i64, _u64, _u64, _u64, _u64, _f64, _f64, _f64]
        L.syn_host_fill_bf16_normal.restype = None
        L.syn_host_fill_u16_uniform.argtypes = [_vp, _i64, _i64, _u64, _u64, _u64, _u64]
        L.syn_host_fill_u16_uniform.restype = None
        L.syn_dev_fill_bf16_normal.argtypes = [_vp, _i64, _i64, _u64, _u64, _u64, _u64, _f64, _f64, _f64, _vp]
        L.syn_dev_fill_bf16_normal.restype = ctypes.c_int
        L.syn_dev_fill_u16_uniform.argtypes = [_vp, _i64, _i64, _u64, _u64, _u64, _u64, _vp]
        L.syn_dev_fill_u16_uniform.restype = ctypes.c_int
        _lib = L
    return _lib


def host_bf16_normal(n, seed, stream, tensor, step, sigma, outlier_p=0.0, outlier_scale=1.0, start=0):
    out = np.empty(n, dtype=np.uint16)
    lib().syn_host_fill_bf16_normal(out.ctypes.data, start, n, seed, stream, tensor, step, sigma,
                                    outlier_p, outlier_scale)
    return out


def host_u16_uniform(n, seed, stream, tensor, step, start=0):
    out = np.empty(n, dtype=np.uint16)
    lib().syn_host_fill_u16_uniform(out.ctypes.data, start, n, seed, stream, tensor, step)
    return out


def _stream_handle(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def dev_bf16_normal(t, seed, stream, tensor, step, sigma, outlier_p=0.0, outlier_scale=1.0, start=0):
    """Fill the 16-bit device tensor `t` (any 2-byte dtype, contiguous)."""
    assert t.is_cuda and t.element_size() == 2 and t.is_contiguous()
    rc = lib().syn_dev_fill_bf16_normal(t.data_ptr(), start, t.numel(), seed, stream, tensor, step, sigma,
                                        outlier_p, outlier_scale, _stream_handle(t))
    if rc != 0:
        raise RuntimeError(f"syn_dev_fill_bf16_normal failed: hip error {rc}")


def dev_u16_uniform(t, seed, stream, tensor, step, start=0):
    assert t.is_cuda and t.element_size() == 2 and t.is_contiguous()
    rc = lib().syn_dev_fill_u16_uniform(t.data_ptr(), start, t.numel(), seed, stream, tensor, step,
                                        _stream_handle(t))
    if rc != 0:
        raise RuntimeError(f"syn_dev_fill_u16_uniform failed: hip error {rc}")
