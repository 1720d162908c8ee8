"""ctypes front end of the reference oracle (oracle/ps_oracle.c).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module. All arrays are host numpy arrays;
every function mirrors one C entry point of ps_oracle.c.
"""
import ctypes
import dataclasses
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libps_oracle.so")

ALGO_ADAM, ALGO_NADAM = 0, 1
SPLIT_TRUNC, SPLIT_NEAREST_AWAY, SPLIT_STOCHASTIC = 0, 1, 2
SIGNED, UNSIGNED = 0, 1
BLOCK = 256

_vp, _i64, _int, _f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float


class _HP(ctypes.Structure):
    _fields_ = [("algo", ctypes.c_int32), ("split_mode", ctypes.c_int32), ("lr", ctypes.c_double),
                ("beta1", ctypes.c_double), ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("momentum_decay", ctypes.c_double),
                ("seed", ctypes.c_uint64), ("tensor", ctypes.c_int64), ("elem0", ctypes.c_int64)]


class _FHP(ctypes.Structure):
    _fields_ = [("split_mode", ctypes.c_int32), ("reserved", ctypes.c_int32), ("lr", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps1", ctypes.c_double), ("clip_threshold", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("decay_rate", ctypes.c_double), ("beta1", ctypes.c_double),
                ("seed", ctypes.c_uint64), ("tensor", ctypes.c_int64)]


class _Coeffs(ctypes.Structure):
    _fields_ = [(k, ctypes.c_float) for k in ("B1", "C1", "B2", "C2", "EPS", "A", "RS2", "AG", "AM", "CWD")]


@dataclass
class HParams:
    algo: int = ALGO_NADAM
    split_mode: int = SPLIT_TRUNC
    lr: float = 3.5e-6
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    momentum_decay: float = 4e-3
    seed: int = 0      # stochastic rounding only
    tensor: int = 0    # stochastic rounding only: the tensor's index in the step's list
    elem0: int = 0     # stochastic rounding only: tensor index of the arrays' first element

    def c(self):
        return _HP(self.algo, self.split_mode, self.lr, self.beta1, self.beta2, self.eps, self.weight_decay,
                   self.momentum_decay, self.seed, self.tensor, self.elem0)


@dataclass
class FHParams:
    split_mode: int = SPLIT_TRUNC
    lr: float = 3.5e-6
    beta2: float = 0.999
    eps1: float = 1e-30
    clip_threshold: float = 1.0
    weight_decay: float = 0.0
    decay_rate: float = 0.0   # < 0: beta2 at update t is 1 - t^decay_rate (Adafactor's schedule)
    beta1: float = 0.0        # > 0: first moment of the clipped update, in mc/ms (signed codec)
    seed: int = 0             # stochastic rounding only
    tensor: int = 0           # stochastic rounding only: the tensor's index in the step's list

    def c(self):
        return _FHP(self.split_mode, 0, self.lr, self.beta2, self.eps1, self.clip_threshold, self.weight_decay,
                    self.decay_rate, self.beta1, self.seed, self.tensor)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB_PATH)
        sig = {
            "orc_join": ([_vp, _vp, _vp, _i64, _int], None),
            "orc_split": ([_vp, _vp, _vp, _i64, _int], None),
            "orc_encode": ([_vp, _i64, _int, _vp, _vp], None),
            "orc_decode": ([_vp, _vp, _i64, _int, _vp], None),
            "orc_dec_mag": ([_f32, _int], _f32),
            "orc_code_mag": ([_f32, _int], ctypes.c_uint32),
            "orc_dec_mag_array": ([_vp, _i64, _int, _vp], None),
            "orc_code_mag_array": ([_vp, _i64, _int, _vp], None),
            "orc_coeffs_for": ([ctypes.POINTER(_HP), _i64, ctypes.POINTER(_Coeffs)], None),
            "orc_core_step": ([_vp, _vp, _vp, _vp, _i64, ctypes.POINTER(_HP), _i64], None),
            "orc_opt_step": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, ctypes.POINTER(_HP), _i64], None),
            "orc_opt_step_flags": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, ctypes.c_uint32, ctypes.POINTER(_HP),
                                    _i64], None),
            "orc_f24_encode": ([_vp, _i64, _vp], None),
            "orc_splitmix64_mix": ([ctypes.c_uint64], ctypes.c_uint64),
            "orc_splitmix64_at": ([ctypes.c_uint64, ctypes.c_uint64], ctypes.c_uint64),
            "orc_sr_rand16": ([ctypes.c_uint64, _i64, _i64, _i64], ctypes.c_uint16),
            "orc_sr_bf16": ([ctypes.c_float, ctypes.c_uint16], ctypes.c_uint16),
            "orc_sr_rand16_array": ([ctypes.c_uint64, _i64, _i64, _i64, _i64, _vp], None),
            "orc_f24_decode": ([_vp, _i64, _vp], None),
            "orc_factored_2d": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, ctypes.POINTER(_FHP), _i64], None),
            "orc_factored_1d": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, ctypes.POINTER(_FHP), _i64], None),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _p(a, dtype):
    assert a.dtype == dtype and a.flags.c_contiguous, (a.dtype, dtype)
    return a.ctypes.data


def join(hi, lo, mode=SPLIT_TRUNC, out=None):
    w = np.empty(hi.shape, np.float32) if out is None else out
    lib().orc_join(_p(hi, np.uint16), _p(lo, np.uint16), _p(w, np.float32), hi.size, mode)
    return w


def split(w, mode=SPLIT_TRUNC, out=None):
    hi, lo = (np.empty(w.shape, np.uint16), np.empty(w.shape, np.uint16)) if out is None else out
    lib().orc_split(_p(w, np.float32), _p(hi, np.uint16), _p(lo, np.uint16), w.size, mode)
    return hi, lo


def nblocks(n):
    return (n + BLOCK - 1) // BLOCK


def encode(x, kind):
    code = np.empty(x.shape, np.uint16)
    scale = np.empty(nblocks(x.size), np.float32)
    lib().orc_encode(_p(x, np.float32), x.size, kind, _p(code, np.uint16), _p(scale, np.float32))
    return code, scale


def decode(code, scale, kind):
    x = np.empty(code.shape, np.float32)
    lib().orc_decode(_p(code, np.uint16), _p(scale, np.float32), code.size, kind, _p(x, np.float32))
    return x


def dec_mag(h, kind):
    h = np.ascontiguousarray(h, np.float32)
    out = np.empty(h.shape, np.float32)
    lib().orc_dec_mag_array(_p(h, np.float32), h.size, kind, _p(out, np.float32))
    return out


def code_mag(x, kind):
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint32)
    lib().orc_code_mag_array(_p(x, np.float32), x.size, kind, _p(out, np.uint32))
    return out


def coeffs(hp: HParams, step: int):
    c = _Coeffs()
    h = hp.c()
    lib().orc_coeffs_for(ctypes.byref(h), step, ctypes.byref(c))
    return {k: np.float32(getattr(c, k)) for k, _ in _Coeffs._fields_}


def core_step(w, m, v, g, hp: HParams, step: int):
    """In place on fp32 arrays w, m, v; g fp32."""
    h = hp.c()
    lib().orc_core_step(_p(w, np.float32), _p(m, np.float32), _p(v, np.float32), _p(g, np.float32), w.size,
                        ctypes.byref(h), step)


@dataclass
class TensorState:
    """Host copy of one tensor's optimizer state (all numpy, C-contiguous)."""
    hi: np.ndarray
    lo: np.ndarray
    mc: np.ndarray = None
    ms: np.ndarray = None
    vc: np.ndarray = None
    vs: np.ndarray = None
    row: np.ndarray = None
    col: np.ndarray = None

    def copy(self):
        return TensorState(*[None if a is None else a.copy() for a in
                             (self.hi, self.lo, self.mc, self.ms, self.vc, self.vs, self.row, self.col)])


def zero_moments(n):
    nb = nblocks(n)
    return (np.full(n, 32768, np.uint16), np.zeros(nb, np.float32), np.zeros(n, np.uint16),
            np.zeros(nb, np.float32))


def opt_step(st: TensorState, g, hp: HParams, step: int):
    """In place on `st`; g is a uint16 bf16 pattern array or None."""
    h = hp.c()
    gp = None if g is None else _p(g, np.uint16)
    lib().orc_opt_step(_p(st.hi, np.uint16), _p(st.lo, np.uint16), gp, _p(st.mc, np.uint16),
                       _p(st.ms, np.float32), _p(st.vc, np.uint16), _p(st.vs, np.float32), st.hi.size,
                       ctypes.byref(h), step)


FP32_MOMENTS, FP32_PARAM, F24_MOMENTS = 1, 2, 4


def splitmix64_at(state, k):
    """Output k (0-based) of the SplitMix64 stream starting at `state`."""
    return lib().orc_splitmix64_at(state, k)


def sr_rand16(seed, step, tensor, e0, n):
    """The stochastic-rounding random 16-bit values of elements e0 .. e0+n-1."""
    out = np.empty(n, np.uint16)
    lib().orc_sr_rand16_array(seed, step, tensor, e0, n, out.ctypes.data)
    return out


def sr_bf16(x, r):
    """Stochastic rounding of the fp32 value x to bf16 bits with the random 16 bits r."""
    return lib().orc_sr_bf16(float(np.float32(x)), int(r))


def f24_encode(x):
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(3 * x.size, np.uint8)
    lib().orc_f24_encode(x.ctypes.data, x.size, out.ctypes.data)
    return out


def f24_decode(b):
    b = np.ascontiguousarray(b, np.uint8)
    out = np.empty(b.size // 3, np.float32)
    lib().orc_f24_decode(b.ctypes.data, out.size, out.ctypes.data)
    return out


def opt_step_flags(w, lo, g, m, ms, v, vs, flags, hp: HParams, step: int):
    """In place. w/g: uint16 (bf16 bits) or float32 when FP32_PARAM; m/v: uint16
    codes with scales ms/vs, float32 arrays when FP32_MOMENTS, or uint8 f24
    arrays (3 bytes per value) when F24_MOMENTS."""
    h = hp.c()
    ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
    n = w.size
    lib().orc_opt_step_flags(ptr(w), ptr(lo), ptr(g), ptr(m), ptr(ms), ptr(v), ptr(vs), n, flags,
                             ctypes.byref(h), step)


def opt_step_multi(states, grads, hp: HParams, step: int):
    """The list step: tensor i is keyed by its index for stochastic rounding."""
    for i, (st, g) in enumerate(zip(states, grads)):
        opt_step(st, g, dataclasses.replace(hp, tensor=i), step)


def factored_step(st: TensorState, g, rows: int, cols: int, hp: FHParams, step: int):
    """rows == 0: 1-D tensor (codec second moment); else 2-D [rows, cols]."""
    h = hp.c()
    gp = None if g is None else _p(g, np.uint16)
    if hp.beta1 != 0.0:
        mcp, msp = _p(st.mc, np.uint16), _p(st.ms, np.float32)
    else:
        mcp = msp = None
    if rows > 0:
        lib().orc_factored_2d(_p(st.hi, np.uint16), _p(st.lo, np.uint16), gp, _p(st.row, np.float32),
                              _p(st.col, np.float32), mcp, msp, rows, cols, ctypes.byref(h), step)
    else:
        lib().orc_factored_1d(_p(st.hi, np.uint16), _p(st.lo, np.uint16), gp, _p(st.vc, np.uint16),
                              _p(st.vs, np.float32), mcp, msp, st.hi.size, ctypes.byref(h), step)


def bf16_to_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_bits(x):
    return np.ascontiguousarray(x, np.float32).view(np.uint32)
