"""Python binding of libps.so, the MI355X fused low-precision optimizer step.

Argument marshalling only: every function takes torch tensors that live in
device memory, passes their pointers and the current HIP stream to the C ABI
declared in include/ps.h, and raises PSError on a non-zero status. No step
of the computation runs in Python or PyTorch; if libps.so is missing the
import fails.

16-bit arrays (bf16 weights and gradients, residuals, moment codes) may be any
2-byte dtype (torch.int16, torch.uint16, torch.bfloat16): only their bits
matter. Scale and EMA arrays are torch.float32.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libps.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")

# libps.so needs libamdhip64.so.7. PyTorch ships a HIP runtime of its own:
# with torch loaded first the library binds to that one, and the process has a
# single HIP runtime whose device pointers and streams both sides share.
# Loaded first, the library would map the system runtime and torch its own
# afterwards: two runtimes on one GPU, each unable to use the other's memory
# and streams. So torch is imported before the library whenever it exists.
try:
    import torch  # noqa: F401
except ImportError:
    pass

_lib = ctypes.CDLL(LIB_PATH)

ALGO_ADAM, ALGO_NADAM = 0, 1
SPLIT_TRUNC, SPLIT_NEAREST_AWAY, SPLIT_STOCHASTIC = 0, 1, 2
MOMENT_SIGNED, MOMENT_UNSIGNED = 0, 1
TENSOR_FP32_MOMENTS, TENSOR_FP32_PARAM, TENSOR_F24_MOMENTS = 1, 2, 4
BLOCK = 256

STATUS = {0: "PS_OK", 1: "PS_ERR_INVALID_ARG", 2: "PS_ERR_ALIGNMENT", 3: "PS_ERR_SHAPE",
          4: "PS_ERR_UNSUPPORTED", 5: "PS_ERR_HIP", 6: "PS_ERR_NO_MEMORY", 7: "PS_ERR_WORKSPACE"}

EXPORTED = ["ps_opt_step_multi", "ps_step_scalars", "ps_split", "ps_join", "ps_encode_moments",
            "ps_decode_moments", "ps_factored_workspace_size", "ps_factored_step", "ps_factored_step_noalloc",
            "ps_offload_plan_create", "ps_offload_plan_create_ex",
            "ps_offload_run", "ps_offload_bytes", "ps_offload_plan_destroy", "ps_status_string",
            "ps_last_error", "ps_version"]


class PSError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class CTensor(ctypes.Structure):
    _fields_ = [("w_hi", ctypes.c_void_p), ("w_lo", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("m_code", ctypes.c_void_p), ("m_scale", ctypes.c_void_p), ("v_code", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("row_ema", ctypes.c_void_p), ("col_ema", ctypes.c_void_p),
                ("numel", ctypes.c_int64), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("flags", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class CHParams(ctypes.Structure):
    _fields_ = [("algo", ctypes.c_int32), ("split_mode", ctypes.c_int32), ("lr", ctypes.c_double),
                ("beta1", ctypes.c_double), ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("momentum_decay", ctypes.c_double), ("seed", ctypes.c_uint64)]


class CFHParams(ctypes.Structure):
    _fields_ = [("split_mode", ctypes.c_int32), ("reserved", ctypes.c_int32), ("lr", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps1", ctypes.c_double), ("clip_threshold", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("decay_rate", ctypes.c_double), ("beta1", ctypes.c_double),
                ("seed", ctypes.c_uint64)]


class COffloadGroup(ctypes.Structure):
    _fields_ = [("tensors", ctypes.POINTER(CTensor)), ("n_tensors", ctypes.c_int32)]


class COffloadOptions(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("n_cus", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("reserved1", ctypes.c_int32)]


OFFLOAD_DIRECT, OFFLOAD_STAGED = 0, 1
OFFLOAD_DEFAULT_CUS = 8


_vp, _i64, _i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
_sig = {
    "ps_opt_step_multi": [ctypes.POINTER(CTensor), _i32, ctypes.POINTER(CHParams), _i64, _vp],
    "ps_step_scalars": [ctypes.POINTER(CHParams), _i64, ctypes.POINTER(ctypes.c_float)],
    "ps_split": [_vp, _vp, _vp, _i64, _i32, _vp],
    "ps_join": [_vp, _vp, _vp, _i64, _i32, _vp],
    "ps_encode_moments": [_vp, _vp, _vp, _i64, _i32, _vp],
    "ps_decode_moments": [_vp, _vp, _vp, _i64, _i32, _vp],
    "ps_factored_workspace_size": [ctypes.POINTER(CTensor), _i32, ctypes.POINTER(ctypes.c_size_t)],
    "ps_factored_step": [ctypes.POINTER(CTensor), _i32, ctypes.POINTER(CFHParams), _i64, _vp, ctypes.c_size_t, _vp],
    "ps_factored_step_noalloc": [ctypes.POINTER(CTensor), _i32, ctypes.POINTER(CFHParams), _i64, _vp],
    "ps_offload_plan_create": [ctypes.POINTER(COffloadGroup), _i32, ctypes.POINTER(ctypes.c_void_p)],
    "ps_offload_plan_create_ex": [ctypes.POINTER(COffloadGroup), _i32, ctypes.POINTER(COffloadOptions),
                                  ctypes.POINTER(ctypes.c_void_p)],
    "ps_offload_run": [_vp, ctypes.POINTER(CHParams), _i64, _vp],
    "ps_offload_bytes": [_vp, ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint64)],
    "ps_offload_plan_destroy": [_vp],
}
for _name, _args in _sig.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_int32
_lib.ps_status_string.argtypes = [ctypes.c_int32]
_lib.ps_status_string.restype = ctypes.c_char_p
_lib.ps_last_error.argtypes = []
_lib.ps_last_error.restype = ctypes.c_char_p
_lib.ps_version.argtypes = []
_lib.ps_version.restype = ctypes.c_char_p


def lib():
    return _lib


def version():
    return _lib.ps_version().decode()


def last_error():
    return _lib.ps_last_error().decode()


def _check(status):
    if status != 0:
        raise PSError(status, last_error())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


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
    seed: int = 0          # SPLIT_STOCHASTIC: the random stream's seed (see ps_hparams in include/ps.h)

    def c(self):
        return CHParams(self.algo, self.split_mode, self.lr, self.beta1, self.beta2, self.eps,
                        self.weight_decay, self.momentum_decay, self.seed)


@dataclass
class FactoredHParams:
    split_mode: int = SPLIT_TRUNC
    lr: float = 3.5e-6
    beta2: float = 0.999
    eps1: float = 1e-30
    clip_threshold: float = 1.0
    weight_decay: float = 0.0
    decay_rate: float = 0.0   # < 0: beta2 of update t is 1 - t^decay_rate (Adafactor's schedule)
    beta1: float = 0.0        # > 0: first moment of the clipped update in m_code / m_scale
    seed: int = 0             # SPLIT_STOCHASTIC: the random stream's seed

    def c(self):
        return CFHParams(self.split_mode, 0, self.lr, self.beta2, self.eps1, self.clip_threshold,
                         self.weight_decay, self.decay_rate, self.beta1, self.seed)


@dataclass
class TensorState:
    """Device state of one parameter tensor (see ps_tensor in include/ps.h)."""
    w_hi: object
    w_lo: object
    m_code: object = None
    m_scale: object = None
    v_code: object = None
    v_scale: object = None
    row_ema: object = None
    col_ema: object = None
    rows: int = 0
    cols: int = 0
    flags: int = 0

    @property
    def numel(self):
        return self.w_hi.numel()


class StateSlab:
    """Optimizer state of a whole tensor list in one contiguous device
    allocation per stream (bf16 weights, residuals, gradients, m codes, v codes,
    m scales, v scales); each tensor gets 256-byte-aligned views. Streaming
    the step over a few large allocations needs far fewer address translations
    than one allocation per tensor and stream.

    numels: element count of each tensor. Moments start as the zero codes with
    zero scales; weights, residuals and gradients are left uninitialised for
    the caller to fill (or copy into)."""

    ALIGN = 128    # elements of a 16-bit stream = 256 bytes

    def __init__(self, numels, device="cuda", with_grads=True, shapes2d=None, host_state=False, moments="codec"):
        """host_state=True puts residuals, codes and scales in pinned host
        memory (the layout ps_offload_* expects); weights and gradients stay
        on `device`. moments="f24" stores both moments as f24 arrays (3 bytes
        per value, zero-initialised, no scales; TENSOR_F24_MOMENTS)."""
        import torch
        self.numels = list(numels)
        offs, boffs, n_tot, nb_tot = [], [], 0, 0
        for n in self.numels:
            offs.append(n_tot)
            boffs.append(nb_tot)
            n_tot += (n + self.ALIGN - 1) // self.ALIGN * self.ALIGN
            nb_tot += ((n + BLOCK - 1) // BLOCK + 63) // 64 * 64
        if moments not in ("codec", "f24"):
            raise ValueError("moments must be 'codec' or 'f24'")
        f24 = moments == "f24"
        names = ["hi", "lo"] + ([] if f24 else ["mc", "vc"]) + (["g"] if with_grads else [])

        def where(k):
            return dict(device="cpu", pin_memory=True) if host_state and k in ("lo", "mc", "vc", "ms", "vs") \
                else dict(device=device)
        self.slab = {k: torch.empty(max(1, n_tot), dtype=torch.int16, **where(k)) for k in names}
        if f24:
            for k in ("mc", "vc"):
                self.slab[k] = torch.zeros(max(1, 3 * n_tot), dtype=torch.uint8, **where(k))
            self.scales = {}
        else:
            self.slab["mc"].fill_(-32768)          # 0x8000: the zero code of the signed kind
            self.slab["vc"].zero_()
            self.scales = {k: torch.zeros(max(1, nb_tot), dtype=torch.float32, **where(k)) for k in ("ms", "vs")}
        self.states, self.grads = [], []
        for i, n in enumerate(self.numels):
            o, bo, nb = offs[i], boffs[i], (n + BLOCK - 1) // BLOCK
            rows, cols = shapes2d[i] if shapes2d else (0, 0)
            if f24:
                self.states.append(TensorState(self.slab["hi"][o:o + n], self.slab["lo"][o:o + n],
                                               self.slab["mc"][3 * o:3 * (o + n)], None,
                                               self.slab["vc"][3 * o:3 * (o + n)], None,
                                               rows=rows, cols=cols, flags=TENSOR_F24_MOMENTS))
            else:
                self.states.append(TensorState(self.slab["hi"][o:o + n], self.slab["lo"][o:o + n],
                                               self.slab["mc"][o:o + n], self.scales["ms"][bo:bo + nb],
                                               self.slab["vc"][o:o + n], self.scales["vs"][bo:bo + nb],
                                               rows=rows, cols=cols))
            self.grads.append(self.slab["g"][o:o + n] if with_grads else None)

    def records(self, grads=None):
        return make_records(self.states, self.grads if grads is None else grads)


def make_records(states: Sequence[TensorState], grads: Sequence[Optional[object]]):
    """ctypes array of ps_tensor records (reusable while the tensors live)."""
    if len(states) != len(grads):
        raise ValueError("states and grads differ in length")
    arr = (CTensor * max(1, len(states)))()
    for i, (s, g) in enumerate(zip(states, grads)):
        arr[i] = CTensor(_ptr(s.w_hi), _ptr(s.w_lo), _ptr(g), _ptr(s.m_code), _ptr(s.m_scale), _ptr(s.v_code),
                         _ptr(s.v_scale), _ptr(s.row_ema), _ptr(s.col_ema), s.numel, s.rows, s.cols,
                         s.flags, 0)
    return arr, len(states)


def step_scalars(hp: HParams, step: int):
    out = (ctypes.c_float * 10)()
    h = hp.c()
    _check(_lib.ps_step_scalars(ctypes.byref(h), step, out))
    names = ("B1", "C1", "B2", "C2", "EPS", "A", "RS2", "AG", "AM", "CWD")
    return dict(zip(names, list(out)))


def opt_step_multi(states, grads=None, hp: HParams = None, step: int = 1, stream=None, records=None):
    """One fused (N)AdamW step over all tensors in one launch. Pass either
    (states, grads) or `records` from make_records()."""
    arr, n = records if records is not None else make_records(states, grads)
    h = (hp or HParams()).c()
    _check(_lib.ps_opt_step_multi(arr, n, ctypes.byref(h), step, _stream(stream)))


def split(w32, hi, lo, mode=SPLIT_TRUNC, stream=None):
    _check(_lib.ps_split(_ptr(w32), _ptr(hi), _ptr(lo), w32.numel(), mode, _stream(stream)))


def join(hi, lo, w32, mode=SPLIT_TRUNC, stream=None):
    _check(_lib.ps_join(_ptr(hi), _ptr(lo), _ptr(w32), hi.numel(), mode, _stream(stream)))


def encode_moments(x, code, scale, kind, stream=None):
    _check(_lib.ps_encode_moments(_ptr(x), _ptr(code), _ptr(scale), x.numel(), kind, _stream(stream)))


def decode_moments(code, scale, x, kind, stream=None):
    _check(_lib.ps_decode_moments(_ptr(code), _ptr(scale), _ptr(x), code.numel(), kind, _stream(stream)))


def factored_workspace_size(states, grads=None, records=None):
    arr, n = records if records is not None else make_records(states, grads)
    out = ctypes.c_size_t(0)
    _check(_lib.ps_factored_workspace_size(arr, n, ctypes.byref(out)))
    return out.value


def factored_step(states, grads=None, hp: FactoredHParams = None, step: int = 1, workspace=None, stream=None,
                  records=None):
    arr, n = records if records is not None else make_records(states, grads)
    h = (hp or FactoredHParams()).c()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.ps_factored_step(arr, n, ctypes.byref(h), step, _ptr(workspace), ws_bytes, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20   # PS_NOALLOC_SCRATCH_BYTES


def factored_step_noalloc(states, grads=None, hp: FactoredHParams = None, step: int = 1, stream=None, records=None):
    """ps_factored_step_noalloc: the factored step with the library's built-in
    scratch as its workspace (no device allocation)."""
    arr, n = records if records is not None else make_records(states, grads)
    h = (hp or FactoredHParams()).c()
    _check(_lib.ps_factored_step_noalloc(arr, n, ctypes.byref(h), step, _stream(stream)))


class OffloadPlan:
    """Host-offload plan (ps_offload_*): groups of tensors whose residual and
    moment state live in pinned host memory. mode OFFLOAD_DIRECT (the step
    kernel works on the host arrays in place, on n_cus compute units) or
    OFFLOAD_STAGED (copies through two device staging slots)."""

    def __init__(self, groups, mode=OFFLOAD_DIRECT, n_cus=OFFLOAD_DEFAULT_CUS):
        # groups: list of (states, grads) with host-pinned lo/codes/scales
        self._recs = [make_records(s, g) for s, g in groups]
        garr = (COffloadGroup * max(1, len(groups)))()
        for i, (arr, n) in enumerate(self._recs):
            garr[i] = COffloadGroup(ctypes.cast(arr, ctypes.POINTER(CTensor)), n)
        self._garr = garr
        h = ctypes.c_void_p()
        opt = COffloadOptions(mode, n_cus, 0, 0)
        _check(_lib.ps_offload_plan_create_ex(garr, len(groups), ctypes.byref(opt), ctypes.byref(h)))
        self._h = h

    def run(self, hp: HParams, step: int, stream=None):
        h = hp.c()
        _check(_lib.ps_offload_run(self._h, ctypes.byref(h), step, _stream(stream)))

    def bytes(self):
        a, b = ctypes.c_uint64(0), ctypes.c_uint64(0)
        _check(_lib.ps_offload_bytes(self._h, ctypes.byref(a), ctypes.byref(b)))
        return a.value, b.value

    def close(self):
        if self._h:
            _check(_lib.ps_offload_plan_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
