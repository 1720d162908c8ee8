"""Host-side checks of libps.so that need no GPU: every symbol of
include/ps.h is exported, the host-computed step scalars equal the oracle's,
and invalid arguments are rejected before any device call."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def ps():
    import precision_state_amd as ps
    return ps


def test_library_exports_every_declared_symbol(ps):
    hdr = open(os.path.join(ROOT, "include", "ps.h")).read()
    declared = set(re.findall(r"\b(ps_[a-z0-9_]+)\s*\(", hdr))
    assert len(declared) >= 15
    missing = [s for s in sorted(declared) if not hasattr(ps.lib(), s)]
    assert not missing, missing
    assert set(ps.EXPORTED) == declared


@pytest.mark.parametrize("algo", [0, 1])
@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_step_scalars_equal_oracle(ps, algo, wd):
    for lr, b1, b2 in ((3.5e-6, 0.9, 0.999), (1e-3, 0.95, 0.99), (0.1, 0.0, 0.5)):
        for step in (1, 2, 3, 10, 57, 1000, 123456):
            hp = ps.HParams(algo=algo, lr=lr, beta1=b1, beta2=b2, weight_decay=wd)
            got = ps.step_scalars(hp, step)
            ref = oracle.coeffs(oracle.HParams(algo=algo, lr=lr, beta1=b1, beta2=b2, weight_decay=wd), step)
            for k, v in ref.items():
                assert np.float32(got[k]).view(np.uint32) == v.view(np.uint32), (k, step, got[k], v)


def _rec(ps, n=1024, **kw):
    base = dict(w_hi=16, w_lo=32, grad=48, m_code=64, m_scale=80, v_code=96, v_scale=112, row_ema=0, col_ema=0,
                numel=n, rows=0, cols=0)
    base.update(kw)
    return ps.CTensor(**base)


def _call(ps, recs, hp=None, step=1):
    arr = (ps.CTensor * max(1, len(recs)))(*recs)
    h = (hp or ps.HParams()).c()
    return ps.lib().ps_opt_step_multi(arr, len(recs), ctypes.byref(h), step, None)


def test_invalid_arguments_rejected_on_host(ps):
    L = ps.lib()
    assert _call(ps, [_rec(ps)], step=0) == 1
    assert _call(ps, [_rec(ps)], hp=ps.HParams(algo=7)) == 1
    assert _call(ps, [_rec(ps)], hp=ps.HParams(split_mode=3)) == 1
    assert _call(ps, [_rec(ps)], hp=ps.HParams(beta1=1.0)) == 1
    assert _call(ps, [_rec(ps)], hp=ps.HParams(beta2=-0.1)) == 1
    assert _call(ps, [_rec(ps)], hp=ps.HParams(eps=0.0)) == 1
    assert _call(ps, [_rec(ps)], hp=ps.HParams(eps=1e-50)) == 1   # 0 once rounded to fp32
    assert "fp32" in ps.last_error()
    assert _call(ps, [_rec(ps)], hp=ps.HParams(lr=float("nan"))) == 1
    assert _call(ps, [_rec(ps)], hp=ps.HParams(weight_decay=-1.0)) == 1
    assert _call(ps, [_rec(ps, numel=-1)]) == 3
    assert _call(ps, [_rec(ps, numel=(1 << 40) + 1)]) == 3
    assert _call(ps, [_rec(ps, w_lo=0)]) == 1
    assert "w_lo" in ps.last_error()
    assert _call(ps, [_rec(ps, m_code=66)]) == 2
    assert _call(ps, [_rec(ps, v_scale=114)]) == 2
    assert _call(ps, [_rec(ps, flags=8)]) == 1
    assert _call(ps, [_rec(ps)], hp=ps.HParams(split_mode=3)) == 1
    # stochastic rounding keeps no residual: a NULL w_lo passes validation (the
    # next check, m_scale's alignment, is the one that fails here)
    assert _call(ps, [_rec(ps, w_lo=0, m_scale=81)], hp=ps.HParams(split_mode=ps.SPLIT_STOCHASTIC)) == 2
    assert "m_scale" in ps.last_error()
    assert _call(ps, [_rec(ps, w_lo=0, m_scale=81)], hp=ps.HParams(split_mode=ps.SPLIT_TRUNC)) == 1
    assert "w_lo" in ps.last_error()
    assert L.ps_split(16, 32, 48, 10, ps.SPLIT_STOCHASTIC, None) == 4
    assert L.ps_join(16, 32, 48, 10, ps.SPLIT_STOCHASTIC, None) == 4
    assert _call(ps, [_rec(ps, flags=ps.TENSOR_FP32_MOMENTS | ps.TENSOR_F24_MOMENTS)]) == 1
    assert "exclusive" in ps.last_error()
    assert _call(ps, [_rec(ps, flags=ps.TENSOR_F24_MOMENTS, m_code=8)]) == 2
    h = ps.HParams().c()
    assert L.ps_opt_step_multi(None, 3, ctypes.byref(h), 1, None) == 1
    assert L.ps_opt_step_multi(None, 0, None, 1, None) == 1
    assert L.ps_split(None, None, None, -1, 0, None) == 3
    assert L.ps_split(16, 32, 48, 10, 5, None) == 1
    assert L.ps_join(16, 32, 40, 10, 0, None) == 2
    assert L.ps_encode_moments(16, 32, 0, 10, 0, None) == 1
    assert L.ps_decode_moments(16, 32, 48, 10, 9, None) == 1


def test_empty_and_gradless_lists_are_noops(ps):
    """Nothing to do means no device call at all, so this runs without a GPU."""
    assert _call(ps, []) == 0
    assert _call(ps, [_rec(ps, numel=0, w_hi=0, w_lo=0, grad=0)]) == 0
    assert _call(ps, [_rec(ps, grad=0, w_hi=0)]) == 0
    L = ps.lib()
    assert L.ps_split(None, None, None, 0, 0, None) == 0
    assert L.ps_encode_moments(None, None, None, 0, 1, None) == 0


def test_status_strings(ps):
    L = ps.lib()
    for s in range(8):
        assert L.ps_status_string(s)
    assert b"gfx950" in L.ps_version()


def _frec(ps, n=1024, rows=32, cols=32, **kw):
    base = dict(w_hi=16, w_lo=32, grad=48, m_code=0, m_scale=0, v_code=96, v_scale=112, row_ema=128, col_ema=144,
                numel=n, rows=rows, cols=cols)
    base.update(kw)
    return ps.CTensor(**base)


def test_factored_workspace_size_and_validation(ps):
    L = ps.lib()
    size = ctypes.c_size_t(0)
    arr = (ps.CTensor * 2)(_frec(ps), _frec(ps, n=300, rows=0, cols=0))
    assert L.ps_factored_workspace_size(arr, 2, ctypes.byref(size)) == 0
    # 2-D 32x32: rowpart 1x32, colpart 1x32 doubles, rpart 1, rho 32, kap 32 floats, rinv 32, cinv 32
    # doubles, upart 1, f; 1-D 300: v 300 floats, upart 1, f -- each region rounded up to 256 bytes
    assert size.value == 256 * (1 + 1 + 1 + 1 + 1 + 1 + 1 + 1 + 1) + 1280 + 256 + 256
    # 16384x512 takes the row-strip pass (256 groups of 64 rows, one segment each): rowpart 16384,
    # colpart and qpart 256x512 doubles, rpart 64, rho 16384, kap 512 floats, upart 2 column chunks, f
    strip = (ps.CTensor * 1)(_frec(ps, n=16384 * 512, rows=16384, cols=512))
    assert L.ps_factored_workspace_size(strip, 1, ctypes.byref(size)) == 0
    assert size.value == 131072 + 1048576 + 1048576 + 512 + 65536 + 2048 + 256 + 256
    # one row fewer takes the tiles: rowpart 2x16383, colpart 64x512, rpart 64 doubles, rho, kap,
    # rinv 16383, cinv 512 doubles, upart 2048 row tiles (8 rows each), f
    tiles = (ps.CTensor * 1)(_frec(ps, n=16383 * 512, rows=16383, cols=512))
    assert L.ps_factored_workspace_size(tiles, 1, ctypes.byref(size)) == 0
    up = lambda b: (b + 255) // 256 * 256
    assert size.value == (up(8 * 2 * 16383) + up(8 * 64 * 512) + up(8 * 64) + up(4 * 16383) + up(4 * 512)
                          + up(8 * 16383) + up(8 * 512) + up(8 * 2048) + 256)
    bad = (ps.CTensor * 1)(_frec(ps, rows=33))
    assert L.ps_factored_workspace_size(bad, 1, ctypes.byref(size)) == 3
    bad = (ps.CTensor * 1)(_frec(ps, row_ema=0))
    assert L.ps_factored_workspace_size(bad, 1, ctypes.byref(size)) == 1
    bad = (ps.CTensor * 1)(_frec(ps, n=300, rows=0, cols=0, v_code=98))
    assert L.ps_factored_workspace_size(bad, 1, ctypes.byref(size)) == 2
    hp = ps.FactoredHParams().c()
    assert L.ps_factored_step(arr, 2, ctypes.byref(hp), 1, None, 0, None) == 7
    assert L.ps_factored_step(arr, 2, ctypes.byref(hp), 1, 4096 + 16, 1 << 20, None) == 2
    assert L.ps_factored_step(arr, 2, ctypes.byref(hp), 1, 4096, 100, None) == 7
    assert L.ps_factored_step(arr, 2, ctypes.byref(hp), 0, 4096, 1 << 20, None) == 1
    for k, v in (("eps1", 0.0), ("clip_threshold", -1.0), ("beta2", 1.0), ("lr", float("inf")),
                 ("decay_rate", 0.5), ("beta1", 1.0), ("beta1", -0.1)):
        h = ps.FactoredHParams(**{k: v}).c()
        assert L.ps_factored_step(arr, 2, ctypes.byref(h), 1, 4096, 1 << 20, None) == 1, k
    # a first moment needs m_code / m_scale and, for 2-D tensors, fewer than 2^31 elements
    h = ps.FactoredHParams(beta1=0.9).c()
    assert L.ps_factored_step((ps.CTensor * 1)(_frec(ps, m_code=0)), 1, ctypes.byref(h), 1, 4096, 1 << 20,
                              None) == 1
    assert L.ps_factored_step((ps.CTensor * 1)(_frec(ps, m_code=160, m_scale=82)), 1, ctypes.byref(h), 1, 4096,
                              1 << 20, None) == 2
    big = (ps.CTensor * 1)(_frec(ps, n=1 << 31, rows=1 << 16, cols=1 << 15, m_code=160, m_scale=176))
    assert L.ps_factored_step(big, 1, ctypes.byref(h), 1, 4096, 1 << 40, None) == 4
    assert "numel < 2^31" in ps.last_error()
    # stochastic rounding keeps no residual: w_lo may be NULL
    hs = ps.FactoredHParams(split_mode=ps.SPLIT_STOCHASTIC).c()
    assert L.ps_factored_step((ps.CTensor * 1)(_frec(ps, w_lo=0, row_ema=0)), 1, ctypes.byref(hs), 1, 4096,
                              1 << 20, None) == 1
    assert "row_ema" in ps.last_error()
    assert L.ps_factored_step((ps.CTensor * 1)(_frec(ps, w_lo=0, row_ema=0)), 1, ctypes.byref(h0 := ps.FactoredHParams().c()),
                              1, 4096, 1 << 20, None) == 1
    assert "w_lo" in ps.last_error()
    # without a first moment m_code is not read (workspace check fails next)
    assert L.ps_factored_step((ps.CTensor * 1)(_frec(ps, m_code=0)), 1, ctypes.byref(h0), 1, None, 0, None) == 7
    empty = (ps.CTensor * 1)(_frec(ps, grad=0))
    assert L.ps_factored_step(empty, 1, ctypes.byref(hp), 1, None, 0, None) == 0


def test_build_scripts_load_without_the_built_library():
    """build() must work in a tree where libps.so does not exist yet: the
    package refuses to import until it is built, so its build script is loaded
    by path. Checked in a fresh interpreter that the package stays unimported."""
    import subprocess
    import sys
    code = ("import sys, __graft_entry__ as g\n"
            "for p in ('precision_state_amd', 'synth', 'oracle'):\n"
            "    m = g._load_build_module(p)\n"
            "    assert callable(m.build) and m.LIB.endswith('.so'), p\n"
            "assert 'precision_state_amd' not in sys.modules\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_noalloc_factored_step_rejects_on_host(ps):
    """The allocation-free factored step validates and sizes the call before
    any HIP call: a list whose workspace exceeds the built-in scratch, bad
    hyperparameters and bad shapes are rejected here, with no GPU."""
    L = ps.lib()
    big = (ps.CTensor * 1)(ps.CTensor(256, 256, 256, 256, 256, 256, 256, 256, 256, 1048576 * 4096, 1048576, 4096, 0, 0))
    h = ps.FactoredHParams().c()
    assert L.ps_factored_step_noalloc(big, 1, ctypes.byref(h), 1, None) == 7      # PS_ERR_WORKSPACE
    assert "scratch" in ps.last_error()
    tiny = ps.FactoredHParams(eps1=1e-50).c()                                     # 0 once rounded to fp32
    assert L.ps_factored_step_noalloc(big, 1, ctypes.byref(tiny), 1, None) == 1
    bad = ps.FactoredHParams(clip_threshold=0.0).c()
    assert L.ps_factored_step_noalloc(big, 1, ctypes.byref(bad), 1, None) == 1    # PS_ERR_INVALID_ARG
    assert L.ps_factored_step_noalloc(big, 1, ctypes.byref(h), 0, None) == 1
    shape = (ps.CTensor * 1)(ps.CTensor(256, 256, 256, 256, 256, 256, 256, 256, 256, 100, 7, 13, 0, 0))
    assert L.ps_factored_step_noalloc(shape, 1, ctypes.byref(h), 1, None) == 3    # PS_ERR_SHAPE
    assert L.ps_factored_step_noalloc(shape, 0, ctypes.byref(h), 1, None) == 0    # empty list: no-op
