"""Pins of the oracle's residual split/join (the "Kahan summation" master
weight of sd-scripts PR #2159, 'Kahan summation for Adafactor-optimized Flux
FFT')."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from figures import page_figure
from oracle import SPLIT_NEAREST_AWAY, SPLIT_TRUNC


def _roundtrip_range(mode, starts, chunk):
    base = np.arange(chunk, dtype=np.uint32)
    bits = np.empty(chunk, np.uint32)
    hi, lo = np.empty(chunk, np.uint16), np.empty(chunk, np.uint16)
    back = np.empty(chunk, np.float32)
    for start in starts:
        np.add(base, np.uint32(start), out=bits)
        oracle.split(bits.view(np.float32), mode, out=(hi, lo))
        oracle.join(hi, lo, mode, out=back)
        if not np.array_equal(back.view(np.uint32), bits):
            bad = np.flatnonzero(back.view(np.uint32) != bits)
            return int(bits[bad[0]])
    return None


@pytest.mark.parametrize("mode", [SPLIT_TRUNC, SPLIT_NEAREST_AWAY])
def test_roundtrip_exhaustive_all_fp32_patterns(mode):
    """The residual restores the identical fp32 bits, for every 32-bit pattern
    (ctypes releases the GIL, so worker threads split the range)."""
    chunk, workers = 1 << 24, 8
    starts = list(range(0, 1 << 32, chunk))
    with ThreadPoolExecutor(workers) as ex:
        res = list(ex.map(lambda k: _roundtrip_range(mode, starts[k::workers], chunk), range(workers)))
    bad = [r for r in res if r is not None]
    assert not bad, f"mode {mode}: mismatch at {bad[0]:#010x}"


def _finite_samples(n, seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    w = bits.view(np.float32)
    keep = np.isfinite(w) & (np.abs(w) < 3.0e38)
    return np.ascontiguousarray(w[keep])


def test_trunc_is_truncation_toward_zero():
    w = _finite_samples(1 << 20, 1)
    hi, _ = oracle.split(w, SPLIT_TRUNC)
    b = oracle.bf16_to_f32(hi).astype(np.float64)
    wd = w.astype(np.float64)
    assert np.all(np.abs(b) <= np.abs(wd))
    assert np.all(np.sign(b) * np.sign(wd) >= 0)
    # the dropped part is less than one bf16 ulp of the magnitude
    nxt = oracle.bf16_to_f32((hi.astype(np.uint32) + 1).astype(np.uint16)).astype(np.float64)
    ok = np.isfinite(nxt)
    assert np.all(np.abs(wd[ok]) < np.abs(nxt[ok]))


def test_nearest_away_matches_library_rounding_off_ties():
    """Off exact ties, NEAREST_AWAY's bf16 equals torch's round-to-nearest cast;
    on ties (residual low half exactly 0x8000) it rounds away from zero."""
    w = _finite_samples(1 << 20, 2)
    hi, lo = oracle.split(w, SPLIT_NEAREST_AWAY)
    ref = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bits = w.view(np.uint32)
    tie = (bits & 0xFFFF) == 0x8000
    assert np.array_equal(hi[~tie], ref[~tie])
    # constructed ties: both neighbours equally near, pick the larger magnitude
    tb = (np.arange(1, 5001, dtype=np.uint32) * 0x10001 + 0x3F000000) & 0xFFFF0000 | 0x8000
    tb = np.concatenate([tb, tb | 0x80000000]).astype(np.uint32)
    th, _ = oracle.split(tb.view(np.float32), SPLIT_NEAREST_AWAY)
    assert np.all(oracle.bf16_to_f32(th).view(np.uint32) & 0x7FFFFFFF ==
                  ((tb & 0x7FFFFFFF) + 0x8000) & 0xFFFF0000)


def _page_period_case():
    fig = page_figure("kahan_subulp_update_period")
    f, k = fig["update_fraction_of_ulp"], fig["period_steps"]
    # at w = 1.0 the fp32 increment is 13107 units of 2^-23 (a fifth of the 65536-unit bf16 step,
    # rounded down), so k steps fall one unit short of a full step and the moves come at k*j + 1
    return f, [k + 1 + i * k for i in range(5)]


@pytest.mark.parametrize("frac,bumps", [(0.25, [4, 8, 12, 16, 20, 24]), _page_period_case()])
def test_residual_accumulates_subulp_updates(frac, bumps):
    """PR #2159's closing explanation: an update worth 20% of a bf16 step moves
    the stored bf16 once every five steps (deterministically), where plain
    bf16 rounding never moves. Here: w = 1.0, bf16 ulp = 2^-7."""
    delta = np.float32(frac * 2.0 ** -7)
    hi, lo = oracle.split(np.array([1.0], np.float32), SPLIT_TRUNC)
    plain = np.array([1.0], np.float32).astype(np.float32)
    moved = []
    for step in range(1, 27):
        w = oracle.join(hi, lo, SPLIT_TRUNC) + delta
        new_hi, lo = oracle.split(np.ascontiguousarray(w, np.float32), SPLIT_TRUNC)
        if new_hi[0] != hi[0]:
            moved.append(step)
        hi = new_hi
        plain = torch.from_numpy(plain + delta).to(torch.bfloat16).float().numpy()
    assert moved == [s for s in bumps if s <= 26]
    assert plain[0] == 1.0
