"""Pins of the oracle's companded uint16 moment codec (sd-scripts PR #2187,
'(N)AdamW / Adan with fused backwards pass & CPU offloading', second post:
moments scaled, biased and pow()-companded into 0..65535)."""
import numpy as np
import pytest
import torch

import oracle
from figures import page_figure
from oracle import SIGNED, UNSIGNED

Q = {SIGNED: 32767, UNSIGNED: 65535}


def _thresholds(kind):
    k = np.arange(1, Q[kind] + 1, dtype=np.float32)
    return oracle.dec_mag(k - np.float32(0.5), kind)


@pytest.mark.parametrize("kind", [SIGNED, UNSIGNED])
def test_thresholds_are_quarter_power_midpoints(kind):
    """The boundary between codes k-1 and k is ((k - 1/2)/Q)^4 up to fp32
    rounding, strictly increasing in k. Relative error bound with u = 2^-24:
    1/Q rounded (u, raised to the 4th power: 4u), h*K (4u), a*a (2u), t*t (u)."""
    T = _thresholds(kind).astype(np.float64)
    k = np.arange(1, Q[kind] + 1, dtype=np.float64)
    exact = ((k - 0.5) / Q[kind]) ** 4
    assert np.max(np.abs(T / exact - 1.0)) <= 11 * 2.0 ** -24
    assert np.all(np.diff(T) > 0)


@pytest.mark.parametrize("kind", [SIGNED, UNSIGNED])
def test_code_mag_steps_exactly_at_thresholds(kind):
    T = _thresholds(kind)
    k = np.arange(1, Q[kind] + 1)
    assert np.array_equal(oracle.code_mag(T, kind), k)
    below = np.nextafter(T, np.float32(0))
    assert np.array_equal(oracle.code_mag(below, kind), k - 1)
    assert oracle.code_mag(np.float32(0.0), kind) == 0
    assert oracle.code_mag(np.float32(1.0), kind) == Q[kind]
    assert oracle.code_mag(np.float32(1.0 + 2 ** -23), kind) == Q[kind]


@pytest.mark.parametrize("kind", [SIGNED, UNSIGNED])
def test_code_mag_vs_double_quarter_power(kind):
    """Codes agree with round(Q * x^(1/4)) evaluated in double: within 1
    everywhere, and equal unless Q * x^(1/4) lies within the thresholds'
    rounding band of a .5 boundary (relative threshold error <= 11u, u = 2^-24,
    which is Q * 11u / 4 < Q * 3u in code units)."""
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.random(500_000), 10.0 ** rng.uniform(-30, 0, 500_000)]).astype(np.float32)
    c = oracle.code_mag(x, kind).astype(np.int64)
    y = Q[kind] * x.astype(np.float64) ** 0.25
    ref = np.floor(y + 0.5).astype(np.int64)
    assert np.max(np.abs(c - ref)) <= 1
    far = np.abs(y - np.floor(y) - 0.5) > Q[kind] * 3 * 2.0 ** -24
    assert np.array_equal(c[far], ref[far])
    order = np.argsort(x, kind="stable")
    assert np.all(np.diff(c[order]) >= 0)


@pytest.mark.parametrize("kind", [SIGNED, UNSIGNED])
@pytest.mark.parametrize("e", [-60, -20, -3, 0, 7])
def test_decode_then_encode_is_identity_at_power_of_two_scale(kind, e):
    """Every code survives decode -> encode when the block scale is a power of
    two (so value * (1/scale) is exact) and decoded values stay normal."""
    s = np.float32(2.0 ** e)
    if kind == SIGNED:
        mags = np.arange(0, 32768, dtype=np.uint32)
        codes = np.concatenate([32768 + mags, 32768 - mags[1:]]).astype(np.uint16)
        zero = 32768
    else:
        codes = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
        zero = 0
    # 255 codes per block behind a leading top code, so every block's scale is s
    pad = (-codes.size) % 255
    body = np.concatenate([codes, np.full(pad, zero, np.uint16)]).reshape(-1, 255)
    flat = np.concatenate([np.full((body.shape[0], 1), 65535, np.uint16), body], axis=1).reshape(-1)
    flat = np.ascontiguousarray(flat)
    scale = np.full(oracle.nblocks(flat.size), s, np.float32)
    x = oracle.decode(flat, scale, kind)
    c2, s2 = oracle.encode(x, kind)
    assert np.all(s2 == s)
    assert np.array_equal(c2, flat)


@pytest.mark.parametrize("kind", [SIGNED, UNSIGNED])
def test_zero_and_subnormal_blocks_flush(kind):
    zero_code = 32768 if kind == SIGNED else 0
    x = np.zeros(300, np.float32)
    c, s = oracle.encode(x, kind)
    assert np.all(c == zero_code) and np.all(s == 0)
    x = np.full(256, np.float32(1e-39), np.float32)   # subnormal max
    x[5] = np.float32(2.0 ** -127)
    c, s = oracle.encode(x, kind)
    assert np.all(c == zero_code) and s[0] == 0
    back = oracle.decode(c, s, kind)
    assert np.all(back == 0)


def test_block_max_gets_top_code_and_decodes_exactly():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(1000) * 1e-3).astype(np.float32)
    for kind, vals in ((SIGNED, x), (UNSIGNED, np.abs(x) ** 2)):
        vals = np.ascontiguousarray(vals, np.float32)
        c, s = oracle.encode(vals, kind)
        back = oracle.decode(c, s, kind)
        for b in range(oracle.nblocks(vals.size)):
            blk = vals[b * 256:(b + 1) * 256]
            i = int(np.argmax(np.abs(blk)))
            assert s[b] == np.abs(blk).max()
            assert back[b * 256 + i] == blk[i]
            assert c[b * 256 + i] in ((65535, 1) if kind == SIGNED else (65535,))


def test_signed_codes_are_symmetric():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(4096) * 1e-4).astype(np.float32)
    c, s = oracle.encode(x, SIGNED)
    cn, sn = oracle.encode(np.ascontiguousarray(-x), SIGNED)
    assert np.array_equal(s, sn)
    assert np.array_equal(cn.astype(np.int64), 65536 - c.astype(np.int64))


def test_l1_error_at_least_90pct_below_bf16_storage():
    """PR #2187 reports the companded u16 format cutting the L1 error of
    bf16 moment storage by about 90%. Moments from 10 fp32 NAdam steps."""
    rng = np.random.default_rng(6)
    n = 1 << 16
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    hp = oracle.HParams()
    for t in range(1, 11):
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        oracle.core_step(w, m, v, g, hp, t)
    for kind, val in ((SIGNED, m), (UNSIGNED, v)):
        c, s = oracle.encode(val, kind)
        e_u16 = np.abs(oracle.decode(c, s, kind).astype(np.float64) - val).sum()
        bf = torch.from_numpy(val).to(torch.bfloat16).float().numpy()
        e_bf16 = np.abs(bf.astype(np.float64) - val).sum()
        assert e_u16 <= page_figure("codec_l1_error_vs_bf16")["max_error_ratio"] * e_bf16, (kind, e_u16 / e_bf16)


# ---------------------------------------------------------------------------
# f24 moment storage (PR #2187, third post: the upper three bytes of fp32)
# ---------------------------------------------------------------------------

def test_f24_is_fp32_rounded_to_16_significant_bits():
    """decode(encode(x)) keeps sign, exponent and the top 15 mantissa bits:
    relative error <= 2^-16, exact for values whose low byte is already 0,
    and never more than half a 24-bit step away."""
    rng = np.random.default_rng(31)
    x = (rng.standard_normal(1 << 20) * 10.0 ** rng.uniform(-30, 5, 1 << 20)).astype(np.float32)
    y = oracle.f24_decode(oracle.f24_encode(x))
    rel = np.abs(y.astype(np.float64) / x.astype(np.float64) - 1.0)
    assert rel.max() <= 2.0 ** -16
    assert np.all(y.view(np.uint32) & 0xFF == 0)
    step = np.abs(x).astype(np.float64) * 0 + 2.0 ** (np.floor(np.log2(np.abs(x).astype(np.float64))) - 15)
    assert np.all(np.abs(y.astype(np.float64) - x.astype(np.float64)) <= 0.5 * step * (1 + 1e-12))
    z = (x.view(np.uint32) & 0xFFFFFF00).view(np.float32)
    assert np.array_equal(oracle.f24_decode(oracle.f24_encode(z)).view(np.uint32), z.view(np.uint32))


def test_f24_is_about_256x_more_accurate_than_bf16():
    """PR #2187's third post: f24 moments are ~256 times more accurate than
    bf16 (8 more mantissa bits). Mean relative error ratio on moments from 10
    fp32 NAdam steps."""
    rng = np.random.default_rng(32)
    n = 1 << 16
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t in range(1, 11):
        oracle.core_step(w, m, v, (rng.standard_normal(n) * 1e-3).astype(np.float32), oracle.HParams(), t)
    for val in (m, v):
        f24 = oracle.f24_decode(oracle.f24_encode(val)).astype(np.float64)
        bf = torch.from_numpy(val).to(torch.bfloat16).float().numpy().astype(np.float64)
        nz = val != 0
        e24 = np.mean(np.abs(f24[nz] / val[nz] - 1))
        e16 = np.mean(np.abs(bf[nz] / val[nz] - 1))
        lo, hi = page_figure("f24_accuracy_vs_bf16")["accepted_range"]
        assert lo < e16 / e24 < hi, e16 / e24
