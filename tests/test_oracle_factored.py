"""Pins of the oracle's factored second-moment step with update clipping
(sd-scripts commit 7983d3d 'Fused backward pass', adafactor_step_param;
konstmish/prodigy PR #25 'no first moment and factored second moment')."""
import numpy as np
import pytest

import oracle
from oracle import UNSIGNED, FHParams


def ulp32(x):
    x = np.abs(np.asarray(x, np.float32))
    return (np.nextafter(x, np.float32(np.inf)) - x).astype(np.float64)


def _bf16(x):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _state2d(R, C, w=None, seed=0):
    n = R * C
    if w is None:
        hi, lo = np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    else:
        hi, lo = oracle.split(np.ascontiguousarray(w, np.float32))
    return oracle.TensorState(hi, lo, row=np.zeros(R, np.float32), col=np.zeros(C, np.float32))


def _state1d(n, w=None):
    hi, lo = (np.zeros(n, np.uint16), np.zeros(n, np.uint16)) if w is None else oracle.split(w)
    _, _, vc, vs = oracle.zero_moments(n)
    return oracle.TensorState(hi, lo, vc=vc, vs=vs)


def test_rank_one_gradient_first_step_is_lr_sign_g():
    """For g_ij = a_i b_j the factored estimate is exact, U = sign(g)/sqrt(1-b2)
    has RMS 31.6 > 1, and clipping leaves a step of exactly lr*sign(g)."""
    rng = np.random.default_rng(1)
    R, C = 48, 64
    a = rng.choice([1.0, 1.5, 2.0, 3.0], R) * rng.choice([-1, 1], R) * 2.0 ** -6
    b = rng.choice([1.0, 1.5, 2.0, 3.0], C) * rng.choice([-1, 1], C) * 2.0 ** -5
    g = np.outer(a, b).astype(np.float32).reshape(-1)
    gb = _bf16(g)
    assert np.array_equal(oracle.bf16_to_f32(gb), g)      # exact in bf16
    hp = FHParams(lr=3.5e-6)
    st = _state2d(R, C)
    oracle.factored_step(st, gb, R, C, hp, 1)
    w = oracle.join(st.hi, st.lo).astype(np.float64)
    assert np.max(np.abs(w + hp.lr * np.sign(g)) / hp.lr) < 1e-6


def test_one_d_first_step_is_lr_sign_g():
    rng = np.random.default_rng(2)
    n = 1000
    g = _bf16(rng.standard_normal(n) * 1e-3)
    hp = FHParams(lr=3.5e-6)
    st = _state1d(n)
    oracle.factored_step(st, g, 0, 0, hp, 1)
    w = oracle.join(st.hi, st.lo).astype(np.float64)
    gf = oracle.bf16_to_f32(g).astype(np.float64)
    assert np.max(np.abs(w + hp.lr * np.sign(gf)) / hp.lr) < 1e-6


@pytest.mark.parametrize("two_d", [True, False])
def test_zero_gradient_no_nan_and_weights_identical(two_d):
    """Zero rows/columns were the NaN case of the Prodigy thread; eps1 on g^2
    before the means keeps every factor finite and U exactly 0."""
    rng = np.random.default_rng(3)
    R, C = 32, 40
    w = (rng.standard_normal(R * C) * 0.02).astype(np.float32)
    st = _state2d(R, C, w) if two_d else _state1d(R * C, w)
    hi0, lo0 = st.hi.copy(), st.lo.copy()
    g = np.zeros(R * C, np.uint16)
    for t in range(1, 11):
        oracle.factored_step(st, g, R if two_d else 0, C if two_d else 0, FHParams(), t)
    assert np.array_equal(st.hi, hi0) and np.array_equal(st.lo, lo0)
    if two_d:
        assert np.all(np.isfinite(st.row)) and np.all(np.isfinite(st.col)) and np.all(st.row > 0)
    else:
        assert np.all(np.isfinite(st.vs)) and np.all(st.vs > 0)


def test_tensor_without_gradient_is_untouched():
    st = _state2d(8, 16, np.ones(128, np.float32))
    before = st.copy()
    oracle.factored_step(st, None, 8, 16, FHParams(), 1)
    assert np.array_equal(st.hi, before.hi) and np.array_equal(st.row, before.row)


def _dbl_factored_2d(w, g, r, c, hp: FHParams, beta2=None):
    R, C = g.shape
    b2 = hp.beta2 if beta2 is None else beta2
    q = g * g + hp.eps1
    r = b2 * r + (1 - b2) * q.mean(axis=1)
    c = b2 * c + (1 - b2) * q.mean(axis=0)
    vhat = np.outer(r, c) / r.mean()                # Adafactor's factored estimate
    U = g / np.sqrt(vhat)
    rms = np.sqrt(np.mean(U * U))
    U = U / max(1.0, rms / hp.clip_threshold)
    w2 = w - hp.lr * U - hp.lr * hp.weight_decay * w
    return w2, r, c, rms


@pytest.mark.parametrize("preset", [0.0, 1.0])
@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_factored_vs_double_brute_force(preset, wd):
    """[64, 48], 10 lockstep steps, grads N(0,1e-3) with 100x outliers. preset
    row/col EMAs of 1.0 keep RMS(U) < 1 so the clip is inactive (f = lr)."""
    rng = np.random.default_rng(4)
    R, C = 64, 48
    hp = FHParams(lr=3.5e-6, weight_decay=wd)
    st = _state2d(R, C, (rng.standard_normal(R * C) * 0.02).astype(np.float32))
    st.row[:] = preset
    st.col[:] = preset
    clipped = []
    for t in range(1, 11):
        gf = rng.standard_normal(R * C) * 1e-3
        gf[rng.random(R * C) < 0.01] *= 100
        g = _bf16(gf)
        w = oracle.join(st.hi, st.lo).astype(np.float64)
        gd = oracle.bf16_to_f32(g).astype(np.float64).reshape(R, C)
        w2, r, c, rms = _dbl_factored_2d(w.reshape(R, C), gd, st.row.astype(np.float64),
                                         st.col.astype(np.float64), hp)
        clipped.append(rms > 1)
        oracle.factored_step(st, g, R, C, hp, t)
        assert np.allclose(st.row, r, rtol=1e-6, atol=0) and np.allclose(st.col, c, rtol=1e-6, atol=0)
        wo = oracle.join(st.hi, st.lo).astype(np.float64)
        w2 = w2.reshape(-1)
        du = np.abs(w2 - w)
        assert np.all(np.abs(wo - w2) <= 2 * ulp32(w2) + 1e-5 * du), t
    assert all(clipped) if preset == 0.0 else not any(clipped)


def test_one_d_vs_double_brute_force():
    """Unfactored 1-D path with the uint16 codec for v: weights and v codes."""
    rng = np.random.default_rng(5)
    n = 700
    hp = FHParams(lr=3.5e-6)
    st = _state1d(n, (rng.standard_normal(n) * 0.02).astype(np.float32))
    for t in range(1, 11):
        g = _bf16(rng.standard_normal(n) * 1e-3)
        gd = oracle.bf16_to_f32(g).astype(np.float64)
        w = oracle.join(st.hi, st.lo).astype(np.float64)
        nb = oracle.nblocks(n)
        v0 = (st.vc.astype(np.float64) / 65535) ** 4 * np.repeat(st.vs.astype(np.float64), 256)[:n]
        v = hp.beta2 * v0 + (1 - hp.beta2) * (gd * gd + hp.eps1)
        U = gd / np.sqrt(v)
        rms = np.sqrt(np.mean(U * U))
        w2 = w - hp.lr * U / max(1.0, rms)
        oracle.factored_step(st, g, 0, 0, hp, t)
        wo = oracle.join(st.hi, st.lo).astype(np.float64)
        assert np.all(np.abs(wo - w2) <= 2 * ulp32(w2) + 1e-5 * np.abs(w2 - w)), t
        for b in range(nb):
            vb = v[b * 256:(b + 1) * 256]
            assert abs(st.vs[b] / vb.max() - 1) < 1e-6
            k = np.floor(65535 * (vb / vb.max()) ** 0.25 + 0.5)
            assert np.max(np.abs(st.vc[b * 256:(b + 1) * 256].astype(np.int64) - k)) <= 1


# ---------------------------------------------------------------------------
# Adafactor's beta2 schedule and the optional first moment (commit 7983d3d,
# adafactor_step_param: beta2t = 1 - step^decay_rate; exp_avg of the clipped,
# lr-scaled update when beta1 is set)
# ---------------------------------------------------------------------------

def test_schedule_first_update_keeps_exactly_this_steps_means():
    """At update 1 the schedule gives beta2 = 1 - 1 = 0, so whatever the EMAs
    held before, they become this step's row and column means of g^2 + eps1
    (means of the fp32 squares, accumulated exactly and rounded once)."""
    rng = np.random.default_rng(21)
    R, C = 40, 56
    g = _bf16(rng.standard_normal(R * C) * 1e-3)
    st = _state2d(R, C)
    st.row[:] = 123.0
    st.col[:] = 7.0
    oracle.factored_step(st, g, R, C, FHParams(decay_rate=-0.8), 1)
    gf = oracle.bf16_to_f32(g).reshape(R, C)
    q = (gf * gf + np.float32(1e-30)).astype(np.float64)
    assert np.array_equal(st.row, q.mean(axis=1).astype(np.float32))
    assert np.array_equal(st.col, q.mean(axis=0).astype(np.float32))
    st1 = _state1d(300)
    g1 = _bf16(rng.standard_normal(300) * 1e-3)
    st1.vs[:] = 5.0
    st1.vc[:] = 40000
    oracle.factored_step(st1, g1, 0, 0, FHParams(decay_rate=-0.8), 1)
    v = oracle.decode(st1.vc, st1.vs, UNSIGNED)
    g1f = oracle.bf16_to_f32(g1).astype(np.float64)
    assert np.allclose(v, g1f * g1f + 1e-30, rtol=1e-3, atol=0)


def test_schedule_vs_double_brute_force():
    """Ten steps with beta2_t = 1 - t^-0.8 against the same step in double."""
    rng = np.random.default_rng(22)
    R, C = 32, 48
    hp = FHParams(lr=1e-4, decay_rate=-0.8)
    st = _state2d(R, C, (rng.standard_normal(R * C) * 0.02).astype(np.float32))
    for t in range(1, 11):
        g = _bf16(rng.standard_normal(R * C) * 1e-3)
        w = oracle.join(st.hi, st.lo).astype(np.float64)
        gd = oracle.bf16_to_f32(g).astype(np.float64).reshape(R, C)
        w2, r, c, _ = _dbl_factored_2d(w.reshape(R, C), gd, st.row.astype(np.float64), st.col.astype(np.float64),
                                       hp, beta2=1.0 - t ** -0.8)
        oracle.factored_step(st, g, R, C, hp, t)
        assert np.allclose(st.row, r, rtol=1e-6, atol=0) and np.allclose(st.col, c, rtol=1e-6, atol=0), t
        wo = oracle.join(st.hi, st.lo).astype(np.float64)
        w2 = w2.reshape(-1)
        assert np.all(np.abs(wo - w2) <= 2 * ulp32(w2) + 1e-5 * np.abs(w2 - w)), t


@pytest.mark.parametrize("two_d", [True, False])
def test_first_moment_scales_the_first_step_and_carries_momentum(two_d):
    """beta1 = 0.9: the first update is (1 - beta1) times the update without a
    first moment (the EMA starts from zero); a following zero-gradient step
    (U = 0) still moves the weight by beta1 times the previous step (momentum),
    up to the signed codec's rounding of the stored moment."""
    rng = np.random.default_rng(23)
    R, C = (24, 40) if two_d else (0, 0)
    n = R * C if two_d else 777
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = _bf16(rng.standard_normal(n) * 1e-3)

    def fresh():
        st = _state2d(R, C, w0) if two_d else _state1d(n, w0)
        st.mc, st.ms, _, _ = oracle.zero_moments(n)
        return st
    st_a, st_b = fresh(), fresh()
    oracle.factored_step(st_a, g, R, C, FHParams(lr=1e-3), 1)
    oracle.factored_step(st_b, g, R, C, FHParams(lr=1e-3, beta1=0.9), 1)
    wa = oracle.join(st_a.hi, st_a.lo).astype(np.float64)
    wb = oracle.join(st_b.hi, st_b.lo).astype(np.float64)
    base = w0.astype(np.float64)
    d_a, d_b = wa - base, wb - base
    assert np.all(np.abs(d_b - 0.1 * d_a) <= 2 * ulp32(wb) + 1e-5 * np.abs(d_a))
    assert np.any(st_b.mc != 32768) and np.all(st_a.mc == 32768)
    oracle.factored_step(st_b, np.zeros(n, np.uint16), R, C, FHParams(lr=1e-3, beta1=0.9), 2)
    wb2 = oracle.join(st_b.hi, st_b.lo).astype(np.float64)
    assert np.all(np.abs((wb2 - wb) - 0.9 * d_b) <= 2 * ulp32(wb2) + 2e-3 * np.abs(d_b))


@pytest.mark.parametrize("two_d", [True, False])
def test_stochastic_rounding_brackets_the_residual_step(two_d):
    """Stochastic rounding in the factored step [ADAF's default]: from a bf16
    weight (residual 0) the result is the fp32 step's weight rounded up in
    magnitude exactly when its low 16 bits plus the element's random bits
    carry; the EMAs and v codes equal the residual step's."""
    rng = np.random.default_rng(24)
    R, C = (20, 36) if two_d else (0, 0)
    n = R * C if two_d else 500
    hi0 = _bf16(rng.standard_normal(n) * 0.02)
    g = _bf16(rng.standard_normal(n) * 1e-3)

    def fresh():
        st = _state2d(R, C) if two_d else _state1d(n)
        st.hi[:] = hi0
        return st
    st_t, st_s = fresh(), fresh()
    oracle.factored_step(st_t, g, R, C, FHParams(lr=1e-3), 1)
    oracle.factored_step(st_s, g, R, C, FHParams(lr=1e-3, split_mode=oracle.SPLIT_STOCHASTIC, seed=5, tensor=3), 1)
    assert np.all(st_s.lo == 0)
    r = oracle.sr_rand16(5, 1, 3, 0, n).astype(np.uint32)
    carry = st_t.lo.astype(np.uint32) + r >= 65536
    assert np.array_equal(st_s.hi, (st_t.hi.astype(np.uint32) + carry).astype(np.uint16))
    if two_d:
        assert np.array_equal(st_s.row, st_t.row) and np.array_equal(st_s.col, st_t.col)
    else:
        assert np.array_equal(st_s.vc, st_t.vc) and np.array_equal(st_s.vs, st_t.vs)


# ---------------------------------------------------------------------------
# The order of adafactor_step_param (commit 7983d3d 'Fused backward pass'):
# divide U by max(1, RMS(U) / clip_threshold), multiply by lr, replace it by
# the first-moment EMA when beta1 is set, decay the weight by wd * lr, then
# subtract. Written here in double from each step's decoded oracle state.
# ---------------------------------------------------------------------------

def _dbl_adaf_update(U, w, m0, hp: FHParams):
    """Clip, lr, optional EMA, decoupled decay and the subtraction, in the
    page's order; returns (new weight, new first moment or None, RMS(U))."""
    rms = np.sqrt(np.mean(U * U))
    x = U / max(1.0, rms / hp.clip_threshold) * hp.lr
    m = None
    if hp.beta1 != 0.0:
        m = hp.beta1 * m0 + (1.0 - hp.beta1) * x
        x = m
    w = w - hp.weight_decay * hp.lr * w
    return w - x, m, rms


def _dbl_adaf_2d(st, g, R, C, hp: FHParams):
    gd = oracle.bf16_to_f32(g).astype(np.float64).reshape(R, C)
    w = oracle.join(st.hi, st.lo).astype(np.float64)
    q = gd * gd + hp.eps1
    r = hp.beta2 * st.row.astype(np.float64) + (1 - hp.beta2) * q.mean(axis=1)
    c = hp.beta2 * st.col.astype(np.float64) + (1 - hp.beta2) * q.mean(axis=0)
    U = (gd / np.sqrt(np.outer(r, c) / r.mean())).reshape(-1)
    m0 = oracle.decode(st.mc, st.ms, oracle.SIGNED).astype(np.float64) if hp.beta1 else None
    w2, m, rms = _dbl_adaf_update(U, w, m0, hp)
    return w, w2, m, rms


def _dbl_adaf_1d(st, g, hp: FHParams):
    gd = oracle.bf16_to_f32(g).astype(np.float64)
    w = oracle.join(st.hi, st.lo).astype(np.float64)
    v0 = oracle.decode(st.vc, st.vs, UNSIGNED).astype(np.float64)
    v = hp.beta2 * v0 + (1 - hp.beta2) * (gd * gd + hp.eps1)
    U = gd / np.sqrt(v)
    m0 = oracle.decode(st.mc, st.ms, oracle.SIGNED).astype(np.float64) if hp.beta1 else None
    w2, m, rms = _dbl_adaf_update(U, w, m0, hp)
    return w, w2, m, rms


def _assert_codes_near(code, scale, want, what):
    """Signed codes within 1 of round(32767 (|m| / block max)^(1/4)), scales
    within 1e-6 of the block max, both from the double brute force."""
    for b in range(oracle.nblocks(want.size)):
        mb = want[b * 256:(b + 1) * 256]
        s = np.max(np.abs(mb))
        assert abs(scale[b] / s - 1) < 1e-6, (what, b)
        k = np.floor(32767 * (np.abs(mb) / s) ** 0.25 + 0.5)
        ref = np.where(mb < 0, 32768 - k, 32768 + k)
        assert np.max(np.abs(code[b * 256:(b + 1) * 256].astype(np.int64) - ref)) <= 1, (what, b)


@pytest.mark.parametrize("two_d", [True, False])
@pytest.mark.parametrize("wd", [0.01, 0.1])
def test_first_moment_with_weight_decay_vs_double_brute_force(two_d, wd):
    """beta1 = 0.9 together with weight decay, 10 lockstep steps against the
    page's order in double: the EMA holds only the clipped, lr-scaled update
    and the decay is applied to the weight outside it. Folding the decay into
    the EMA would scale it by 1 - beta1 on the first step and carry it into
    the stored moment."""
    rng = np.random.default_rng(31)
    R, C = (40, 56) if two_d else (0, 0)
    n = R * C if two_d else 900
    hp = FHParams(lr=1e-3, beta1=0.9, weight_decay=wd)
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    st = _state2d(R, C, w0) if two_d else _state1d(n, w0)
    st.mc, st.ms, _, _ = oracle.zero_moments(n)
    for t in range(1, 11):
        g = _bf16(rng.standard_normal(n) * 1e-3)
        if two_d:
            w, w2, m, _ = _dbl_adaf_2d(st, g, R, C, hp)
        else:
            w, w2, m, _ = _dbl_adaf_1d(st, g, hp)
        oracle.factored_step(st, g, R, C, hp, t)
        wo = oracle.join(st.hi, st.lo).astype(np.float64)
        assert np.all(np.abs(wo - w2) <= 2 * ulp32(w2) + 1e-5 * np.abs(w2 - w)), t
        _assert_codes_near(st.mc, st.ms, m, t)


# (clip threshold, preset of the row/column EMAs or of v, expected clipping):
# RMS(U) is about 1e-3 / sqrt(preset) for N(0, 1e-3) gradients, so presets of
# 1.1e-5 and 2.5e-7 give RMS near 0.3 and 2; a zero preset gives about 31.6.
CLIP_CASES = [(0.5, 1.1e-5, False), (0.5, 2.5e-7, True), (4.0, 2.5e-7, False), (4.0, 0.0, True)]


@pytest.mark.parametrize("two_d", [True, False])
@pytest.mark.parametrize("clip,preset,active", CLIP_CASES)
def test_clip_threshold_vs_double_brute_force(two_d, clip, preset, active):
    """Update clipping divides by max(1, RMS(U) / clip_threshold): at
    thresholds 0.5 and 4.0, with the clip active and inactive, 3 lockstep
    steps against the double brute force (where the clip is inactive the step
    is lr * U exactly)."""
    rng = np.random.default_rng(32)
    R, C = (48, 40) if two_d else (0, 0)
    n = R * C if two_d else 1100
    hp = FHParams(lr=1e-4, clip_threshold=clip, weight_decay=0.01)
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    if two_d:
        st = _state2d(R, C, w0)
        st.row[:] = preset
        st.col[:] = preset
    else:
        st = _state1d(n, w0)
        st.vc[:] = 65535 if preset else 0
        st.vs[:] = preset
    for t in range(1, 4):
        g = _bf16(rng.standard_normal(n) * 1e-3)
        if two_d:
            w, w2, _, rms = _dbl_adaf_2d(st, g, R, C, hp)
        else:
            w, w2, _, rms = _dbl_adaf_1d(st, g, hp)
        if t == 1:
            assert (rms > clip) == active, rms
        oracle.factored_step(st, g, R, C, hp, t)
        wo = oracle.join(st.hi, st.lo).astype(np.float64)
        assert np.all(np.abs(wo - w2) <= 2 * ulp32(w2) + 1e-5 * np.abs(w2 - w)), t
