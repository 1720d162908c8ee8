"""Pins of the oracle's fused (N)AdamW step (sd-scripts PR #2187, '(N)AdamW /
Adan with fused backwards pass & CPU offloading': AdamW with Nesterov momentum,
Kahan residuals, lr 3.5e-6; commit 7983d3d 'Fused backward pass' for the EMA
form and the skip of tensors without a gradient)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import ALGO_ADAM, ALGO_NADAM, SIGNED, UNSIGNED, HParams


def ulp32(x):
    x = np.abs(np.asarray(x, np.float32))
    return (np.nextafter(x, np.float32(np.inf)) - x).astype(np.float64)


def _grads(n, seed, scale=1e-3):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(n) * scale).astype(np.float32)


# ---------------------------------------------------------------------------
# closed forms of the first update
# ---------------------------------------------------------------------------

def test_first_adam_step_is_lr_sign_g():
    """From zero moments, Adam's first update is lr * g / (|g| + eps): lr*sign(g)
    for |g| >> eps. With w = 0 the new weight is exactly -u."""
    n = 4096
    g = _grads(n, 1)
    w, m, v = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    hp = HParams(algo=ALGO_ADAM, lr=3.5e-6)
    oracle.core_step(w, m, v, g, hp, 1)
    gd = g.astype(np.float64)
    expect = -hp.lr * gd / (np.abs(gd) + hp.eps)
    assert np.max(np.abs(w - expect) / hp.lr) < 1e-6


def test_first_nadam_step_closed_form():
    """NAdam's first update from zero moments: lr*sign(g)*(1 + (1-b1) mu2/(1 - mu1 mu2))
    * |g|/(|g|+eps) with mu_t = b1 (1 - 0.5*0.96^(0.004 t)); the bracket is 1.0564518."""
    mu1 = 0.9 * (1 - 0.5 * 0.96 ** 0.004)
    mu2 = 0.9 * (1 - 0.5 * 0.96 ** 0.008)
    factor = 1 + 0.1 * mu2 / (1 - mu1 * mu2)
    assert abs(factor - 1.0564518) < 1e-7
    n = 4096
    g = _grads(n, 2)
    w, m, v = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    hp = HParams(algo=ALGO_NADAM, lr=3.5e-6)
    oracle.core_step(w, m, v, g, hp, 1)
    gd = g.astype(np.float64)
    expect = -hp.lr * factor * gd / (np.abs(gd) + hp.eps)
    assert np.max(np.abs(w - expect) / hp.lr) < 1e-6


def test_coefficients_at_step_one():
    """A = lr/(1-b1), RS2 = 1/sqrt(1-b2), AG = lr (mu1 cancels), CWD = lr*wd."""
    hp = HParams(lr=3.5e-6, weight_decay=0.01)
    c = oracle.coeffs(hp, 1)
    assert c["A"] == np.float32(3.5e-6 / (1 - 0.9))
    assert c["RS2"] == np.float32(1 / math.sqrt(1 - 0.999))
    assert c["AG"] == np.float32(3.5e-6)
    assert c["CWD"] == np.float32(3.5e-8)
    assert c["C1"] == np.float32(0.1) and c["C2"] == np.float32(1 - 0.999)


# ---------------------------------------------------------------------------
# invariants of the full quantized step
# ---------------------------------------------------------------------------

def _state(n, seed):
    rng = np.random.default_rng(seed)
    hi = torch.from_numpy((rng.standard_normal(n) * 0.02).astype(np.float32)).to(torch.bfloat16)
    hi = hi.view(torch.int16).numpy().view(np.uint16).copy()
    lo = rng.integers(0, 65536, n).astype(np.uint16)
    mc, ms, vc, vs = oracle.zero_moments(n)
    return oracle.TensorState(hi, lo, mc, ms, vc, vs)


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


@pytest.mark.parametrize("algo", [ALGO_ADAM, ALGO_NADAM])
def test_zero_gradient_leaves_weights_bit_identical(algo):
    n = 1000
    st = _state(n, 3)
    hi0, lo0 = st.hi.copy(), st.lo.copy()
    g = np.zeros(n, np.uint16)
    for t in range(1, 11):
        oracle.opt_step(st, g, HParams(algo=algo), t)
    assert np.array_equal(st.hi, hi0) and np.array_equal(st.lo, lo0)
    assert np.all(st.mc == 32768) and np.all(st.vc == 0) and np.all(st.ms == 0) and np.all(st.vs == 0)


def test_tensor_without_gradient_is_untouched():
    st = _state(700, 4)
    before = st.copy()
    oracle.opt_step(st, None, HParams(), 1)
    for a, b in zip((st.hi, st.lo, st.mc, st.ms, st.vc, st.vs),
                    (before.hi, before.lo, before.mc, before.ms, before.vc, before.vs)):
        assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# library routines: torch.optim on plain fp32 state (codec and split bypassed)
# ---------------------------------------------------------------------------

def _torch_opt(kind, p, lr, wd):
    if kind == "adam":
        return torch.optim.Adam([p], lr=lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0, foreach=False)
    if kind == "adamw":
        return torch.optim.AdamW([p], lr=lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=wd, foreach=False)
    return torch.optim.NAdam([p], lr=lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=wd,
                             momentum_decay=4e-3, decoupled_weight_decay=True, foreach=False)


@pytest.mark.parametrize("kind,algo,wd", [("adam", ALGO_ADAM, 0.0), ("adamw", ALGO_ADAM, 0.01),
                                          ("nadam", ALGO_NADAM, 0.0), ("nadam", ALGO_NADAM, 0.01)])
def test_core_step_matches_torch_optim(kind, algo, wd):
    """10 steps, lockstep (same state into both each step). lr 1e-3 makes the
    update hundreds of ulps so formula errors cannot hide in rounding."""
    n, lr = 20000, 1e-3
    rng = np.random.default_rng(7)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    p = torch.nn.Parameter(torch.from_numpy(w.copy()))
    opt = _torch_opt(kind, p, lr, wd)
    hp = HParams(algo=algo, lr=lr, weight_decay=wd)
    for t in range(1, 11):
        g = _grads(n, 100 + t)
        w_prev = w.copy()
        m_prev = m.copy()
        oracle.core_step(w, m, v, g, hp, t)
        with torch.no_grad():
            p.copy_(torch.from_numpy(w_prev))
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        st = opt.state[p]
        ref = p.detach().numpy()
        du = np.abs(w_prev.astype(np.float64) - ref)
        err = np.abs(w.astype(np.float64) - ref)
        assert np.all(err <= 2 * ulp32(ref) + 1e-5 * du), (t, np.max(err / (ulp32(ref) + 1e-30)))
        # moments agree too (then both continue from the oracle's moments); torch
        # forms exp_avg by lerp, so the bound scales with the EMA's terms
        scale_m = 0.9 * np.abs(m_prev) + 0.1 * np.abs(g)
        assert np.all(np.abs(m - st["exp_avg"].numpy()) <= 8 * 2.0 ** -24 * scale_m)
        assert np.allclose(v, st["exp_avg_sq"].numpy(), rtol=2e-6, atol=0)
        st["exp_avg"].copy_(torch.from_numpy(m))
        st["exp_avg_sq"].copy_(torch.from_numpy(v))


# ---------------------------------------------------------------------------
# double-precision brute force of the whole quantized step (64-element tensors)
# ---------------------------------------------------------------------------

def _dbl_decode(code, s, Q, signed):
    c = code.astype(np.float64)
    if signed:
        k = c - 32768.0
        return np.sign(k) * (np.abs(k) / Q) ** 4 * s
    return (c / Q) ** 4 * s


def _dbl_step(w, g, m0, v0, hp: HParams, t):
    """PyTorch's documented NAdam (m_hat with the mu schedule) / Adam, in double."""
    b1, b2, lr, eps = hp.beta1, hp.beta2, hp.lr, hp.eps
    m = b1 * m0 + (1 - b1) * g
    v = b2 * v0 + (1 - b2) * g * g
    vhat = v / (1 - b2 ** t)
    if hp.algo == ALGO_ADAM:
        mhat = m / (1 - b1 ** t)
    else:
        mus = [b1 * (1 - 0.5 * 0.96 ** (i * hp.momentum_decay)) for i in range(1, t + 2)]
        p_t = math.prod(mus[:t])
        p_n = p_t * mus[t]
        mhat = mus[t] * m / (1 - p_n) + (1 - mus[t - 1]) * g / (1 - p_t)
    w2 = w - lr * mhat / (np.sqrt(vhat) + eps) - lr * hp.weight_decay * w
    return w2, m, v


@pytest.mark.parametrize("algo,wd", [(ALGO_ADAM, 0.0), (ALGO_NADAM, 0.0), (ALGO_NADAM, 0.01)])
@pytest.mark.parametrize("split_mode", [oracle.SPLIT_TRUNC, oracle.SPLIT_NEAREST_AWAY])
def test_quantized_step_vs_double_brute_force(algo, wd, split_mode):
    """10 lockstep steps on a 64-element tensor (one partial block): master
    weights within 2 fp32 ulp (+ the decode chain's few-ulp moment error
    carried through the update), codes within 1 of the exact quarter-power
    codes of the double moments, scales within 1e-6."""
    n = 64
    hp = HParams(algo=algo, weight_decay=wd, split_mode=split_mode, lr=3.5e-6)
    st = _state(n, 11)
    for t in range(1, 11):
        g = _bf16(_grads(n, 200 + t) * (1 + 50 * (t % 3 == 0)))
        w = oracle.join(st.hi, st.lo, split_mode).astype(np.float64)
        gd = oracle.bf16_to_f32(g).astype(np.float64)
        m0 = _dbl_decode(st.mc, float(st.ms[0]), 32767, True)
        v0 = _dbl_decode(st.vc, float(st.vs[0]), 65535, False)
        w2, m, v = _dbl_step(w, gd, m0, v0, hp, t)
        oracle.opt_step(st, g, hp, t)
        wo = oracle.join(st.hi, st.lo, split_mode).astype(np.float64)
        u = np.abs(w2 - w)
        assert np.all(np.abs(wo - w2) <= 2 * ulp32(w2) + 1e-5 * u), t
        sm, sv = np.abs(m).max(), v.max()
        assert abs(st.ms[0] / sm - 1) < 1e-6 and abs(st.vs[0] / sv - 1) < 1e-6
        km = np.floor(32767 * (np.abs(m) / sm) ** 0.25 + 0.5)
        cm = np.where(m < 0, 32768 - km, 32768 + km)
        cv = np.floor(65535 * (v / sv) ** 0.25 + 0.5)
        assert np.max(np.abs(st.mc.astype(np.int64) - cm)) <= 1
        assert np.max(np.abs(st.vc.astype(np.int64) - cv)) <= 1


# ---------------------------------------------------------------------------
# per-tensor precision policy (fp32 moments for small tensors, fp32 final layer)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("algo", [ALGO_ADAM, ALGO_NADAM])
@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_policy_flags_reduce_to_pinned_steps(algo, wd):
    """fp32 moments + fp32 param is exactly the fp32 core step (pinned to
    torch.optim above); fp32 moments alone is join -> core step -> split;
    fp32 param with coded moments is the coded step on a TRUNC-split copy of
    the same fp32 weights (join(split(w)) == w)."""
    n = 1300
    hp = HParams(algo=algo, weight_decay=wd, lr=1e-4)
    rng = np.random.default_rng(21)
    w32 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g16 = _bf16(rng.standard_normal(n) * 1e-3)
    g32 = oracle.bf16_to_f32(g16).copy()
    # both flags == core step
    w_a, m_a, v_a = w32.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    w_b, m_b, v_b = w32.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, 4):
        oracle.core_step(w_a, m_a, v_a, g32, hp, t)
        oracle.opt_step_flags(w_b, None, g32, m_b, None, v_b, None, oracle.FP32_MOMENTS | oracle.FP32_PARAM, hp, t)
    assert np.array_equal(w_a.view(np.uint32), w_b.view(np.uint32))
    assert np.array_equal(m_a.view(np.uint32), m_b.view(np.uint32)) and np.array_equal(v_a, v_b)
    # fp32 moments with bf16 + residual weights
    hi, lo = oracle.split(w32)
    m_c, v_c = np.zeros(n, np.float32), np.zeros(n, np.float32)
    w_d, m_d, v_d = w32.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, 4):
        oracle.opt_step_flags(hi, lo, g16, m_c, None, v_c, None, oracle.FP32_MOMENTS, hp, t)
        oracle.core_step(w_d, m_d, v_d, g32, hp, t)
    assert np.array_equal(oracle.join(hi, lo).view(np.uint32), w_d.view(np.uint32))
    assert np.array_equal(m_c.view(np.uint32), m_d.view(np.uint32))
    # fp32 param with coded moments == coded step on split weights
    st = oracle.TensorState(*oracle.split(w32), *oracle.zero_moments(n))
    w_e = w32.copy()
    mc, ms, vc, vs = oracle.zero_moments(n)
    for t in range(1, 4):
        oracle.opt_step(st, g16, hp, t)
        oracle.opt_step_flags(w_e, None, g32, mc, ms, vc, vs, oracle.FP32_PARAM, hp, t)
    assert np.array_equal(oracle.join(st.hi, st.lo).view(np.uint32), w_e.view(np.uint32))
    assert np.array_equal(st.mc, mc) and np.array_equal(st.vc, vc) and np.array_equal(st.ms, ms)


def test_f24_moment_step_equals_core_step_on_f24_rounded_moments():
    """With F24 moments each step equals the fp32 core step whose moments are
    rounded to f24 after every update (the storage is the only difference)."""
    n = 999
    hp = HParams(lr=1e-4)
    rng = np.random.default_rng(33)
    w32 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hi, lo = oracle.split(w32)
    m24, v24 = oracle.f24_encode(np.zeros(n, np.float32)), oracle.f24_encode(np.zeros(n, np.float32))
    w_r, m_r, v_r = w32.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, 6):
        g16 = _bf16(rng.standard_normal(n) * 1e-3)
        oracle.opt_step_flags(hi, lo, g16, m24, None, v24, None, oracle.F24_MOMENTS, hp, t)
        oracle.core_step(w_r, m_r, v_r, oracle.bf16_to_f32(g16).copy(), hp, t)
        m_r = oracle.f24_decode(oracle.f24_encode(m_r))
        v_r = oracle.f24_decode(oracle.f24_encode(v_r))
    assert np.array_equal(oracle.join(hi, lo).view(np.uint32), w_r.view(np.uint32))
    assert np.array_equal(oracle.f24_decode(m24).view(np.uint32), m_r.view(np.uint32))
