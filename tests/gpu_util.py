"""Helpers of the GPU parity tests: build the same seeded optimizer state on
the device (through synth's device fills) and on the host (synth's host fills)
and compare device results with the oracle's."""
import math

import numpy as np

import oracle
import synth
from synth import SIGMA_G, SIGMA_W, STREAM_GRAD, STREAM_HI, STREAM_LO

DEV = "cuda"


def torch():
    import torch as _t
    return _t


def ps():
    import precision_state_amd as _ps
    return _ps


def nblocks(n):
    return (n + 255) // 256


def u16(t):
    return t.detach().cpu().numpy().view(np.uint16)


def f32(t):
    return t.detach().cpu().numpy()


def dev_u16_from(a):
    T = torch()
    return T.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).to(DEV)


def dev_state(numel, seed=0, tid=0, rows=0, cols=0, factored=False):
    """Device state: hi ~ bf16(N(0, 0.02)), lo uniform, zero moments."""
    T = torch()
    hi = T.empty(numel, dtype=T.int16, device=DEV)
    lo = T.empty(numel, dtype=T.int16, device=DEV)
    synth.dev_bf16_normal(hi, seed, STREAM_HI, tid, 0, SIGMA_W)
    synth.dev_u16_uniform(lo, seed, STREAM_LO, tid, 0)
    nb = nblocks(numel)
    st = ps().TensorState(hi, lo, rows=rows, cols=cols)
    if factored:
        if rows > 0:
            st.row_ema = T.zeros(rows, dtype=T.float32, device=DEV)
            st.col_ema = T.zeros(cols, dtype=T.float32, device=DEV)
        else:
            st.v_code = T.zeros(numel, dtype=T.int16, device=DEV)
            st.v_scale = T.zeros(nb, dtype=T.float32, device=DEV)
        st.m_code = T.full((numel,), -32768, dtype=T.int16, device=DEV)   # first moment (read only if beta1 > 0)
        st.m_scale = T.zeros(nb, dtype=T.float32, device=DEV)
    else:
        st.m_code = T.full((numel,), -32768, dtype=T.int16, device=DEV)   # 0x8000: zero code
        st.m_scale = T.zeros(nb, dtype=T.float32, device=DEV)
        st.v_code = T.zeros(numel, dtype=T.int16, device=DEV)
        st.v_scale = T.zeros(nb, dtype=T.float32, device=DEV)
    return st


def host_state(numel, seed=0, tid=0, rows=0, factored=False, cols=0):
    hi = synth.host_bf16_normal(numel, seed, STREAM_HI, tid, 0, SIGMA_W)
    lo = synth.host_u16_uniform(numel, seed, STREAM_LO, tid, 0)
    st = oracle.TensorState(hi, lo)
    if factored:
        if rows > 0:
            st.row = np.zeros(rows, np.float32)
            st.col = np.zeros(cols, np.float32)
        else:
            _, _, st.vc, st.vs = oracle.zero_moments(numel)
        st.mc, st.ms, _, _ = oracle.zero_moments(numel)
    else:
        st.mc, st.ms, st.vc, st.vs = oracle.zero_moments(numel)
    return st


def dev_grad(numel, seed, tid, step, outlier_p=0.0, sigma=SIGMA_G):
    T = torch()
    g = T.empty(numel, dtype=T.int16, device=DEV)
    synth.dev_bf16_normal(g, seed, STREAM_GRAD, tid, step, sigma, outlier_p, 100.0)
    return g


def host_grad(numel, seed, tid, step, outlier_p=0.0, sigma=SIGMA_G):
    return synth.host_bf16_normal(numel, seed, STREAM_GRAD, tid, step, sigma, outlier_p, 100.0)


def to_host(st):
    """oracle.TensorState copy of a device TensorState."""
    h = oracle.TensorState(u16(st.w_hi).copy(), u16(st.w_lo).copy())
    if st.m_code is not None:
        h.mc, h.ms = u16(st.m_code).copy(), f32(st.m_scale).copy()
    if st.v_code is not None:
        h.vc, h.vs = u16(st.v_code).copy(), f32(st.v_scale).copy()
    if st.row_ema is not None:
        h.row, h.col = f32(st.row_ema).copy(), f32(st.col_ema).copy()
    return h


def mismatches(dev, host):
    """Per-field counts of differing elements (bitwise; fp32 compared as bits)."""
    d = to_host(dev)
    out = {}
    for name in ("hi", "lo", "mc", "ms", "vc", "vs", "row", "col"):
        a, b = getattr(d, name), getattr(host, name)
        if a is None and b is None:
            continue
        out[name] = int(np.count_nonzero(a.view(np.uint32 if a.dtype == np.float32 else np.uint16) !=
                                         b.view(np.uint32 if b.dtype == np.float32 else np.uint16)))
    return out


def max_code_diff(dev, host):
    d = to_host(dev)
    r = {}
    for name in ("mc", "vc"):
        a, b = getattr(d, name), getattr(host, name)
        if a is not None:
            r[name] = int(np.max(np.abs(a.astype(np.int64) - b.astype(np.int64)), initial=0))
    return r


def sample_blocks(numel, k, rng):
    """k distinct block indices of a tensor (always including the last)."""
    nb = nblocks(numel)
    if nb <= k:
        return np.arange(nb)
    idx = rng.choice(nb - 1, size=k - 1, replace=False)
    return np.sort(np.append(idx, nb - 1))


def block_slice(b, numel):
    return slice(b * 256, min(numel, (b + 1) * 256))


def ohp(hp, tensor=0, elem0=0):
    """oracle.HParams of a precision_state_amd.HParams; tensor = the tensor's
    index in the device call's list and elem0 = the index within the tensor of
    the host arrays' first element (both only matter for stochastic rounding)."""
    return oracle.HParams(hp.algo, hp.split_mode, hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay,
                          hp.momentum_decay, hp.seed, tensor, elem0)


def _host_block_state(tid, b, numel, seed):
    sl = block_slice(b, numel)
    L = sl.stop - sl.start
    hi = synth.host_bf16_normal(L, seed, STREAM_HI, tid, 0, SIGMA_W, start=sl.start)
    lo = synth.host_u16_uniform(L, seed, STREAM_LO, tid, 0, start=sl.start)
    mc, ms, vc, vs = oracle.zero_moments(L)
    return oracle.TensorState(hi, lo, mc, ms, vc, vs)


def _check_f24_block(tid, b, numel, d, hp, steps, seed, outlier_p):
    sl = block_slice(b, numel)
    L = sl.stop - sl.start
    hi = synth.host_bf16_normal(L, seed, STREAM_HI, tid, 0, SIGMA_W, start=sl.start)
    lo = synth.host_u16_uniform(L, seed, STREAM_LO, tid, 0, start=sl.start)
    m, v = np.zeros(3 * L, np.uint8), np.zeros(3 * L, np.uint8)
    for t in range(1, steps + 1):
        g = synth.host_bf16_normal(L, seed, STREAM_GRAD, tid, t, SIGMA_G, outlier_p, 100.0, start=sl.start)
        oracle.opt_step_flags(hi, lo, g, m, None, v, None, oracle.F24_MOMENTS, ohp(hp, tid, sl.start), t)
    b3 = slice(3 * sl.start, 3 * sl.stop)
    got = {"hi": u16(d.w_hi[sl]), "lo": u16(d.w_lo[sl]), "m": d.m_code[b3].cpu().numpy(),
           "v": d.v_code[b3].cpu().numpy()}
    want = {"hi": hi, "lo": lo, "m": m, "v": v}
    for name in got:
        assert np.array_equal(got[name], want[name]), (tid, int(b), name)


def check_sampled_blocks(shapes, devs, hp, steps, seed, per_tensor, outlier_p=0.0):
    """Every 256-block evolves from its own inputs only, so the oracle runs
    sampled blocks alone, free-running from the synthetic initial state.
    Tensors with f24 moments are checked through the oracle's flagged step."""
    rng = np.random.default_rng(seed + 1)
    total = 0
    for tid, (shape, d) in enumerate(zip(shapes, devs)):
        blocks = sample_blocks(shape.numel, per_tensor, rng)
        if d.flags & oracle.F24_MOMENTS:
            for b in blocks:
                _check_f24_block(tid, b, shape.numel, d, hp, steps, seed, outlier_p)
            total += len(blocks)
            continue
        for b in blocks:
            sl = block_slice(b, shape.numel)
            st = _host_block_state(tid, b, shape.numel, seed)
            for t in range(1, steps + 1):
                g = synth.host_bf16_normal(sl.stop - sl.start, seed, STREAM_GRAD, tid, t, SIGMA_G, outlier_p,
                                           100.0, start=sl.start)
                oracle.opt_step(st, g, ohp(hp, tid, sl.start), t)
            got = {"hi": u16(d.w_hi[sl]), "lo": u16(d.w_lo[sl]), "mc": u16(d.m_code[sl]), "vc": u16(d.v_code[sl]),
                   "ms": f32(d.m_scale[b:b + 1]).view(np.uint32), "vs": f32(d.v_scale[b:b + 1]).view(np.uint32)}
            want = {"hi": st.hi, "lo": st.lo, "mc": st.mc, "vc": st.vc, "ms": st.ms.view(np.uint32),
                    "vs": st.vs.view(np.uint32)}
            for name in got:
                assert np.array_equal(got[name], want[name]), (shape.name, int(b), name)
        total += len(blocks)
    return total


def ofhp(hp, tensor=0):
    """oracle.FHParams of a precision_state_amd.FactoredHParams (tensor = the
    tensor's index in the device call's list, for stochastic rounding)."""
    return oracle.FHParams(hp.split_mode, hp.lr, hp.beta2, hp.eps1, hp.clip_threshold, hp.weight_decay,
                           hp.decay_rate, hp.beta1, hp.seed, tensor)


def ulp_dist(a, b):
    """Distance in fp32 ulps between bit patterns (monotone integer mapping)."""
    def key(x):
        x = x.astype(np.int64)
        return np.where(x & 0x80000000, 0x80000000 - (x & 0x7FFFFFFF), x + 0x80000000)
    return np.abs(key(a.view(np.uint32)) - key(b.view(np.uint32)))


def compare_factored(d, h, rows, what, first_moment=False):
    """Factored-step parity of a device state against the oracle's: master
    weights within 4 fp32 ulp, row/column EMAs within 1 ulp, v and m codes
    within 1, m scales within 1 ulp; returns the mismatch report."""
    dh = to_host(d)
    wd = oracle.join(dh.hi, dh.lo).view(np.uint32)
    wh = oracle.join(h.hi, h.lo).view(np.uint32)
    ud = ulp_dist(wd, wh)
    rep = {"w_exact": int(np.count_nonzero(ud == 0)), "w_n": int(ud.size), "w_max_ulp": int(ud.max(initial=0))}
    if rows > 0:
        rd = np.concatenate([ulp_dist(dh.row, h.row), ulp_dist(dh.col, h.col)])
        rep["rowcol_max_ulp"] = int(rd.max(initial=0))
        assert rep["rowcol_max_ulp"] <= 1, (what, rep)
    else:
        cd = np.abs(dh.vc.astype(np.int64) - h.vc.astype(np.int64))
        rep["v_code_max_diff"] = int(cd.max(initial=0))
        rep["v_scale_max_ulp"] = int(ulp_dist(dh.vs, h.vs).max(initial=0))
        assert rep["v_code_max_diff"] <= 1, (what, rep)
    if first_moment:
        md = np.abs(dh.mc.astype(np.int64) - h.mc.astype(np.int64))
        rep["m_code_max_diff"] = int(md.max(initial=0))
        rep["m_scale_max_ulp"] = int(ulp_dist(dh.ms, h.ms).max(initial=0))
        assert rep["m_code_max_diff"] <= 1 and rep["m_scale_max_ulp"] <= 1, (what, rep)
    assert rep["w_max_ulp"] <= 4, (what, rep)
    return rep
