"""GPU parity: the HIP path through the C ABI against the oracle, on seeded
synthetic inputs. Bar: bit-exact residual/join bits and block scales, codes
within 1, master weights within 4 fp32 ulp after 10 steps; the kernels are
built to match the oracle bit for bit, so every case here also reports and
asserts exact equality."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (DEV, check_sampled_blocks, dev_grad, dev_state, dev_u16_from, f32, host_grad,
                      host_state, max_code_diff, mismatches, nblocks, ohp, to_host, u16)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import precision_state_amd as ps  # noqa: E402


def _assert_exact(dev, host, what):
    mm = mismatches(dev, host)
    print(f"  {what}: mismatches {mm} max code diff {max_code_diff(dev, host)}", flush=True)
    assert all(v == 0 for v in mm.values()), (what, mm)


# ---------------------------------------------------------------------------
# split / join
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [ps.SPLIT_TRUNC, ps.SPLIT_NEAREST_AWAY])
@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 255, 1000, 65541, (1 << 22) + 3])
def test_split_join_match_oracle(mode, n):
    rng = np.random.default_rng(n)
    bits = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    w = torch.from_numpy(bits.view(np.int32)).to(DEV).view(torch.float32)
    hi = torch.empty(n, dtype=torch.int16, device=DEV)
    lo = torch.empty(n, dtype=torch.int16, device=DEV)
    ps.split(w, hi, lo, mode)
    rhi, rlo = oracle.split(bits.view(np.float32), mode)
    assert np.array_equal(u16(hi), rhi) and np.array_equal(u16(lo), rlo)
    back = torch.empty(n, dtype=torch.float32, device=DEV)
    ps.join(hi, lo, back, mode)
    assert np.array_equal(f32(back).view(np.uint32), bits)
    # join of arbitrary (hi, lo) pairs, not only split outputs
    h2 = rng.integers(0, 65536, n).astype(np.uint16)
    l2 = rng.integers(0, 65536, n).astype(np.uint16)
    ps.join(dev_u16_from(h2), dev_u16_from(l2), back, mode)
    assert np.array_equal(f32(back).view(np.uint32), oracle.join(h2, l2, mode).view(np.uint32))


@pytest.mark.parametrize("mode", [ps.SPLIT_TRUNC, ps.SPLIT_NEAREST_AWAY])
def test_split_join_roundtrip_all_patterns(mode):
    """Every 32-bit pattern survives split then join on the device."""
    chunk = 1 << 28
    base = torch.arange(chunk, dtype=torch.int64, device=DEV)
    hi = torch.empty(chunk, dtype=torch.int16, device=DEV)
    lo = torch.empty(chunk, dtype=torch.int16, device=DEV)
    back = torch.empty(chunk, dtype=torch.float32, device=DEV)
    for start in range(0, 1 << 32, chunk):
        w = (base + start).to(torch.int32)          # wraps to the 32-bit pattern
        ps.split(w.view(torch.float32), hi, lo, mode)
        ps.join(hi, lo, back, mode)
        assert torch.equal(back.view(torch.int32), w), hex(start)


# ---------------------------------------------------------------------------
# moment codec
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind", [ps.MOMENT_UNSIGNED, ps.MOMENT_SIGNED])
def test_codec_exhaustive_all_x_in_unit_interval(kind):
    """Every fp32 x in [0, 1] (1,065,353,217 patterns) encodes to the oracle's
    code: each 256-block is [1.0, 255 consecutive patterns], so the scale is 1
    and x' = x exactly; the device codes must step exactly at the oracle's
    thresholds D(k - 1/2)."""
    Q = 65535 if kind == ps.MOMENT_UNSIGNED else 32767
    nx = 0x3F800000 + 1
    per = 255
    nblk = (nx + per - 1) // per
    x = torch.ones(nblk, 256, dtype=torch.float32, device=DEV)
    pat = torch.arange(nblk * per, dtype=torch.int64, device=DEV).clamp_(max=nx - 1).to(torch.int32)
    x[:, 1:] = pat.view(torch.float32).view(nblk, per)
    del pat
    code = torch.empty(nblk * 256, dtype=torch.int16, device=DEV)
    scale = torch.empty(nblk, dtype=torch.float32, device=DEV)
    ps.encode_moments(x.view(-1), code, scale, kind)
    assert bool((scale == 1.0).all())
    del x
    c = u16(code).reshape(nblk, 256)[:, 1:].reshape(-1)[:nx].astype(np.int32)
    if kind == ps.MOMENT_SIGNED:
        assert c.min() >= 32768
        c -= 32768
    assert c[0] == 0 and c[-1] == Q
    assert int(np.max(np.diff(c))) <= 1 and int(np.min(np.diff(c))) >= 0
    thr = oracle.dec_mag(np.arange(1, Q + 1, dtype=np.float32) - np.float32(0.5),
                         oracle.SIGNED if kind == ps.MOMENT_SIGNED else oracle.UNSIGNED).view(np.uint32)
    first = np.searchsorted(c, np.arange(1, Q + 1), side="left")
    bad = np.flatnonzero(first != thr)
    assert bad.size == 0, f"{bad.size} thresholds differ; first k={bad[0] + 1}: dev {first[bad[0]]:#x} oracle {thr[bad[0]]:#x}"


@pytest.mark.parametrize("kind", [ps.MOMENT_SIGNED, ps.MOMENT_UNSIGNED])
@pytest.mark.parametrize("n", [0, 1, 255, 256, 257, 1000, 4096, 100003, 5000011])
def test_encode_decode_match_oracle(kind, n):
    rng = np.random.default_rng(1000 + n)
    x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-12, 2, n)).astype(np.float32)
    if kind == ps.MOMENT_UNSIGNED:
        x = np.abs(x)
    if n > 600:
        x[256:512] = 0.0                                # a zero block
        x[512:600] = np.float32(1e-40)                  # subnormal block max
        x[512:768] = np.where(np.arange(256) < 88, x[512:768], np.float32(-3e-39))
    okind = oracle.SIGNED if kind == ps.MOMENT_SIGNED else oracle.UNSIGNED
    rc, rs = oracle.encode(x, okind)
    xd = torch.from_numpy(x).to(DEV)
    code = torch.empty(n, dtype=torch.int16, device=DEV)
    scale = torch.empty(nblocks(n), dtype=torch.float32, device=DEV)
    ps.encode_moments(xd, code, scale, kind)
    assert np.array_equal(u16(code), rc)
    assert np.array_equal(f32(scale).view(np.uint32), rs.view(np.uint32))
    back = torch.empty(n, dtype=torch.float32, device=DEV)
    ps.decode_moments(code, scale, back, kind)
    assert np.array_equal(f32(back).view(np.uint32), oracle.decode(rc, rs, okind).view(np.uint32))


@pytest.mark.parametrize("kind", [ps.MOMENT_SIGNED, ps.MOMENT_UNSIGNED])
def test_decode_all_codes(kind):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    okind = oracle.SIGNED if kind == ps.MOMENT_SIGNED else oracle.UNSIGNED
    for s in (0.0, 1.0, 3.7e-5, 2.0 ** -126, 1.7e38):
        scale = np.full(256, s, np.float32)
        back = torch.empty(65536, dtype=torch.float32, device=DEV)
        ps.decode_moments(dev_u16_from(codes), torch.from_numpy(scale).to(DEV), back, kind)
        assert np.array_equal(f32(back).view(np.uint32), oracle.decode(codes, scale, okind).view(np.uint32))


# ---------------------------------------------------------------------------
# fused step
# ---------------------------------------------------------------------------

def test_single_1024x3072_nadam_10_steps_free_running():
    """One [1024, 3072] tensor, 10 NAdam steps (lr 3.5e-6, betas 0.9/0.999,
    eps 1e-8, wd 0, seed 0), device and oracle each running on their own."""
    n = 1024 * 3072
    dev = dev_state(n, 0, 0)
    host = host_state(n, 0, 0)
    _assert_exact(dev, host, "initial state")
    hp = ps.HParams(algo=ps.ALGO_NADAM, lr=3.5e-6, weight_decay=0.0)
    for t in range(1, 11):
        ps.opt_step_multi([dev], [dev_grad(n, 0, 0, t)], hp, t)
        oracle.opt_step(host, host_grad(n, 0, 0, t), ohp(hp), t)
        _assert_exact(dev, host, f"step {t}")


@pytest.mark.parametrize("split_mode", [ps.SPLIT_TRUNC, ps.SPLIT_STOCHASTIC])
def test_single_1024x3072_200_steps_sampled(split_mode):
    """A long run: 200 NAdamW steps on the [1024, 3072] tensor (lr 1e-4 so
    that the weights move every few steps; 0.1% gradient outliers x100), then
    96 sampled 256-blocks, each replayed alone by the oracle over all 200
    steps from the synthetic start."""
    n = 1024 * 3072
    hp = ps.HParams(algo=ps.ALGO_NADAM, lr=1e-4, weight_decay=0.01, split_mode=split_mode, seed=99)
    dev = dev_state(n, 4, 0)
    g = torch.empty(n, dtype=torch.int16, device=DEV)
    for t in range(1, 201):
        synth.dev_bf16_normal(g, 4, synth.STREAM_GRAD, 0, t, synth.SIGMA_G, 0.001, 100.0)
        ps.opt_step_multi([dev], [g], hp, t)
    torch.cuda.synchronize()
    shape = synth.Shape("w", 1024, 3072, n)
    nblk = check_sampled_blocks([shape], [dev], hp, 200, 4, per_tensor=96, outlier_p=0.001)
    assert nblk == 96


@pytest.mark.parametrize("algo", [ps.ALGO_ADAM, ps.ALGO_NADAM])
@pytest.mark.parametrize("wd", [0.0, 0.01])
@pytest.mark.parametrize("split_mode", [ps.SPLIT_TRUNC, ps.SPLIT_NEAREST_AWAY])
def test_step_variants(algo, wd, split_mode):
    n = 100003
    hp = ps.HParams(algo=algo, weight_decay=wd, split_mode=split_mode, lr=1e-4)
    dev = dev_state(n, 5, 3)
    host = host_state(n, 5, 3)
    for t in range(1, 4):
        ps.opt_step_multi([dev], [dev_grad(n, 5, 3, t, 0.001)], hp, t)
        oracle.opt_step(host, host_grad(n, 5, 3, t, 0.001), ohp(hp), t)
    _assert_exact(dev, host, f"algo {algo} wd {wd} split {split_mode}")


# Gradient magnitudes far from the default: subnormal v (below 2^-96, where a
# wave takes the library square root, and block maxima flushed to 0), large
# finite g (g^2 near 1e33), exact zeros, and one tensor at the default scale.
EXTREME_SIGMAS = [1e-20, 1e-3, 1e16, 0.0]
EXTREME_HPARAMS = [dict(algo=ps.ALGO_NADAM, beta1=0.0, beta2=0.5, eps=1e-30, lr=1.0, weight_decay=0.1,
                        momentum_decay=0.0),
                   dict(algo=ps.ALGO_NADAM, beta1=0.99, beta2=0.9999, eps=1.0, lr=1e-6, weight_decay=0.0,
                        momentum_decay=0.1),
                   dict(algo=ps.ALGO_ADAM, beta1=0.5, beta2=0.0, eps=1e-12, lr=0.1, weight_decay=0.5)]


@pytest.mark.parametrize("split_mode", [ps.SPLIT_TRUNC, ps.SPLIT_NEAREST_AWAY, ps.SPLIT_STOCHASTIC])
@pytest.mark.parametrize("which", range(len(EXTREME_HPARAMS)))
def test_step_extreme_magnitudes_and_hparams(which, split_mode):
    """Extreme hyperparameters (beta1 0 or 0.99, beta2 0 to 0.9999, eps from
    1e-30 to 1, lr up to 1, heavy weight decay, the NAdam momentum decay) on a
    list whose tensors' gradients are N(0, sigma) with sigma 1e-20, 1e-3, 1e16
    and 0; ragged sizes, 4 steps, every byte against the oracle."""
    hp = ps.HParams(split_mode=split_mode, seed=5 + which, **EXTREME_HPARAMS[which])
    sizes = [5000, 70001, 3000, 1025]
    devs = [dev_state(n, 8, i) for i, n in enumerate(sizes)]
    hosts = [host_state(n, 8, i) for i, n in enumerate(sizes)]
    for t in range(1, 5):
        grads = []
        for i, (n, sigma) in enumerate(zip(sizes, EXTREME_SIGMAS)):
            g = torch.empty(n, dtype=torch.int16, device=DEV)
            synth.dev_bf16_normal(g, 8, synth.STREAM_GRAD, i, t, sigma)
            grads.append(g)
            oracle.opt_step(hosts[i], synth.host_bf16_normal(n, 8, synth.STREAM_GRAD, i, t, sigma), ohp(hp, i), t)
        ps.opt_step_multi(devs, grads, hp, t)
    torch.cuda.synchronize()
    for i, sigma in enumerate(EXTREME_SIGMAS):
        _assert_exact(devs[i], hosts[i], f"hparams {which} split {split_mode} sigma {sigma}")


RAGGED = [0, 1, 7, 8, 64, 128, 255, 256, 257, 1000, 1023, 1024, 1025, 3000, 4096, 65539, 131089]


@pytest.mark.parametrize("split_mode", [ps.SPLIT_TRUNC, ps.SPLIT_STOCHASTIC])
@pytest.mark.parametrize("count", [len(RAGGED), 9])
def test_multi_tensor_ragged_lists(count, split_mode):
    """Ragged sizes (tails inside a 16-lane row, partial blocks, partial work
    items), tensors without a gradient, an empty tensor; 17 tensors take the
    device-table path, 9 the kernel-argument path. Stochastic rounding: the
    residual arrays stay untouched on both sides."""
    sizes = RAGGED[:count]
    hp = ps.HParams(algo=ps.ALGO_NADAM, weight_decay=0.01, lr=1e-4, split_mode=split_mode, seed=2024)
    devs = [dev_state(n, 7, i) for i, n in enumerate(sizes)]
    hosts = [host_state(n, 7, i) for i, n in enumerate(sizes)]
    for t in range(1, 4):
        has_grad = [(i + t) % 4 != 0 for i in range(count)]
        dg = [dev_grad(n, 7, i, t) if has_grad[i] else None for i, n in enumerate(sizes)]
        hg = [host_grad(n, 7, i, t) if has_grad[i] else None for i, n in enumerate(sizes)]
        ps.opt_step_multi(devs, dg, hp, t)
        oracle.opt_step_multi(hosts, hg, ohp(hp), t)
    for i, (d, h) in enumerate(zip(devs, hosts)):
        _assert_exact(d, h, f"tensor {i} numel {sizes[i]}")


def test_list_past_the_xcd_run_threshold_all_bytes():
    """Every byte of a list long enough for the XCD-aware work order (about
    49,000 work items: two whole rounds of 8 runs of 2048 items, then a tail
    in plain index order), ragged tensors among large ones, 2 NAdamW steps,
    against the oracle."""
    sizes = RAGGED + [3072 * 3072, 3072 * 4096, 3000003]
    items = sum((n + 511) // 512 for n in sizes)
    assert items > 2 * 8 * 2048
    hp = ps.HParams(algo=ps.ALGO_NADAM, weight_decay=0.01, lr=1e-4)
    devs = [dev_state(n, 13, i) for i, n in enumerate(sizes)]
    hosts = [host_state(n, 13, i) for i, n in enumerate(sizes)]
    for t in range(1, 3):
        ps.opt_step_multi(devs, [dev_grad(n, 13, i, t) for i, n in enumerate(sizes)], hp, t)
        oracle.opt_step_multi(hosts, [host_grad(n, 13, i, t) for i, n in enumerate(sizes)], ohp(hp), t)
        print(f"  step {t} done", flush=True)
    for i, (d, h) in enumerate(zip(devs, hosts)):
        _assert_exact(d, h, f"tensor {i} numel {sizes[i]}")


def _clone(st):
    c = ps.TensorState(st.w_hi.clone(), st.w_lo.clone(), st.m_code.clone(), st.m_scale.clone(),
                       st.v_code.clone(), st.v_scale.clone())
    return c


def _equal(a, b):
    return all(torch.equal(getattr(a, k), getattr(b, k)) for k in ("w_hi", "w_lo", "m_code", "m_scale",
                                                                  "v_code", "v_scale"))


def test_batched_equals_per_tensor_calls():
    sizes = RAGGED + [300000, 77]
    hp = ps.HParams(lr=1e-4)
    batch = [dev_state(n, 9, i) for i, n in enumerate(sizes)]
    single = [_clone(s) for s in batch]
    for t in range(1, 3):
        grads = [dev_grad(n, 9, i, t) for i, n in enumerate(sizes)]
        ps.opt_step_multi(batch, grads, hp, t)
        for s, g in zip(single, grads):
            ps.opt_step_multi([s], [g], hp, t)
    assert all(_equal(a, b) for a, b in zip(batch, single))


def test_checkpoint_resume_equals_straight_run():
    """10 straight steps == 5 steps, state copied to host and back, 5 steps."""
    n = 200000
    hp = ps.HParams(weight_decay=0.01, lr=1e-4)
    a = dev_state(n, 11, 0)
    b = _clone(a)
    for t in range(1, 11):
        ps.opt_step_multi([a], [dev_grad(n, 11, 0, t)], hp, t)
    for t in range(1, 6):
        ps.opt_step_multi([b], [dev_grad(n, 11, 0, t)], hp, t)
    saved = {k: getattr(b, k).cpu() for k in ("w_hi", "w_lo", "m_code", "m_scale", "v_code", "v_scale")}
    b = ps.TensorState(**{k: v.to(DEV) for k, v in saved.items()})
    for t in range(6, 11):
        ps.opt_step_multi([b], [dev_grad(n, 11, 0, t)], hp, t)
    assert _equal(a, b)


@pytest.mark.parametrize("split_mode", [ps.SPLIT_TRUNC, ps.SPLIT_STOCHASTIC])
def test_flux_double_block_3_steps_sampled(split_mode):
    """One FLUX double-stream block (24 tensors, 339,831,296 parameters), NAdamW
    wd 0.01, one multi-tensor launch per step; sampled blocks vs the oracle
    (stochastic rounding: the oracle draws each sampled block's random bits at
    the block's own element offsets)."""
    shapes = synth.WORKLOADS["flux_double_block"]()
    hp = ps.HParams(algo=ps.ALGO_NADAM, lr=3.5e-6, weight_decay=0.01, split_mode=split_mode, seed=31337)
    seed = 0
    devs = [dev_state(s.numel, seed, i, s.rows, s.cols) for i, s in enumerate(shapes)]
    recs_dev = None
    for t in range(1, 4):
        grads = [dev_grad(s.numel, seed, i, t) for i, s in enumerate(shapes)]
        recs_dev = ps.make_records(devs, grads)
        ps.opt_step_multi(None, None, hp, t, records=recs_dev)
        del grads
    torch.cuda.synchronize()
    nblk = check_sampled_blocks(shapes, devs, hp, 3, seed, per_tensor=48)
    print(f"  {nblk} sampled blocks bit-exact", flush=True)


# ---------------------------------------------------------------------------
# per-tensor storage flags (fp32 moments for small tensors, fp32 final layer)
# ---------------------------------------------------------------------------

def _flag_mix(sizes, large):
    """fp32 moments for tensors of <= 4096 elements; `large` (0: the codec, or
    f24) for the rest; fp32 parameters on two of them."""
    flag_of = [ps.TENSOR_FP32_MOMENTS if n <= 4096 else large for n in sizes]
    flag_of[5] = ps.TENSOR_FP32_PARAM | large
    flag_of[10] = ps.TENSOR_FP32_PARAM | ps.TENSOR_FP32_MOMENTS
    if large:
        flag_of[9] = flag_of[16] = large          # ragged f24 tensors of 5 and 999 elements
    return flag_of


@pytest.mark.parametrize("split_mode,large", [(ps.SPLIT_TRUNC, 0), (ps.SPLIT_NEAREST_AWAY, 0),
                                              (ps.SPLIT_TRUNC, ps.TENSOR_F24_MOMENTS),
                                              (ps.SPLIT_NEAREST_AWAY, ps.TENSOR_F24_MOMENTS),
                                              (ps.SPLIT_STOCHASTIC, ps.TENSOR_F24_MOMENTS)])
def test_storage_flags_match_oracle(split_mode, large):
    """A list mixing the default format with fp32 moments (tensors of <= 4096
    elements on the pages), f24 moments and fp32 parameters (the final
    layer), ragged sizes, both the kernel-argument and the device-table
    paths, 3 NAdamW steps; bit-exact against the oracle."""
    hp = ps.HParams(algo=ps.ALGO_NADAM, weight_decay=0.01, lr=1e-4, split_mode=split_mode, seed=77)
    _storage_flags_run(hp, large, (synth.SIGMA_G,))


@pytest.mark.parametrize("split_mode,large,which", [(ps.SPLIT_TRUNC, ps.TENSOR_F24_MOMENTS, 0),
                                                    (ps.SPLIT_STOCHASTIC, ps.TENSOR_F24_MOMENTS, 2),
                                                    (ps.SPLIT_NEAREST_AWAY, 0, 1)])
def test_storage_flags_extreme_scales(split_mode, large, which):
    """The same mixed-format list with the extreme hyperparameters and the
    gradient scales 1e-20, 1e-3, 1e16 and 0 taken in turn by its tensors:
    subnormal and near-1e33 moments through fp32, f24 and the codec, and
    through fp32 parameters; bit-exact against the oracle."""
    hp = ps.HParams(split_mode=split_mode, seed=21 + which, **EXTREME_HPARAMS[which])
    _storage_flags_run(hp, large, EXTREME_SIGMAS)


def _storage_flags_run(hp, large, sigmas):
    split_mode = hp.split_mode
    sizes = [64, 128, 3072, 4096, 1000, 300001, 257, 18432, 3000, 5, 6144 * 8, 2048, 100, 4096, 77, 65536, 999]
    flag_of = _flag_mix(sizes, large)
    for count in (len(sizes), 9):
        devs, hosts = [], []
        for i, (n, fl) in enumerate(zip(sizes[:count], flag_of[:count])):
            hi = synth.host_bf16_normal(n, 13, synth.STREAM_HI, i, 0, synth.SIGMA_W)
            lo = synth.host_u16_uniform(n, 13, synth.STREAM_LO, i, 0)
            h = {"flags": fl}
            if fl & ps.TENSOR_FP32_PARAM:
                h["w"] = oracle.join(hi, lo, ps.SPLIT_TRUNC if split_mode == ps.SPLIT_STOCHASTIC else split_mode)
                h["lo"] = None
            else:
                h["w"], h["lo"] = hi.copy(), lo.copy()
            if fl & ps.TENSOR_FP32_MOMENTS:
                h["m"], h["v"], h["ms"], h["vs"] = np.zeros(n, np.float32), np.zeros(n, np.float32), None, None
            elif fl & ps.TENSOR_F24_MOMENTS:
                h["m"], h["v"], h["ms"], h["vs"] = np.zeros(3 * n, np.uint8), np.zeros(3 * n, np.uint8), None, None
            else:
                h["m"], h["ms"], h["v"], h["vs"] = oracle.zero_moments(n)
            hosts.append(h)
            to_dev = lambda a: None if a is None else torch.from_numpy(  # noqa: E731
                a.view(np.int16) if a.dtype == np.uint16 else a.copy()).to(DEV)
            st = ps.TensorState(to_dev(h["w"].copy()), to_dev(h["lo"]), to_dev(h["m"].copy()), to_dev(h["ms"]),
                                to_dev(h["v"].copy()), to_dev(h["vs"]), flags=fl)
            if st.w_lo is None:
                st.w_lo = torch.empty(0, dtype=torch.int16, device=DEV)   # unused for fp32 parameters
            if split_mode == ps.SPLIT_STOCHASTIC and i % 2 == 0:
                st.w_lo = None                                            # no residual array at all
            if st.m_scale is None:
                st.m_scale = st.v_scale = torch.empty(0, dtype=torch.float32, device=DEV)
            devs.append(st)
        for t in range(1, 4):
            grads_d, grads_h = [], []
            for i, (n, fl) in enumerate(zip(sizes[:count], flag_of[:count])):
                g16 = synth.host_bf16_normal(n, 13, synth.STREAM_GRAD, i, t, sigmas[i % len(sigmas)])
                if fl & ps.TENSOR_FP32_PARAM:
                    g32 = oracle.bf16_to_f32(g16).copy()
                    grads_h.append(g32)
                    grads_d.append(torch.from_numpy(g32).to(DEV))
                else:
                    grads_h.append(g16)
                    grads_d.append(torch.from_numpy(g16.view(np.int16)).to(DEV))
            ps.opt_step_multi(devs, grads_d, hp, t)
            for i, (h, g) in enumerate(zip(hosts, grads_h)):
                oracle.opt_step_flags(h["w"], h["lo"], g, h["m"], h["ms"], h["v"], h["vs"], h["flags"], ohp(hp, i), t)
        torch.cuda.synchronize()
        for i, (d, h) in enumerate(zip(devs, hosts)):
            fl = h["flags"]
            got_w = d.w_hi.cpu().numpy()
            assert np.array_equal(got_w.view(np.uint32 if fl & ps.TENSOR_FP32_PARAM else np.uint16),
                                  h["w"].view(np.uint32 if fl & ps.TENSOR_FP32_PARAM else np.uint16)), (count, i, "w")
            if not fl & ps.TENSOR_FP32_PARAM and d.w_lo is not None:
                assert np.array_equal(u16(d.w_lo), h["lo"]), (count, i, "lo")
            for k in ("m", "v"):
                got = getattr(d, k + "_code").cpu().numpy()
                want = h[k]
                as_bits = {np.dtype(np.float32): np.uint32, np.dtype(np.uint16): np.uint16,
                           np.dtype(np.uint8): np.uint8}[want.dtype]
                assert np.array_equal(got.view(as_bits), want.view(as_bits)), (count, i, k)
            if not fl & (ps.TENSOR_FP32_MOMENTS | ps.TENSOR_F24_MOMENTS):
                assert np.array_equal(f32(d.m_scale).view(np.uint32), h["ms"].view(np.uint32)), (count, i, "ms")
                assert np.array_equal(f32(d.v_scale).view(np.uint32), h["vs"].view(np.uint32)), (count, i, "vs")


# ---------------------------------------------------------------------------
# maximum sizes: a tensor beyond 2^31 elements (64-bit element offsets)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("split_mode", [ps.SPLIT_TRUNC, ps.SPLIT_STOCHASTIC])
def test_tensor_beyond_2_31_elements_sampled(split_mode):
    """One tensor of 2^31 + 4097 elements (about 21.5 GB of state), 2 NAdamW
    steps in one launch each; sampled 256-blocks, most of them past element
    2^31, and the partial last block against the oracle."""
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    n = (1 << 31) + 4097
    free, _ = torch.cuda.mem_get_info()
    if free < 40 * 2**30:
        pytest.skip(f"needs ~22 GiB of device memory, {free / 2**30:.0f} GiB free")
    shapes = [synth.Shape("big", 0, 0, n)]
    hp = ps.HParams(algo=ps.ALGO_NADAM, lr=1e-4, weight_decay=0.01, split_mode=split_mode, seed=17)
    dev = [dev_state(n, 3, 0)]
    for t in (1, 2):
        g = dev_grad(n, 3, 0, t)
        ps.opt_step_multi(dev, [g], hp, t)
        del g
    torch.cuda.synchronize()
    nblk = check_sampled_blocks(shapes, dev, hp, 2, 3, per_tensor=64)
    print(f"  {nblk} sampled blocks bit-exact", flush=True)
    del dev
    gc.collect()
    torch.cuda.empty_cache()
