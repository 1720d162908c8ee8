"""GPU parity of the factored-second-moment step (sd-scripts commit 7983d3d
'Fused backward pass', adafactor_step_param; konstmish/prodigy PR #25) against
the oracle. Bar: master weights within 4 fp32 ulp after 10 steps, row/column
EMAs within 1 ulp, v codes within 1. The kernels use the oracle's operation
order except for the order of the double-precision sums (fixed trees instead
of index order) and, for tensors whose rows are whole multiples of 512
columns, the sum of U^2, which they form as rbar * sum_j Q_j / c_j with
Q_j = sum_i g_ij^2 / r_i in double (the same quantity, without the fp32
rounding of rho_i, kap_j and U); mismatch counts are reported."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import synth
from gpu_util import (DEV, compare_factored as _compare, dev_grad, dev_state, host_grad, host_state, ofhp as _ofhp,
                      ulp_dist)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import precision_state_amd as ps  # noqa: E402


# The oracle steps each checked tensor on its own host thread (ctypes releases
# the GIL during each call; the tensors' states are independent).
_POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))


def _run(shapes, hp, steps, seed, outlier_p, check=None, zero_grad=(), sigmas=(synth.SIGMA_G,)):
    devs = [dev_state(s.numel, seed, i, s.rows, s.cols, factored=True) for i, s in enumerate(shapes)]
    check = list(range(len(shapes)) if check is None else check)
    hosts = {i: host_state(shapes[i].numel, seed, i, shapes[i].rows, factored=True, cols=shapes[i].cols)
             for i in check}
    ws = None

    def oracle_step(i, t):
        s = shapes[i]
        g = (np.zeros(s.numel, np.uint16) if i in zero_grad else
             host_grad(s.numel, seed, i, t, outlier_p, sigmas[i % len(sigmas)]))
        oracle.factored_step(hosts[i], g, s.rows, s.cols, _ofhp(hp, i), t)

    for t in range(1, steps + 1):
        dg = [torch.zeros(s.numel, dtype=torch.int16, device=DEV) if i in zero_grad else
              dev_grad(s.numel, seed, i, t, outlier_p, sigmas[i % len(sigmas)]) for i, s in enumerate(shapes)]
        recs = ps.make_records(devs, dg)
        need = ps.factored_workspace_size(None, records=recs)
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
        ps.factored_step(None, None, hp, t, workspace=ws, records=recs)
        # largest tensors first, so the longest oracle calls start at once
        for f in [_POOL.submit(oracle_step, i, t) for i in sorted(check, key=lambda i: -shapes[i].numel)]:
            f.result()
        print(f"  step {t} done", flush=True)
    torch.cuda.synchronize()
    reps = {}
    for i in check:
        reps[shapes[i].name] = _compare(devs[i], hosts[i], shapes[i].rows, shapes[i].name, hp.beta1 != 0.0)
    for k, v in reps.items():
        print(f"  {k}: {v}", flush=True)
    return reps


def test_factored_double_block_shapes_10_steps():
    """The FLUX double-block shapes (10 2-D factored + 14 1-D), grads N(0,1e-3)
    with 0.1% outliers at 100x, beta2 0.999, eps1 1e-30, clip 1.0, lr 3.5e-6,
    wd 0, 10 steps, one call per step; every tensor checked."""
    shapes = synth.WORKLOADS["flux_double_block"]()
    hp = ps.FactoredHParams(lr=3.5e-6, beta2=0.999, eps1=1e-30, clip_threshold=1.0, weight_decay=0.0)
    reps = _run(shapes, hp, 10, 0, 0.001)
    assert len(reps) == 24


RAGGED = [synth.Shape("a", 1, 1, 1), synth.Shape("b", 1, 300, 300), synth.Shape("c", 300, 1, 300),
          synth.Shape("d", 65, 257, 65 * 257), synth.Shape("e", 129, 8, 129 * 8), synth.Shape("f", 64, 256, 64 * 256),
          synth.Shape("g", 100, 3000, 300000), synth.Shape("h", 0, 0, 1), synth.Shape("i", 0, 0, 255),
          synth.Shape("j", 0, 0, 257), synth.Shape("k", 0, 0, 5000), synth.Shape("l", 70, 130, 9100),
          synth.Shape("m", 0, 0, 3000)]


@pytest.mark.parametrize("split_mode", [ps.SPLIT_TRUNC, ps.SPLIT_NEAREST_AWAY, ps.SPLIT_STOCHASTIC])
@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_factored_ragged_shapes(split_mode, wd):
    """Partial tiles, C % 8 != 0 rows, 1xC and Rx1 tensors, partial codec
    blocks, and all-zero gradients in one 2-D and one 1-D tensor; stochastic
    rounding draws the same stream as the oracle in the flat, tiled and 1-D
    kernels."""
    hp = ps.FactoredHParams(split_mode=split_mode, lr=1e-4, weight_decay=wd, seed=4242)
    _run(RAGGED, hp, 5, 3, 0.01, zero_grad=(11, 12))


def test_zero_gradient_leaves_weights_identical():
    shapes = [synth.Shape("w", 96, 320, 96 * 320), synth.Shape("b", 0, 0, 320)]
    hp = ps.FactoredHParams()
    devs = [dev_state(s.numel, 1, i, s.rows, s.cols, factored=True) for i, s in enumerate(shapes)]
    before = [(d.w_hi.clone(), d.w_lo.clone()) for d in devs]
    zeros = [torch.zeros(s.numel, dtype=torch.int16, device=DEV) for s in shapes]
    recs = ps.make_records(devs, zeros)
    ws = torch.empty(ps.factored_workspace_size(None, records=recs), dtype=torch.uint8, device=DEV)
    for t in range(1, 4):
        ps.factored_step(None, None, hp, t, workspace=ws, records=recs)
    for d, (h, l) in zip(devs, before):
        assert torch.equal(d.w_hi, h) and torch.equal(d.w_lo, l)
    assert bool(torch.isfinite(devs[0].row_ema).all()) and bool(torch.isfinite(devs[0].col_ema).all())


def test_factored_schedule_and_first_moment_double_block_6_steps():
    """Adafactor's beta2 schedule (1 - t^-0.8) and a first moment (beta1 0.9)
    on the FLUX double-block shapes (all 24 in one call per step), 6 steps,
    wd 0.01; weights, EMAs, v codes and the first-moment codes and scales of
    every tensor against the oracle."""
    shapes = synth.WORKLOADS["flux_double_block"]()
    hp = ps.FactoredHParams(lr=1e-5, eps1=1e-30, clip_threshold=1.0, weight_decay=0.01, decay_rate=-0.8, beta1=0.9)
    reps = _run(shapes, hp, 6, 5, 0.001)
    assert len(reps) == 24


@pytest.mark.parametrize("clip,decay_rate", [(0.5, 0.0), (4.0, -0.8), (2.5, 0.0)])
def test_factored_clip_threshold(clip, decay_rate):
    """Update clipping at thresholds other than 1 (adafactor_step_param divides
    U by max(1, RMS(U) / clip_threshold)): with zero EMAs and constant beta2
    the first step's RMS is about 31.6 (clipped at 0.5 and 2.5); with the
    schedule, beta2 is 0 at update 1 and RMS(U) is near 1, so 4.0 mostly
    leaves the update unclipped. Ragged shapes (with a first moment at 2.5),
    4 steps."""
    hp = ps.FactoredHParams(lr=1e-4, clip_threshold=clip, weight_decay=0.01, decay_rate=decay_rate,
                            beta1=0.9 if clip == 2.5 else 0.0, seed=3)
    _run(RAGGED if clip != 2.5 else FM_RAGGED, hp, 4, 13, 0.01)


FM_RAGGED = [synth.Shape("e", 129, 8, 129 * 8), synth.Shape("f", 64, 256, 64 * 256), synth.Shape("g", 100, 3000, 300000),
             synth.Shape("n", 3, 8, 24), synth.Shape("o", 33, 1032, 33 * 1032), synth.Shape("h", 0, 0, 1),
             synth.Shape("i", 0, 0, 255), synth.Shape("j", 0, 0, 257), synth.Shape("k", 0, 0, 5000),
             synth.Shape("m", 0, 0, 3000)]


@pytest.mark.parametrize("split_mode", [ps.SPLIT_TRUNC, ps.SPLIT_NEAREST_AWAY, ps.SPLIT_STOCHASTIC])
def test_factored_first_moment_ragged(split_mode):
    """Partial items and blocks (flattened 2-D tensors ending inside a block,
    1-D tails), a zero gradient in one 2-D and one 1-D tensor (momentum keeps
    moving them), with the schedule on."""
    hp = ps.FactoredHParams(split_mode=split_mode, lr=1e-4, weight_decay=0.01, decay_rate=-0.8, beta1=0.8, seed=99)
    _run(FM_RAGGED, hp, 5, 9, 0.01, zero_grad=(3, 9))


FM_ANY_COLS = [synth.Shape("a", 1, 1, 1), synth.Shape("b", 1, 300, 300), synth.Shape("c", 300, 1, 300),
               synth.Shape("d", 65, 257, 65 * 257), synth.Shape("l", 70, 130, 9100), synth.Shape("p", 5, 3, 15),
               synth.Shape("q", 401, 499, 401 * 499), synth.Shape("f", 64, 256, 64 * 256),
               synth.Shape("j", 0, 0, 257)]


@pytest.mark.parametrize("split_mode", [ps.SPLIT_TRUNC, ps.SPLIT_NEAREST_AWAY, ps.SPLIT_STOCHASTIC])
def test_factored_first_moment_any_column_count(split_mode):
    """A first moment on 2-D tensors whose column count is not a multiple of 8
    (runs of 8 elements that cross one or several rows, tensors ending inside
    a run, a block and an item; 1 x C, R x 1 and 1 x 1), next to a 16-byte-row
    tensor and a 1-D tensor in the same call; a zero gradient in one of them."""
    hp = ps.FactoredHParams(split_mode=split_mode, lr=1e-4, weight_decay=0.01, decay_rate=-0.8, beta1=0.8, seed=7)
    _run(FM_ANY_COLS, hp, 5, 11, 0.01, zero_grad=(4,))


@pytest.mark.parametrize("split_mode", [ps.SPLIT_TRUNC, ps.SPLIT_NEAREST_AWAY, ps.SPLIT_STOCHASTIC])
def test_single_one_d_tensor_calls(split_mode):
    """Per-hook calls with one 1-D tensor each (biases and norm scales are
    stepped this way from their gradient hooks): 1 to 70000 elements, partial
    items and blocks, with a first moment and the schedule, 4 steps, every
    call against the oracle."""
    sizes = [1, 255, 256, 1025, 18432, 32768, 32769, 70000]
    hp = ps.FactoredHParams(split_mode=split_mode, lr=1e-4, weight_decay=0.01, decay_rate=-0.8, beta1=0.9, seed=17)
    for i, n in enumerate(sizes):
        shape = synth.Shape(f"v{n}", 0, 0, n)
        d = dev_state(n, 21, i, 0, 0, factored=True)
        h = host_state(n, 21, i, 0, factored=True)
        ws = torch.empty(max(ps.factored_workspace_size([d], [d.w_hi]), 256), dtype=torch.uint8, device=DEV)
        for t in range(1, 5):
            g = dev_grad(n, 21, i, t, 0.01)
            ps.factored_step([d], [g], hp, t, workspace=ws)
            oracle.factored_step(h, host_grad(n, 21, i, t, 0.01), 0, 0, _ofhp(hp, 0), t)
        torch.cuda.synchronize()
        _compare(d, h, 0, shape.name, first_moment=True)


@pytest.mark.parametrize("split_mode", [ps.SPLIT_TRUNC, ps.SPLIT_STOCHASTIC])
def test_one_d_only_lists(split_mode):
    """Lists of 1-D tensors only (no 2-D tensor, so no statistics or strip
    pass: the stats items ride the finalize launch and the clip factors the
    factor launch): ragged sizes from 1 to 32768 elements, then the same list
    with a tensor of 34 items added; a zero gradient, first moment and
    schedule, 4 steps, every tensor against the oracle."""
    small = [synth.Shape(f"v{n}", 0, 0, n) for n in (1, 128, 255, 1024, 1025, 3072, 9216, 32768)]
    hp = ps.FactoredHParams(split_mode=split_mode, lr=1e-4, weight_decay=0.01, decay_rate=-0.8, beta1=0.9, seed=41)
    _run(small, hp, 4, 37, 0.01, zero_grad=(2,))
    _run(small + [synth.Shape("v33793", 0, 0, 33793)], hp, 4, 37, 0.01, zero_grad=(2,))


# Row-strip stats pass (C % 512 == 0, C <= 12288; taken when the list's
# eligible tensors have at least 256 x 64 rows): 12, 6, 2 and 1 rows per
# step, idle waves (C = 4096), a partial second run per thread (C = 8192), two
# full runs (C = 12288), single-row segments, steps past a segment's last row,
# tensors cut across many groups and groups holding several tensors, next to
# a tensor of the tile path and a 1-D tensor.
STRIP = [synth.Shape("s512x1", 1, 512, 512), synth.Shape("s512x13", 13, 512, 13 * 512),
         synth.Shape("s1024x7", 7, 1024, 7 * 1024), synth.Shape("s3072x3", 3, 3072, 3 * 3072),
         synth.Shape("s3072x257", 257, 3072, 257 * 3072), synth.Shape("s4096x5", 5, 4096, 5 * 4096),
         synth.Shape("s8192x3", 3, 8192, 3 * 8192), synth.Shape("s12288x33", 33, 12288, 33 * 12288),
         synth.Shape("s1024x2000", 2000, 1024, 2000 * 1024), synth.Shape("s512x16384", 16384, 512, 16384 * 512),
         synth.Shape("s12288x1", 1, 12288, 12288), synth.Shape("t520x9", 9, 520, 9 * 520),
         synth.Shape("v3000", 0, 0, 3000)]


@pytest.mark.parametrize("split_mode,beta1", [(ps.SPLIT_TRUNC, 0.0), (ps.SPLIT_NEAREST_AWAY, 0.9),
                                              (ps.SPLIT_STOCHASTIC, 0.9)])
def test_factored_row_strip_shapes(split_mode, beta1):
    """Tensors of the row-strip pass in every thread layout it has, 4 steps,
    wd 0.01, a zero gradient in one of them; every tensor against the oracle."""
    hp = ps.FactoredHParams(split_mode=split_mode, lr=1e-4, weight_decay=0.01, beta1=beta1, seed=31)
    _run(STRIP, hp, 4, 17, 0.01, zero_grad=(2,))


@pytest.mark.parametrize("eps1", [1e-40, 1e-3])
def test_factored_eps1_extremes(eps1):
    """eps1 at a subnormal fp32 value (rows of zero gradient then carry
    subnormal q, row EMAs near 1e-43 and 1/r_i near 1e43 through the row-strip
    pass, the tiles and the 1-D path) and at 1e-3 (eps1 dominates q): the
    strip shapes, zero gradients in two tensors, 3 steps, every tensor against
    the oracle."""
    hp = ps.FactoredHParams(lr=1e-4, eps1=eps1, weight_decay=0.01, seed=3)
    _run(STRIP, hp, 3, 19, 0.01, zero_grad=(2, 5))


@pytest.mark.parametrize("split_mode,beta1", [(ps.SPLIT_TRUNC, 0.0), (ps.SPLIT_STOCHASTIC, 0.9)])
def test_factored_extreme_gradient_scales(split_mode, beta1):
    """Gradients N(0, sigma) with sigma 1e-20 (g^2 subnormal in fp32, so q is
    eps1 plus a subnormal), 1e16 (g^2 near 1e33, row sums near 1e37) and 1e-3
    taken in turn by the strip shapes' tensors, lr 0.1, clip 0.5, the
    schedule: 3 steps, every tensor against the oracle."""
    hp = ps.FactoredHParams(split_mode=split_mode, lr=0.1, clip_threshold=0.5, weight_decay=0.01,
                            decay_rate=-0.8, beta1=beta1, seed=9)
    _run(STRIP, hp, 3, 27, 0.0, sigmas=(1e-20, 1e16, 1e-3))


def test_factored_row_strip_threshold():
    """The same strip-eligible shapes in a list of 16383 rows (statistics
    tiles) and of 16384 rows (row-strip pass), clip threshold 4 with the
    schedule: both against the oracle."""
    base = [synth.Shape("a", 3, 3072, 3 * 3072), synth.Shape("b", 1, 12288, 12288),
            synth.Shape("c", 2, 1536, 2 * 1536), synth.Shape("v", 0, 0, 700)]
    hp = ps.FactoredHParams(lr=1e-4, clip_threshold=4.0, decay_rate=-0.8, seed=5)
    for rows in (16383 - 6, 16384 - 6):
        _run(base + [synth.Shape("d", rows, 512, rows * 512)], hp, 3, 23, 0.01)


# ---------------------------------------------------------------------------
# maximum sizes: one 2-D tensor beyond 2^31 elements. It takes neither the
# row-strip pass nor flat items: statistics tiles, U^2 row tiles and apply
# tiles, all with 64-bit element offsets, and R / 256 = 8129 row chunks in
# mean(r).
# ---------------------------------------------------------------------------

def test_factored_tensor_beyond_2_31_elements():
    """One [2080903, 1032] tensor (2,147,491,896 elements, about 13 GB of
    weights, residuals and gradient with 0.1% outliers), one factored step
    with weight decay, against the oracle on the same bytes (generated on the
    device, copied to the host): every weight and residual, and the row and
    column EMAs."""
    import gc
    R, C = 2080903, 1032
    n = R * C
    assert n > 1 << 31
    gc.collect()
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    if free < 40 * 2**30:
        pytest.skip(f"needs ~14 GiB of device memory, {free / 2**30:.0f} GiB free")
    seed, tid = 29, 0
    hi = torch.empty(n, dtype=torch.int16, device=DEV)
    lo = torch.empty(n, dtype=torch.int16, device=DEV)
    synth.dev_bf16_normal(hi, seed, synth.STREAM_HI, tid, 0, synth.SIGMA_W)
    synth.dev_u16_uniform(lo, seed, synth.STREAM_LO, tid, 0)
    g = dev_grad(n, seed, tid, 1, 0.001)
    st = ps.TensorState(hi, lo, rows=R, cols=C)
    st.row_ema = torch.zeros(R, dtype=torch.float32, device=DEV)
    st.col_ema = torch.zeros(C, dtype=torch.float32, device=DEV)
    host = oracle.TensorState(hi.cpu().numpy().view(np.uint16), lo.cpu().numpy().view(np.uint16))
    host.row, host.col = np.zeros(R, np.float32), np.zeros(C, np.float32)
    g_host = g.cpu().numpy().view(np.uint16)
    print("  inputs on device and host", flush=True)

    hp = ps.FactoredHParams(lr=1e-4, weight_decay=0.01, seed=7)
    recs = ps.make_records([st], [g])
    ws = torch.empty(ps.factored_workspace_size(None, records=recs), dtype=torch.uint8, device=DEV)
    ps.factored_step(None, None, hp, 1, workspace=ws, records=recs)
    torch.cuda.synchronize()
    del g, ws
    print("  device step done", flush=True)
    oracle.factored_step(host, g_host, R, C, _ofhp(hp, 0), 1)
    del g_host
    print("  oracle step done", flush=True)

    rd = np.concatenate([ulp_dist(st.row_ema.cpu().numpy(), host.row), ulp_dist(st.col_ema.cpu().numpy(), host.col)])
    assert rd.max() <= 1, ("row/col EMA ulp", int(rd.max()))
    d_hi = st.w_hi.cpu().numpy().view(np.uint16)
    d_lo = st.w_lo.cpu().numpy().view(np.uint16)
    bad = np.flatnonzero((d_hi != host.hi) | (d_lo != host.lo))
    worst = 0
    if bad.size:
        wd = oracle.join(d_hi[bad], d_lo[bad]).view(np.uint32)
        wh = oracle.join(host.hi[bad], host.lo[bad]).view(np.uint32)
        worst = int(ulp_dist(wd, wh).max())
    print(f"  {n - bad.size} of {n} weights bit-identical, max {worst} ulp; EMAs max {int(rd.max())} ulp", flush=True)
    assert worst <= 4


def test_factored_steps_are_deterministic():
    """The same three steps run twice from the same state (the double-block
    shapes, whose 2-D tensors take the row-strip pass, plus a tile-path
    tensor and ragged 1-D tensors; first moment, schedule, stochastic
    rounding): every output byte is equal, with a fresh workspace the first
    time and the first run's workspace, still holding its values, the second.
    All reductions are fixed trees, so no run-to-run variation is allowed."""
    shapes = synth.WORKLOADS["flux_double_block"]() + [synth.Shape("t", 300, 1000, 300000),
                                                       synth.Shape("v", 0, 0, 4097)]
    hp = ps.FactoredHParams(split_mode=ps.SPLIT_STOCHASTIC, lr=1e-4, weight_decay=0.01, decay_rate=-0.8,
                            beta1=0.9, seed=11)
    grads = {t: [dev_grad(s.numel, 43, i, t, 0.001) for i, s in enumerate(shapes)] for t in (1, 2, 3)}
    ws = None
    outs = []
    for run in range(2):
        devs = [dev_state(s.numel, 43, i, s.rows, s.cols, factored=True) for i, s in enumerate(shapes)]
        for t in (1, 2, 3):
            recs = ps.make_records(devs, grads[t])
            if ws is None:
                ws = torch.zeros(ps.factored_workspace_size(None, records=recs), dtype=torch.uint8, device=DEV)
            ps.factored_step(None, None, hp, t, workspace=ws, records=recs)
        torch.cuda.synchronize()
        outs.append([[a.clone() for a in (d.w_hi, d.w_lo, d.m_code, d.m_scale,
                                         d.row_ema if d.row_ema is not None else d.v_code,
                                         d.col_ema if d.col_ema is not None else d.v_scale)] for d in devs])
        del devs
    for i, (a, b) in enumerate(zip(*outs)):
        for k, (x, y) in enumerate(zip(a, b)):
            assert torch.equal(x, y), (shapes[i].name, k)
