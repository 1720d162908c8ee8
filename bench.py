#!/usr/bin/env python3
"""Benchmark of the fused low-precision optimizer step on one MI355X.

One step = one fused NAdam update (one kernel launch) over a whole parameter
set whose state is resident in HBM: bf16 weight + uint16 residual + bf16
gradient + uint16 exp_avg / exp_avg_sq codes + per-256 fp32 block scales.
Inputs are seeded synthetic data of the FLUX shapes (no trained weights or
datasets are needed). Prints ONE JSON line on stdout; progress goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload flux_dev_12b]

Reported:
  value      optimizer-updated params/s over the timed steps (wall clock,
             bracketed by device synchronisation)
  roofline   the step kernel's average duration from HIP events recorded on
             its stream around each launch; algorithmic bytes per launch =
             18 B/param (read hi, lo, grad, m, v; write hi, lo, m, v) + 16 B
             per 256-block (two scales read and written), against 8 TB/s
  roofline.practical_peak  a streaming kernel with the step's exact access
             pattern and no arithmetic (tests/kernels/stream_ceiling.hip) over
             the same state, timed the same way right after the step: the
             rate this memory system gives that 5-read/4-write 16-byte mix;
             frac_of_practical is the step's share of it
  cpu_baseline  the C oracle as it stands on a bounded sample of the same
             workload, on one thread and on the host threads (the leading
             tensors of the set for the NAdam step, here and in the
             per-tensor and offload modes; the whole double block for the
             factored step; 2^24 elements for the standalone kernels)
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "optimizer-updated params/sec + achieved HBM GB/s (% of MI355X peak), Flux-12B set"
PEAK_HBM_GBS = 8000.0
BYTES_PER_BLOCK = 16
KERNEL_SOURCES = ["precision_state_amd/csrc/k_adam.hip", "precision_state_amd/csrc/dev_common.h"]
FACTORED_SOURCES = ["precision_state_amd/csrc/k_factored.hip", "precision_state_amd/csrc/dev_common.h",
                    "precision_state_amd/csrc/ps_internal.h"]


def step_bytes(numel, flags=0, residual=True):
    """Algorithmic HBM bytes of one step of one tensor: the weight words read
    and written (bf16 + residual, bf16 alone under stochastic rounding, or
    fp32), the gradient read, the two moments read and written (uint16 codes +
    per-256 scales, fp32, or f24)."""
    import precision_state_amd as ps
    nblk = -(-numel // 256)
    w = (8 if residual or flags & ps.TENSOR_FP32_PARAM else 4) * numel
    g = (4 if flags & ps.TENSOR_FP32_PARAM else 2) * numel
    if flags & ps.TENSOR_FP32_MOMENTS:
        mv = 16 * numel
    elif flags & getattr(ps, "TENSOR_F24_MOMENTS", 0):
        mv = 12 * numel
    else:
        mv = 8 * numel + BYTES_PER_BLOCK * nblk
    return w + g + mv


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_text(src):
    """Source text with comments removed and whitespace collapsed: what the
    compiler sees of it, so that an edit to a comment does not change it."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash(sources=None):
    """First 16 hex digits of the SHA-256 of the kernel sources' code text
    (comments and whitespace removed), in the listed order. A committed
    counter summary carries the hash of the sources it was taken on."""
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, p)) as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def gpu_pci_bus_id():
    """PCI bus id (domain:bus:device.function) of the current HIP device, from
    the HIP runtime already loaded in this process, or None."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        dev = ctypes.c_int(0)
        buf = ctypes.create_string_buffer(64)
        if hip.hipGetDevice(ctypes.byref(dev)) != 0 or hip.hipDeviceGetPCIBusId(buf, 64, dev) != 0:
            return None
        return buf.value.decode().lower()
    except (OSError, AttributeError):
        return None


def gpu_clocks():
    """Current shader and memory clock levels of the GPU this process runs on:
    the amdgpu sysfs files (pp_dpm_sclk / pp_dpm_mclk, active level marked
    '*') of the PCI device whose bus id HIP reports for the current device.
    Read from files: no helper program is started from this GPU process."""
    bdf = gpu_pci_bus_id()
    if bdf is None:
        return None
    out = {"pci_bus_id": bdf}
    for kind in ("sclk", "mclk"):
        path = f"/sys/bus/pci/devices/{bdf}/pp_dpm_{kind}"
        try:
            with open(path) as f:
                cur = [ln.split(":", 1)[1].replace("*", "").strip() for ln in f if ln.rstrip().endswith("*")]
        except OSError:
            continue
        if cur:
            out[kind] = cur[0]
    return out


def stream_ceiling(slab, steps, stream, stochastic=False):
    """Practical HBM ceiling of the step's access pattern on this GPU: the
    no-arithmetic streaming kernels of tests/kernels/stream_ceiling.hip over the
    same slab arrays as the step, timed with HIP events on the same stream.
    mode 0 is the step's mix (five 16-byte reads and four 16-byte writes per
    lane, block scales read and written: 18 B per element + 16 B per block);
    mode 1 the reads alone (10 B per element + 8 B per block); with stochastic
    rounding, mode 2 is the step's mix without the residual stream (14 B per
    element + 16 B per block) and is reported as step_mix. Overwrites the
    state, so it runs after the step's timing."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "tests", "kernels", "libps_probe.so")
    if slab is None or not os.path.exists(path):
        log(f"[bench] no ceiling measurement ({'no slab' if slab is None else path + ' is not built'})")
        return None
    L = ctypes.CDLL(path)
    L.probe_stream_ceiling.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 8 + [ctypes.c_uint32, ctypes.c_void_p]
    L.probe_stream_ceiling.restype = ctypes.c_int
    sl, sc = slab.slab, slab.scales
    n_items = min(sl["hi"].numel() // 512, sc["ms"].numel() // 2, sc["vs"].numel() // 2)
    sink = torch.zeros(4, dtype=torch.int32, device=sl["hi"].device)
    ptrs = [sl[k].data_ptr() for k in ("hi", "lo", "g", "mc", "vc")] + [sc["ms"].data_ptr(), sc["vs"].data_ptr(),
                                                                      sink.data_ptr()]
    hs = ctypes.c_void_p(stream.cuda_stream)
    res = {"elements": n_items * 512}
    modes = ((2, "step_mix", 512 * 14 + 32),) if stochastic else \
        ((0, "step_mix", 512 * 18 + 32), (1, "reads_only", 512 * 10 + 16))
    for mode, name, per_item in modes:
        for _ in range(5):
            if L.probe_stream_ceiling(mode, *ptrs, n_items, hs) != 0:
                raise RuntimeError("stream ceiling kernel launch failed")
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            L.probe_stream_ceiling(mode, *ptrs, n_items, hs)
            b.record(stream)
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in ev) / steps
        res[name] = {"ms": ms, "gbs": n_items * per_item / (ms * 1e-3) / 1e9}
        log(f"[bench] ceiling {name}: {ms:.3f} ms per launch, {res[name]['gbs']:.0f} GB/s")
    return res


def ew_ceiling(n, bufs, steps, stream):
    """Practical ceilings of the four standalone kernels: probe_ew_ceiling of
    tests/kernels/stream_ceiling.hip runs each one's grid, lane layout and
    cache hints with no arithmetic (same bytes per element), timed with HIP
    events on the same stream. bufs maps split/join/encode/decode to their
    (in0, in1, out0, out1) tensors; overwrites the outputs, so it runs after
    the kernels' own timing."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "tests", "kernels", "libps_probe.so")
    if n % 4096 or not os.path.exists(path):
        log(f"[bench] no elementwise ceilings ({'n not a multiple of 4096' if n % 4096 else path + ' is not built'})")
        return None
    L = ctypes.CDLL(path)
    if not hasattr(L, "probe_ew_ceiling"):
        log("[bench] no elementwise ceilings (probe library predates them)")
        return None
    L.probe_ew_ceiling.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_void_p]
    L.probe_ew_ceiling.restype = ctypes.c_int
    hs = ctypes.c_void_p(stream.cuda_stream)
    res = {}
    for kind, name in enumerate(("split", "join", "encode", "decode")):
        ptrs = [None if t is None else t.data_ptr() for t in bufs[name]]
        for _ in range(5):
            if L.probe_ew_ceiling(kind, *ptrs, n, hs) != 0:
                raise RuntimeError("elementwise ceiling kernel launch failed")
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            L.probe_ew_ceiling(kind, *ptrs, n, hs)
        b.record(stream)
        torch.cuda.synchronize()
        res[name] = {"ms": a.elapsed_time(b) / steps}
        log(f"[bench] ceiling {name}: {res[name]['ms']:.3f} ms per launch")
    return res


def read_counter_summary(name, key, sources=None):
    """A figure from a committed rocprofv3 counter summary under profiles/, if
    the summary was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    try:
        return float(kv[key])
    except (KeyError, ValueError):
        return None


def read_traffic(workload, moments="codec", split="trunc"):
    """HBM bytes per launch of the fused step from the committed counter summary."""
    tag = {("codec", "trunc"): "", ("f24", "trunc"): "_f24", ("codec", "stochastic"): "_sr"}.get((moments, split))
    if tag is None:
        return None
    return read_counter_summary(f"adam_step_{workload}{tag}_counters.txt", "hbm_bytes_per_launch")


def build_state(shapes, seed, dev, layout="slab", moments="codec"):
    """Optimizer state for every tensor of the set, filled on the device.

    layout "slab": one contiguous allocation per state stream
    (precision_state_amd.StateSlab, also returned); "separate": one allocation
    per tensor and stream (slab None). moments "f24" (slab only): f24 moment
    arrays instead of codes."""
    import torch

    import precision_state_amd as ps
    import synth
    if layout == "slab":
        slab = ps.StateSlab([s.numel for s in shapes], dev, shapes2d=[(s.rows, s.cols) for s in shapes],
                            moments=moments)
        states, grads = slab.states, slab.grads
    else:
        slab = None
        if moments != "codec":
            raise ValueError("f24 moments need the slab layout")
        states, grads = [], []
        for s in shapes:
            n, nb = s.numel, (s.numel + 255) // 256
            hi, lo, g = (torch.empty(n, dtype=torch.int16, device=dev) for _ in range(3))
            states.append(ps.TensorState(hi, lo, torch.full((n,), -32768, dtype=torch.int16, device=dev),
                                         torch.zeros(nb, dtype=torch.float32, device=dev),
                                         torch.zeros(n, dtype=torch.int16, device=dev),
                                         torch.zeros(nb, dtype=torch.float32, device=dev), rows=s.rows, cols=s.cols))
            grads.append(g)
    for tid, (st, g) in enumerate(zip(states, grads)):
        synth.dev_bf16_normal(st.w_hi, seed, synth.STREAM_HI, tid, 0, synth.SIGMA_W)
        synth.dev_u16_uniform(st.w_lo, seed, synth.STREAM_LO, tid, 0)
        synth.dev_bf16_normal(g, seed, synth.STREAM_GRAD, tid, 1, synth.SIGMA_G)
    return states, grads, slab


def apply_policy(shapes, states, grads, dev):
    """The pages' storage policy: tensors of at most 4096 elements keep fp32
    moments, final-layer tensors keep an fp32 parameter and gradient (no
    residual). Changes states and grads in place; returns the two counts."""
    import torch

    import precision_state_amd as ps
    n_small = n_final = 0
    for i, (s, st) in enumerate(zip(shapes, states)):
        if s.name.startswith("final_layer."):
            w32 = torch.empty(s.numel, dtype=torch.float32, device=dev)
            ps.join(st.w_hi, st.w_lo, w32)
            st.w_hi, st.w_lo = w32, torch.empty(0, dtype=torch.int16, device=dev)
            grads[i] = grads[i].view(torch.bfloat16).float()
            st.flags |= ps.TENSOR_FP32_PARAM
            n_final += 1
        if s.numel <= 4096:
            st.m_code = torch.zeros(s.numel, dtype=torch.float32, device=dev)
            st.v_code = torch.zeros(s.numel, dtype=torch.float32, device=dev)
            st.flags = (st.flags & ~ps.TENSOR_F24_MOMENTS) | ps.TENSOR_FP32_MOMENTS
            n_small += 1
    torch.cuda.synchronize()
    log(f"[bench] policy: {n_small} tensors with fp32 moments, {n_final} fp32 final-layer tensors")
    return n_small, n_final


def host_threads():
    """Host threads this process may use (its CPU affinity, at most 16: the
    share of the host that goes with one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(shapes, seed, target_params=60_000_000, weight_decay=0.0):
    """The oracle as it stands, one NAdam step over the leading tensors of the
    set (about target_params parameters): timed on one thread, then on all the
    host threads of this process over block-aligned chunks of the same sample
    (256-element blocks are independent; the oracle has no shared state and
    ctypes releases the GIL during each call). The oracle itself is unchanged."""
    import concurrent.futures

    import numpy as np

    import oracle
    import synth
    sample, total = [], 0
    for tid, s in enumerate(shapes):
        if total >= target_params:
            break
        sample.append((tid, s))
        total += s.numel
    inputs = []
    for tid, s in sample:
        n = s.numel
        st = oracle.TensorState(synth.host_bf16_normal(n, seed, synth.STREAM_HI, tid, 0, synth.SIGMA_W),
                                synth.host_u16_uniform(n, seed, synth.STREAM_LO, tid, 0), *oracle.zero_moments(n))
        inputs.append((st, synth.host_bf16_normal(n, seed, synth.STREAM_GRAD, tid, 1, synth.SIGMA_G)))
    copies = [(st.copy(), g) for st, g in inputs]
    hp = oracle.HParams(algo=oracle.ALGO_NADAM, lr=3.5e-6, weight_decay=weight_decay)
    t0 = time.perf_counter()
    for st, g in inputs:
        oracle.opt_step(st, g, hp, 1)
    dt1 = time.perf_counter() - t0

    chunk = 4096 * 256
    parts = []
    for st, g in copies:
        n = st.hi.size
        for a in range(0, n, chunk):
            b = min(n, a + chunk)
            sb = slice(a // 256, (b + 255) // 256)
            parts.append((oracle.TensorState(st.hi[a:b], st.lo[a:b], st.mc[a:b], st.ms[sb], st.vc[a:b], st.vs[sb]),
                          g[a:b]))
    threads = host_threads()
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as pool:
        t0 = time.perf_counter()
        list(pool.map(lambda p: oracle.opt_step(p[0], p[1], hp, 1), parts))
        dtn = time.perf_counter() - t0
    for (x, _), (y, _) in zip(inputs, copies):   # the chunked run must give the same bytes
        if not (np.array_equal(x.hi, y.hi) and np.array_equal(x.lo, y.lo) and np.array_equal(x.mc, y.mc)
                and np.array_equal(x.vc, y.vc) and np.array_equal(x.ms, y.ms) and np.array_equal(x.vs, y.vs)):
            raise RuntimeError("chunked oracle run differs from the single-thread run")
    return {"value": total / dtn, "unit": "params/s", "cores": threads, "kind": "oracle",
            "sample": f"first {len(sample)} tensors of the set ({total} params), one NAdam step, "
                      f"{threads} threads over {len(parts)} block-aligned chunks, {dtn:.2f} s; "
                      f"single thread {total / dt1:.3e} params/s ({dt1:.1f} s)"}


def cpu_baseline_factored(shapes, seed, hp):
    """The oracle's factored step as it stands, one step over every tensor of
    the set (with a first moment, whose exact encode is slow, over the leading
    tensors up to about 60M parameters): timed on one thread, then on this
    process's host threads with one tensor per task (each tensor's step is
    independent; ctypes releases the GIL during each call). The oracle itself
    is unchanged."""
    import concurrent.futures
    import dataclasses

    import numpy as np

    import oracle
    import synth
    ohp = oracle.FHParams(hp.split_mode, hp.lr, hp.beta2, hp.eps1, hp.clip_threshold, hp.weight_decay,
                          hp.decay_rate, hp.beta1, hp.seed, 0)
    if hp.beta1:
        lead, total = [], 0
        for s in shapes:
            if total >= 60_000_000:
                break
            lead.append(s)
            total += s.numel
        shapes = lead
    inputs = []
    for tid, s in enumerate(shapes):
        n = s.numel
        st = oracle.TensorState(synth.host_bf16_normal(n, seed, synth.STREAM_HI, tid, 0, synth.SIGMA_W),
                                synth.host_u16_uniform(n, seed, synth.STREAM_LO, tid, 0))
        if s.is_2d:
            st.row, st.col = np.zeros(s.rows, np.float32), np.zeros(s.cols, np.float32)
        else:
            _, _, st.vc, st.vs = oracle.zero_moments(n)
        if hp.beta1:
            st.mc, st.ms, _, _ = oracle.zero_moments(n)
        g = synth.host_bf16_normal(n, seed, synth.STREAM_GRAD, tid, 1, synth.SIGMA_G, 0.001, 100.0)
        inputs.append((tid, s, st, g))
    copies = [(tid, s, st.copy(), g) for tid, s, st, g in inputs]

    def one(item):
        tid, s, st, g = item
        oracle.factored_step(st, g, s.rows, s.cols, dataclasses.replace(ohp, tensor=tid), 1)

    t0 = time.perf_counter()
    for item in inputs:
        one(item)
    dt1 = time.perf_counter() - t0
    threads = min(host_threads(), len(copies))
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as pool:
        t0 = time.perf_counter()
        list(pool.map(one, sorted(copies, key=lambda it: -it[1].numel)))   # largest first
        dtn = time.perf_counter() - t0
    for (_, _, x, _), (_, _, y, _) in zip(inputs, copies):   # the threaded run must give the same bytes
        if not (np.array_equal(x.hi, y.hi) and np.array_equal(x.lo, y.lo)):
            raise RuntimeError("threaded oracle run differs from the single-thread run")
    total = sum(s.numel for s in shapes)
    return {"value": total / dtn, "unit": "params/s", "cores": threads, "kind": "oracle",
            "sample": f"{'the first' if hp.beta1 else 'all'} {len(shapes)} tensors of the set ({total} params), "
                      f"one factored step, {threads} threads "
                      f"with one tensor per task, {dtn:.2f} s; single thread {total / dt1:.3e} params/s ({dt1:.1f} s)"}


def cpu_baseline_elementwise(seed, n=1 << 24):
    """The oracle's split and join (both modes) and moment encode and decode
    (both kinds) as they stand, on n elements of the same values as the GPU
    run: timed on one thread, then on this process's host threads over
    block-aligned chunks. Value: algorithmic GB/s over the eight calls, as the
    GPU line counts them."""
    import concurrent.futures

    import numpy as np

    import oracle
    import synth
    hi = synth.host_bf16_normal(n, seed, synth.STREAM_HI, 0, 0, synth.SIGMA_W)
    lo = synth.host_u16_uniform(n, seed, synth.STREAM_LO, 0, 0)
    w = oracle.join(hi, lo)
    m = w * np.float32(1e-3)
    v = m * m
    cs, ss = oracle.encode(m, oracle.SIGNED)
    cu, su = oracle.encode(v, oracle.UNSIGNED)
    nb = (n + 255) // 256

    def blk(a, b):
        return slice(a // 256, (b + 255) // 256)
    ops = [(lambda a, b: oracle.split(w[a:b], oracle.SPLIT_TRUNC), 8 * n),
           (lambda a, b: oracle.join(hi[a:b], lo[a:b], oracle.SPLIT_TRUNC), 8 * n),
           (lambda a, b: oracle.split(w[a:b], oracle.SPLIT_NEAREST_AWAY), 8 * n),
           (lambda a, b: oracle.join(hi[a:b], lo[a:b], oracle.SPLIT_NEAREST_AWAY), 8 * n),
           (lambda a, b: oracle.encode(m[a:b], oracle.SIGNED), 6 * n + 4 * nb),
           (lambda a, b: oracle.decode(cs[a:b], ss[blk(a, b)], oracle.SIGNED), 6 * n + 4 * nb),
           (lambda a, b: oracle.encode(v[a:b], oracle.UNSIGNED), 6 * n + 4 * nb),
           (lambda a, b: oracle.decode(cu[a:b], su[blk(a, b)], oracle.UNSIGNED), 6 * n + 4 * nb)]
    total = sum(nbytes for _, nbytes in ops)
    t0 = time.perf_counter()
    for fn, _ in ops:
        fn(0, n)
    dt1 = time.perf_counter() - t0
    chunk = 1 << 20
    threads = host_threads()
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as pool:
        t0 = time.perf_counter()
        for fn, _ in ops:
            list(pool.map(lambda a: fn(a, min(n, a + chunk)), range(0, n, chunk)))
        dtn = time.perf_counter() - t0
    return {"value": total / dtn / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} elements, the eight calls, {threads} threads over {(n + chunk - 1) // chunk} "
                      f"block-aligned chunks each, {dtn:.2f} s; single thread {total / dt1 / 1e9:.3f} GB/s "
                      f"({dt1:.1f} s)"}


def calibrate_copy(gib, stream, dev):
    """Three plain device copies of `gib` GiB (the counter calibration of the
    profiles: a copy's FETCH_SIZE and WRITE_SIZE against the bytes it moves);
    returns the best copy rate in GB/s (read + write), or None when gib is 0."""
    if gib <= 0:
        return None
    import torch
    nbytes = int(gib * 2**30) // 16 * 16
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    times = []
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    copy_gbs = 2 * nbytes / (min(times) * 1e-3) / 1e9
    log(f"[bench] plain copy of {nbytes} bytes: best {min(times):.3f} ms = {copy_gbs:.0f} GB/s (read + write)")
    return copy_gbs


def bench_factored(args):
    """Adafactor-style step (beta1 = 0, factored v, clip 1.0, beta2 0.999,
    eps1 1e-30, lr 3.5e-6) on the FLUX double-block shapes: 2-D tensors
    factored, 1-D tensors with the uint16 codec. Grads N(0, 1e-3) with 0.1%
    outliers at 100x. Algorithmic bytes: 10 B/param (read hi, lo, grad; write
    hi, lo); the kernels read the gradient twice (12 B/param) for tensors of
    the row-strip statistics pass and the 1-D tensors, three times for the
    other 2-D tensors (14 B/param)."""
    import torch

    import precision_state_amd as ps
    import synth
    dev = "cuda:0"
    wl = "flux_double_block" if args.workload == "flux_dev_12b" else args.workload
    shapes = synth.WORKLOADS[wl]()
    n_params = synth.total_params(shapes)
    states, grads = [], []
    for tid, s in enumerate(shapes):
        n = s.numel
        hi, lo, g = (torch.empty(n, dtype=torch.int16, device=dev) for _ in range(3))
        synth.dev_bf16_normal(hi, args.seed, synth.STREAM_HI, tid, 0, synth.SIGMA_W)
        synth.dev_u16_uniform(lo, args.seed, synth.STREAM_LO, tid, 0)
        synth.dev_bf16_normal(g, args.seed, synth.STREAM_GRAD, tid, 1, synth.SIGMA_G, 0.001, 100.0)
        st = ps.TensorState(hi, lo, rows=s.rows, cols=s.cols)
        if s.is_2d:
            st.row_ema = torch.zeros(s.rows, dtype=torch.float32, device=dev)
            st.col_ema = torch.zeros(s.cols, dtype=torch.float32, device=dev)
        else:
            st.v_code = torch.zeros(n, dtype=torch.int16, device=dev)
            st.v_scale = torch.zeros((n + 255) // 256, dtype=torch.float32, device=dev)
        if args.beta1:
            st.m_code = torch.full((n,), -32768, dtype=torch.int16, device=dev)
            st.m_scale = torch.zeros((n + 255) // 256, dtype=torch.float32, device=dev)
        states.append(st)
        grads.append(g)
    recs = ps.make_records(states, grads)
    ws = torch.empty(ps.factored_workspace_size(None, records=recs), dtype=torch.uint8, device=dev)
    split = {"trunc": ps.SPLIT_TRUNC, "nearest_away": ps.SPLIT_NEAREST_AWAY,
             "stochastic": ps.SPLIT_STOCHASTIC}[args.split]
    hp = ps.FactoredHParams(lr=3.5e-6, beta2=0.999, eps1=1e-30, clip_threshold=1.0, weight_decay=0.0,
                            decay_rate=args.decay_rate, beta1=args.beta1, split_mode=split, seed=args.seed)
    stream = torch.cuda.current_stream()
    step = 0
    for _ in range(args.warmup):
        step += 1
        ps.factored_step(None, None, hp, step, workspace=ws, stream=stream, records=recs)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(args.steps):
        step += 1
        ps.factored_step(None, None, hp, step, workspace=ws, stream=stream, records=recs)
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clocks = gpu_clocks()
    step_ms = a.elapsed_time(b) / args.steps
    log(f"[bench] factored: {args.steps} steps, {step_ms:.3f} ms/step (events), {wall * 1e3 / args.steps:.3f} wall")
    per_tensor = None
    if args.per_tensor_calls:
        per_tensor = time_factored_per_tensor(ps, states, grads, hp, ws, stream, step, args.steps)
    copy_gbs = calibrate_copy(args.calibrate_copy, stream, dev)
    n_blocks = sum((s.numel + 255) // 256 for s in shapes)
    alg = (10 if split != ps.SPLIT_STOCHASTIC else 6) * n_params + ((4 * n_params + 8 * n_blocks) if args.beta1 else 0)
    gbs10 = alg / (step_ms * 1e-3) / 1e9
    # gradient re-reads of the design: the row-strip pass (2-D tensors with C % 512 == 0, C <= 12288 and
    # fewer than 2^31 elements, when they have 256 x 64 rows in all) reads it once more, the tiles twice
    strip = [s for s in shapes if s.is_2d and s.cols % 512 == 0 and s.cols <= 12288 and s.numel < 2 ** 31]
    strip = strip if sum(s.rows for s in strip) >= 256 * 64 else []
    rereads = sum(2 * s.numel for s in shapes) + sum(2 * s.numel for s in shapes if s.is_2d and s not in strip)
    gbs_design = (alg + rereads) / (step_ms * 1e-3) / 1e9
    baseline = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host (cpu_baseline)")
        baseline = cpu_baseline_factored(shapes, args.seed, hp)
        log(f"[bench] cpu_baseline: {baseline}")
    traffic = None
    if not args.beta1 and not args.decay_rate and split == ps.SPLIT_TRUNC and wl == "flux_double_block":
        traffic = read_counter_summary("factored_step_flux_double_block_counters.txt", "hbm_bytes_per_step",
                                       FACTORED_SOURCES)
    print(json.dumps({
        "metric": "factored optimizer-updated params/sec (Adafactor-style step, FLUX double-block shapes)",
        "value": n_params * args.steps / wall, "unit": "params/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl + "_factored", "params": n_params, "tensors": len(shapes), "step_ms": step_ms,
                   "gpu_clocks_after_timing": clocks,
                   "beta1": args.beta1, "decay_rate": args.decay_rate, "split": args.split, "algorithmic_bytes": alg,
                   "gbs_algorithmic": gbs10, "gbs_with_gradient_rereads": gbs_design,
                   "gradient_reread_bytes": rereads, "per_tensor_calls": per_tensor,
                   "copy_gbs": copy_gbs},
        "roofline": {"bound": "hbm", "achieved": gbs10, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs10 / PEAK_HBM_GBS, "traffic": traffic},
        "cpu_baseline": baseline}), flush=True)


def time_factored_per_tensor(ps, states, grads, hp, ws, stream, step, steps):
    """Per-hook granularity of the factored step: one call per tensor, one
    workspace (sized for the largest single-tensor call) shared by all calls."""
    import torch
    recs_one = [ps.make_records([st], [g]) for st, g in zip(states, grads)]
    need = max(ps.factored_workspace_size(None, records=r) for r in recs_one)
    if need > ws.numel():
        ws = torch.empty(need, dtype=torch.uint8, device=ws.device)
    for r in recs_one:
        step += 1
        ps.factored_step(None, None, hp, step, workspace=ws, stream=stream, records=r)
    torch.cuda.synchronize()
    a1, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    issue = 0.0
    t0 = time.perf_counter()
    a1.record(stream)
    for _ in range(steps):
        step += 1
        t1 = time.perf_counter()
        for r in recs_one:
            ps.factored_step(None, None, hp, step, workspace=ws, stream=stream, records=r)
        issue += time.perf_counter() - t1
    b1.record(stream)
    torch.cuda.synchronize()
    res = {"wall_ms": (time.perf_counter() - t0) * 1e3 / steps, "gpu_ms": a1.elapsed_time(b1) / steps,
           "issue_ms": issue * 1e3 / steps}
    log(f"[bench] factored, one call per tensor: {res}")
    return res


def bench_per_tensor(args):
    """Per-hook granularity: the pages step each parameter inside its gradient
    hook, one call per tensor. Same set, slab layout and NAdam step as the
    headline, but each step is one ps_opt_step_multi call per tensor (records
    built once, as a hook would keep them). Also times the single launch over
    all tensors on the same state, and back-to-back single calls on small
    tensors (host issue time and GPU time per call)."""
    import torch

    import precision_state_amd as ps
    import synth
    dev = "cuda:0"
    shapes = synth.WORKLOADS[args.workload]()
    n_params = synth.total_params(shapes)
    states, grads, _ = build_state(shapes, args.seed, dev, "slab")
    n_small = n_final = 0
    if args.policy:   # flagged tensors go through the device table cache, one table per tensor
        n_small, n_final = apply_policy(shapes, states, grads, dev)
    recs_one = [ps.make_records([st], [g]) for st, g in zip(states, grads)]
    recs_all = ps.make_records(states, grads)
    hp = ps.HParams(algo=ps.ALGO_NADAM, lr=3.5e-6)
    stream = torch.cuda.current_stream()
    step = 0

    def per_tensor_step():
        nonlocal step
        step += 1
        for r in recs_one:
            ps.opt_step_multi(None, None, hp, step, stream=stream, records=r)

    def one_launch():
        nonlocal step
        step += 1
        ps.opt_step_multi(None, None, hp, step, stream=stream, records=recs_all)

    for _ in range(args.warmup):
        one_launch()
    per_tensor_step()
    torch.cuda.synchronize()
    res = {}
    for name, fn in (("per_tensor", per_tensor_step), ("one_launch", one_launch)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        issue = 0.0
        t0 = time.perf_counter()
        a.record(stream)
        for _ in range(args.steps):
            t1 = time.perf_counter()
            fn()
            issue += time.perf_counter() - t1
        b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        res[name] = {"wall_ms": wall * 1e3 / args.steps, "gpu_ms": a.elapsed_time(b) / args.steps,
                     "issue_ms": issue * 1e3 / args.steps}
        log(f"[bench] {name}: {res[name]}")
    clocks = gpu_clocks()
    # back-to-back calls on single small tensors
    lat = {}
    for n in (4096, 65536, 3072 * 3072):
        st, g, _ = build_state([synth.Shape("t", 0, 0, n)], args.seed, dev, "slab")
        r = ps.make_records(st, g)
        calls = 400
        for k in range(20):
            ps.opt_step_multi(None, None, hp, k + 1, stream=stream, records=r)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record(stream)
        for k in range(calls):
            ps.opt_step_multi(None, None, hp, k + 21, stream=stream, records=r)
        t_issue = time.perf_counter() - t0
        b.record(stream)
        torch.cuda.synchronize()
        lat[n] = {"host_us_per_call": t_issue * 1e6 / calls, "gpu_us_per_call": a.elapsed_time(b) * 1e3 / calls}
        log(f"[bench] {n} elements, {calls} back-to-back calls: {lat[n]}")
        del st, g
    # the binding's own cost per call: an empty list returns after validation
    empty = ps.make_records([], [])
    t0 = time.perf_counter()
    for k in range(2000):
        ps.opt_step_multi(None, None, hp, 1, stream=stream, records=empty)
    lat["empty_list"] = {"host_us_per_call": (time.perf_counter() - t0) * 1e6 / 2000}
    log(f"[bench] empty list (binding + validation only): {lat['empty_list']}")
    pt = res["per_tensor"]
    # the same bytes as the single launch: the roofline of the per-tensor calls' GPU time
    alg = sum(step_bytes(sh.numel, st.flags) for sh, st in zip(shapes, states))
    gbs = alg / (pt["gpu_ms"] * 1e-3) / 1e9
    baseline = None
    if not args.no_cpu_baseline:   # the same NAdam step as the headline's, so the same oracle sample
        log("[bench] timing the oracle on the host (cpu_baseline)")
        baseline = cpu_baseline(shapes, args.seed)
    print(json.dumps({
        "metric": "per-hook optimizer step: params/sec with one call per tensor (FLUX-12B set)",
        "value": n_params / (pt["wall_ms"] * 1e-3), "unit": "params/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": pt["wall_ms"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload + "_per_tensor", "params": n_params, "calls_per_step": len(shapes),
                   "gpu_clocks_after_timing": clocks,
                   "policy": {"fp32_moment_tensors": n_small, "fp32_param_tensors": n_final} if args.policy else None,
                   "per_tensor": pt, "one_launch": res["one_launch"],
                   "per_tensor_over_one_launch": pt["wall_ms"] / res["one_launch"]["wall_ms"],
                   "small_tensor_calls": {str(k): v for k, v in lat.items()}, "algorithmic_bytes": alg},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": None},
        "cpu_baseline": baseline}), flush=True)


def pcie_ceiling(dev, nbytes=2 << 30):
    """Pinned host <-> device copy rates: both directions at once, then each
    alone (hipMemcpyAsync of 2 GiB, best of a few). Each direction runs on a
    stream created with a CU mask, which gets a hardware queue of its own: on
    a shared queue (HIP's pool of GPU_MAX_HW_QUEUES, 4 by default) the two
    copies would run one after the other, as the offload pipeline's did before
    its copy streams got queues of their own."""
    import ctypes

    import torch
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32, ctypes.c_void_p]
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    hip.hipStreamSynchronize.argtypes = [ctypes.c_void_p]
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(torch.device(dev)).multi_processor_count
    words = (cus + 31) // 32
    mask = (ctypes.c_uint32 * words)(*([0xFFFFFFFF] * words))
    streams = []
    for _ in range(2):
        s = ctypes.c_void_p()
        if hip.hipExtStreamCreateWithCUMask(ctypes.byref(s), words, mask) != 0:
            raise RuntimeError("hipExtStreamCreateWithCUMask failed")
        streams.append(s)
    h = [torch.empty(nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
    d = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(2)]
    torch.cuda.synchronize()
    H2D, D2H = 1, 2

    def copy(k, kind):
        dst, src = (d[k], h[k]) if kind == H2D else (h[k], d[k])
        if hip.hipMemcpyAsync(dst.data_ptr(), src.data_ptr(), nbytes, kind, streams[k]) != 0:
            raise RuntimeError("hipMemcpyAsync failed")

    def timed(ops):
        t0 = time.perf_counter()
        for k, kind in ops:
            copy(k, kind)
        for k, _ in ops:
            hip.hipStreamSynchronize(streams[k])
        return time.perf_counter() - t0
    # both directions at once first: once each stream had copied alone, its
    # later copies in the two directions ran one after the other (28.7 + 28.7
    # GB/s against 48.7 + 48.7 timed first, same box)
    t_dup = min(timed([(0, H2D), (1, D2H)]) for _ in range(3))
    t_h2d = min(timed([(0, H2D)]) for _ in range(2))
    t_d2h = min(timed([(1, D2H)]) for _ in range(2))
    for s in streams:
        hip.hipStreamDestroy(s)
    return {"h2d": nbytes / t_h2d / 1e9, "d2h": nbytes / t_d2h / 1e9, "dup_h2d": nbytes / t_dup / 1e9,
            "dup_d2h": nbytes / t_dup / 1e9}


def bench_offload(args, n_blocks=57):
    """Host offload: the FLUX double-block tensor set repeated 57 times; each
    block's bf16 weights and gradients in HBM, its residuals, codes and scales
    in pinned host memory, moved over PCIe every step by ps_offload_run (the
    step kernel on the host arrays in place, or the staged pipeline). To bound pinned memory, the 57 blocks cycle
    over --host-blocks distinct host state sets (block k uses set k mod H);
    the pipeline's ordering makes this race-free and the bytes moved are the
    same as with 57 distinct sets."""
    import torch

    import precision_state_amd as ps
    import synth
    dev = "cuda:0"
    # The copy ceiling first, before the state's pinned buffers exist: measured
    # after them, on some boxes the two directions of the probe ran one after
    # the other while the pipeline's overlapped.
    pcie = pcie_ceiling(dev)
    log(f"[bench] pinned-copy ceiling: H2D {pcie['h2d']:.1f} GB/s, D2H {pcie['d2h']:.1f} GB/s, "
        f"both at once {pcie['dup_h2d']:.1f} + {pcie['dup_d2h']:.1f} GB/s")
    shapes = synth.WORKLOADS["flux_double_block"]()
    numels = [s.numel for s in shapes]
    H = max(1, min(args.host_blocks, n_blocks))
    host_sets = [ps.StateSlab(numels, dev, with_grads=False, host_state=True) for _ in range(H)]
    for h, hs in enumerate(host_sets):      # filled on the host: no copies before the timed runs
        for tid, st in enumerate(hs.states):
            st.w_lo.numpy()[:] = synth.host_u16_uniform(st.numel, args.seed, synth.STREAM_LO, 1000 * h + tid,
                                                        0).view("int16")
    groups = []
    for k in range(n_blocks):
        hs = host_sets[k % H]
        hi = torch.empty(sum(numels), dtype=torch.int16, device=dev)
        g = torch.empty_like(hi)
        synth.dev_bf16_normal(hi, args.seed, synth.STREAM_HI, k, 0, synth.SIGMA_W)
        synth.dev_bf16_normal(g, args.seed, synth.STREAM_GRAD, k, 1, synth.SIGMA_G)
        sts, gs, o = [], [], 0
        for st in hs.states:
            n = st.numel
            sts.append(ps.TensorState(hi[o:o + n], st.w_lo, st.m_code, st.m_scale, st.v_code, st.v_scale))
            gs.append(g[o:o + n])
            o += n
        groups.append((sts, gs))
    # device views must stay 16-byte aligned: all FLUX double-block sizes are multiples of 8
    torch.cuda.synchronize()
    mode = {"direct": ps.OFFLOAD_DIRECT, "staged": ps.OFFLOAD_STAGED}[args.offload_mode]
    plan = ps.OffloadPlan(groups, mode, args.offload_cus)
    n_params = n_blocks * synth.total_params(shapes)
    sr = args.split == "stochastic"
    hp = ps.HParams(algo=ps.ALGO_NADAM, lr=3.5e-6, split_mode=ps.SPLIT_STOCHASTIC if sr else ps.SPLIT_TRUNC,
                    seed=args.seed)
    stream = torch.cuda.current_stream()
    step = 0
    for _ in range(args.warmup):
        step += 1
        plan.run(hp, step, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step += 1
        plan.run(hp, step, stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    clocks = gpu_clocks()
    h2d, d2h = plan.bytes()       # of the last run (no residuals under stochastic rounding)
    log(f"[bench] offload ({args.offload_mode}): {n_blocks} blocks, {wall * 1e3:.1f} ms/step, PCIe {h2d / wall / 1e9:.1f} GB/s up + "
        f"{d2h / wall / 1e9:.1f} GB/s down")
    baseline = None
    if not args.no_cpu_baseline:   # the offloaded step is the resident NAdam step: the same oracle on one block
        log("[bench] timing the oracle on the host (cpu_baseline)")
        baseline = cpu_baseline(shapes, args.seed)
    print(json.dumps({
        "metric": "offloaded optimizer-updated params/sec (host-resident residuals and moments over PCIe)",
        "value": n_params / wall, "unit": "params/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"flux_double_block_x{n_blocks}_offload", "params": n_params, "split": args.split,
                   "offload_mode": args.offload_mode, "gpu_clocks_after_timing": clocks,
                   "offload_cus": args.offload_cus if args.offload_mode == "direct" else None,
                   "host_state_sets": H, "pcie_h2d_gbs": h2d / wall / 1e9, "pcie_d2h_gbs": d2h / wall / 1e9,
                   "pcie_total_gbs": (h2d + d2h) / wall / 1e9, "h2d_bytes_per_step": h2d,
                   "hbm_gbs_kernel_18B": (14 if sr else 18) * n_params / wall / 1e9,
                   "pinned_copy_ceiling_gbs": pcie,
                   "frac_of_duplex_ceiling": min(h2d, d2h) / wall / 1e9 / pcie["dup_h2d"]},
        "roofline": {"bound": "pcie", "achieved": (h2d + d2h) / wall / 1e9, "peak": 128.0, "unit": "GB/s",
                     "frac": (h2d + d2h) / wall / 1e9 / 128.0, "traffic": None},
        "cpu_baseline": baseline}), flush=True)
    plan.close()


def bench_elementwise(args):
    """The standalone kernels: residual split and join (8 B/elem each: fp32 <-> two 16-bit halves) and
    moment encode and decode (6 B/elem + 4 B per 256-block: fp32 <-> uint16 codes + scales), both modes
    or kinds, on one array of --elements values (default 2^30: a 4 GiB fp32 array)."""
    import torch

    import precision_state_amd as ps
    import synth
    dev = "cuda:0"
    n = args.elements
    nb = (n + 255) // 256
    hi = torch.empty(n, dtype=torch.int16, device=dev)
    lo = torch.empty(n, dtype=torch.int16, device=dev)
    synth.dev_bf16_normal(hi, args.seed, synth.STREAM_HI, 0, 0, synth.SIGMA_W)
    synth.dev_u16_uniform(lo, args.seed, synth.STREAM_LO, 0, 0)
    w32 = torch.empty(n, dtype=torch.float32, device=dev)
    ps.join(hi, lo, w32)
    m32 = w32 * 1e-3                     # moment-like values of both signs
    v32 = m32 * m32
    code = torch.empty(n, dtype=torch.int16, device=dev)
    scale = torch.empty(nb, dtype=torch.float32, device=dev)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    cases = [
        ("split_trunc", lambda: ps.split(w32, hi, lo, ps.SPLIT_TRUNC, stream=stream), 8 * n),
        ("join_trunc", lambda: ps.join(hi, lo, out, ps.SPLIT_TRUNC, stream=stream), 8 * n),
        ("split_nearest_away", lambda: ps.split(w32, hi, lo, ps.SPLIT_NEAREST_AWAY, stream=stream), 8 * n),
        ("join_nearest_away", lambda: ps.join(hi, lo, out, ps.SPLIT_NEAREST_AWAY, stream=stream), 8 * n),
        ("encode_signed", lambda: ps.encode_moments(m32, code, scale, ps.MOMENT_SIGNED, stream=stream), 6 * n + 4 * nb),
        ("decode_signed", lambda: ps.decode_moments(code, scale, out, ps.MOMENT_SIGNED, stream=stream), 6 * n + 4 * nb),
        ("encode_unsigned", lambda: ps.encode_moments(v32, code, scale, ps.MOMENT_UNSIGNED, stream=stream), 6 * n + 4 * nb),
        ("decode_unsigned", lambda: ps.decode_moments(code, scale, out, ps.MOMENT_UNSIGNED, stream=stream), 6 * n + 4 * nb),
    ]
    res = {}
    tot_bytes = tot_ms = 0.0
    for name, fn, nbytes in cases:
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / args.steps
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"ms": ms, "bytes": nbytes, "gbs": gbs, "frac": gbs / PEAK_HBM_GBS}
        tot_bytes += nbytes
        tot_ms += ms
        log(f"[bench] {name}: {ms:.3f} ms, {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS:.3f} of 8 TB/s)")
    clocks = gpu_clocks()
    ceil = ew_ceiling(n, {"split": (w32, None, hi, lo), "join": (hi, lo, out, None),
                          "encode": (m32, None, code, scale), "decode": (code, scale, out, None)},
                      args.steps, stream)
    if ceil:
        for name, r in res.items():
            c = ceil[name.split("_")[0]]
            r["practical_peak_gbs"] = r["bytes"] / (c["ms"] * 1e-3) / 1e9
            r["frac_of_practical"] = c["ms"] / r["ms"]
    worst = min(res, key=lambda k: res[k]["gbs"])
    baseline = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host (cpu_baseline)")
        baseline = cpu_baseline_elementwise(args.seed)
        log(f"[bench] cpu_baseline: {baseline}")
    print(json.dumps({
        "metric": "standalone split/join/encode/decode: algorithmic HBM GB/s over the eight kernels",
        "value": tot_bytes / (tot_ms * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": tot_ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"elementwise_{n}", "elements": n, "kernels": res, "gpu_clocks_after_timing": clocks},
        "roofline": {"bound": "hbm", "achieved": res[worst]["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": res[worst]["frac"], "traffic": None, "kernel": worst},
        "cpu_baseline": baseline}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default 30, offload mode 1): the GPU needs about a second of "
                         "this load to reach steady clocks")
    ap.add_argument("--workload", default="flux_dev_12b",
                    choices=["flux_dev_12b", "flux_double_block", "single_1024x3072"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--layout", default="slab", choices=["slab", "separate"],
                    help="state in one contiguous allocation per stream (slab) or one per tensor")
    ap.add_argument("--host-blocks", type=int, default=4,
                    help="offload mode: distinct pinned host state sets, reused cyclically by the 57 blocks")
    ap.add_argument("--elements", type=int, default=1 << 30,
                    help="elementwise mode: array length")
    ap.add_argument("--mode", default="nadam", choices=["nadam", "factored", "offload", "per_tensor", "elementwise"],
                    help="nadam: the fused (N)AdamW step (headline); factored: the Adafactor-style step "
                         "(factored second moment, update clipping; --beta1, --decay-rate) on the double-block "
                         "shapes; offload: host-resident state over PCIe; per_tensor: one call per tensor, as a "
                         "gradient hook would step; elementwise: the standalone split/join/encode/decode kernels")
    ap.add_argument("--offload-mode", default="direct", choices=["direct", "staged"],
                    help="offload mode: the step kernel on the host arrays in place over PCIe (direct) or copies "
                         "through two device staging slots (staged)")
    ap.add_argument("--offload-cus", type=int, default=8,
                    help="offload mode direct: compute units the step kernels may use (0 = all)")
    ap.add_argument("--per-tensor-calls", action="store_true",
                    help="factored mode: also time one call per tensor (the per-hook granularity)")
    ap.add_argument("--policy", action="store_true",
                    help="nadam mode: fp32 moments for tensors of <= 4096 elements and an fp32 final layer "
                         "(PS_TENSOR_FP32_MOMENTS / PS_TENSOR_FP32_PARAM)")
    ap.add_argument("--moments", default="codec", choices=["codec", "f24"],
                    help="nadam mode: moment storage, uint16 codes + per-256 scales (codec) or the upper three "
                         "bytes of fp32 (f24, PS_TENSOR_F24_MOMENTS)")
    ap.add_argument("--split", default="trunc", choices=["trunc", "nearest_away", "stochastic"],
                    help="nadam mode: residual split mode; stochastic = stochastic rounding to bf16 with no "
                         "residual (PS_SPLIT_STOCHASTIC, 14 B/param)")
    ap.add_argument("--weight-decay", type=float, default=0.0,
                    help="nadam mode: decoupled weight decay (0.01 makes it the NAdamW step of the double-block "
                         "workload's parity tests)")
    ap.add_argument("--beta1", type=float, default=0.0,
                    help="factored mode: first moment of the clipped update (0 = none)")
    ap.add_argument("--decay-rate", type=float, default=0.0,
                    help="factored mode: beta2 of update t is 1 - t^decay_rate (0 = constant 0.999)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="nadam mode: skip the streaming-ceiling kernels timed after the step")
    ap.add_argument("--calibrate-copy", type=float, default=0.0, metavar="GIB",
                    help="after the timed steps, run 3 plain device copies of GIB GiB (counter calibration "
                         "and the practical copy bandwidth)")
    args = ap.parse_args()
    if args.warmup is None:
        args.warmup = 1 if args.mode == "offload" else 30

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only (the optimizer step has no cross-GPU "
              "communication here); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import precision_state_amd as ps
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.mode == "factored":
        return bench_factored(args)
    if args.mode == "offload":
        return bench_offload(args)
    if args.mode == "per_tensor":
        return bench_per_tensor(args)
    if args.mode == "elementwise":
        return bench_elementwise(args)
    shapes = synth.WORKLOADS[args.workload]()
    n_params = synth.total_params(shapes)
    log(f"[bench] {args.workload}: {len(shapes)} tensors, {n_params} params; generating state on {dev}")
    t0 = time.perf_counter()
    states, grads, slab = build_state(shapes, args.seed, dev, args.layout, args.moments)
    torch.cuda.synchronize()
    log(f"[bench] state ready in {time.perf_counter() - t0:.1f} s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated)")

    split = {"trunc": ps.SPLIT_TRUNC, "nearest_away": ps.SPLIT_NEAREST_AWAY,
             "stochastic": ps.SPLIT_STOCHASTIC}[args.split]
    hp = ps.HParams(algo=ps.ALGO_NADAM, lr=3.5e-6, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=args.weight_decay,
                    split_mode=split, seed=args.seed)
    n_small = n_final = 0
    if args.policy:
        n_small, n_final = apply_policy(shapes, states, grads, dev)
    recs = ps.make_records(states, grads)
    stream = torch.cuda.current_stream()
    step = 0
    wev = []
    for _ in range(args.warmup):
        step += 1
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        ps.opt_step_multi(None, None, hp, step, stream=stream, records=recs)
        b.record(stream)
        wev.append((a, b))
    torch.cuda.synchronize()
    wt = [a.elapsed_time(b) for a, b in wev]
    log(f"[bench] warmup {args.warmup} done" + (f": first {wt[0]:.3f} ms, last {wt[-1]:.3f} ms" if wt else ""))

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step += 1
        ev[k][0].record(stream)
        ps.opt_step_multi(None, None, hp, step, stream=stream, records=recs)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = [a.elapsed_time(b) for a, b in ev]
    kernel_ms = sum(per_step) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    log(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step wall, {kernel_ms:.3f} ms/launch (events); "
        f"per launch min {min(per_step):.3f} max {max(per_step):.3f}")

    copy_gbs = calibrate_copy(args.calibrate_copy, stream, dev)

    alg_bytes = sum(step_bytes(s.numel, st.flags, split != ps.SPLIT_STOCHASTIC) for s, st in zip(shapes, states))
    achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9
    traffic = None if args.policy else read_traffic(args.workload, args.moments, args.split)
    clocks = gpu_clocks()
    ceiling = None
    if not args.no_ceiling and not args.policy and args.moments == "codec":
        ceiling = stream_ceiling(slab, max(5, min(args.steps, 20)), stream, stochastic=args.split == "stochastic")

    baseline = None
    if not args.no_cpu_baseline:
        del states, grads, recs
        torch.cuda.empty_cache()
        log("[bench] timing the oracle on the host (cpu_baseline)")
        baseline = cpu_baseline(shapes, args.seed, weight_decay=args.weight_decay)
        log(f"[bench] oracle: {baseline['value']:.3e} params/s ({baseline['sample']})")

    out = {
        "metric": METRIC,
        "value": n_params * args.steps / wall,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "params": n_params, "tensors": len(shapes),
                   "algo": "nadam", "lr": 3.5e-6, "weight_decay": args.weight_decay, "layout": args.layout,
                   "policy": {"fp32_moment_tensors": n_small, "fp32_param_tensors": n_final} if args.policy else None,
                   "moments": args.moments, "split": args.split,
                   "state": ("bf16 weight (stochastic rounding, no residual)" if args.split == "stochastic"
                             else "bf16 weight + u16 residual") + " + bf16 grad + " +
                            ("u16 m/v codes + fp32 per-256 scales" if args.moments == "codec" else
                             "f24 m/v (upper 3 bytes of fp32)"),
                   "kernel_ms": kernel_ms, "copy_gbs": copy_gbs, "kernel_source_sha256": kernel_source_hash(),
                   "gbs_18B_per_param": 18 * n_params / (kernel_ms * 1e-3) / 1e9,
                   "bytes_per_param_algorithmic": alg_bytes / n_params,
                   "gpu_clocks_after_timing": clocks, "stream_ceiling": ceiling},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "practical_peak": ceiling["step_mix"]["gbs"] if ceiling else None,
                     "frac_of_practical": achieved / ceiling["step_mix"]["gbs"] if ceiling else None},
        "cpu_baseline": baseline,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
