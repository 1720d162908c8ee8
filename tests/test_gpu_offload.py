"""The host-offload pipeline (sd-scripts PR #2187 '(N)AdamW / Adan with fused
backwards pass & CPU offloading', opening post: state offloaded to host memory
between steps) must give exactly the bytes of the device-resident step, and
of the oracle's replay of every tensor."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import DEV, check_sampled_blocks, f32, ohp, u16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import precision_state_amd as ps  # noqa: E402

GROUPS = [[1000, 128, 65536, 64, 300000], [7, 256, 257, 1025], [131072, 3000, 0, 4096, 77]]


def _fill(slab, gid):
    for i, st in enumerate(slab.states):
        tid = 100 * gid + i
        h = torch.empty(st.numel, dtype=torch.int16, device=DEV)
        synth.dev_bf16_normal(st.w_hi, 5, synth.STREAM_HI, tid, 0, synth.SIGMA_W)
        synth.dev_u16_uniform(h, 5, synth.STREAM_LO, tid, 0)
        st.w_lo.copy_(h.cpu() if not st.w_lo.is_cuda else h)


def _resident_copy(slab):
    out = []
    for st in slab.states:
        out.append(ps.TensorState(st.w_hi.clone(), st.w_lo.to(DEV), st.m_code.to(DEV), st.m_scale.to(DEV),
                                  st.v_code.to(DEV), st.v_scale.to(DEV)))
    return out


MODES = [(ps.OFFLOAD_DIRECT, ps.OFFLOAD_DEFAULT_CUS), (ps.OFFLOAD_DIRECT, 3), (ps.OFFLOAD_DIRECT, 0),
         (ps.OFFLOAD_STAGED, 0)]


@pytest.mark.parametrize("mode,cus", MODES)
@pytest.mark.parametrize("split_mode", [ps.SPLIT_TRUNC, ps.SPLIT_NEAREST_AWAY])
def test_offload_equals_resident_bitwise(split_mode, mode, cus):
    slabs = [ps.StateSlab(sizes, DEV, host_state=True) for sizes in GROUPS]
    for gid, sl in enumerate(slabs):
        _fill(sl, gid)
    torch.cuda.synchronize()
    resident = [_resident_copy(sl) for sl in slabs]
    hp = ps.HParams(algo=ps.ALGO_NADAM, lr=1e-4, weight_decay=0.01, split_mode=split_mode)
    grads = [[None if (gid == 1 and i == 1) else g for i, g in enumerate(sl.grads)] for gid, sl in enumerate(slabs)]
    plan = ps.OffloadPlan([(sl.states, grads[gid]) for gid, sl in enumerate(slabs)], mode, cus)
    h2d, d2h = plan.bytes()
    moved = sum(2 * 3 * n + 8 * ((n + 255) // 256) for gid, sizes in enumerate(GROUPS) for i, n in enumerate(sizes)
                if not (gid == 1 and i == 1))
    assert h2d == d2h == moved
    for t in range(1, 4):
        for gid, sl in enumerate(slabs):
            for i, g in enumerate(sl.grads):
                synth.dev_bf16_normal(g, 5, synth.STREAM_GRAD, 100 * gid + i, t, synth.SIGMA_G)
        plan.run(hp, t)
        for gid in range(len(slabs)):
            ps.opt_step_multi(resident[gid], grads[gid], hp, t)
    torch.cuda.synchronize()
    for gid, sl in enumerate(slabs):
        for a, b in zip(sl.states, resident[gid]):
            for k in ("w_hi", "w_lo", "m_code", "m_scale", "v_code", "v_scale"):
                x, y = getattr(a, k).cpu(), getattr(b, k).cpu()
                assert torch.equal(x, y), (gid, a.numel, k)
    plan.close()


@pytest.mark.parametrize("mode", [ps.OFFLOAD_DIRECT, ps.OFFLOAD_STAGED])
def test_offload_stochastic_rounding_moves_no_residual_and_equals_resident(mode):
    """Stochastic rounding through the pipeline (the pages' setting when the
    residual does not fit in host memory): some tensors have no residual at
    all, the run moves only codes and scales, and the bytes equal one resident
    step over the concatenated group lists (whose positions key the random
    streams)."""
    slabs = [ps.StateSlab(sizes, DEV, host_state=True) for sizes in GROUPS]
    for gid, sl in enumerate(slabs):
        _fill(sl, gid)
    torch.cuda.synchronize()
    resident = [_resident_copy(sl) for sl in slabs]
    lo_before = [[st.w_lo.clone() for st in sl.states] for sl in slabs]
    for sl in slabs[1:]:
        sl.states[0].w_lo = None                       # no residual array for these tensors
    hp = ps.HParams(algo=ps.ALGO_NADAM, lr=1e-4, weight_decay=0.01, split_mode=ps.SPLIT_STOCHASTIC, seed=808)
    plan = ps.OffloadPlan([(sl.states, sl.grads) for sl in slabs], mode)
    all_res = [st for group in resident for st in group]
    all_grads = [g for sl in slabs for g in sl.grads]
    for t in range(1, 4):
        for gid, sl in enumerate(slabs):
            for i, g in enumerate(sl.grads):
                synth.dev_bf16_normal(g, 5, synth.STREAM_GRAD, 100 * gid + i, t, synth.SIGMA_G)
        plan.run(hp, t)
        ps.opt_step_multi(all_res, all_grads, hp, t)
    torch.cuda.synchronize()
    h2d, d2h = plan.bytes()
    moved = sum(2 * 2 * n + 8 * ((n + 255) // 256) for sizes in GROUPS for n in sizes)
    assert h2d == d2h == moved
    for gid, sl in enumerate(slabs):
        for i, (a, b) in enumerate(zip(sl.states, resident[gid])):
            for k in ("w_hi", "m_code", "m_scale", "v_code", "v_scale"):
                x, y = getattr(a, k).cpu(), getattr(b, k).cpu()
                assert torch.equal(x, y), (gid, a.numel, k)
            if a.w_lo is not None:
                assert torch.equal(a.w_lo.cpu(), lo_before[gid][i].cpu())   # residuals untouched
    with pytest.raises(ps.PSError):
        plan.run(ps.HParams(algo=ps.ALGO_NADAM), 4)     # a residual mode needs every w_lo
    plan.close()


# ---------------------------------------------------------------------------
# Against the oracle: every tensor of every group regenerated on the host
# from the same seeded recipe and replayed through the oracle's step.
# ---------------------------------------------------------------------------

def _oracle_groups(groups, hp, steps, skip=(), seed=5, tid_of=lambda gid, i, pos: 100 * gid + i):
    """Oracle replay of the offloaded groups. tid_of gives each tensor's
    synthetic-input key; stochastic rounding is keyed by the tensor's position
    in the concatenated group lists, as the pipeline keys it."""
    out, pos = [], 0
    for gid, sizes in enumerate(groups):
        grp = []
        for i, n in enumerate(sizes):
            tid = tid_of(gid, i, pos + i)
            st = oracle.TensorState(synth.host_bf16_normal(n, seed, synth.STREAM_HI, tid, 0, synth.SIGMA_W),
                                    synth.host_u16_uniform(n, seed, synth.STREAM_LO, tid, 0), *oracle.zero_moments(n))
            if (gid, i) not in skip:
                for t in range(1, steps + 1):
                    g = synth.host_bf16_normal(n, seed, synth.STREAM_GRAD, tid, t, synth.SIGMA_G)
                    oracle.opt_step(st, g, ohp(hp, pos + i), t)
            grp.append(st)
        out.append(grp)
        pos += len(sizes)
    return out


@pytest.mark.parametrize("mode", [ps.OFFLOAD_DIRECT, ps.OFFLOAD_STAGED])
@pytest.mark.parametrize("split_mode", [ps.SPLIT_TRUNC, ps.SPLIT_NEAREST_AWAY, ps.SPLIT_STOCHASTIC])
def test_offload_matches_oracle_every_byte(split_mode, mode):
    """Three ragged groups (a tensor without a gradient, an empty tensor), 3
    NAdamW steps through the pipeline; weights, residuals, codes and scales of
    every tensor equal the oracle's replay."""
    slabs = [ps.StateSlab(sizes, DEV, host_state=True) for sizes in GROUPS]
    for gid, sl in enumerate(slabs):
        _fill(sl, gid)
    torch.cuda.synchronize()
    hp = ps.HParams(algo=ps.ALGO_NADAM, lr=1e-4, weight_decay=0.01, split_mode=split_mode, seed=77)
    grads = [[None if (gid == 1 and i == 1) else g for i, g in enumerate(sl.grads)] for gid, sl in enumerate(slabs)]
    plan = ps.OffloadPlan([(sl.states, grads[gid]) for gid, sl in enumerate(slabs)], mode)
    for t in range(1, 4):
        for gid, sl in enumerate(slabs):
            for i, g in enumerate(sl.grads):
                synth.dev_bf16_normal(g, 5, synth.STREAM_GRAD, 100 * gid + i, t, synth.SIGMA_G)
        plan.run(hp, t)
    torch.cuda.synchronize()
    plan.close()
    want = _oracle_groups(GROUPS, hp, 3, skip={(1, 1)})
    for gid, sl in enumerate(slabs):
        for i, (a, h) in enumerate(zip(sl.states, want[gid])):
            got = {"hi": u16(a.w_hi), "lo": u16(a.w_lo), "mc": u16(a.m_code), "vc": u16(a.v_code),
                   "ms": f32(a.m_scale).view(np.uint32), "vs": f32(a.v_scale).view(np.uint32)}
            exp = {"hi": h.hi, "lo": h.lo, "mc": h.mc, "vc": h.vc, "ms": h.ms.view(np.uint32),
                   "vs": h.vs.view(np.uint32)}
            for k in got:
                assert np.array_equal(got[k], exp[k]), (gid, i, a.numel, k)


@pytest.mark.parametrize("mode", [ps.OFFLOAD_DIRECT, ps.OFFLOAD_STAGED])
def test_offload_double_blocks_distinct_host_sets_sampled(mode):
    """Three groups of unequal size built from FLUX double-block shapes (a
    whole block, its first 10 tensors, a whole block plus 5 tensors of
    another), each with its own pinned host state, run for 2 steps so that
    both staging slots are reused (staged mode); sampled 256-blocks of every
    tensor against the oracle (each block evolves from its own inputs only)."""
    blk = synth.WORKLOADS["flux_double_block"]()
    group_shapes = [blk, blk[:10], blk + blk[:5]]
    slabs = [ps.StateSlab([s.numel for s in shapes], DEV, host_state=True) for shapes in group_shapes]
    pos = 0
    all_shapes, all_states = [], []
    for sl, shapes in zip(slabs, group_shapes):
        for i, st in enumerate(sl.states):
            tid = pos + i                      # synthetic key = position in the concatenated list
            h = torch.empty(st.numel, dtype=torch.int16, device=DEV)
            synth.dev_bf16_normal(st.w_hi, 0, synth.STREAM_HI, tid, 0, synth.SIGMA_W)
            synth.dev_u16_uniform(h, 0, synth.STREAM_LO, tid, 0)
            st.w_lo.copy_(h.cpu())
        pos += len(shapes)
        all_shapes += shapes
        all_states += sl.states
    torch.cuda.synchronize()
    hp = ps.HParams(algo=ps.ALGO_NADAM, lr=3.5e-6, weight_decay=0.01)
    plan = ps.OffloadPlan([(sl.states, sl.grads) for sl in slabs], mode)
    for t in range(1, 3):
        pos = 0
        for sl in slabs:
            for i, g in enumerate(sl.grads):
                synth.dev_bf16_normal(g, 0, synth.STREAM_GRAD, pos + i, t, synth.SIGMA_G)
            pos += len(sl.grads)
        plan.run(hp, t)
        print(f"  offload step {t} done", flush=True)
    torch.cuda.synchronize()
    plan.close()
    n = check_sampled_blocks(all_shapes, all_states, hp, 2, 0, 6)
    print(f"  {n} sampled blocks of {len(all_shapes)} tensors exact", flush=True)


def test_offload_plan_rejects_unmapped_host_arrays_and_bad_options():
    """The direct mode takes each host array's device address at plan
    creation: pageable (not pinned) host memory is rejected there, and so are
    unknown modes and negative CU counts."""
    sl = ps.StateSlab([1000], DEV, host_state=True)
    st = sl.states[0]
    pageable = torch.empty(st.numel, dtype=torch.int16)          # not pinned
    bad = ps.TensorState(st.w_hi, pageable, st.m_code, st.m_scale, st.v_code, st.v_scale)
    for mode in (ps.OFFLOAD_DIRECT, ps.OFFLOAD_STAGED):
        with pytest.raises(ps.PSError):
            ps.OffloadPlan([([bad], sl.grads)], mode)
    with pytest.raises(ps.PSError):
        ps.OffloadPlan([(sl.states, sl.grads)], 7)
    with pytest.raises(ps.PSError):
        ps.OffloadPlan([(sl.states, sl.grads)], ps.OFFLOAD_DIRECT, -1)
