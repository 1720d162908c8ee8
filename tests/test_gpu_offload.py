"""The host-offload pipeline (sd-scripts PR #2187 '(N)AdamW / Adan with fused
backwards pass & CPU offloading', opening post: state offloaded to host memory
between steps) must give exactly the bytes of the device-resident step."""
import numpy as np
import pytest

import synth
from gpu_util import DEV

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


@pytest.mark.parametrize("split_mode", [ps.SPLIT_TRUNC, ps.SPLIT_NEAREST_AWAY])
def test_offload_equals_resident_bitwise(split_mode):
    slabs = [ps.StateSlab(sizes, DEV, host_state=True) for sizes in GROUPS]
    for gid, sl in enumerate(slabs):
        _fill(sl, gid)
    torch.cuda.synchronize()
    resident = [_resident_copy(sl) for sl in slabs]
    hp = ps.HParams(algo=ps.ALGO_NADAM, lr=1e-4, weight_decay=0.01, split_mode=split_mode)
    grads = [[None if (gid == 1 and i == 1) else g for i, g in enumerate(sl.grads)] for gid, sl in enumerate(slabs)]
    plan = ps.OffloadPlan([(sl.states, grads[gid]) for gid, sl in enumerate(slabs)])
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


def test_offload_stochastic_rounding_moves_no_residual_and_equals_resident():
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
    plan = ps.OffloadPlan([(sl.states, sl.grads) for sl in slabs])
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
