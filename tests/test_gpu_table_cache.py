"""Per-tensor calls through the device table cache. A fused backward pass
(sd-scripts commit 7983d3d 'Fused backward pass': the optimizer steps each
parameter from its gradient hook) calls the library once per tensor, so a
model brings hundreds of distinct tensor tables; these tests check that such
calls give exactly the bytes of one call over the whole list, and that results
stay exact across the point where the cache is emptied and refilled."""
import numpy as np
import pytest

import oracle
from gpu_util import DEV, compare_factored, dev_grad, dev_state, host_grad, host_state, ofhp, ohp, u16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import precision_state_amd as ps  # noqa: E402

N_TENSORS = 100


def _shapes():
    out = []
    for i in range(N_TENSORS):
        if i % 3 == 0:
            out.append((100 + 37 * i, 0, 0))
        else:
            r, c = 3 + i % 7, 8 * (5 + i % 11)
            out.append((r * c, r, c))
    return out


def _fields(st):
    return [x for x in (st.w_hi, st.w_lo, st.m_code, st.m_scale, st.v_code, st.v_scale, st.row_ema, st.col_ema)
            if x is not None]


def test_per_tensor_factored_calls_equal_one_list_call():
    shapes = _shapes()
    a = [dev_state(n, 31, i, r, c, factored=True) for i, (n, r, c) in enumerate(shapes)]
    b = [dev_state(n, 31, i, r, c, factored=True) for i, (n, r, c) in enumerate(shapes)]
    hp = ps.FactoredHParams(lr=1e-3, weight_decay=0.01, decay_rate=-0.8, beta1=0.9)
    ws_one = ws_all = None
    for t in range(1, 4):
        g = [dev_grad(n, 31, i, t) for i, (n, _, _) in enumerate(shapes)]
        if ws_one is None:
            need = max(ps.factored_workspace_size(a, g), 256)
            ws_one = torch.empty(need, dtype=torch.uint8, device=DEV)   # reused by every per-tensor call
            ws_all = torch.empty(need, dtype=torch.uint8, device=DEV)
        for st, gi in zip(a, g):
            ps.factored_step([st], [gi], hp, t, workspace=ws_one)
        ps.factored_step(b, g, hp, t, workspace=ws_all)
        print(f"  step {t} done", flush=True)
    torch.cuda.synchronize()
    for i, (x, y) in enumerate(zip(a, b)):
        for fx, fy in zip(_fields(x), _fields(y)):
            assert torch.equal(fx, fy), (i, shapes[i])
    # and both against the oracle, tensor by tensor
    for i, (n, r, c) in enumerate(shapes):
        h = host_state(n, 31, i, r, factored=True, cols=c)
        for t in range(1, 4):
            oracle.factored_step(h, host_grad(n, 31, i, t), r, c, ofhp(hp), t)
        compare_factored(a[i], h, r, (i, shapes[i]), first_moment=True)


def _flagged_state(numel, tid, seed=47):
    st = dev_state(numel, seed, tid)
    st.m_code = torch.zeros(numel, dtype=torch.float32, device=DEV)
    st.v_code = torch.zeros(numel, dtype=torch.float32, device=DEV)
    st.m_scale = st.v_scale = None
    st.flags = ps.TENSOR_FP32_MOMENTS
    return st


def test_per_tensor_flagged_calls_equal_one_list_call():
    shapes = _shapes()
    a = [_flagged_state(n, i) for i, (n, _, _) in enumerate(shapes)]
    b = [_flagged_state(n, i) for i, (n, _, _) in enumerate(shapes)]
    hp = ps.HParams(algo=ps.ALGO_NADAM, lr=1e-3, weight_decay=0.01)
    for t in range(1, 4):
        g = [dev_grad(n, 47, i, t) for i, (n, _, _) in enumerate(shapes)]
        for st, gi in zip(a, g):
            ps.opt_step_multi([st], [gi], hp, t)
        ps.opt_step_multi(b, g, hp, t)
    torch.cuda.synchronize()
    for i, (x, y) in enumerate(zip(a, b)):
        for fx, fy in zip(_fields(x), _fields(y)):
            assert torch.equal(fx, fy), (i, shapes[i])


def test_results_stay_exact_across_a_cache_flush():
    """More distinct tensor tables than the cache holds (16384 per device):
    each call steps prefixes of two flagged tensors, with every (prefix,
    prefix) pair distinct, and the final state must equal the oracle's replay
    of the same calls."""
    n0, n1, calls = 128, 160, 16384 + 256
    s0, s1 = _flagged_state(n0, 0), _flagged_state(n1, 1)
    g0, g1 = dev_grad(n0, 47, 0, 1), dev_grad(n1, 47, 1, 1)
    host = []
    for st, g in ((s0, g0), (s1, g1)):
        host.append([u16(st.w_hi).copy(), u16(st.w_lo).copy(), u16(g).copy(), np.zeros(st.numel, np.float32),
                     np.zeros(st.numel, np.float32)])
    hp = ps.HParams(algo=ps.ALGO_NADAM, lr=1e-3, weight_decay=0.01)
    for k in range(calls):
        a, b, t = 1 + k % n0, 1 + (k // n0) % n1, 1 + k % 5
        views = [ps.TensorState(s.w_hi[:m], s.w_lo[:m], s.m_code[:m], None, s.v_code[:m], None,
                                flags=ps.TENSOR_FP32_MOMENTS) for s, m in ((s0, a), (s1, b))]
        ps.opt_step_multi(views, [g0[:a], g1[:b]], hp, t)
        for tid, m in ((0, a), (1, b)):
            w, lo, g, mm, vv = host[tid]
            oracle.opt_step_flags(w[:m], lo[:m], g[:m], mm[:m], None, vv[:m], None, oracle.FP32_MOMENTS,
                                  ohp(hp, tid), t)
        if (k + 1) % 4096 == 0:
            print(f"  {k + 1} calls", flush=True)
    torch.cuda.synchronize()
    for tid, st in enumerate((s0, s1)):
        w, lo, _, mm, vv = host[tid]
        assert np.array_equal(u16(st.w_hi), w), tid
        assert np.array_equal(u16(st.w_lo), lo), tid
        assert np.array_equal(st.m_code.cpu().numpy().view(np.uint32), mm.view(np.uint32)), tid
        assert np.array_equal(st.v_code.cpu().numpy().view(np.uint32), vv.view(np.uint32)), tid
