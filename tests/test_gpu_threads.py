"""Calls from several host threads at once, each on its own stream: the
library keeps per-thread argument buffers and a locked device table cache, so
concurrent (N)AdamW and factored steps over distinct tensors must give exactly
the bytes of the same calls made one after another on one stream."""
import threading

import pytest

from gpu_util import DEV, dev_grad, dev_state

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import precision_state_amd as ps  # noqa: E402

SIZES = [5000, 257, 1, 65536, 1024, 3000, 131089, 4096, 100, 255, 256, 70000, 8, 9, 1023, 1025, 20000, 4097]
# the last shape puts 16384 rows of 512 columns in each list, so every list
# runs the row-strip statistics pass as well as the tiles of the others
SHAPES2D = [(64, 96), (3, 1000), (128, 256), (17, 40), (16384, 512)]
STEPS = 3
THREADS = 4


def _adam_set(tid):
    sts = []
    for i, n in enumerate(SIZES):
        st = dev_state(n, 90 + tid, i)
        if i % 3 == 0:                               # flagged tensors take the cached-table kernel
            st.m_code = torch.zeros(n, dtype=torch.float32, device=DEV)
            st.v_code = torch.zeros(n, dtype=torch.float32, device=DEV)
            st.m_scale = st.v_scale = None
            st.flags = ps.TENSOR_FP32_MOMENTS
        sts.append(st)
    grads = [[dev_grad(n, 90 + tid, i, t) for i, n in enumerate(SIZES)] for t in range(1, STEPS + 1)]
    return sts, grads


def _fact_set(tid):
    sts = [dev_state(r * c, 70 + tid, i, r, c, factored=True) for i, (r, c) in enumerate(SHAPES2D)]
    sts.append(dev_state(3333, 70 + tid, 9, factored=True))
    grads = [[dev_grad(s.numel, 70 + tid, i, t) for i, s in enumerate(sts)] for t in range(1, STEPS + 1)]
    ws = torch.empty(max(ps.factored_workspace_size(sts, grads[0]), 256), dtype=torch.uint8, device=DEV)
    return sts, grads, ws


def _fields(st):
    return [x for x in (st.w_hi, st.w_lo, st.m_code, st.m_scale, st.v_code, st.v_scale, st.row_ema, st.col_ema)
            if x is not None]


def _clone(sts):
    out = []
    for st in sts:
        c = ps.TensorState(*[None if x is None else x.clone() for x in
                             (st.w_hi, st.w_lo, st.m_code, st.m_scale, st.v_code, st.v_scale, st.row_ema,
                              st.col_ema)], rows=st.rows, cols=st.cols, flags=st.flags)
        out.append(c)
    return out


def _work(a_sts, a_grads, f_sts, f_grads, ws, stream):
    hp = ps.HParams(algo=ps.ALGO_NADAM, lr=1e-3, weight_decay=0.01)
    fhp = ps.FactoredHParams(lr=1e-3, decay_rate=-0.8, beta1=0.9)
    for t in range(1, STEPS + 1):
        ps.opt_step_multi(a_sts, a_grads[t - 1], hp, t, stream=stream)
        ps.factored_step(f_sts, f_grads[t - 1], fhp, t, workspace=ws, stream=stream)


def test_concurrent_threads_equal_sequential_calls():
    sets = []
    for tid in range(THREADS):
        a_sts, a_grads = _adam_set(tid)
        f_sts, f_grads, ws = _fact_set(tid)
        sets.append((a_sts, a_grads, f_sts, f_grads, ws))
    refs = [(_clone(a), _clone(f), torch.empty_like(ws)) for a, _, f, _, ws in sets]
    torch.cuda.synchronize()
    # reference: the same calls one after another on the current stream
    for (a_ref, f_ref, ws_ref), (_, a_grads, _, f_grads, _) in zip(refs, sets):
        _work(a_ref, a_grads, f_ref, f_grads, ws_ref, torch.cuda.current_stream())
    torch.cuda.synchronize()
    print("  sequential reference done", flush=True)
    streams = [torch.cuda.Stream() for _ in range(THREADS)]
    errors = []

    def run(k):
        try:
            a_sts, a_grads, f_sts, f_grads, ws = sets[k]
            _work(a_sts, a_grads, f_sts, f_grads, ws, streams[k])
        except Exception as e:          # reported after the join
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=run, args=(k,)) for k in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    torch.cuda.synchronize()
    print("  concurrent run done", flush=True)
    assert not errors, errors
    for k, ((a_sts, _, f_sts, _, _), (a_ref, f_ref, _)) in enumerate(zip(sets, refs)):
        for i, (x, y) in enumerate(zip(a_sts + f_sts, a_ref + f_ref)):
            for fx, fy in zip(_fields(x), _fields(y)):
                assert torch.equal(fx, fy), (k, i)
