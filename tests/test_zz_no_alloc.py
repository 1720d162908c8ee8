"""ps_factored_step_noalloc (the factored step with the library's built-in
scratch instead of a caller workspace, for callers that cannot allocate)
against ps_factored_step on the same inputs: two calls in a row, the second
over a smaller tensor list, so the second runs on scratch the first left
behind. Both use the same kernels, so every byte must agree."""
import pytest

import synth
from gpu_util import DEV, dev_grad, dev_state

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import precision_state_amd as ps  # noqa: E402

SMALL = [synth.Shape("a", 1, 1, 1), synth.Shape("b", 1, 300, 300), synth.Shape("d", 65, 257, 65 * 257),
         synth.Shape("f", 64, 256, 64 * 256), synth.Shape("g", 100, 3000, 300000), synth.Shape("h", 0, 0, 1),
         synth.Shape("j", 0, 0, 257), synth.Shape("k", 0, 0, 5000), synth.Shape("l", 70, 130, 9100)]


def _fields(st):
    return [x for x in (st.w_hi, st.w_lo, st.m_code, st.m_scale, st.v_code, st.v_scale, st.row_ema, st.col_ema)
            if x is not None]


def _one_call(shapes, hp, seed, step):
    a = [dev_state(s.numel, seed, i, s.rows, s.cols, factored=True) for i, s in enumerate(shapes)]
    b = [dev_state(s.numel, seed, i, s.rows, s.cols, factored=True) for i, s in enumerate(shapes)]
    g = [dev_grad(s.numel, seed, i, step, 0.001) for i, s in enumerate(shapes)]
    ws = torch.empty(max(ps.factored_workspace_size(b, g), 256), dtype=torch.uint8, device=DEV)
    for t in range(1, step + 1):
        ps.factored_step_noalloc(a, g, hp, t)
        ps.factored_step(b, g, hp, t, workspace=ws)
    torch.cuda.synchronize()
    for i, (x, y) in enumerate(zip(a, b)):
        for fx, fy in zip(_fields(x), _fields(y)):
            assert torch.equal(fx, fy), (shapes[i].name, i)


def test_noalloc_equals_workspace_call_twice_second_smaller():
    blk = synth.WORKLOADS["flux_double_block"]()
    hp = ps.FactoredHParams(lr=1e-5, weight_decay=0.01, decay_rate=-0.8, beta1=0.9)
    print("  noalloc: FLUX double block (24 tensors), 2 steps", flush=True)
    _one_call(blk, hp, 3, 2)
    hp2 = ps.FactoredHParams(split_mode=ps.SPLIT_STOCHASTIC, lr=1e-4, clip_threshold=2.0, seed=9)
    print("  noalloc: 9 ragged tensors, 2 steps", flush=True)
    _one_call(SMALL, hp2, 4, 2)


def test_noalloc_rejects_a_list_beyond_the_scratch():
    """The records carry placeholder addresses, so the call must be turned away
    on the host: the list's workspace alone is checked to exceed the scratch
    (a host-only size query) before the call is made. A 262144 x 4104 tensor
    takes the statistics tiles, whose row sums alone need 17 x 262144 doubles
    (34 MiB)."""
    blk = synth.WORKLOADS["flux_double_block"]()
    shapes = blk + [synth.Shape("wide", 262144, 4104, 262144 * 4104)]
    recs = (ps.CTensor * len(shapes))()
    for i, s in enumerate(shapes):
        recs[i] = ps.CTensor(256, 256, 256, 256, 256, 256, 256, 256, 256, s.numel, s.rows, s.cols, 0, 0)
    need = ps.factored_workspace_size(None, records=(recs, len(shapes)))
    assert need > ps.NOALLOC_SCRATCH_BYTES, need          # else the call below would reach the GPU
    with pytest.raises(ps.PSError) as e:
        ps.factored_step_noalloc(None, None, ps.FactoredHParams(), 1, records=(recs, len(shapes)))
    assert e.value.status == 7 and "scratch" in str(e.value)
