"""Pins of the oracle's stochastic-rounding split (no residual).

The rounding is defined by its probability (PR #2159 body: the value moves to
the upper or lower neighbouring bf16 with a chance set by its distance to
them); the random bits come from a SplitMix64 stream (Steele, Lea, Flood,
OOPSLA 2014). Each pin checks one of those facts against something other than
the oracle's own formula: the generator's published outputs, exhaustive counts
over all 2^16 random values, distribution statistics, and the relation to the
deterministic fp32 step."""
import numpy as np
import pytest

import oracle
from figures import page_figure
from oracle import HParams


def _bf16_bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_splitmix64_published_outputs():
    """The first three outputs of SplitMix64 from state 0, as the generator's
    reference definition fixes them."""
    for k, want in enumerate(page_figure("splitmix64_state0_outputs")["outputs"]):
        assert oracle.splitmix64_at(0, k) == int(want, 16), k


def test_sr_stream_of_key_zero_is_the_published_sequence():
    """With seed 0, update 0 and tensor 0 the stream starts at state 0
    (mix(0) = 0), so the random 16-bit values of elements 4k..4k+3, read as
    one little-endian 64-bit word, are the generator's k-th published output
    from state 0: this fixes which output word and which 16 bits each element
    takes."""
    outs = [int(x, 16) for x in page_figure("splitmix64_state0_outputs")["outputs"]]
    r = oracle.sr_rand16(0, 0, 0, 0, 4 * len(outs)).astype(np.uint64)
    for k, want in enumerate(outs):
        word = sum(int(r[4 * k + j]) << (16 * j) for j in range(4))
        assert word == want, (k, hex(word))
    # an offset request reads the same values
    assert np.array_equal(oracle.sr_rand16(0, 0, 0, 5, 6).astype(np.uint64), r[5:11])


@pytest.mark.parametrize("bits", [0x3F800001, 0x3F80FFFF, 0x3F808000, 0xBF812345, 0x3F7FFFFF, 0x7F7F8001,
                                  0x00001234, 0x80017FFF, 0x4B7FC000])
def test_sr_rounds_away_with_probability_of_the_fractional_distance(bits):
    """Over all 2^16 random values exactly low16(x) of them round away from
    zero (probability = distance / spacing), the rest truncate, and the result
    is always one of the two neighbouring bf16 values."""
    x = np.uint32(bits).view(np.float32)
    lo = bits & 0xFFFF
    trunc = bits >> 16
    res = np.array([oracle.sr_bf16(x, r) for r in range(65536)], np.uint32)
    away = (res == trunc + 1)
    assert np.all(away | (res == trunc))
    assert int(away.sum()) == lo
    # the away results are the largest random values
    assert np.all(away[65536 - lo:]) and not np.any(away[:65536 - lo])


def test_sr_leaves_bf16_values_unchanged():
    rng = np.random.default_rng(41)
    hi = rng.integers(0, 0x7F80, 64, dtype=np.uint32)
    for h in hi:
        x = np.uint32(h << 16).view(np.float32)
        for r in (0, 1, 12345, 65535):
            assert oracle.sr_bf16(x, r) == h


def test_sr_random_stream_is_uniform_and_keyed():
    """Chi-square on the 2^16 values split into 256 bins (high and low byte);
    different seeds, steps and tensors give unrelated streams."""
    n = 1 << 20
    r = oracle.sr_rand16(7, 3, 5, 0, n).astype(np.int64)
    for part in (r >> 8, r & 0xFF):
        counts = np.bincount(part, minlength=256)
        exp = n / 256
        chi2 = float(((counts - exp) ** 2 / exp).sum())
        assert 170 < chi2 < 350, chi2         # 255 dof: mean 255, sd 22.6
    base = oracle.sr_rand16(7, 3, 5, 0, 4096)
    for other in (oracle.sr_rand16(8, 3, 5, 0, 4096), oracle.sr_rand16(7, 4, 5, 0, 4096),
                  oracle.sr_rand16(7, 3, 6, 0, 4096), oracle.sr_rand16(7, 3, 5, 4096, 4096)):
        assert np.mean(base == other) < 0.01
        c = np.corrcoef(base.astype(np.float64), other.astype(np.float64))[0, 1]
        assert abs(c) < 0.06
    # offsets: element e's value does not depend on where the request starts
    assert np.array_equal(oracle.sr_rand16(7, 3, 5, 100, 50), r[100:150].astype(np.uint16))


def test_sr_moves_a_fifth_of_an_ulp_update_once_in_five_steps_on_average():
    """PR #2159 body: an update of 20% of the distance to the next bf16 makes
    the Kahan-summed value move once every 5 steps; stochastic rounding moves it
    with probability 0.2 per step, so once in five steps on average."""
    n = 1 << 18
    hi = np.full(n, 0x3F80, np.uint32)                     # 1.0
    ulp = 2.0 ** -7
    fig = page_figure("kahan_subulp_update_period")
    p = fig["update_fraction_of_ulp"]
    assert p == 1.0 / fig["period_steps"]
    x = np.float32(1.0 + p * ulp)                          # exactly representable in fp32
    r = oracle.sr_rand16(11, 1, 0, 0, n)
    res = ((np.uint32(np.float32(x).view(np.uint32)) + r.astype(np.uint32)) >> 16)
    # the same through the oracle's function on a sample
    for i in range(0, n, 4099):
        assert oracle.sr_bf16(x, r[i]) == res[i]
    frac = float(np.mean(res == hi + 1))
    assert abs(frac - p) < 4 * np.sqrt(p * (1 - p) / n), frac


def test_sr_step_brackets_the_fp32_step_and_keeps_the_moments():
    """The stochastic-rounding step equals the fp32 core step on the widened
    bf16 weight, rounded to one of its two bf16 neighbours; its moments equal
    those of the residual step (they do not depend on the weight when wd = 0),
    and the residual array is not touched."""
    n = 3000
    rng = np.random.default_rng(43)
    hi = _bf16_bits(rng.standard_normal(n) * 0.02)
    g = _bf16_bits(rng.standard_normal(n) * 1e-3)
    hp_sr = HParams(split_mode=oracle.SPLIT_STOCHASTIC, lr=1e-3, seed=99, tensor=4)
    st = oracle.TensorState(hi.copy(), np.full(n, 0xABCD, np.uint16), *oracle.zero_moments(n))
    oracle.opt_step(st, g, hp_sr, 1)
    assert np.all(st.lo == 0xABCD)
    w = (hi.astype(np.uint32) << 16).view(np.float32).copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    oracle.core_step(w, m, v, oracle.bf16_to_f32(g).copy(), HParams(lr=1e-3), 1)
    wb = w.view(np.uint32)
    trunc = (wb >> 16).astype(np.uint16)
    assert np.all((st.hi == trunc) | (st.hi == trunc + 1))
    moved = st.hi == trunc + 1
    assert np.all(moved <= ((wb & 0xFFFF) != 0))
    r = oracle.sr_rand16(99, 1, 4, 0, n)
    assert np.array_equal(moved, (wb & 0xFFFF).astype(np.uint32) + r >= 65536)
    st_k = oracle.TensorState(hi.copy(), np.zeros(n, np.uint16), *oracle.zero_moments(n))
    oracle.opt_step(st_k, g, HParams(lr=1e-3), 1)
    assert np.array_equal(st.mc, st_k.mc) and np.array_equal(st.vc, st_k.vc)
    assert np.array_equal(st.ms, st_k.ms) and np.array_equal(st.vs, st_k.vs)


def test_sr_is_unbiased_over_many_elements():
    """The mean of the rounded weights equals the mean of the fp32 weights
    within the sampling error of the rounding."""
    n = 1 << 18
    rng = np.random.default_rng(44)
    x = (1.0 + rng.random(n) * 0.5).astype(np.float32)
    r = oracle.sr_rand16(5, 2, 1, 0, n)
    res = ((x.view(np.uint32) + r.astype(np.uint32)) >> 16 << 16).view(np.float32)
    err = res.astype(np.float64) - x.astype(np.float64)
    ulp = 2.0 ** -7
    assert abs(err.mean()) < 4 * (ulp / 2) / np.sqrt(n)
