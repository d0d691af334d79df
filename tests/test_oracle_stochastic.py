"""Pins of the oracle's stochastic-rounding quantizer and its ceiling scale
rule (CPU only).  The pages cite stochastic rounding as part of an MXFP4
training recipe ("MXFP4 기반 MoE (Mixture-of-Experts) 기술 리뷰", section 2)
without details; the readings pinned here: the upper neighbour is taken with
probability equal to the fractional distance, the draw of element
i = row * K + col is the top 24 bits of output i + 1 of a SplitMix64 stream
started at the seed, and scale rule 2 = ceil(log2(amax / 6)) keeps every
element within +-6 so the rounding is unbiased."""

import numpy as np

from oracle import oracle as O
from synth import moe_inputs as MI
from tests import pinlib as PL

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_scale_rule2_all_bf16_maxima():
    for bits in range(1, 0x7F80):
        amax = PL.bf16_to_f64(np.array([bits]))[0]
        assert O.scale_exponent(amax, 2) == PL.scale_exponent_from_bits(bits, 2), hex(bits)
    assert O.scale_exponent(0.0, 2) == -127


def test_scale_rule2_is_the_smallest_scale_without_clipping():
    for j in range(-100, 100):
        for m in (1.0, 1.25, 1.5, 1.5078125, 1.9921875):
            amax = m * 2.0 ** j
            s = O.scale_exponent(amax, 2)
            assert amax <= 6.0 * 2.0 ** s and amax > 6.0 * 2.0 ** (s - 1), (m, j)


def test_splitmix64_reference_outputs():
    # The first outputs of SplitMix64 started from state 0, as the generator's
    # reference implementation (S. Vigna's splitmix64.c; the mix64 of the
    # JDK's java.util.SplittableRandom) produces them.
    assert [O.splitmix64(0, n) for n in (1, 2, 3)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_stochastic_rounding_threshold():
    # between neighbours lo <= y < hi the upper one is taken exactly when
    # u < 2^24 (y - lo) / (hi - lo): both sides of that threshold
    for c in range(7):
        lo, hi = GRID[c], GRID[c + 1]
        for num in (1, 3, 8, 13, 15):
            y = lo + (hi - lo) * num / 16
            thr = (1 << 24) * num // 16
            for sign in (0, 8):
                v = -y if sign else y
                assert O.e2m1_encode_stochastic(v, thr - 1) == sign | (c + 1)
                assert O.e2m1_encode_stochastic(v, thr) == sign | c
                assert O.e2m1_encode_stochastic(v, 0) == sign | (c + 1)
                assert O.e2m1_encode_stochastic(v, (1 << 24) - 1) == sign | c


def test_stochastic_rounding_grid_values_are_exact():
    for c, y in enumerate(GRID):
        for u in (0, 1, 1 << 23, (1 << 24) - 1):
            assert O.e2m1_encode_stochastic(y, u) == c
            assert O.e2m1_encode_stochastic(-y, u) == 8 | c
    assert O.e2m1_encode_stochastic(7.5, 0) == 7          # beyond 6: saturates
    assert O.e2m1_encode_stochastic(1e-30, 0) == 1        # any positive fraction can round up
    assert O.e2m1_encode_stochastic(1e-30, 1) == 0


def test_stochastic_quantize_picks_a_neighbour_and_is_unbiased():
    # Rule 2 never clips, so E[dequantized] equals the input.  Over many seeds
    # the mean of each element must match it within 5 sigma of the draws'
    # spread, and every value must be one of the input's two neighbours.
    rng = np.random.default_rng(11)
    w = MI.f32_to_bf16_bits((rng.standard_normal((2, 64)) * 0.02).astype(np.float32))
    v = PL.bf16_to_f64(w)
    nseed = 1500
    acc = np.zeros_like(v)
    acc2 = np.zeros_like(v)
    q0, s0 = O.quantize(w, rule=2)
    scale = np.repeat(2.0 ** (s0.astype(np.int64) - 127), 32, axis=-1)
    y = np.abs(v) / scale
    step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0)) * scale
    for seed in range(nseed):
        q, s = O.quantize(w, rule=2, stochastic=True, seed=seed)
        assert np.array_equal(s, s0)                      # the scales do not depend on the draw
        d = O.dequantize(q, s)
        assert np.all(np.abs(d - v) < step)              # one of the two neighbours
        acc += d
        acc2 += d * d
    mean = acc / nseed
    var = np.maximum(acc2 / nseed - mean ** 2, 0)
    assert np.all(np.abs(mean - v) <= 5 * np.sqrt(var / nseed) + 1e-15)
    # rounding to nearest moves some elements, so the check above is not vacuous
    assert np.abs(O.dequantize(q0, s0) - v).max() > 0


def test_stochastic_quantize_uses_each_elements_own_draw():
    # element i = row * K + col uses output i + 1 of the seed's stream
    rng = np.random.default_rng(12)
    w = MI.f32_to_bf16_bits(rng.standard_normal((3, 64)).astype(np.float32))
    seed = 0x1234ABCD5678
    q, s = O.quantize(w, rule=2, stochastic=True, seed=seed)
    v = PL.bf16_to_f64(w)
    for r in range(3):
        for c in range(64):
            y = v[r, c] * 2.0 ** -(int(s[r, c // 32]) - 127)
            u = O.splitmix64(seed, r * 64 + c + 1) >> 40
            code = (int(q[r, c // 2]) >> (4 * (c % 2))) & 0xF
            assert code == O.e2m1_encode_stochastic(y, u), (r, c)


def test_stochastic_with_a_clipping_rule_saturates():
    # rule 0 puts the block maximum in [6, 12): it saturates whatever the draw
    w = MI.f32_to_bf16_bits(np.array([[7.0] + [0.5] * 31], np.float32))
    for seed in range(20):
        q, s = O.quantize(w, rule=0, stochastic=True, seed=seed)
        assert int(s[0, 0]) - 127 == 0 and (int(q[0, 0]) & 0xF) == 7
