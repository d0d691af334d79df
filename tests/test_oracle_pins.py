"""Pins of the CPU oracle against facts fixed by the format and the maths.

None of these compare the oracle with itself: expected values come from the
golden E2M1 table, the bf16 bit fields, exact rational arithmetic, NumPy
library routines on special cases, or pure-Python brute force.
"""

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O
from synth import moe_inputs as MI
from tests import pinlib as PL

FINITE_BF16 = [b for b in range(1 << 16) if ((b >> 7) & 0xFF) != 0xFF]


# ---------------------------------------------------------------- E2M1 / E8M0

def test_e2m1_decode_table_matches_golden():
    table = PL.load_e2m1_table()
    got = np.array([O.e2m1_value(c) for c in range(16)])
    assert np.array_equal(got, table)
    assert np.array_equal(np.signbit(got), np.arange(16) >= 8)
    # the 8 magnitudes are exactly +-{0, .5, 1, 1.5, 2, 3, 4, 6}
    assert sorted(set(np.abs(got).tolist())) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_midpoints_are_those_of_the_golden_grid():
    t = PL.load_e2m1_table()[:8]
    mids = [Fraction(t[i]) / 2 + Fraction(t[i + 1]) / 2 for i in range(7)]
    assert mids == PL._MIDPOINTS


def test_e8m0_values():
    for b in range(255):
        assert O.e8m0_value(b) == math.ldexp(1.0, b - 127)
    assert math.isnan(O.e8m0_value(255))


@pytest.mark.parametrize("rule", [0, 1])
def test_scale_exponent_all_bf16_maxima(rule):
    for bits in range(1, 0x7F80):
        amax = PL.bf16_to_f64(np.array([bits]))[0]
        assert O.scale_exponent(amax, rule) == PL.scale_exponent_from_bits(bits, rule), hex(bits)
    assert O.scale_exponent(0.0, rule) == -127


def test_scale_rule0_is_floor_log2_amax_over_6_at_boundaries():
    # amax = 1.5 * 2^j is the only mantissa where amax/6 is a power of two
    for j in range(-100, 100):
        assert O.scale_exponent(1.5 * 2.0 ** j, 0) == j - 2
        assert O.scale_exponent(math.nextafter(1.5 * 2.0 ** j, 0), 0) == j - 3


def test_e2m1_encode_exhaustive_over_bf16():
    """Every finite bf16 value as an already-scaled element."""
    xs = PL.bf16_to_f64(np.array(FINITE_BF16, dtype=np.uint16))
    for bits, y in zip(FINITE_BF16, xs):
        sign = bits >> 15
        mag = PL.e2m1_magnitude_code_exact(abs(PL.bf16_exact(bits)))
        assert O.e2m1_encode(float(y)) == (sign << 3 | mag), hex(bits)


def test_e2m1_encode_ties_and_saturation():
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for y, c in ties.items():
        assert O.e2m1_encode(y) == c
        assert O.e2m1_encode(-y) == 8 | c
    assert O.e2m1_encode(1e30) == 7 and O.e2m1_encode(-1e30) == 15
    assert O.e2m1_encode(-0.0) == 8 and O.e2m1_encode(-0.1) == 8


# ---------------------------------------------------------------- quantize

def _random_blocks(rng, nblk):
    """bf16 blocks with mixed magnitudes: normal, tiny, subnormal, huge, zero."""
    out = []
    for i in range(nblk):
        kind = i % 6
        if kind == 0:
            v = rng.standard_normal(32) * 0.02
        elif kind == 1:
            v = rng.standard_normal(32) * 10.0 ** rng.uniform(-30, 30)
        elif kind == 2:
            v = rng.standard_normal(32) * 1e-39          # bf16 subnormals
        elif kind == 3:
            v = rng.standard_normal(32) * 1e37
        elif kind == 4:
            v = np.zeros(32)
            v[rng.integers(0, 32)] = rng.standard_normal()
        else:
            v = rng.choice([-6, -4, -3, -2, -1.5, -1, -.5, 0, .5, 1, 1.5, 2, 3, 4, 6], 32) \
                * 2.0 ** rng.integers(-20, 20)
        out.append(MI.f32_to_bf16_bits(v.astype(np.float32)))
    return np.stack(out)


@pytest.mark.parametrize("rule", [0, 1])
def test_quantize_matches_bruteforce(rule):
    rng = np.random.default_rng(11)
    w = _random_blocks(rng, 600).reshape(20, 30 * 32)     # rows=20, K=960
    q, s = O.quantize(w, rule)
    assert q.shape == (20, 480) and s.shape == (20, 30)
    table = PL.load_e2m1_table()
    for r in range(20):
        for b in range(30):
            blk = [int(v) for v in w[r, b * 32:(b + 1) * 32]]
            amax_bits = max(v & 0x7FFF for v in blk)
            se = PL.scale_exponent_from_bits(amax_bits, rule)
            assert s[r, b] == se + 127
            scale = Fraction(2) ** se
            codes = []
            for v in blk:
                a = abs(PL.bf16_exact(v)) / scale
                codes.append((v >> 15) << 3 | PL.e2m1_magnitude_code_exact(a))
            packed = [codes[2 * i] | codes[2 * i + 1] << 4 for i in range(16)]
            assert list(q[r, b * 16:(b + 1) * 16]) == packed, (r, b)
            # nearest-value property: no grid value times the scale is closer
            for v, c in zip(blk, codes):
                x = PL.bf16_exact(v)
                err = abs(Fraction(table[c]) * scale - x)
                for g in table:
                    assert err <= abs(Fraction(g) * scale - x)


def test_quantize_rejects_bad_shapes():
    with pytest.raises(ValueError):
        O.quantize(np.zeros((2, 48), np.uint16))
    with pytest.raises(ValueError):
        O.quantize(np.zeros((2, 64), np.uint16), rule=7)


def _representable_blocks(rng, n, top_mag):
    """Blocks of E2M1 grid values times 2^j whose largest magnitude is top_mag * 2^j."""
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    blocks, js = [], []
    for _ in range(n):
        j = int(rng.integers(-60, 60))
        v = rng.choice(grid[grid <= top_mag[-1]], 32) * rng.choice([-1, 1], 32)
        v[rng.integers(0, 32)] = rng.choice(top_mag) * rng.choice([-1, 1])
        blocks.append(MI.f32_to_bf16_bits((v * 2.0 ** j).astype(np.float32)))
        js.append(j)
    return np.stack(blocks), js


def test_roundtrip_rule1_exact_for_representable_blocks():
    rng = np.random.default_rng(3)
    w, js = _representable_blocks(rng, 400, [4.0, 6.0])      # max in [4, 6]: s = j
    q, s = O.quantize(w, 1)
    assert list(s.ravel().astype(int) - 127) == js
    assert np.array_equal(O.dequantize(q, s), PL.bf16_to_f64(w))


def test_roundtrip_rule0_exact_when_block_max_is_6():
    rng = np.random.default_rng(4)
    w, js = _representable_blocks(rng, 400, [6.0])
    q, s = O.quantize(w, 0)
    assert list(s.ravel().astype(int) - 127) == js
    assert np.array_equal(O.dequantize(q, s), PL.bf16_to_f64(w))


def test_rule0_saturates_a_power_of_two_maximum():
    """floor(log2(4/6)) = -1, so 4 scales to 8 and saturates to 6 * 2^-1 = 3."""
    w = np.zeros((1, 32), np.uint16)
    w[0, 0] = MI.f32_to_bf16_bits(np.array([4.0], np.float32))[0]
    q, s = O.quantize(w, 0)
    assert s[0, 0] == 126 and q[0, 0] == 0x07
    assert O.dequantize(q, s)[0, 0] == 3.0


@pytest.mark.parametrize("rule", [0, 1])
def test_quantize_idempotent(rule):
    rng = np.random.default_rng(5)
    w = _random_blocks(rng, 300).reshape(10, 960)
    q, s = O.quantize(w, rule)
    d = O.dequantize(q, s)
    w2 = MI.f32_to_bf16_bits(d.astype(np.float32))
    assert np.array_equal(PL.bf16_to_f64(w2), d)              # D(Q(w)) is exact in bf16
    q2, s2 = O.quantize(w2, rule)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_rule0_every_unclamped_nonzero_block_holds_a_saturated_code():
    cfg = MI.CONFIGS["tiny"]
    w13, w2 = MI.gen_experts(cfg, 0)
    q, s = O.quantize(w13.reshape(-1, cfg.D), 0)
    mags = np.stack([q & 7, (q >> 4) & 7], -1).reshape(q.shape[0], -1, 32)
    assert np.all((mags == 7).any(axis=-1))


def test_dequantize_matches_numpy_decode():
    rng = np.random.default_rng(6)
    w = _random_blocks(rng, 120).reshape(4, 960)
    for rule in (0, 1):
        q, s = O.quantize(w, rule)
        assert np.array_equal(O.dequantize(q, s), PL.dequant_numpy(q, s))


# ---------------------------------------------------------------- routing

def _tiny_router(T=16, D=64, E=8, seed=0, bias=None):
    rng = np.random.default_rng(seed)
    x = MI.f32_to_bf16_bits(rng.standard_normal((T, D)).astype(np.float32))
    wr = (rng.standard_normal((E, D)) * 0.02).astype(np.float32)
    b = np.zeros(E, np.float32) if bias is None else np.asarray(bias, np.float32)
    return x, wr, b


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_route_against_numpy(k):
    x, wr, b = _tiny_router(T=40, D=96, E=8, seed=k)
    b = (np.arange(8) * 0.01).astype(np.float32)
    r = O.route(x, wr, b, k)
    L = PL.bf16_to_f64(x) @ wr.astype(np.float64).T + b.astype(np.float64)
    np.testing.assert_allclose(r["logits"], L, rtol=0, atol=1e-12)
    order = np.lexsort((np.broadcast_to(np.arange(8), L.shape), -L), axis=-1)
    assert np.array_equal(r["ids"], order[:, :k])
    sel = np.take_along_axis(L, order[:, :k], 1)
    ez = np.exp(sel - sel.max(1, keepdims=True))
    np.testing.assert_allclose(r["w"], ez / ez.sum(1, keepdims=True), rtol=1e-13)
    np.testing.assert_allclose(r["w"].sum(1), 1.0, rtol=1e-14)
    ids = r["ids"].ravel()
    assert np.array_equal(r["counts"], np.bincount(ids, minlength=8))
    assert np.array_equal(r["offsets"], np.concatenate([[0], np.cumsum(np.bincount(ids, minlength=8))]))
    assert np.array_equal(r["sorted"], np.argsort(ids, kind="stable"))
    assert np.array_equal(r["pos"][r["sorted"]], np.arange(len(ids)))
    srt = np.sort(L, axis=1)[:, ::-1][:, :min(k + 1, 8)]
    np.testing.assert_allclose(r["gap"], np.diff(-srt, axis=1).min(1), rtol=1e-12)


def test_route_k_equals_E_is_full_softmax():
    import scipy.special
    x, wr, b = _tiny_router(T=10, D=64, E=6, seed=2)
    r = O.route(x, wr, b, 6)
    L = r["logits"]
    full = scipy.special.softmax(L, axis=1)
    np.testing.assert_allclose(np.take_along_axis(full, r["ids"], 1), r["w"], rtol=1e-13)


def test_route_k1_weight_is_one_and_ties_go_to_lower_id():
    x = np.zeros((3, 32), np.uint16)                    # all logits equal the bias
    wr = np.zeros((4, 32), np.float32)
    r = O.route(x, wr, np.array([0.5, 2.0, 2.0, 1.0], np.float32), 2)
    assert np.array_equal(r["ids"], [[1, 2]] * 3)
    assert np.all(r["gap"] == 0.0)
    r1 = O.route(x, wr, np.array([0.5, 2.0, 2.0, 1.0], np.float32), 1)
    assert np.array_equal(r1["ids"], [[1]] * 3) and np.all(r1["w"] == 1.0)


# ---------------------------------------------------------------- expert MLP

def _tiny_experts(E, D, F, seed=0):
    rng = np.random.default_rng(seed)
    w13 = MI.f32_to_bf16_bits((rng.standard_normal((E, 2 * F, D)) * 0.05).astype(np.float32))
    w2 = MI.f32_to_bf16_bits((rng.standard_normal((E, D, F)) * 0.05).astype(np.float32))
    q13, s13 = O.quantize(w13, 0)
    q2, s2 = O.quantize(w2, 0)
    return q13, s13, q2, s2


def test_one_hot_route_is_dense_swiglu_mlp():
    T, D, F, E = 12, 64, 96, 5
    x, wr, _ = _tiny_router(T=T, D=D, E=E, seed=7)
    q13, s13, q2, s2 = _tiny_experts(E, D, F, seed=8)
    X = PL.bf16_to_f64(x)
    for e in range(E):
        bias = np.full(E, -1e3, np.float32)
        bias[e] = 1e3                                   # forces every token to expert e
        r = O.route(x, wr, bias, 1)
        assert np.all(r["ids"] == e) and np.all(r["w"] == 1.0)
        out = O.moe(x, q13, s13, q2, s2, r["ids"], r["w"], F)
        W13 = PL.dequant_numpy(q13[e], s13[e])
        W2 = PL.dequant_numpy(q2[e], s2[e])
        g, u = X @ W13[:F].T, X @ W13[F:].T
        dense = (PL.silu(g) * u) @ W2.T
        np.testing.assert_allclose(out, dense, rtol=1e-12, atol=1e-12)


def test_identical_experts_make_output_routing_independent():
    T, D, F, E = 8, 32, 64, 4
    x, wr, _ = _tiny_router(T=T, D=D, E=E, seed=9)
    q13, s13, q2, s2 = _tiny_experts(1, D, F, seed=10)
    rep = lambda a: np.repeat(a, E, axis=0)
    r = O.route(x, wr, None, 2)
    out = O.moe(x, rep(q13), rep(s13), rep(q2), rep(s2), r["ids"], r["w"], F)
    dense = O.moe(x, q13, s13, q2, s2, np.zeros((T, 1), np.int32), np.ones((T, 1)), F)
    np.testing.assert_allclose(out, dense, rtol=1e-12, atol=1e-14)


def test_zero_input_gives_zero_output():
    T, D, F, E = 4, 32, 32, 3
    q13, s13, q2, s2 = _tiny_experts(E, D, F, seed=12)
    x = np.zeros((T, D), np.uint16)
    r = O.route(x, np.ones((E, D), np.float32), None, 2)
    assert np.all(O.moe(x, q13, s13, q2, s2, r["ids"], r["w"], F) == 0.0)


def test_token_subset_matches_full_run():
    T, D, F, E = 10, 32, 64, 4
    x, wr, _ = _tiny_router(T=T, D=D, E=E, seed=13)
    q13, s13, q2, s2 = _tiny_experts(E, D, F, seed=14)
    r = O.route(x, wr, None, 2)
    full = O.moe(x, q13, s13, q2, s2, r["ids"], r["w"], F)
    sub = O.moe(x, q13, s13, q2, s2, r["ids"], r["w"], F, tokens=[7, 2, 9])
    assert np.array_equal(sub, full[[7, 2, 9]])


# ---------------------------------------------------------------- brute force

def _pure_python_layer(x, wr, b, q13, s13, q2, s2, k, F):
    """Scalar loops over Python floats; decode via the golden table."""
    table = PL.load_e2m1_table().tolist()
    T, D = x.shape
    E = wr.shape[0]

    def xv(t, d):
        return float(PL.bf16_exact(int(x[t, d])))

    def wq(q, s, K, e, r, c):
        byte = int(q[e, r, c // 2])
        code = byte & 15 if c % 2 == 0 else byte >> 4
        return table[code] * 2.0 ** (int(s[e, r, c // 32]) - 127)

    outs = []
    for t in range(T):
        L = [sum(xv(t, d) * float(wr[e, d]) for d in range(D)) + float(b[e]) for e in range(E)]
        ranked = sorted(range(E), key=lambda e: (-L[e], e))[:k]
        m = max(L[e] for e in ranked)
        z = sum(math.exp(L[e] - m) for e in ranked)
        out = [0.0] * D
        for e in ranked:
            wt = math.exp(L[e] - m) / z
            h = []
            for f in range(F):
                g = sum(wq(q13, s13, D, e, f, d) * xv(t, d) for d in range(D))
                u = sum(wq(q13, s13, D, e, F + f, d) * xv(t, d) for d in range(D))
                h.append(g / (1 + math.exp(-g)) * u)
            for d in range(D):
                out[d] += wt * sum(wq(q2, s2, F, e, d, f) * h[f] for f in range(F))
        outs.append(out)
    return np.array(outs)


def test_bruteforce_tiny_layer_all_forced_routings():
    T, D, F, E, k = 3, 32, 32, 4, 2
    x, wr, _ = _tiny_router(T=T, D=D, E=E, seed=15)
    q13, s13, q2, s2 = _tiny_experts(E, D, F, seed=16)
    for pair in itertools.combinations(range(E), k):
        bias = np.full(E, -50.0, np.float32)
        bias[list(pair)] = [50.0, 49.0]
        r = O.route(x, wr, bias, k)
        got = O.moe(x, q13, s13, q2, s2, r["ids"], r["w"], F)
        want = _pure_python_layer(x, wr, bias, q13, s13, q2, s2, k, F)
        np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-13)
        assert set(r["ids"].ravel()) == set(pair)


def test_bruteforce_tiny_layer_free_routing():
    T, D, F, E, k = 4, 64, 32, 4, 2
    x, wr, b = _tiny_router(T=T, D=D, E=E, seed=17)
    q13, s13, q2, s2 = _tiny_experts(E, D, F, seed=18)
    r = O.route(x, wr, b, k)
    got = O.moe(x, q13, s13, q2, s2, r["ids"], r["w"], F)
    want = _pure_python_layer(x, wr, b, q13, s13, q2, s2, k, F)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-13)


def test_tiny_workload_has_no_near_ties():
    cfg = MI.CONFIGS["tiny"]
    wr, b = MI.gen_router(cfg, 0)
    r = O.route(MI.gen_x(cfg, 0), wr, b, cfg.k)
    assert r["gap"].min() > 1e-4
    assert r["counts"].sum() == cfg.P


def test_threaded_harness_equals_plain_oracle():
    T, D, F, E, k = 9, 64, 96, 5, 2
    x, wr, b = _tiny_router(T=T, D=D, E=E, seed=19)
    q13, s13, q2, s2 = _tiny_experts(E, D, F, seed=20)
    r = O.route(x, wr, b, k)
    plain = O.moe(x, q13, s13, q2, s2, r["ids"], r["w"], F)
    thr = O.moe_threaded(x, lambda e: (q13[e], s13[e], q2[e], s2[e]), r["ids"], r["w"], F,
                         threads=3)
    assert np.array_equal(plain, thr)
    sub = O.moe_threaded(x, lambda e: (q13[e], s13[e], q2[e], s2[e]), r["ids"], r["w"], F,
                         tokens=[4, 0], threads=2)
    assert np.array_equal(sub, plain[[4, 0]])
