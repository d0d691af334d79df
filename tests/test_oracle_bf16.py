"""Pins of the oracle's bf16-weight expert (oracle_expert_mlp_bf16), the
reference of the bf16 comparison path.

Expected values come from NumPy dense algebra, pure-Python scalar loops, a
closed form, and the MXFP4 oracle on weights whose bf16 values are exactly
the dequantized MXFP4 ones -- not from the function itself.
"""

import math

import numpy as np
import pytest

from oracle import oracle as O
from synth import moe_inputs as MI
from tests import pinlib as PL


def _bf16(rng, shape, scale):
    return MI.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _case(T, D, F, seed):
    rng = np.random.default_rng(seed)
    x = _bf16(rng, (T, D), 1.0)
    w13 = _bf16(rng, (2 * F, D), 0.05)
    w2 = _bf16(rng, (D, F), 0.05)
    return x, w13, w2


@pytest.mark.parametrize("T,D,F", [(5, 32, 32), (7, 96, 160), (3, 2880, 64)])
def test_bf16_expert_is_dense_swiglu_mlp(T, D, F):
    x, w13, w2 = _case(T, D, F, 31)
    toks = np.arange(T)[::-1].copy()
    got = O.expert_mlp_bf16(x, w13, w2, F, toks)
    X = PL.bf16_to_f64(x)[toks]
    W13, W2 = PL.bf16_to_f64(w13), PL.bf16_to_f64(w2)
    g, u = X @ W13[:F].T, X @ W13[F:].T
    want = (PL.silu(g) * u) @ W2.T
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-13)


def test_bf16_expert_pure_python_loops():
    T, D, F = 2, 32, 32
    x, w13, w2 = _case(T, D, F, 32)
    got = O.expert_mlp_bf16(x, w13, w2, F, [1, 0])
    xv = lambda t, d: float(PL.bf16_exact(int(x[t, d])))
    wv = lambda a, r, c: float(PL.bf16_exact(int(a[r, c])))
    for i, t in enumerate([1, 0]):
        h = []
        for f in range(F):
            g = sum(wv(w13, f, d) * xv(t, d) for d in range(D))
            u = sum(wv(w13, F + f, d) * xv(t, d) for d in range(D))
            h.append(g / (1.0 + math.exp(-g)) * u)
        for d in range(D):
            want = sum(wv(w2, d, f) * h[f] for f in range(F))
            assert abs(got[i, d] - want) <= 1e-12 * (1.0 + abs(want))


def test_bf16_expert_single_weight_closed_form():
    # one gate weight a, one up weight b (row f, column d), one down weight c
    # (row o, column f): y[o] = c silu(a x_d) b x_d, every other output 0
    D, F, f, d, o = 64, 32, 5, 17, 40
    a, b, c = 1.5, -0.75, 2.0
    w13 = np.zeros((2 * F, D), np.uint16)
    w2 = np.zeros((D, F), np.uint16)
    enc = lambda v: MI.f32_to_bf16_bits(np.array([v], np.float32))[0]
    w13[f, d], w13[F + f, d], w2[o, f] = enc(a), enc(b), enc(c)
    x = np.zeros((1, D), np.uint16)
    x[0, d] = enc(0.8125)
    y = O.expert_mlp_bf16(x, w13, w2, F, [0])[0]
    z = a * 0.8125
    want = c * (z / (1.0 + math.exp(-z))) * (b * 0.8125)
    assert abs(y[o] - want) <= 1e-15 * abs(want)
    assert np.all(np.delete(y, o) == 0.0)


def test_bf16_expert_equals_mxfp4_expert_on_the_same_values():
    # MXFP4 values e2m1 * 2^(s - 127) with normal scales are bf16 numbers:
    # written as bf16, the two oracles see identical weights
    T, D, F = 6, 64, 96
    x, w13, w2 = _case(T, D, F, 33)
    q13, s13 = O.quantize(w13, 0)
    q2, s2 = O.quantize(w2, 0)
    d13, d2 = O.dequantize(q13, s13), O.dequantize(q2, s2)
    b13 = MI.f32_to_bf16_bits(d13.astype(np.float32))
    b2 = MI.f32_to_bf16_bits(d2.astype(np.float32))
    assert np.array_equal(PL.bf16_to_f64(b13), d13) and np.array_equal(PL.bf16_to_f64(b2), d2)
    toks = [0, 3, 5, 1]
    assert np.array_equal(O.expert_mlp_bf16(x, b13, b2, F, toks),
                          O.expert_mlp(x, q13, s13, q2, s2, F, toks))


def test_bf16_threaded_layer_combines_in_slot_order():
    T, D, F, E, k = 5, 32, 64, 3, 2
    rng = np.random.default_rng(34)
    x = _bf16(rng, (T, D), 1.0)
    w13 = _bf16(rng, (E, 2 * F, D), 0.05)
    w2 = _bf16(rng, (E, D, F), 0.05)
    ids = np.array([[0, 2], [1, 0], [2, 1], [0, 1], [2, 0]], np.int32)
    w = rng.uniform(0.1, 0.9, (T, k))
    out = O.moe_threaded(x, lambda e: (w13[e], w2[e]), ids, w, F, threads=2)
    X, W13, W2 = PL.bf16_to_f64(x), PL.bf16_to_f64(w13), PL.bf16_to_f64(w2)
    for t in range(T):
        want = np.zeros(D)
        for j in range(k):
            e = ids[t, j]
            g, u = W13[e, :F] @ X[t], W13[e, F:] @ X[t]
            want = want + w[t, j] * (W2[e] @ (PL.silu(g) * u))
        np.testing.assert_allclose(out[t], want, rtol=1e-12, atol=1e-14)


def test_bf16_expert_rejects_bad_weight_shapes():
    x, w13, w2 = _case(2, 32, 32, 35)
    with pytest.raises(ValueError):
        O.expert_mlp_bf16(x, w13[:32], w2, 32, [0])
