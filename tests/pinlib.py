"""Independent checks used to pin the oracle (test-side only).

Everything here is derived from the format's bit fields or from exact
rational arithmetic, not from the oracle's own formulas, so that a mistake in
the oracle (a wrong bias, a dropped term, a transposed operand, a wrong tie
rule) shows up as a disagreement.
"""

from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def load_e2m1_table() -> np.ndarray:
    """The 16 E2M1 values from tests/golden/e2m1_codes.txt (index = code)."""
    vals = {}
    with open(os.path.join(HERE, "golden", "e2m1_codes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c, 16)] = float(v)
    assert sorted(vals) == list(range(16))
    return np.array([vals[c] for c in range(16)], dtype=np.float64)


# Round-to-nearest-even decision boundaries of the E2M1 magnitude grid
# {0, .5, 1, 1.5, 2, 3, 4, 6}: the midpoints between neighbours, and at each
# midpoint the neighbour whose mantissa bit is 0 (even code) wins.
_MIDPOINTS = [Fraction(1, 4), Fraction(3, 4), Fraction(5, 4), Fraction(7, 4),
              Fraction(5, 2), Fraction(7, 2), Fraction(5)]


def e2m1_magnitude_code_exact(a: Fraction) -> int:
    """Magnitude code of |a| under RNE with saturation, in exact arithmetic."""
    assert a >= 0
    code = 0
    for i, m in enumerate(_MIDPOINTS):      # m sits between codes i and i+1
        if a > m or (a == m and (i + 1) % 2 == 0):
            code = i + 1
        else:
            break
    return code


def bf16_fields(bits: int) -> tuple[int, int, int]:
    return (bits >> 15) & 1, (bits >> 7) & 0xFF, bits & 0x7F


def bf16_exact(bits: int) -> Fraction:
    """Exact rational value of a finite bf16 bit pattern."""
    s, E, M = bf16_fields(bits)
    assert E != 0xFF
    if E == 0:
        v = Fraction(M, 1) * Fraction(1, 2 ** 133)
    else:
        v = Fraction(128 + M, 1) * (Fraction(2) ** (E - 134))
    return -v if s else v


def scale_exponent_from_bits(amax_bits: int, rule: int) -> int:
    """Shared exponent derived from the bf16 fields of the block maximum.

    rule 0, floor(log2(amax/6)): amax = (1 + M/128) 2^(E-127), and
    log2((1+M/128)/6) lies in [-3, -2) when M < 64 (1+m < 1.5) and in
    [-2, -1) otherwise, so s = E - 130 + [M >= 64].
    rule 1, floor(log2 amax) - 2 = E - 127 - 2.
    rule 2, ceil(log2(amax/6)): log2((1+M/128)/1.5) lies in (-1, 0] when
    M <= 64 and in (0, 1) otherwise, so s = E - 129 + [M > 64].
    A subnormal or zero maximum lies below 2^-126, so every rule gives a value
    under -127, clamped to -127.  Results are clamped to [-127, 127].
    """
    _, E, M = bf16_fields(amax_bits)
    if E == 0:
        return -127
    if rule == 0:
        s = E - 130 + (1 if M >= 64 else 0)
    elif rule == 1:
        s = E - 129
    else:
        s = E - 129 + (1 if M > 64 else 0)
    return max(-127, min(127, s))


def dequant_numpy(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Packed codes (low nibble = even element) + E8M0 -> float64, via the
    golden table and exact powers of two."""
    table = load_e2m1_table()
    lo = (q & 0xF).astype(np.int64)
    hi = (q >> 4).astype(np.int64)
    codes = np.stack([lo, hi], axis=-1).reshape(q.shape[:-1] + (q.shape[-1] * 2,))
    vals = table[codes]
    scale = np.ldexp(1.0, s.astype(np.int64) - 127)
    return vals * np.repeat(scale, 32, axis=-1)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))
