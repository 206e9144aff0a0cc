"""Pins of the oracle's INT8 rows (oracle.quantize_int8 / dequantize_int8).

The scheme is the library's own (no page fixes one): symmetric codes with one float32 scale per
row.  Pinned by hand-worked rows (tests/golden/int8_rows_hand.txt), by exact rational arithmetic
of the same rule, by the bounds the rule implies, and by the special rows.
"""
import os
from fractions import Fraction

import numpy as np

import oracle
from conftest import GOLDEN


def _hand_rows():
    rows = []
    for line in open(os.path.join(GOLDEN, "int8_rows_hand.txt")):
        if line.startswith("#") or not line.strip():
            continue
        x, c, s = (part.strip() for part in line.split("|"))
        num, den = s.split("/")
        rows.append(([float(v) for v in x.split(",")], [int(v) for v in c.split(",")], float(num) / float(den)))
    return rows


def test_hand_worked_rows():
    rows = _hand_rows()
    assert len(rows) == 4
    for x, codes, scale in rows:
        c, s = oracle.quantize_int8(np.array([x], np.float32))
        assert c[0].tolist() == codes, (x, c)
        assert s[0] == np.float32(np.float32(scale)), (x, s)


def test_codes_follow_exact_rounding_of_x_over_scale():
    """code = round(127 x / amax) in exact rationals, except where the float32 rounding of
    127 / amax moves a product across a half-integer: then the codes differ by one."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((400, 64)).astype(np.float32) * np.exp(rng.uniform(-8, 8, (400, 1))).astype(np.float32)
    codes, scales = oracle.quantize_int8(x)
    diff = 0
    for r in range(x.shape[0]):
        amax = max(abs(Fraction(float(v))) for v in x[r])
        for j in range(x.shape[1]):
            q = Fraction(float(x[r, j])) * 127 / amax
            fl = q.numerator // q.denominator
            rem = q - fl
            exact = fl + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2) else 0)
            if exact != codes[r, j]:
                diff += 1
                assert abs(exact - int(codes[r, j])) == 1
        assert scales[r] == np.float32(np.float32(float(amax)) / np.float32(127))
    assert diff <= x.size // 1000


def test_bounds_and_extremes():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((1000, 128)) * 3).astype(np.float32)
    codes, scales = oracle.quantize_int8(x)
    assert np.abs(codes.astype(np.int32)).max() <= 127
    # the largest magnitude of every row maps to +-127
    arg = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(codes[np.arange(1000), arg].astype(np.int32)) == 127)
    # dequantisation error: at most half a step (plus the float32 rounding of the scale)
    err = np.abs(oracle.dequantize_int8(codes, scales) - x.astype(np.float64))
    assert np.all(err <= scales[:, None].astype(np.float64) * (0.5 + 1e-5))


def test_special_rows():
    c, s = oracle.quantize_int8(np.array([[np.nan, 1.0, -1.0, 0.0]], np.float32))
    # a NaN element is ignored by the max and clamps to -127; the rest as usual
    assert c[0].tolist() == [-127, 127, -127, 0] and s[0] == np.float32(1) / np.float32(127)
    c, s = oracle.quantize_int8(np.array([[np.inf, 1.0]], np.float32))
    # amax inf -> inv 0 -> inf * 0 = NaN clamps to -127, 1 * 0 = 0; scale inf
    assert c[0].tolist() == [-127, 0] and np.isinf(s[0])
