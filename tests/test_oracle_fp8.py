"""Pins of the oracle's FP8 E4M3 codec and scaled rows (oracle.e4m3_to_f64, f64_to_e4m3,
quantize_e4m3, dequantize_e4m3).

The format is fixed by its definition (OCP E4M3, the "FN" variant: bias 7, no infinities, one
NaN pattern per sign, largest finite 448); the scaling scheme is the library's own (no page
fixes one).  Pinned by the format's landmark values, by torch's own float8_e4m3fn conversion in
both directions, by hand-worked rows (tests/golden/e4m3_rows_hand.txt), by the error bound the
rule implies, and by the special rows.
"""
import os
from fractions import Fraction

import numpy as np
import torch

import oracle
from conftest import GOLDEN


def test_landmark_values():
    v = oracle.e4m3_to_f64
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0          # largest finite
    assert v(0x01) == 2.0**-9 and v(0x07) == 7 * 2.0**-9     # subnormals m * 2^-9
    assert v(0x08) == 2.0**-6                                 # smallest normal
    assert v(0x38) == 1.0 and v(0x39) == 1.125 and v(0x40) == 2.0
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    assert v(0x00) == 0.0 and np.signbit(v(0x80))


def test_decode_matches_torch_on_every_code():
    c = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(c)
    ref = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_encode_matches_torch_in_range():
    """Random float32 values over every binade up to 448, every exact midpoint between adjacent
    codes (ties to even), and the codes' own values: the same code as torch's RNE cast."""
    rng = np.random.default_rng(0)
    mags = np.exp2(rng.uniform(-14, np.log2(448.0), size=20000)).astype(np.float32)
    x = mags * rng.choice([-1, 1], size=mags.size).astype(np.float32)
    ladder = oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = ((ladder[:-1] + ladder[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, ladder.astype(np.float32), np.float32([0.0, -0.0])])
    ours = oracle.f64_to_e4m3(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(ours[i]), hex(ref[i])) for i in bad[:5]]


def test_encode_saturates_and_maps_nan():
    e = oracle.f64_to_e4m3
    assert e(np.float64(464.0)) == 0x7E and e(np.float64(1e30)) == 0x7E and e(np.float64(np.inf)) == 0x7E
    assert e(np.float64(-500.0)) == 0xFE and e(np.float64(-np.inf)) == 0xFE
    assert e(np.float64(np.nan)) == 0x7F and e(np.float64(-np.nan)) == 0x7F
    assert e(np.float64(2.0**-10)) == 0x00          # halfway between 0 and 2^-9: even code 0
    assert e(np.float64(3 * 2.0**-10)) == 0x02      # halfway between 2^-9 and 2^-8: even code 2


def _hand_rows():
    rows = []
    for line in open(os.path.join(GOLDEN, "e4m3_rows_hand.txt")):
        if line.startswith("#") or not line.strip():
            continue
        x, c, s = (part.strip() for part in line.split("|"))
        num, den = s.split("/")
        rows.append(([float(v) for v in x.split(",")], [int(v, 16) for v in c.split(",")], (float(num), float(den))))
    return rows


def test_hand_worked_rows():
    rows = _hand_rows()
    assert len(rows) == 4
    for x, codes, (num, den) in rows:
        c, s = oracle.quantize_e4m3(np.array([x], np.float32))
        assert c[0].tolist() == codes, (x, [hex(v) for v in c[0]])
        assert s[0] == np.float32(np.float32(num) / np.float32(den))


def test_error_bound():
    """Each dequantised value is within half a step of x: 2^-4 |x| for normal codes, half the
    subnormal step (2^-10 of the scaled unit) below them."""
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((500, 128)) * np.exp(rng.uniform(-6, 6, (500, 1)))).astype(np.float32)
    c, s = oracle.quantize_e4m3(x)
    deq = oracle.dequantize_e4m3(c, s)
    err = np.abs(deq - x.astype(np.float64))
    bound = np.maximum(2.0**-4 * np.abs(x.astype(np.float64)), 2.0**-10 * s[:, None].astype(np.float64)) * (1 + 1e-6)
    assert np.all(err <= bound)
    # the largest magnitude of every row maps to +-448
    arg = np.abs(x).argmax(axis=1)
    assert np.all((c[np.arange(500), arg] & 0x7F) == 0x7E)


def test_products_are_rounded_exactly_once():
    """The code is the E4M3 rounding of the float32 product x * inv, checked with exact rationals
    on the float32 values."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((50, 32)) * 3).astype(np.float32)
    c, s = oracle.quantize_e4m3(x)
    ladder = [Fraction(float(v)) for v in oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))]
    for r in range(x.shape[0]):
        amax = np.float32(np.abs(x[r]).max())
        inv = np.float32(np.float32(448) / amax)
        for j in range(x.shape[1]):
            y = Fraction(float(np.float32(x[r, j] * inv)))
            a = abs(y)
            k = min(range(len(ladder)), key=lambda i: (abs(ladder[i] - a), i % 2))
            want = (0x80 if y < 0 else 0) | k
            assert c[r, j] == want, (x[r, j], hex(c[r, j]), hex(want))


def test_special_rows():
    c, s = oracle.quantize_e4m3(np.array([[np.nan, 1.0, -0.5, 0.0]], np.float32))
    # amax 1 ignoring NaN; inv 448: 1 -> 448, -0.5 -> -224; NaN -> 0x7f
    assert c[0].tolist() == [0x7F, 0x7E, 0xF6, 0x00] and s[0] == np.float32(1) / np.float32(448)
    c, s = oracle.quantize_e4m3(np.array([[np.inf, 1.0]], np.float32))
    # amax inf -> inv 0: inf * 0 = NaN -> 0x7f, 1 * 0 = 0; scale inf
    assert c[0].tolist() == [0x7F, 0x00] and np.isinf(s[0])
    c, s = oracle.quantize_e4m3(np.full((1, 4), np.nan, np.float32))
    assert c[0].tolist() == [0x7F] * 4 and np.isnan(s[0])
