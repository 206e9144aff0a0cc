"""Pins for the oracle's E5M2 codec (CPU only).

The fp8 KV cache stores E5M2 codes written by a cast on store and read back by
a cast to a wider type (Colossal-Inference release post, section "KV缓存量化
(KVCache Quant)").  The oracle's encoder is a nearest-value search; it is
checked against (1) spot values derived from the format by hand
(tests/golden/e5m2_codes.txt), (2) a bit-level rounding routine written here
(a different algorithm), and (3) torch's own CPU cast as a third witness,
over all 65,536 bf16 bit patterns.
"""
import os

import numpy as np
import pytest
import torch

from conftest import GOLDEN
from oracle import bf16_to_f64, e5m2_to_f64, f64_to_e5m2

ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _parse_value(tok: str) -> float:
    tok = tok.strip()
    if tok in ("inf", "-inf"):
        return float(tok)
    if "2^" in tok:
        coef, _, exp = tok.partition("2^")
        c = float(coef.rstrip("*")) if coef else 1.0
        return c * 2.0 ** float(exp)
    return float(tok)


def _golden_codes():
    rows = []
    with open(os.path.join(GOLDEN, "e5m2_codes.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((_parse_value(parts[0]), int(parts[1], 16)))
    return rows


def _bitwise_bf16_to_e5m2(b: int) -> int:
    """Round a bf16 bit pattern to E5M2 with integer operations only."""
    s = (b >> 15) & 1
    a = b & 0x7FFF
    if a > 0x7F80:
        return (s << 7) | 0x7F
    if a == 0x7F80:
        return (s << 7) | 0x7C
    e = a >> 7
    m = a & 0x7F
    if e >= 113:  # at or above 2^-14: re-bias 127 -> 15, drop 5 mantissa bits
        x = a - (112 << 7)
        q, r = x >> 5, x & 31
        if r > 16 or (r == 16 and (q & 1)):
            q += 1
        return (s << 7) | min(q, 0x7C)
    if e == 0:
        return s << 7
    # below 2^-14: code = value / 2^-16 rounded to nearest even
    mant = m | 0x80
    sh = 118 - e
    if sh > 9:
        return s << 7
    q, r, half = mant >> sh, mant & ((1 << sh) - 1), 1 << (sh - 1)
    if r > half or (r == half and (q & 1)):
        q += 1
    return (s << 7) | q


def test_golden_spot_values():
    for value, code in _golden_codes():
        got = int(f64_to_e5m2(np.array([value]))[0])
        assert got == code, (value, hex(got), hex(code))


def test_decode_all_codes_against_format_and_torch():
    codes = np.arange(256, dtype=np.uint32).astype(np.uint8)
    val = e5m2_to_f64(codes)
    # format facts
    assert val[0x3C] == 1.0 and val[0x7B] == 57344.0 and val[0x01] == 2.0**-16
    assert val[0x04] == 2.0**-14 and val[0x03] == 3 * 2.0**-16
    assert np.isinf(val[0x7C]) and val[0x7C] > 0 and np.isinf(val[0xFC]) and val[0xFC] < 0
    assert np.all(np.isnan(val[[0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]]))
    assert val[0x80] == 0.0 and np.signbit(val[0x80])
    # ascending magnitude over the finite positive codes
    assert np.all(np.diff(val[:0x7C]) > 0)
    # third-party witness: torch's e5m2 -> float32
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e5m2).to(torch.float64).numpy()
    same = (val == ref) | (np.isnan(val) & np.isnan(ref))
    assert same.all()


def test_round_trip_identity_on_non_nan_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) <= 0x7C], dtype=np.uint8)
    back = f64_to_e5m2(e5m2_to_f64(codes))
    assert np.array_equal(back, codes)


def test_exhaustive_bf16_against_bitwise_rounding():
    x = bf16_to_f64(ALL_BF16)
    got = f64_to_e5m2(x)
    want = np.array([_bitwise_bf16_to_e5m2(int(b)) for b in ALL_BF16], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(int(ALL_BF16[i])), hex(int(got[i])), hex(int(want[i]))) for i in bad[:10]]


def test_exhaustive_bf16_against_torch_cast():
    t = torch.from_numpy(ALL_BF16.view(np.int16).copy()).view(torch.bfloat16)
    ref = t.to(torch.float8_e5m2).view(torch.uint8).numpy()
    got = f64_to_e5m2(bf16_to_f64(ALL_BF16))
    nan = np.isnan(bf16_to_f64(ALL_BF16))
    # NaN payload/sign conventions may differ between libraries: compare NaN-ness there
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(e5m2_to_f64(ref[nan]))) and np.all(np.isnan(e5m2_to_f64(got[nan])))


def test_rounding_is_nearest_and_monotone():
    x = bf16_to_f64(ALL_BF16)
    finite = np.isfinite(x) & (np.abs(x) < 57344.0)
    code = f64_to_e5m2(x[finite])
    back = e5m2_to_f64(code)
    # no finite E5M2 value is strictly closer than the chosen one
    mags = e5m2_to_f64(np.arange(0x7C, dtype=np.uint8))
    cand = np.concatenate([mags, -mags])
    best = np.min(np.abs(x[finite][:, None] - cand[None, :]), axis=1)
    assert np.all(np.abs(x[finite] - back) == best)
    pos = np.sort(x[finite & (x >= 0)])
    assert np.all(np.diff(e5m2_to_f64(f64_to_e5m2(pos))) >= 0)


@pytest.mark.parametrize("v", [1e-30, -1e-30, 7.62939453125e-06])
def test_tiny_values_flush_with_sign(v):
    c = int(f64_to_e5m2(np.array([v]))[0])
    assert c & 0x7F == 0 and (c >> 7) == (1 if v < 0 else 0)
