"""Pins for the oracle's element codecs (E2M1, E4M3, bf16).

Each encoder is checked against something other than itself: hand-written
tables under tests/golden/, exhaustive enumeration of the code space,
brute-force nearest-value search in exact rational arithmetic, and torch's own
float8_e4m3fn / bfloat16 casts (library routines) on float32 inputs.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- E2M1
def test_e2m1_decode_matches_handwritten_table():
    for code_s, val_s in _read_table("e2m1_table.txt"):
        code = int(code_s, 16)
        val = float(val_s)
        got = float(F.e2m1_decode(code))
        assert got == val and math.copysign(1, got) == math.copysign(1, val), (code, got, val)


def _brute_e2m1(x: Fraction):
    """Nearest E2M1 magnitude by exhaustive search, ties -> even code."""
    mags = [(c, Fraction(v).limit_denominator(4)) for c, v in
            [(0, 0), (1, 0.5), (2, 1), (3, 1.5), (4, 2), (5, 3), (6, 4), (7, 6)]]
    a = abs(x)
    best = min(mags, key=lambda cv: (abs(cv[1] - a), cv[0] & 1))
    return best[0]


def test_e2m1_encode_bruteforce_at_thresholds():
    # every midpoint, and one float64 ulp either side of it
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    xs = []
    for m in mids:
        xs += [m, np.nextafter(m, 0), np.nextafter(m, 10)]
    xs += [0.0, 0.5, 6.0, 6.5, 7.0, 100.0, 1e-300]
    for x in xs:
        for sgn in (1.0, -1.0):
            v = sgn * x
            want = _brute_e2m1(Fraction(v)) if abs(v) <= 6 else 7
            got = int(F.e2m1_encode(v))
            assert got & 7 == want, (v, got, want)
            assert (got >> 3) == (1 if np.signbit(v) else 0)


@settings(max_examples=400, deadline=None)
@given(st.floats(min_value=-8, max_value=8, allow_nan=False))
def test_e2m1_encode_bruteforce_random(x):
    got = int(F.e2m1_encode(x))
    want = _brute_e2m1(Fraction(x)) if abs(x) <= 6 else 7
    assert got & 7 == want


def test_e2m1_decode_encode_identity():
    for c in range(16):
        assert int(F.e2m1_encode(F.e2m1_decode(c))) == c


# ---------------------------------------------------------------- E4M3
def _e4m3_positive_values():
    vals = [float(F.e4m3_decode(c)) for c in range(0x7F)]  # 0x00 .. 0x7E
    return vals


def test_e4m3_code_space():
    vals = [float(F.e4m3_decode(c)) for c in range(256)]
    nan_codes = [c for c, v in enumerate(vals) if math.isnan(v)]
    assert nan_codes == [0x7F, 0xFF]
    pos = _e4m3_positive_values()
    assert sum(1 for v in pos if v > 0) == 126
    assert max(pos) == 448.0 and pos.index(448.0) == 0x7E
    assert min(v for v in pos if v > 0) == 2.0 ** -9 and pos.index(2.0 ** -9) == 0x01
    assert all(a < b for a, b in zip(pos, pos[1:])), "positive codes must be monotone"
    for c in range(0x7F):
        assert float(F.e4m3_decode(c | 0x80)) == -pos[c]


def _brute_e4m3(x: Fraction):
    a = abs(x)
    if a >= 448:
        return 0x7E
    cands = [(c, Fraction(v)) for c, v in enumerate(_E4M3_POS)]
    best = min(cands, key=lambda cv: (abs(cv[1] - a), cv[0] & 1))
    return best[0]


_E4M3_POS = None


@pytest.fixture(autouse=True, scope="module")
def _e4m3_table():
    global _E4M3_POS
    _E4M3_POS = _e4m3_positive_values()


def test_e4m3_encode_bruteforce_at_midpoints():
    pos = _E4M3_POS
    xs = []
    for a, b in zip(pos, pos[1:]):
        m = (a + b) / 2
        xs += [m, np.nextafter(m, 0), np.nextafter(m, 1e9), a]
    xs += [448.0, 460.0, 464.0, 470.0, 1e6, 0.0]
    for x in xs:
        for sgn in (1.0, -1.0):
            v = sgn * x
            got = int(F.e4m3_encode(v))
            assert got & 0x7F == _brute_e4m3(Fraction(v)), (v, hex(got))
            assert (got >> 7) == (1 if np.signbit(v) else 0)


def test_e4m3_encode_matches_golden():
    for x_s, code_s in _read_table("fp8_values.txt"):
        assert int(F.e4m3_encode(float(x_s))) == int(code_s, 16), x_s


def test_e4m3_encode_matches_torch_cast():
    # torch's float8_e4m3fn cast rounds to nearest even but does not saturate,
    # so the comparison clamps to +-448 first (library cross-check).
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(50),
        (rng.standard_normal(20000) * 2.0 ** rng.integers(-14, 9, 20000)).astype(np.float32),
        np.array([0.0, -0.0, 448.0, -448.0, 2 ** -9, 2 ** -10, 3 * 2 ** -10], np.float32),
    ])
    xc = np.clip(x, -448, 448)
    want = torch.from_numpy(xc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_e4m3_decode_encode_identity():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert int(F.e4m3_encode(F.e4m3_decode(c))) == c


# ---------------------------------------------------------------- bf16 / fp32
def test_bf16_round_matches_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(50000) * 2.0 ** rng.integers(-30, 30, 50000)).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(F.bf16_round(x.astype(np.float64)), want)


def test_bf16_ulp():
    assert F.bf16_ulp(1.0) == 2.0 ** -7
    assert F.bf16_ulp(1.99) == 2.0 ** -7
    assert F.bf16_ulp(0.5) == 2.0 ** -8
    assert F.bf16_ulp(60.0) == 2.0 ** -2


def test_fp32_round_is_ieee():
    x = np.array([1 / 3, 2 / 3, 1e-40, 123456789.0])
    assert np.array_equal(F.fp32_round(x), x.astype(np.float32).astype(np.float64))


def test_e4m3_decode_matches_torch_view():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(np.arange(256))
    both_nan = np.isnan(want) & np.isnan(got)
    assert np.array_equal(np.where(both_nan, 0, got), np.where(both_nan, 0, want))
    assert np.array_equal(np.signbit(got[~both_nan]), np.signbit(want[~both_nan]))
