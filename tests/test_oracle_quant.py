"""Pins for the oracle's calibration and NVFP4 / FP8 packing.

Pinned against: hand-worked blocks (tests/golden/nvfp4_blocks.txt,
tests/golden/fp8_values.txt), a brute-force packer in exact rational
arithmetic written independently of the oracle, and the format invariants the
method fixes (every dequantized value on the E2M1 grid times its block scale,
block scales exact E4M3 values, the block max mapping to 6, idempotence).
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import kvq_synth
from oracle import formats as F
from oracle import quant as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

E2M1_GRID = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])


# ------------------------------------------------------------ brute force
def _torch_e4m3_values():
    codes = torch.arange(0x7F, dtype=torch.int32).to(torch.uint8)
    return [Fraction(float(v)) for v in codes.view(torch.float8_e4m3fn).to(torch.float64)]


E4M3_FRAC = _torch_e4m3_values()          # library decode of codes 0x00..0x7E
E2M1_FRAC = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
             Fraction(3), Fraction(4), Fraction(6)]


def _nearest(cands, a):
    """index of the nearest candidate, ties to the even index (= even code)."""
    return min(range(len(cands)), key=lambda i: (abs(cands[i] - a), i & 1))


def brute_nvfp4_block(xs, s_t):
    """Exhaustive NVFP4 packing of one 16-block in exact rationals.
    Returns (scale_code, [16 element codes])."""
    s_t = Fraction(s_t)
    bamax = max(abs(Fraction(x)) for x in xs)
    target = bamax / (6 * s_t)
    sc = 0x7E if target >= 448 else _nearest(E4M3_FRAC, target)
    s_hat = E4M3_FRAC[sc]
    if s_hat == 0:
        return 0, [0] * 16
    out = []
    for x in xs:
        r = abs(Fraction(x)) / (s_hat * s_t)
        c = 7 if r >= 6 else _nearest(E2M1_FRAC, r)
        if np.signbit(x):
            c |= 8
        out.append(c)
    return sc, out


def _unpack_nibbles(packed):
    packed = np.asarray(packed, np.uint8)
    return np.stack([packed & 0xF, packed >> 4], -1).reshape(packed.shape[:-1] + (-1,))


# ------------------------------------------------------------ golden
def _golden_blocks():
    cases = []
    with open(os.path.join(GOLDEN, "nvfp4_blocks.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if not line:
                continue
            head, xs, sc, codes = [p.strip() for p in line.split("|")]
            amax = float(head.split("amax=")[1])
            cases.append((head.split()[0], amax, [float(v) for v in xs.split()], int(sc, 16),
                          [int(c, 16) for c in codes.split()]))
    return cases


@pytest.mark.parametrize("case", _golden_blocks(), ids=lambda c: c[0])
def test_nvfp4_golden_blocks(case):
    _, amax, xs, sc, codes = case
    packed, scales, s_t = Q.nvfp4_pack(np.array([xs]), amax)
    assert list(packed[0]) == codes
    assert int(scales[0, 0]) == sc


@pytest.mark.parametrize("case", _golden_blocks(), ids=lambda c: c[0])
def test_bruteforce_agrees_with_golden(case):
    # the independent brute-force packer reproduces the hand-worked bytes
    _, amax, xs, sc, codes = case
    s_t = float(np.float32(amax / 2688.0))
    bsc, bcodes = brute_nvfp4_block(xs, s_t)
    assert bsc == sc
    assert [bcodes[2 * j] | (bcodes[2 * j + 1] << 4) for j in range(8)] == codes


def test_fp8_golden_values():
    rows = []
    with open(os.path.join(GOLDEN, "fp8_values.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    x = np.array([float(r[0]) for r in rows])
    codes, scale = Q.fp8_pack(x, 448.0)
    assert scale == 1.0
    assert [int(c) for c in codes] == [int(r[1], 16) for r in rows]


# ------------------------------------------------------------ tensor scale
def test_tensor_scales():
    assert Q.nvfp4_tensor_scale(2688.0) == 1.0
    assert Q.nvfp4_tensor_scale(0.0) == 1.0
    assert Q.fp8_tensor_scale(0.0) == 1.0
    assert Q.fp8_tensor_scale(448.0) == 1.0
    a = np.float32(7.53125)  # a printed latent amax (PR #714)
    assert Q.nvfp4_tensor_scale(a) == float(np.float32(np.float64(a) / 2688.0))
    assert Q.fp8_tensor_scale(a) == float(np.float32(np.float64(a) / 448.0))


# ------------------------------------------------------------ brute force vs oracle
def test_nvfp4_matches_bruteforce_random_blocks():
    rng = np.random.default_rng(11)
    for trial in range(300):
        amax = float(np.float32(np.abs(rng.standard_normal()) * 10 + 1e-3))
        scale_exp = rng.integers(-12, 3)
        xs = (rng.standard_normal(16) * 2.0 ** scale_exp).astype(np.float32)
        xs = np.clip(xs, -amax, amax).astype(np.float64)
        packed, scales, s_t = Q.nvfp4_pack(xs[None], amax)
        bsc, bcodes = brute_nvfp4_block(list(xs), s_t)
        assert int(scales[0, 0]) == bsc, (trial, xs, amax)
        assert list(_unpack_nibbles(packed)[0]) == bcodes, (trial, xs, amax)


@settings(max_examples=150, deadline=None)
@given(st.lists(st.floats(min_value=-1000, max_value=1000, width=32), min_size=16, max_size=16),
       st.floats(min_value=0.0009765625, max_value=3000, width=32))
def test_nvfp4_matches_bruteforce_hypothesis(xs, amax):
    xs = np.array(xs, dtype=np.float64)
    amax = max(amax, float(np.abs(xs).max()))
    packed, scales, s_t = Q.nvfp4_pack(xs[None], amax)
    bsc, bcodes = brute_nvfp4_block(list(xs), s_t)
    assert int(scales[0, 0]) == bsc
    assert list(_unpack_nibbles(packed)[0]) == bcodes


def test_nvfp4_threshold_ties_exact():
    # elements placed exactly on, and one ulp around, every E2M1 midpoint
    # times s_hat * s_t, for several block scales: brute force decides.
    s_t = float(np.float32(3.0 / 2688.0))
    for s_hat in [1.0, 0.875, 2.0 ** -7, 3 * 2.0 ** -9, 448.0, 13 * 2.0 ** -8]:
        d = s_hat * s_t
        for mid in [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]:
            for x in [mid * d, np.nextafter(mid * d, 0), np.nextafter(mid * d, 1)]:
                xs = np.zeros(16)
                xs[0] = 6 * d  # pins the block scale to s_hat
                xs[1] = x
                xs[2] = -x
                bsc, bcodes = brute_nvfp4_block(list(xs), s_t)
                packed, scales, _ = Q.nvfp4_pack(xs[None], 3.0)
                assert int(scales[0, 0]) == bsc
                assert list(_unpack_nibbles(packed)[0]) == bcodes


# ------------------------------------------------------------ invariants
def _gqa_small():
    inp = kvq_synth.gqa_inputs(2, 8, 2, 128, 64, outliers=True, config="gqa", salt=99)
    return kvq_synth.f64(inp.k)


def test_grid_fact_and_scale_bytes():
    x = _gqa_small()
    a = Q.amax(x)
    packed, scales, s_t = Q.nvfp4_pack(x, a)
    s_hat = F.e4m3_decode(scales)
    assert np.all(np.isfinite(s_hat)) and np.all(s_hat >= 0)
    xhat = Q.nvfp4_unpack(packed, scales, s_t)
    ratio = xhat / (np.repeat(s_hat, 16, -1) * s_t)
    ratio = np.where(np.repeat(s_hat, 16, -1) == 0, 0, ratio)
    assert np.all(np.isin(np.abs(ratio), E2M1_GRID))


def test_block_max_maps_to_six():
    x = _gqa_small()
    a = Q.amax(x)
    packed, scales, s_t = Q.nvfp4_pack(x, a)
    codes = _unpack_nibbles(packed).reshape(x.shape[:-1] + (8, 16))
    s_hat = F.e4m3_decode(scales)
    normal = s_hat >= 2.0 ** -6
    maxmag = (codes & 7).max(-1)
    assert np.all(maxmag[normal] == 7)
    # the block holding the tensor amax gets the largest scale 448 (0x7E)
    flat_idx = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert scales[flat_idx[:-1] + (flat_idx[-1] // 16,)] == 0x7E


def test_idempotence_normal_blocks():
    x = _gqa_small()
    a = Q.amax(x)
    packed, scales, s_t = Q.nvfp4_pack(x, a)
    xhat = Q.nvfp4_unpack(packed, scales, s_t)
    # re-calibrating from the dequantized tensor reproduces s_t
    assert Q.nvfp4_tensor_scale(Q.amax(xhat)) == s_t
    packed2, scales2, s_t2 = Q.nvfp4_pack(xhat, Q.amax(xhat))
    s_hat = F.e4m3_decode(scales)
    ok = (s_hat == 0) | (s_hat >= 2.0 ** -6)
    assert np.array_equal(scales2[ok], scales[ok])
    pk = _unpack_nibbles(packed).reshape(x.shape[:-1] + (8, 16))
    pk2 = _unpack_nibbles(packed2).reshape(x.shape[:-1] + (8, 16))
    assert np.array_equal(pk2[ok], pk[ok])


def test_idempotence_documented_exception():
    # a subnormal block scale whose block max lands on code 4: re-packing the
    # dequantized block picks a smaller scale (documented exception).
    s_t = 1.0
    xs = np.zeros(16)
    xs[0] = 6 * s_t * 1.6 * 2.0 ** -9       # bamax/(6 s_t) = 1.6 * 2^-9 -> s_hat = 2^-8
    packed, scales, st_ = Q.nvfp4_pack(xs[None], 2688.0)
    assert float(F.e4m3_decode(scales[0, 0])) == 2.0 ** -8
    assert int(packed[0, 0] & 0xF) == 6     # 9.6 * 2^-9 / 2^-8 = 4.8 -> 4
    xhat = Q.nvfp4_unpack(packed, scales, st_)
    _, scales2, _ = Q.nvfp4_pack(xhat, 2688.0)
    # x_hat max = 4 * 2^-8 = 2^-6; 2^-6 / 6 = 1.33 * 2^-9 -> s_hat' = 2^-9, not 2^-8
    assert float(F.e4m3_decode(scales2[0, 0])) == 2.0 ** -9
    assert scales2[0, 0] != scales[0, 0]


def test_on_grid_round_trip():
    rng = np.random.default_rng(5)
    rows, nb = 32, 8
    codes = rng.integers(0, 16, size=(rows, nb, 16))
    codes[:, :, 0] = 7 | (rng.integers(0, 2, size=(rows, nb)) << 3)   # block max 6
    sc = rng.integers(0x08, 0x7F, size=(rows, nb))                     # normal scales
    amax_x = 6 * F.e4m3_decode(sc).max()
    s_t = Q.nvfp4_tensor_scale(np.float32(amax_x))
    # choose s_t so that the largest block scale maps to itself: amax = 2688 s_t
    x = F.e2m1_decode(codes) * F.e4m3_decode(sc)[..., None] * s_t
    x = x.reshape(rows, nb * 16)
    a = np.float32(Q.amax(x))
    packed, scales, s_t2 = Q.nvfp4_pack(x, a)
    # the tensor's own amax gives a different s_t unless max scale is 448; we
    # therefore pack with amax = 2688 * s_t directly
    packed, scales, s_t3 = Q.nvfp4_pack(x, np.float32(2688.0 * s_t))
    assert s_t3 == s_t
    assert np.array_equal(scales, sc.astype(np.uint8))
    assert np.array_equal(_unpack_nibbles(packed).reshape(rows, nb, 16), codes)


def test_fp8_idempotent_and_bruteforce():
    x = _gqa_small()
    a = Q.amax(x)
    codes, scale = Q.fp8_pack(x, a)
    xhat = Q.fp8_unpack(codes, scale)
    codes2, scale2 = Q.fp8_pack(xhat, Q.amax(xhat))
    assert scale2 == scale
    assert np.array_equal(codes2, codes)
    flat = x.reshape(-1)[:2000]
    fs = Fraction(scale)
    for xv, cv in zip(flat, codes.reshape(-1)[:2000]):
        r = abs(Fraction(float(xv))) / fs
        want = 0x7E if r >= 448 else _nearest(E4M3_FRAC, r)
        assert int(cv) & 0x7F == want
        assert (int(cv) >> 7) == int(np.signbit(xv))


# ------------------------------------------------------------ amax
def test_amax_masks_padding():
    x = np.zeros((2, 3, 10, 4))
    x[0, 1, 2, 3] = -5.0
    x[1, 0, 7, 0] = 9.0       # beyond kv_len of request 1
    x[1, 2, 3, 1] = 4.0
    assert Q.amax(x) == 9.0
    assert Q.amax(x, kv_lens=[10, 5]) == 5.0
    assert Q.amax(x, kv_lens=[0, 0]) == 0.0
    # MLA layout [B, L, D]
    y = np.zeros((2, 6, 8))
    y[1, 5, 0] = 3.0
    y[0, 2, 7] = -2.0
    assert Q.amax(y, kv_lens=[6, 5], token_axis=1) == 2.0


# ------------------------------------------------------------ FP8 per kv head
def test_fp8_heads_worked_example():
    """Hand-worked: head 0 has amax 448 (scale 1), head 1 amax 3.5 (scale
    2^-7, exact).  0.78125 sits on an E4M3 midpoint in both heads: in head 0
    between 0.75 and 0.8125 -> 0.75 (even mantissa, code 0x34); in head 1
    0.78125 / 2^-7 = 100 lies between 96 and 104 -> 96 (code 0x6C).  Each
    head's max maps to 448 (0x7E); a negative value keeps the sign bit."""
    x = np.zeros((1, 2, 2, 4))
    x[0, 0, 0, 0], x[0, 1, 1, 3] = 448.0, -3.5
    x[0, 0, 1, 2] = x[0, 1, 0, 1] = 0.78125
    a = Q.amax_heads(x)
    assert list(a) == [448.0, 3.5]
    codes, scales = Q.fp8_pack_heads(x, a)
    assert list(scales) == [1.0, 2.0 ** -7]
    assert codes[0, 0, 1, 2] == 0x34 and codes[0, 1, 0, 1] == 0x6C
    assert codes[0, 0, 0, 0] == 0x7E and codes[0, 1, 1, 3] == 0xFE
    # per tensor the same value in head 1 would use scale 1
    pt, _ = Q.fp8_pack(x, Q.amax(x))
    assert pt[0, 1, 0, 1] == 0x34
    back = Q.fp8_unpack_heads(codes, scales)
    assert back[0, 1, 0, 1] == 96 * 2.0 ** -7 and back[0, 1, 1, 3] == -3.5


def test_fp8_heads_reduce_to_per_tensor():
    """Invariants: the largest head amax is the tensor amax; with every head
    given the tensor amax, per-head packing equals per-tensor packing; each
    head's codes equal the per-tensor packing of that head alone."""
    rng = np.random.default_rng(5)
    x = kvq_synth.f64(torch.from_numpy(rng.standard_normal((3, 4, 33, 16)) * rng.uniform(0.1, 30, (1, 4, 1, 1))).to(torch.bfloat16))
    lens = np.array([33, 7, 1], dtype=np.int32)
    a = Q.amax_heads(x, lens)
    assert a.max() == Q.amax(x, lens)
    for h in range(4):
        assert a[h] == Q.amax(x[:, h], lens)
    full = np.full(4, Q.amax(x, lens))
    c_all, s_all = Q.fp8_pack_heads(x, full)
    c_pt, s_pt = Q.fp8_pack(x, Q.amax(x, lens))
    assert np.array_equal(c_all, c_pt) and np.all(s_all == s_pt)
    c_h, s_h = Q.fp8_pack_heads(x, a)
    for h in range(4):
        c1, s1 = Q.fp8_pack(x[:, h], a[h])
        assert np.array_equal(c_h[:, h], c1) and s_h[h] == s1


def test_fp8_query_worked_example():
    """FP8 query, hand-worked E4M3 codes (bias 7, 3 mantissa bits, ties to
    even).  Per tensor: amax 448 gives scale 1; 448 = 1.75 * 2^8 -> 0x7E,
    1.0625 (midway 1.0 / 1.125) -> 1.0 = 0x38, 1.1875 (midway 1.125 / 1.25)
    -> 1.25 = 0x3A, -3 = -1.5 * 2^1 -> 0xC4, 224 = 1.75 * 2^7 -> 0x76,
    0.5 -> 0x30.  Per head: head 1 has amax 224, scale 0.5, so 224 -> 0x7E
    and 0.5 -> 1.0 = 0x38, dequantized back to 224 and 0.5."""
    q = np.zeros((1, 2, 16))
    q[0, 0, :5] = [448.0, 1.0625, 1.1875, -3.0, 0.0]
    q[0, 1, :2] = [224.0, 0.5]
    codes, scales, qhat = Q.fp8_quantize_query(q)
    assert scales.tolist() == [1.0]
    assert codes[0, 0, :5].tolist() == [0x7E, 0x38, 0x3A, 0xC4, 0x00]
    assert codes[0, 1, :2].tolist() == [0x76, 0x30]
    assert qhat[0, 0, :4].tolist() == [448.0, 1.0, 1.25, -3.0]
    codes, scales, qhat = Q.fp8_quantize_query(q, per_head=True)
    assert scales.tolist() == [1.0, 0.5]
    assert codes[0, 1, :2].tolist() == [0x7E, 0x38]
    assert qhat[0, 1, :2].tolist() == [224.0, 0.5]
    assert codes[0, 0, :5].tolist() == [0x7E, 0x38, 0x3A, 0xC4, 0x00]


def test_fp8_query_properties():
    """Values already on the E4M3 grid times the scale come back unchanged;
    per head equals per tensor when every head has the same amax; the
    per-tensor error is at most half a code step (relative 2^-4) above the
    E4M3 subnormal range."""
    rng = np.random.default_rng(11)
    grid = F.e4m3_decode(np.arange(0x08, 0x7F, dtype=np.uint8))   # positive normal E4M3 values
    q = rng.choice(grid, size=(2, 4, 32)) * rng.choice([-1.0, 1.0], size=(2, 4, 32))
    q[:, :, 0] = 448.0   # every head's amax is 448: scale 1
    codes, scales, qhat = Q.fp8_quantize_query(q)
    assert scales.tolist() == [1.0] and np.array_equal(qhat, q)
    c2, s2, qh2 = Q.fp8_quantize_query(q, per_head=True)
    assert np.array_equal(c2, codes) and np.array_equal(qh2, qhat) and s2.tolist() == [1.0] * 4
    x = rng.standard_normal((2, 4, 64))
    _, sc, xh = Q.fp8_quantize_query(x)
    big = np.abs(x) / sc[0] >= 2.0 ** -6
    assert np.all(np.abs(xh - x)[big] <= 2.0 ** -4 * np.abs(x)[big] * (1 + 1e-12))
