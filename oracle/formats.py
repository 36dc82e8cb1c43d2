"""Element formats used by the quantized KV cache, in exact float64 arithmetic.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg only.

Formats (Model-Optimizer PR #714, Testing section: "(2, 1) bit" elements with
"scale_bits (4, 3)"; compressed-tensors PR #436 ``kv_cache_scheme``:
``num_bits 8, type float``):

* E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit, no inf/NaN.
  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* E4M3 (the "FN" variant: max 448, NaN only at S.1111.111, no inf):
  1 sign, 4 exponent bits (bias 7), 3 mantissa bits, subnormals 2^-9 .. 7*2^-9.

Encoding is round-to-nearest, ties to the even code (ties to an even
mantissa), saturating to the largest finite magnitude, sign kept (a negative
value that rounds to zero encodes as the negative-zero code).  Every operation
below is a power-of-two scaling, ``np.rint`` (round half to even) or a compare,
so the result is the exact real-number rounding of the float64 input.
"""
import numpy as np

E2M1_MAX = 6.0
E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# generic minifloat rounding
# --------------------------------------------------------------------------
def _rne_minifloat(mag, mbits, emin, maxval):
    """Round non-negative float64 ``mag`` to the nearest value of a binary
    float format with ``mbits`` explicit mantissa bits and minimum normal
    exponent ``emin`` (subnormals below 2**emin), ties to even, saturating at
    ``maxval``.

    The binade exponent e = floor(log2 mag) comes from frexp; the quantum of
    that binade is 2**(e - mbits) (clamped to the subnormal quantum); mag/q is
    an exact power-of-two scaling and rint rounds half to even, which is the
    even-mantissa tie rule.  A carry into the next binade (n == 2**(mbits+1))
    is still the correct grid value.
    """
    mag = np.asarray(mag, dtype=np.float64)
    if np.any(mag < 0) or not np.all(np.isfinite(mag)):
        raise ValueError("_rne_minifloat expects finite non-negative magnitudes")
    _, ex = np.frexp(mag)              # mag = f * 2**ex, f in [0.5, 1)
    e = np.maximum(ex - 1, emin)       # floor(log2 mag), clamped to the subnormal binade
    q = np.ldexp(1.0, e - mbits)
    n = np.rint(mag / q)
    return np.minimum(n * q, maxval)


# --------------------------------------------------------------------------
# E2M1
# --------------------------------------------------------------------------
def e2m1_decode(code):
    """E2M1 code (0..15, bit 3 = sign) -> float64 value."""
    c = np.asarray(code, dtype=np.int64)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where((c & 8) != 0, -mag, mag)


def e2m1_round(r):
    """Value of the E2M1 rounding of float64 ``r`` (sign kept, saturating)."""
    r = np.asarray(r, dtype=np.float64)
    v = _rne_minifloat(np.abs(r), mbits=1, emin=0, maxval=E2M1_MAX)
    return np.where(np.signbit(r), -v, v)


def e2m1_encode(r):
    """E2M1 code (uint8 0..15) of float64 ``r``: RNE, ties to even, saturating,
    sign kept (negative values that round to 0 give code 0x8)."""
    r = np.asarray(r, dtype=np.float64)
    v = _rne_minifloat(np.abs(r), mbits=1, emin=0, maxval=E2M1_MAX)
    # value -> magnitude bits: v < 1 is subnormal (code = v / 0.5), else
    # e = floor(log2 v), code = (e + 1) << 1 | mantissa bit.
    _, ex = np.frexp(np.where(v >= 1.0, v, 1.0))
    e = ex - 1
    frac = np.where(v >= 1.0, v / np.ldexp(1.0, e), 1.0)
    normal = ((e + 1) << 1) | np.rint((frac - 1.0) * 2.0).astype(np.int64)
    mag = np.where(v >= 1.0, normal, np.rint(v / 0.5).astype(np.int64))
    sign = np.where(np.signbit(r), 8, 0)
    return (mag | sign).astype(np.uint8)


# --------------------------------------------------------------------------
# E4M3 (FN)
# --------------------------------------------------------------------------
def e4m3_decode(code):
    """E4M3FN code (0..255) -> float64 value (NaN for 0x7F / 0xFF)."""
    c = np.asarray(code, dtype=np.int64)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where((c & 0x80) != 0, -mag, mag)


def e4m3_round(r):
    """Value of the E4M3 rounding of float64 ``r`` (sign kept, saturating)."""
    r = np.asarray(r, dtype=np.float64)
    v = _rne_minifloat(np.abs(r), mbits=3, emin=-6, maxval=E4M3_MAX)
    return np.where(np.signbit(r), -v, v)


def e4m3_encode(r):
    """E4M3FN code (uint8) of float64 ``r``: RNE, ties to even, saturating at
    448 (never NaN), sign kept (-0 and negative underflow give 0x80)."""
    r = np.asarray(r, dtype=np.float64)
    v = _rne_minifloat(np.abs(r), mbits=3, emin=-6, maxval=E4M3_MAX)
    normal_mask = v >= np.ldexp(1.0, -6)
    _, ex = np.frexp(np.where(normal_mask, v, 1.0))
    e = ex - 1
    frac = np.where(normal_mask, v / np.ldexp(1.0, e), 1.0)
    normal = ((e + 7) << 3) | np.rint((frac - 1.0) * 8.0).astype(np.int64)
    sub = np.rint(v / np.ldexp(1.0, -9)).astype(np.int64)
    mag = np.where(normal_mask, normal, sub)
    sign = np.where(np.signbit(r), 0x80, 0)
    return (mag | sign).astype(np.uint8)


# --------------------------------------------------------------------------
# bf16 / fp32
# --------------------------------------------------------------------------
def fp32_round(r):
    """float64 -> nearest float32 (IEEE RNE), returned as float64."""
    return np.asarray(r, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_round(r):
    """float64 -> nearest bfloat16 (8 significant bits, 8 exponent bits, RNE),
    returned as float64.  Finite inputs inside bf16's range only."""
    r = np.asarray(r, dtype=np.float64)
    v = _rne_minifloat(np.abs(r), mbits=7, emin=-126, maxval=np.float64(3.3895313892515355e38))
    return np.where(np.signbit(r), -v, v)


def bf16_ulp(r):
    """Spacing of bfloat16 values at |r| (the ulp of the binade holding r)."""
    r = np.abs(np.asarray(r, dtype=np.float64))
    _, ex = np.frexp(np.where(r > 0, r, 1.0))
    e = np.maximum(ex - 1, -126)
    return np.ldexp(1.0, e - 7)
