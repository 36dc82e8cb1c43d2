"""KV-cache quantization: max calibration, NVFP4 and FP8 E4M3 pack / unpack.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definitions followed
--------------------
* Max calibration: the per-tensor ``amax`` is the maximum absolute value of
  the tensor (Model-Optimizer PR #714, Testing section: ``calibrator=
  MaxCalibrator`` with a printed per-tensor ``amax``; compressed-tensors
  PR #436 ``kv_cache_scheme``: ``observer minmax``, ``symmetric true``,
  ``dynamic false``).  Only valid tokens (t < kv_len of the request) count.

* NVFP4 (PR #714 quantizer dump: E2M1 elements, ``block_sizes={-1: 16}`` with
  ``'type': 'dynamic'`` and ``scale_bits (4, 3)``, plus the per-tensor amax):
  two-level scale.  The per-tensor fp32 scale maps the tensor amax onto the
  largest representable product of an E4M3 scale and an E2M1 element,
  s_t = amax / (448 * 6); each block of 16 consecutive elements along the last
  (head) dimension gets an E4M3 scale chosen dynamically from the block's own
  max, s_hat = E4M3(bamax / (6 * s_t)); elements are E2M1(x / (s_hat * s_t)).
  Reading taken where the page is silent: rounding decisions are made on the
  exact real quotient (float64 here is exact for them, see below), RNE ties to
  even, saturating; an all-zero / underflowing block stores scale 0 and
  codes 0; amax == 0 gives s_t = 1.

* FP8 per-tensor (compressed-tensors PR #436 ``kv_cache_scheme``: 8-bit float,
  ``strategy tensor``, symmetric, static min-max): scale = amax / 448,
  code = E4M3(x / scale); amax == 0 gives scale 1 (Model-Optimizer PR #673:
  a missing KV scale is served as 1).

* FP8 per kv head (compressed-tensors PR #436, "Changes": the ``attn_head``
  strategy of ``_flatten_attention``; "Testing": ``strategy="attn_head"``,
  symmetric, ``static_minmax`` observer, the KV-FP8-Head rows of the GSM8K
  table).  Reading taken: the K (or V) tensor is split along the kv-head
  axis and each head's slice is quantized exactly as a per-tensor FP8 tensor
  of its own: amax_h over the head's valid tokens of every request, scale_h =
  amax_h / 448.

* FP8 query (compressed-tensors PR #436, "Changes": an ``attention`` scheme
  whose ``input_activations`` are 8-bit float with ``strategy tensor``;
  "Testing": the QKV-FP8-Tensor and QKV-FP8-Head rows of the GSM8K table).
  Reading taken: the decode step's query [B, Hq, D] is quantized exactly
  like a KV tensor — per tensor (amax over every element of the query
  batch) or per attention head (amax over that head's elements), scale =
  amax / 448, code = E4M3(q / scale) — and the attention then uses the
  dequantized query code * scale.

Why float64 decides exactly: x has at most 24 significant bits; a threshold
(E2M1 midpoint * s_hat * s_t, or E4M3 midpoint * 6 * s_t) has at most 32.  Two
such dyadic numbers that differ do so by at least 2^-32 relative, far above
float64's 2^-53 quotient error, so comparing the float64 quotient against the
grid midpoints reproduces the real-number decision, ties included.

Packed layout: element 2j of a row goes in the low nibble of code byte j,
element 2j+1 in the high nibble; scale byte k holds the E4M3 bits of block k.
"""
import numpy as np

from . import formats as F

NVFP4_BLOCK = 16
NVFP4_RANGE = F.E4M3_MAX * F.E2M1_MAX  # 2688


def amax(x, kv_lens=None, token_axis=-2):
    """Per-tensor max |x| over valid tokens.

    ``x``: float array whose axis 0 is the request and ``token_axis`` the
    token position; tokens t >= kv_lens[b] are excluded.  Returns float64
    (an element of x, hence exact).  An empty selection gives 0.
    """
    x = np.abs(np.asarray(x, dtype=np.float64))
    if kv_lens is not None:
        ta = token_axis % x.ndim
        t = np.arange(x.shape[ta])
        shape = [1] * x.ndim
        shape[0] = x.shape[0]
        shape[ta] = x.shape[ta]
        valid = (t[None, :] < np.asarray(kv_lens)[:, None]).reshape(shape)
        x = np.where(valid, x, 0.0)
    return float(x.max()) if x.size else 0.0


def nvfp4_tensor_scale(amax_value):
    """s_t = fp32(amax / 2688) for amax > 0, else 1."""
    a = np.float64(np.float32(amax_value))
    if a > 0:
        return float(F.fp32_round(a / NVFP4_RANGE))
    return 1.0


def fp8_tensor_scale(amax_value):
    """scale = fp32(amax / 448) for amax > 0, else 1."""
    a = np.float64(np.float32(amax_value))
    if a > 0:
        return float(F.fp32_round(a / F.E4M3_MAX))
    return 1.0


def nvfp4_pack(x, amax_value):
    """Quantize rows of ``x`` (last dim D, D % 16 == 0) to NVFP4.

    Returns (codes uint8 [..., D/2], scales uint8 [..., D/16], s_t float).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % NVFP4_BLOCK:
        raise ValueError("head dim must be a multiple of 16")
    s_t = nvfp4_tensor_scale(amax_value)
    blocks = x.reshape(x.shape[:-1] + (d // NVFP4_BLOCK, NVFP4_BLOCK))
    bamax = np.abs(blocks).max(axis=-1)
    # block scale: E4M3 rounding of the exact quotient bamax / (6 s_t)
    s_hat = F.e4m3_round(bamax / (F.E2M1_MAX * s_t))
    scale_bytes = F.e4m3_encode(s_hat)
    zero_block = s_hat == 0.0
    scale_bytes = np.where(zero_block, np.uint8(0), scale_bytes).astype(np.uint8)
    denom = np.where(zero_block, 1.0, s_hat * s_t)[..., None]   # exact product
    codes = F.e2m1_encode(blocks / denom)
    codes = np.where(zero_block[..., None], np.uint8(0), codes).astype(np.uint8)
    codes = codes.reshape(x.shape[:-1] + (d,))
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, scale_bytes, s_t


def nvfp4_unpack(codes, scales, s_t):
    """Exact float64 dequantization: E2M1(code) * E4M3(scale) * s_t.

    ``codes`` uint8 [..., D/2], ``scales`` uint8 [..., D/16]."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = codes & 0xF
    hi = codes >> 4
    c = np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
    e = F.e2m1_decode(c)
    s = F.e4m3_decode(np.asarray(scales, dtype=np.uint8))
    s = np.repeat(s, NVFP4_BLOCK, axis=-1)
    return e * s * np.float64(s_t)


def fp8_pack(x, amax_value):
    """Per-tensor FP8 E4M3: returns (codes uint8 [..., D], scale float)."""
    x = np.asarray(x, dtype=np.float64)
    scale = fp8_tensor_scale(amax_value)
    return F.e4m3_encode(x / scale), scale


def fp8_unpack(codes, scale):
    """Exact float64 dequantization E4M3(code) * scale."""
    return F.e4m3_decode(np.asarray(codes, dtype=np.uint8)) * np.float64(scale)


def amax_heads(x, kv_lens=None, head_axis=1, token_axis=-2):
    """Per-kv-head max |x| over valid tokens: one float per index of
    ``head_axis`` (the ``attn_head`` observer), each an element of x."""
    x = np.asarray(x, dtype=np.float64)
    ha = head_axis % x.ndim
    return np.array([amax(np.take(x, h, axis=ha), kv_lens, token_axis=token_axis if token_axis < 0 else token_axis - (token_axis > ha))
                     for h in range(x.shape[ha])], dtype=np.float64)


def fp8_pack_heads(x, amax_values, head_axis=1):
    """FP8 E4M3 with one scale per kv head: head h's slice is quantized as a
    per-tensor FP8 tensor with amax_values[h].  Returns (codes uint8, same
    shape as x; scales float64 [H])."""
    x = np.asarray(x, dtype=np.float64)
    ha = head_axis % x.ndim
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[ha], dtype=np.float64)
    for h in range(x.shape[ha]):
        c, sc = fp8_pack(np.take(x, h, axis=ha), amax_values[h])
        idx = [slice(None)] * x.ndim
        idx[ha] = h
        codes[tuple(idx)] = c
        scales[h] = sc
    return codes, scales


def fp8_unpack_heads(codes, scales, head_axis=1):
    """Exact float64 dequantization with one scale per kv head."""
    codes = np.asarray(codes, dtype=np.uint8)
    ha = head_axis % codes.ndim
    shape = [1] * codes.ndim
    shape[ha] = codes.shape[ha]
    return F.e4m3_decode(codes) * np.asarray(scales, dtype=np.float64).reshape(shape)


def fp8_quantize_query(q, per_head=False):
    """FP8 E4M3 query [B, Hq, D], per tensor or per attention head (axis 1).
    Returns (codes uint8 [B, Hq, D], scales float64 [1] or [Hq], dequantized
    query float64)."""
    q = np.asarray(q, dtype=np.float64)
    if per_head:
        codes, scales = fp8_pack_heads(q, amax_heads(q, None, head_axis=1), head_axis=1)
        return codes, scales, fp8_unpack_heads(codes, scales, head_axis=1)
    codes, scale = fp8_pack(q, amax(q))
    return codes, np.array([scale], dtype=np.float64), fp8_unpack(codes, scale)
