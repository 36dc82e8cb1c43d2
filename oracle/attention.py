"""Exact softmax decode attention over a dequantized KV cache, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed (one query token per request, "decode"):

* GQA / MHA (Model-Optimizer PR #1832, Testing section: decode over
  (request, head) with GQA 4:1 and MHA configurations compared against
  PyTorch SDPA): query head h reads kv head floor(h / G), G = Hq / Hkv (the
  repeat-interleave convention of SDPA's grouped-query mode).
  sigma_t = alpha * q . K_t for t < kv_len, P = softmax(sigma),
  o = sum_t P_t V_t, lse = max + log(sum exp(sigma - max)).
* MLA latent cache (Model-Optimizer PR #714, Testing section: only the latent
  ``kv_c_bmm_quantizer`` is enabled, ``q_bmm_quantizer`` is disabled): with
  absorbed query parts q_c (latent width) and q_r (rope width),
  sigma_t = alpha * (q_c . c_t + q_r . k_r,t) and o = sum_t P_t c_t; the
  latent c is the (dequantized) NVFP4 cache, k_r the unquantized rope key.
* Split emulation (PR #1832, Testing section, split-KV description): split j
  of s covers the contiguous chunk [j*c, min((j+1)*c, L)), c = ceil(L / s);
  each split produces its own normalized partial o_j and lse_j (running max
  and denominator over its chunk); an empty split has lse_j = -inf, o_j = 0.
  The combine merges them: M = max_j lse_j, w_j = exp(lse_j - M),
  o = sum_j w_j o_j / sum_j w_j, LSE = M + log(sum_j w_j).
* FP8 probabilities (vLLM PR #15734, item 2: softmax(QK^T) quantized to FP8
  inside the attention loop with a probability scale): reading taken, the
  normalized probabilities P are quantized, P~ = E4M3(P / prob_scale) *
  prob_scale, and o = sum_t P~_t V_t without renormalization.
* FP8 output (vLLM PR #15734, item 1: attention output kept in FP8 with an
  output scale): code = E4M3(o / out_scale), value = code * out_scale.

All arithmetic is float64; q, K and V are used exactly as given (the caller
passes dequantized caches from ``oracle.quant``).
"""
import math

import numpy as np

from . import formats as F


def _softmax_stats(scores):
    """(P, lse) of a 1-D float64 score vector; empty -> (empty, -inf)."""
    if scores.size == 0:
        return scores, -math.inf
    m = scores.max()
    p = np.exp(scores - m)
    lsum = p.sum()
    return p / lsum, float(m + math.log(lsum))


def decode_gqa(q, k, v, kv_lens, softmax_scale):
    """Exact decode attention.

    q: [B, Hq, D]; k: [B, Hkv, Lmax, D]; v: [B, Hkv, Lmax, Dv] (float64,
    dequantized); kv_lens: [B] ints; softmax_scale: alpha.
    Returns (o [B, Hq, Dv], lse [B, Hq]); a request with kv_len 0 gives o = 0
    and lse = -inf.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Hq, _ = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    o = np.zeros((B, Hq, v.shape[-1]))
    lse = np.full((B, Hq), -math.inf)
    for b in range(B):
        L = int(kv_lens[b])
        for h in range(Hq):
            kvh = h // G
            s = softmax_scale * (k[b, kvh, :L] @ q[b, h])
            p, lse[b, h] = _softmax_stats(s)
            if L:
                o[b, h] = p @ v[b, kvh, :L]
    return o, lse


def decode_mla(q_c, q_r, c, k_r, kv_lens, softmax_scale):
    """Exact MLA decode: q_c [B, H, Dc], q_r [B, H, Dr], c [B, Lmax, Dc]
    (dequantized latent), k_r [B, Lmax, Dr].  Returns (o [B, H, Dc], lse)."""
    q_c = np.asarray(q_c, np.float64)
    q_r = np.asarray(q_r, np.float64)
    c = np.asarray(c, np.float64)
    k_r = np.asarray(k_r, np.float64)
    B, H, Dc = q_c.shape
    o = np.zeros((B, H, Dc))
    lse = np.full((B, H), -math.inf)
    for b in range(B):
        L = int(kv_lens[b])
        s_all = softmax_scale * (c[b, :L] @ q_c[b].T + k_r[b, :L] @ q_r[b].T)  # [L, H]
        for h in range(H):
            p, lse[b, h] = _softmax_stats(s_all[:, h])
            if L:
                o[b, h] = p @ c[b, :L]
    return o, lse


def split_bounds(L, s):
    """Chunk boundaries [(start, end)] of the s contiguous splits of L tokens."""
    c = -(-L // s) if L else 0
    return [(min(j * c, L), min((j + 1) * c, L)) for j in range(s)]


def decode_gqa_split(q, k, v, kv_lens, softmax_scale, s):
    """Per-split partials: (o_part [B, Hq, s, Dv], lse_part [B, Hq, s])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Hq, _ = q.shape
    G = Hq // k.shape[1]
    o = np.zeros((B, Hq, s, v.shape[-1]))
    lse = np.full((B, Hq, s), -math.inf)
    for b in range(B):
        for h in range(Hq):
            kvh = h // G
            for j, (t0, t1) in enumerate(split_bounds(int(kv_lens[b]), s)):
                sc = softmax_scale * (k[b, kvh, t0:t1] @ q[b, h])
                p, lse[b, h, j] = _softmax_stats(sc)
                if t1 > t0:
                    o[b, h, j] = p @ v[b, kvh, t0:t1]
    return o, lse


def combine(o_part, lse_part):
    """Merge split partials: o_part [..., s, Dv], lse_part [..., s].
    All splits empty -> o = 0, LSE = -inf."""
    o_part = np.asarray(o_part, np.float64)
    lse_part = np.asarray(lse_part, np.float64)
    out_shape = o_part.shape[:-2] + (o_part.shape[-1],)
    o = np.zeros(out_shape)
    lse = np.full(lse_part.shape[:-1], -math.inf)
    for idx in np.ndindex(*lse_part.shape[:-1]):
        ls = lse_part[idx]
        live = np.isfinite(ls)
        if not live.any():
            continue
        m = ls[live].max()
        w = np.where(live, np.exp(np.where(live, ls, m) - m), 0.0)
        wsum = w.sum()
        o[idx] = (w[:, None] * o_part[idx]).sum(axis=0) / wsum
        lse[idx] = m + math.log(wsum)
    return o, lse


def gqa_probs(q, k, kv_lens, softmax_scale):
    """Normalized softmax probabilities of GQA decode: P [B, Hq, Lmax] with
    P[b, h, t] = softmax_t(alpha * q_h . K_{floor(h/G), t}) for t < kv_len,
    0 past it (float64)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    B, Hq, _ = q.shape
    G = Hq // k.shape[1]
    P = np.zeros((B, Hq, k.shape[2]))
    for b in range(B):
        L = int(kv_lens[b])
        for h in range(Hq):
            if L:
                P[b, h, :L], _ = _softmax_stats(softmax_scale * (k[b, h // G, :L] @ q[b, h]))
    return P


def decode_gqa_fp8p(q, k, v, kv_lens, softmax_scale, prob_scale):
    """GQA decode with the normalized probabilities quantized to E4M3:
    P~ = E4M3(P / prob_scale) * prob_scale, o = sum_t P~_t V_t (not
    renormalized).  Returns o [B, Hq, Dv]."""
    v = np.asarray(v, np.float64)
    P = gqa_probs(q, k, kv_lens, softmax_scale)
    B, Hq, _ = P.shape
    G = Hq // v.shape[1]
    o = np.zeros((B, Hq, v.shape[-1]))
    for b in range(B):
        L = int(kv_lens[b])
        for h in range(Hq):
            if L:
                pq = F.e4m3_round(P[b, h, :L] / prob_scale) * prob_scale
                o[b, h] = pq @ v[b, h // G, :L]
    return o


def fp8_output(o, out_scale):
    """E4M3 codes of o / out_scale (saturating, RNE)."""
    return F.e4m3_encode(np.asarray(o, np.float64) / np.float64(out_scale))


def prefill_gqa(q, k, v, kv_lens, softmax_scale):
    """Chunked prefill over the (dequantized) cache: the Sq query tokens of
    request b are its last Sq positions, p_i = kv_lens[b] - Sq + i, and query
    i attends causally to the cached tokens t <= p_i (the chunk's own tokens
    are in the cache already).  A query with p_i < 0 sees nothing: o = 0,
    lse = -inf.  GQA head mapping as decode_gqa.

    q: [B, Sq, Hq, D]; k: [B, Hkv, Lmax, D]; v: [B, Hkv, Lmax, Dv] (float64).
    Returns (o [B, Sq, Hq, Dv], lse [B, Sq, Hq])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Sq, Hq, _ = q.shape
    G = Hq // k.shape[1]
    o = np.zeros((B, Sq, Hq, v.shape[-1]))
    lse = np.full((B, Sq, Hq), -math.inf)
    for b in range(B):
        for i in range(Sq):
            n = int(kv_lens[b]) - Sq + i + 1   # keys 0 .. p_i
            if n <= 0:
                continue
            for h in range(Hq):
                s = softmax_scale * (k[b, h // G, :n] @ q[b, i, h])
                p, lse[b, i, h] = _softmax_stats(s)
                o[b, i, h] = p @ v[b, h // G, :n]
    return o, lse
