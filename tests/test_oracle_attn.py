"""Pins for the oracle's decode attention, split emulation and combine.

Pinned against closed forms (L = 1, q = 0, equal keys, a dominant score),
torch's scaled_dot_product_attention in float64 (library routine), 50-digit
mpmath brute force on tiny inputs, split invariance, the MLA == GQA(Hkv = 1)
reduction and hand-worked FP8-probability cases.
"""
import math

import mpmath
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import formats as F


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_single_token_returns_v0():
    q = _rand((1, 4, 16), 0)
    k = _rand((1, 2, 5, 16), 1)
    v = _rand((1, 2, 5, 16), 2)
    o, lse = A.decode_gqa(q, k, v, [1], 0.25)
    for h in range(4):
        assert np.array_equal(o[0, h], v[0, h // 2, 0])
        assert lse[0, h] == pytest.approx(0.25 * k[0, h // 2, 0] @ q[0, h], rel=1e-15)


def test_zero_query_and_equal_keys_give_mean():
    k = _rand((1, 1, 7, 8), 3)
    v = _rand((1, 1, 7, 8), 4)
    o, lse = A.decode_gqa(np.zeros((1, 2, 8)), k, v, [7], 1.0)
    assert np.allclose(o[0, 0], v[0, 0].mean(0), rtol=0, atol=1e-15)
    assert lse[0, 0] == pytest.approx(math.log(7), rel=1e-15)
    keq = np.repeat(_rand((1, 1, 1, 8), 5), 7, axis=2)
    o2, _ = A.decode_gqa(_rand((1, 2, 8), 6), keq, v, [7], 0.3)
    assert np.allclose(o2[0, 1], v[0, 0].mean(0), rtol=0, atol=1e-14)


def test_dominant_score_selects_row():
    k = np.zeros((1, 1, 6, 4))
    k[0, 0, 3, 0] = 1000.0
    q = np.zeros((1, 1, 4))
    q[0, 0, 0] = 1.0
    v = _rand((1, 1, 6, 4), 7)
    o, _ = A.decode_gqa(q, k, v, [6], 1.0)
    assert np.array_equal(o[0, 0], v[0, 0, 3])


def test_empty_request():
    o, lse = A.decode_gqa(_rand((2, 2, 4), 1), _rand((2, 1, 3, 4), 2), _rand((2, 1, 3, 4), 3), [0, 3], 1.0)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))


@pytest.mark.parametrize("B,Hq,Hkv,D,L", [(2, 8, 2, 32, 50), (1, 4, 4, 16, 9), (3, 6, 1, 8, 17)])
def test_matches_torch_sdpa_float64(B, Hq, Hkv, D, L):
    q = _rand((B, Hq, D), 10)
    k = _rand((B, Hkv, L, D), 11)
    v = _rand((B, Hkv, L, D), 12)
    lens = np.full(B, L)
    lens[0] = L - 3  # ragged: padding must be ignored
    alpha = 1 / math.sqrt(D)
    o, _ = A.decode_gqa(q, k, v, lens, alpha)
    G = Hq // Hkv
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1)
    for b in range(B):
        Lb = int(lens[b])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b:b + 1, :, None, :]), kt[b:b + 1, :, :Lb], vt[b:b + 1, :, :Lb],
            scale=alpha)[0, :, 0].numpy()
        np.testing.assert_allclose(o[b], ref, rtol=1e-12, atol=1e-13)


def test_mpmath_bruteforce_tiny():
    mpmath.mp.dps = 50
    q = _rand((1, 2, 16), 20)
    k = _rand((1, 1, 8, 16), 21)
    v = _rand((1, 1, 8, 16), 22)
    alpha = 0.3
    for L in (1, 3, 8):
        o, lse = A.decode_gqa(q, k, v, [L], alpha)
        for h in range(2):
            sc = [mpmath.mpf(alpha) * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b))
                                                  for a, b in zip(k[0, 0, t], q[0, h])) for t in range(L)]
            m = max(sc)
            w = [mpmath.e ** (s - m) for s in sc]
            tot = mpmath.fsum(w)
            for d in range(16):
                ref = mpmath.fsum(w[t] * mpmath.mpf(float(v[0, 0, t, d])) for t in range(L)) / tot
                assert abs(o[0, h, d] - float(ref)) <= 1e-14 * max(1.0, abs(float(ref)))
            assert abs(lse[0, h] - float(m + mpmath.log(tot))) <= 1e-14 * abs(float(m + mpmath.log(tot))) + 1e-15


@pytest.mark.parametrize("s", [1, 2, 3, 8, 40])
def test_split_invariance(s):
    B, Hq, Hkv, D = 2, 8, 2, 32
    q = _rand((B, Hq, D), 30)
    k = _rand((B, Hkv, 33, D), 31) * 3
    v = _rand((B, Hkv, 33, D), 32)
    lens = [33, 20]
    o, lse = A.decode_gqa(q, k, v, lens, 0.2)
    op, lp = A.decode_gqa_split(q, k, v, lens, 0.2, s)
    oc, lc = A.combine(op, lp)
    np.testing.assert_allclose(oc, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lc, lse, rtol=1e-12, atol=1e-14)
    if s > 33:
        assert np.isneginf(lp[0, 0, -1])  # chunk past the end is empty


def test_split_bounds_cover_exactly():
    for L in (0, 1, 7, 64, 1000):
        for s in (1, 2, 3, 7, 64):
            b = A.split_bounds(L, s)
            assert len(b) == s
            covered = [t for t0, t1 in b for t in range(t0, t1)]
            assert covered == list(range(L))


def test_combine_skips_empty_and_all_empty():
    o_part = np.zeros((1, 3, 2))
    o_part[0, 1] = [1.0, 2.0]
    o_part[0, 2] = [5.0, 6.0]
    lse_part = np.array([[-np.inf, 0.0, math.log(3.0)]])
    o, lse = A.combine(o_part, lse_part)
    np.testing.assert_allclose(o[0], (np.array([1.0, 2.0]) + 3 * np.array([5.0, 6.0])) / 4, rtol=1e-15)
    assert lse[0] == pytest.approx(math.log(4.0), rel=1e-15)
    o2, l2 = A.combine(np.ones((1, 2, 2)), np.full((1, 2), -np.inf))
    assert np.all(o2 == 0) and np.isneginf(l2[0])


def test_mla_equals_gqa_with_one_kv_head():
    B, H, Dc, Dr, L = 2, 4, 32, 8, 19
    q_c, q_r = _rand((B, H, Dc), 40), _rand((B, H, Dr), 41)
    c, k_r = _rand((B, L, Dc), 42), _rand((B, L, Dr), 43)
    lens = [19, 11]
    o, lse = A.decode_mla(q_c, q_r, c, k_r, lens, 0.17)
    qk = np.concatenate([q_c, q_r], -1)
    kk = np.concatenate([c, k_r], -1)[:, None]
    o2, lse2 = A.decode_gqa(qk, kk, c[:, None], lens, 0.17)
    np.testing.assert_allclose(o, o2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, lse2, rtol=1e-13)


def test_fp8_probabilities_closed_forms():
    v = _rand((1, 1, 3, 4), 50)
    k = np.zeros((1, 1, 3, 4))
    q = np.zeros((1, 1, 4))
    # L = 2, equal scores: P = 1/2 -> 224 / 448 is on the E4M3 grid
    o2 = A.decode_gqa_fp8p(q, k, v, [2], 1.0, 1.0 / 448)
    assert np.array_equal(o2[0, 0], 0.5 * v[0, 0, 0] + 0.5 * v[0, 0, 1])
    # L = 3: 448/3 = 149.33 -> E4M3 rounds to 144 (quantum 16 in [128, 256))
    o3 = A.decode_gqa_fp8p(q, k, v, [3], 1.0, 1.0 / 448)
    np.testing.assert_allclose(o3[0, 0], (144.0 / 448.0) * v[0, 0].sum(0), rtol=1e-15)


def test_fp8_output_codes():
    codes = A.fp8_output(np.array([1.0, -3.0, 1000.0, 0.0]), 1.0)
    assert list(codes) == [0x38, 0xC4, 0x7E, 0x00]
    codes = A.fp8_output(np.array([0.5]), 0.25)
    assert int(codes[0]) == int(F.e4m3_encode(2.0))


# ---- FP8 probabilities at query groups of more than one head --------------
# gqa_probs and decode_gqa_fp8p are pinned here with G = 4 query heads per kv
# head, kv heads that differ, nonzero scores and softmax_scale != 1, so that a
# wrong head mapping (h % G instead of h // G) or a dropped softmax_scale fails.

def _gqa_case():
    B, Hq, Hkv, D, L = 2, 8, 2, 16, 23
    q = _rand((B, Hq, D), 60) * 2.0
    k = _rand((B, Hkv, L, D), 61)
    k[:, 1] *= 3.0   # kv heads see clearly different score ranges
    v = _rand((B, Hkv, L, D), 62)
    return q, k, v, [L, 14], 0.37


def test_gqa_probs_match_torch_sdpa_on_identity_values():
    # SDPA with V = the identity matrix returns the probability rows
    # themselves (library routine; keys repeat-interleaved by G)
    q, k, _, lens, alpha = _gqa_case()
    P = A.gqa_probs(q, k, lens, alpha)
    G = q.shape[1] // k.shape[1]
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1)
    for b, Lb in enumerate(lens):
        eye = torch.eye(Lb, dtype=torch.float64).expand(1, q.shape[1], Lb, Lb)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b:b + 1, :, None, :]), kt[b:b + 1, :, :Lb], eye, scale=alpha)[0, :, 0].numpy()
        np.testing.assert_allclose(P[b, :, :Lb], ref, rtol=1e-12, atol=1e-15)
        assert np.all(P[b, :, Lb:] == 0)
        np.testing.assert_allclose(P[b, :, :Lb].sum(-1), 1.0, rtol=1e-14)


def test_gqa_probs_weight_values_like_decode_gqa():
    # sum_t P_t V_t reproduces decode_gqa's output (itself pinned by SDPA and
    # mpmath above); P_t = exp(sigma_t - lse) with decode_gqa's lse, where
    # sigma_t comes from the single-token case (L = 1: lse = sigma_0)
    q, k, v, lens, alpha = _gqa_case()
    P = A.gqa_probs(q, k, lens, alpha)
    o, lse = A.decode_gqa(q, k, v, lens, alpha)
    G = q.shape[1] // k.shape[1]
    for b, Lb in enumerate(lens):
        for h in range(q.shape[1]):
            np.testing.assert_allclose(P[b, h, :Lb] @ v[b, h // G, :Lb], o[b, h], rtol=1e-12, atol=1e-14)
            for t in (0, Lb // 2, Lb - 1):
                kt = k[b:b + 1, :, t:t + 1]
                _, sig = A.decode_gqa(q[b:b + 1], kt, v[b:b + 1, :, t:t + 1], [1], alpha)
                assert P[b, h, t] == pytest.approx(math.exp(sig[0, h] - lse[b, h]), rel=1e-12)


def test_fp8_probabilities_closed_form_four_heads_per_kv_head():
    # Hkv = 2, G = 4, L = 3, softmax_scale 0.5, D = 4.
    #  kv head 0: three equal keys -> P = 1/3 for every query head of the
    #    group; 448/3 = 149.33 -> E4M3 144, so o = (144/448) (V0 + V1 + V2).
    #  kv head 1: keys (0, 2 ln 4, -2000) on channel 0.  Query head 4 has
    #    q = e_0: alpha * dscore = ln 4 -> P = (1/5, 4/5, 0); 448/5 = 89.6 ->
    #    88 and 4*448/5 = 358.4 -> 352.  Query head 5 has q = 2 e_0:
    #    P = (1/17, 16/17, 0); 26.35 -> 26 and 421.65 -> 416.  Heads 6 and 7
    #    have q = 0: P = 1/3 each -> 144 each.
    alpha, ps = 0.5, 1.0 / 448.0
    k = np.zeros((1, 2, 3, 4))
    k[0, 0, :, :] = [0.7, -1.2, 0.3, 2.0]
    k[0, 1, :, 0] = [0.0, 2.0 * math.log(4.0), -2000.0]
    q = np.zeros((1, 8, 4))
    q[0, 0:4] = _rand((4, 4), 63)
    q[0, 4, 0] = 1.0
    q[0, 5, 0] = 2.0
    v = _rand((1, 2, 3, 4), 64)
    o = A.decode_gqa_fp8p(q, k, v, [3], alpha, ps)
    V0, V1 = v[0, 0], v[0, 1]
    for h in range(4):
        np.testing.assert_allclose(o[0, h], (144.0 / 448.0) * V0.sum(0), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(o[0, 4], (88.0 * V1[0] + 352.0 * V1[1]) / 448.0, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(o[0, 5], (26.0 * V1[0] + 416.0 * V1[1]) / 448.0, rtol=1e-14, atol=1e-15)
    for h in (6, 7):
        np.testing.assert_allclose(o[0, h], (144.0 / 448.0) * V1.sum(0), rtol=1e-14, atol=1e-15)


# ---- chunked prefill -------------------------------------------------------
def test_prefill_matches_torch_sdpa_with_causal_offset_mask():
    # library routine: SDPA in float64 with an explicit boolean mask in which
    # query i of the chunk sees keys t <= L - Sq + i (keys repeat-interleaved by G)
    B, Sq, Hq, Hkv, D = 2, 5, 8, 2, 16
    q = _rand((B, Sq, Hq, D), 70)
    k = _rand((B, Hkv, 23, D), 71)
    v = _rand((B, Hkv, 23, D), 72)
    lens = [23, 9]
    alpha = 0.21
    o, lse = A.prefill_gqa(q, k, v, lens, alpha)
    G = Hq // Hkv
    for b, L in enumerate(lens):
        kt = torch.from_numpy(k[b:b + 1, :, :L]).repeat_interleave(G, dim=1)
        vt = torch.from_numpy(v[b:b + 1, :, :L]).repeat_interleave(G, dim=1)
        qt = torch.from_numpy(q[b:b + 1]).transpose(1, 2)   # [1, Hq, Sq, D]
        mask = torch.arange(L)[None, :] <= (L - Sq + torch.arange(Sq))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=alpha)
        np.testing.assert_allclose(o[b], ref[0].transpose(0, 1).numpy(), rtol=1e-12, atol=1e-13)
    assert np.all(np.isfinite(lse))


def test_prefill_full_causal_is_sdpa_is_causal():
    # Sq = L: ordinary causal self-attention (torch's is_causal)
    B, Sq, H, D = 1, 12, 4, 8
    q = _rand((B, Sq, H, D), 73)
    k = _rand((B, H, Sq, D), 74)
    v = _rand((B, H, Sq, D), 75)
    o, _ = A.prefill_gqa(q, k, v, [Sq], 0.4)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q).transpose(1, 2), torch.from_numpy(k),
                                                           torch.from_numpy(v), is_causal=True, scale=0.4)
    np.testing.assert_allclose(o, ref.transpose(1, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_prefill_rows_reduce_to_decode():
    # query i is the decode of the cache truncated to p_i + 1 tokens (decode_gqa
    # is pinned above); the first query of a chunk longer than the cache sees nothing
    B, Sq, Hq, Hkv, D = 1, 4, 4, 1, 8
    q = _rand((B, Sq, Hq, D), 76)
    k = _rand((B, Hkv, 6, D), 77)
    v = _rand((B, Hkv, 6, D), 78)
    o, lse = A.prefill_gqa(q, k, v, [6], 0.3)
    for i in range(Sq):
        od, ld = A.decode_gqa(q[:, i], k, v, [6 - Sq + i + 1], 0.3)
        np.testing.assert_array_equal(o[:, i], od)
        np.testing.assert_array_equal(lse[:, i], ld)
    o2, l2 = A.prefill_gqa(q, k, v, [2], 0.3)   # p_i = 2 - 4 + i: queries 0, 1 see nothing
    assert np.all(o2[:, :2] == 0) and np.all(np.isneginf(l2[:, :2]))
    np.testing.assert_allclose(o2[0, 2], np.repeat(v[0, :, 0], 4, axis=0), rtol=0, atol=0)   # one key: o = v_0
