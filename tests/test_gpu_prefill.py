"""GPU parity for the chunked prefill over the packed cache (attn_prefill,
through the C ABI) against the oracle's prefill_gqa on the oracle's own
dequantized cache: query i of an Sq-token chunk sits at position
kv_len - Sq + i and attends causally to the cached tokens up to it.

Cases span several 128-row query blocks and 64-token KV tiles with ragged
tails, every implemented query-group width (1, 2, 4, 8), chunks longer than
the cache (queries that see nothing: output 0, lse -inf), a chunk that is the
whole sequence, one-token chunks, both cache formats, per-head FP8 scales,
paged planes (bit-identical to contiguous), both output dtypes, and the
bench workload's shape (GQA 4:1, 32K cache, 1024-token chunk) on sampled
query rows.  Planes are padded with 0xFF bytes (NaN E4M3 scales), so a read
of a row past a request's length would show."""
import numpy as np
import pytest
import torch

import kvq_synth
from gpu_helpers import DEV, K, announce, err_report, gpu_pack, page_plane
from oracle import formats as OF
from oracle import attention as OA
from oracle import quant as OQ

pytestmark = pytest.mark.gpu


def _oracle_cache(inp, fmt, per_head=False):
    """Oracle packing + dequantization of the cache (fp64)."""
    kf, vf = kvq_synth.f64(inp.k), kvq_synth.f64(inp.v)
    if fmt == "nvfp4":
        kc, ks, kst = OQ.nvfp4_pack(kf, OQ.amax(kf, inp.kv_lens))
        vc, vs, vst = OQ.nvfp4_pack(vf, OQ.amax(vf, inp.kv_lens))
        return OQ.nvfp4_unpack(kc, ks, kst), OQ.nvfp4_unpack(vc, vs, vst)
    if per_head:
        kc, ks = OQ.fp8_pack_heads(kf, OQ.amax_heads(kf, inp.kv_lens))
        vc, vs = OQ.fp8_pack_heads(vf, OQ.amax_heads(vf, inp.kv_lens))
        return OQ.fp8_unpack_heads(kc, ks), OQ.fp8_unpack_heads(vc, vs)
    kc, kst = OQ.fp8_pack(kf, OQ.amax(kf, inp.kv_lens))
    vc, vst = OQ.fp8_pack(vf, OQ.amax(vf, inp.kv_lens))
    return OQ.fp8_unpack(kc, kst), OQ.fp8_unpack(vc, vst)


def _gpu_planes(inp, fmt, per_head=False):
    """K rows + V TOKEN4 planes, padded to whole 4-token groups with 0xFF."""
    k_ = K()
    if not per_head:
        kp, vp, _, _, lens = gpu_pack(inp, fmt)
        return kp, vp, lens
    k, v = inp.k.to(DEV), inp.v.to(DEV)
    lens = torch.from_numpy(inp.kv_lens).to(DEV)
    B, H, L, D = inp.k.shape
    Lp = (L + 3) // 4 * 4

    def plane(x, layout):   # one E4M3 scale per kv head (the amax tensor has H entries)
        p = k_.FP8Plane(torch.full((B, H, Lp, D), 0xFF, dtype=torch.uint8, device=DEV),
                        torch.empty(H, dtype=torch.float32, device=DEV), layout)
        k_.kvq_pack_fp8(x, k_.kvq_amax(x, lens, per_head=True), out=p)
        return p
    return plane(k, k_.KVQ_PLANE_ROWS), plane(v, k_.KVQ_PLANE_TOKEN4), lens


def gpu_prefill(inp, kp, vp, lens, out_dtype=torch.bfloat16, block_table=None, q=None):
    k_ = K()
    q = inp.q.to(DEV) if q is None else q
    out = torch.full(tuple(q.shape), float("nan"), dtype=out_dtype, device=DEV)
    lse = torch.full(tuple(q.shape[:3]), float("nan"), dtype=torch.float32, device=DEV)
    args = k_.make_prefill_args(q, kp, vp, lens, out, max_kv_len=inp.Lmax, softmax_scale=inp.softmax_scale,
                                lse_out=lse, block_table=block_table)
    k_.attn_prefill(args)
    torch.cuda.synchronize()
    return out, lse


# The kernel's probabilities: every P_t enters P.V as one f16 value (RNE,
# relative error d_t <= 2^-11 in f16's normal range) and the denominator is
# the matrix cores' fp32 sum of the same f16 values, so the denominator's
# relative error e is a P-weighted mean of the d_t (|e| <= 2^-11) and every
# normalized weight carries (1 + d_t) / (1 + e): relative error at most
# W_F16 = 2^-10 (1 + 2^-10).  The log-sum-exp carries ln(1 + e), at most
# L_F16 = 2^-11 (1 + 2^-10), plus the f16 subnormal tail: probabilities
# below 2^-14 round with an absolute error up to 2^-25 each, against a
# denominator of at least 1 (the largest probability of a row is >= 1), so
# at most 2^-25 per key.  (That tail's effect on the output, at most 2^-25
# per key times |V_t|, is left out of the output bound, as for the decode.)
W_F16 = 2.0 ** -10 * (1.0 + 2.0 ** -10)
L_F16 = 2.0 ** -11 * (1.0 + 2.0 ** -10)


def _nkeys(inp):
    """the most keys any query row of the chunk sees (its request's kv_len)"""
    return int(np.max(inp.kv_lens)) if len(inp.kv_lens) else 0


def _check(out, lse, o_ref, lse_ref, label, pv_abs, nkeys, eps=None):
    """Output: |o - o_ref| <= (W_F16 e^{2 eps} + e^{2 eps} - 1) sum_t P_t
    |V_t| (the f16 probabilities above) plus 1e-5 (1 + |o|) of fp32
    arithmetic for fp32 output, or plus max(2e-3, 1 bf16 ulp(o_ref)) for bf16
    output (its RNE rounding), and cosine >= 0.9999.  lse: 1e-5 (1 + |lse|)
    + L_F16 + nkeys 2^-25 (nkeys: the most keys any row sees), and exactly
    -inf where the oracle has -inf (queries that see nothing, whose output
    is 0).  eps [B, Sq, Hq]: a bound on every score's error in the row (FP8
    matrix cores, _fp8_score_eps); scores off by at most eps move each
    probability by a factor within exp(+-2 eps), so the output by at most
    (exp(2 eps) - 1) sum_t P_t |V_t| more, and lse by at most eps."""
    o = out.float().cpu().double().numpy()
    eps = np.zeros(lse_ref.shape) if eps is None else eps
    e2 = np.exp(2.0 * eps)[..., None]
    p_round = (W_F16 * e2 + (e2 - 1.0)) * pv_abs
    if out.dtype == torch.bfloat16:
        bound = np.maximum(2e-3, OF.bf16_ulp(o_ref)) + p_round
    else:
        bound = 1e-5 * (1.0 + np.abs(o_ref)) + p_round
    bad = np.abs(o - o_ref) > bound
    assert not bad.any(), f"{label}: {bad.sum()} elements out of the bound; max abs {np.abs(o - o_ref).max():.3g}"
    if np.abs(o_ref).max() > 0:
        _, _, cos = err_report(o, o_ref)
        assert cos >= 0.9999, f"{label}: cosine {cos}"
    g = lse.cpu().double().numpy()
    ninf = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(g), ninf), f"{label}: -inf lse pattern differs"
    assert np.all(o[ninf] == 0.0), f"{label}: queries that see nothing must output 0"
    fin = ~ninf
    lse_tol = 1e-5 * (1.0 + np.abs(lse_ref[fin])) + L_F16 + nkeys * 2.0 ** -25 + eps[fin]
    assert np.all(np.abs(g[fin] - lse_ref[fin]) <= lse_tol), f"{label}: lse"


CASES = [
    # (name, fmt, B, Hq, Hkv, kv_lens, Sq)
    ("gqa4_ragged", "nvfp4", 2, 8, 2, (300, 1000), 200),
    ("mha", "nvfp4", 1, 4, 4, (777,), 300),
    ("gqa8_chunk_longer_than_cache", "nvfp4", 2, 16, 2, (130, 64), 100),
    ("gqa2_whole_sequence", "nvfp4", 1, 8, 4, (513,), 513),
    ("gqa4_one_token", "nvfp4", 3, 8, 2, (1, 65, 700), 1),
    ("fp8_gqa4", "fp8", 2, 8, 2, (700, 69), 96),
    ("fp8_mha_whole", "fp8", 1, 2, 2, (200,), 200),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_matches_oracle(case):
    name, fmt, B, Hq, Hkv, lens, Sq = case
    announce(f"prefill {case}")
    inp = kvq_synth.prefill(B, Hq, Hkv, 128, list(lens), Sq, outliers=True)
    khat, vhat = _oracle_cache(inp, fmt)
    o_ref, lse_ref = OA.prefill_gqa(kvq_synth.f64(inp.q), khat, vhat, inp.kv_lens, inp.softmax_scale)
    kp, vp, klens = _gpu_planes(inp, fmt)
    pv_abs, _ = OA.prefill_gqa(kvq_synth.f64(inp.q), khat, np.abs(vhat), inp.kv_lens, inp.softmax_scale)
    out, lse = gpu_prefill(inp, kp, vp, klens)
    _check(out, lse, o_ref, lse_ref, f"prefill {name} bf16", pv_abs, _nkeys(inp))
    out32, lse32 = gpu_prefill(inp, kp, vp, klens, out_dtype=torch.float32)
    _check(out32, lse32, o_ref, lse_ref, f"prefill {name} f32", pv_abs, _nkeys(inp))
    # the bf16 output is the RNE rounding of the fp32 one (same kernel arithmetic)
    assert torch.equal(out32.to(torch.bfloat16), out)
    assert torch.equal(lse32, lse)


def test_prefill_fp8_per_head_scales():
    announce("prefill fp8 per-head scales")
    inp = kvq_synth.prefill(2, 8, 2, 128, [400, 150], 128, outliers=True)
    khat, vhat = _oracle_cache(inp, "fp8", per_head=True)
    o_ref, lse_ref = OA.prefill_gqa(kvq_synth.f64(inp.q), khat, vhat, inp.kv_lens, inp.softmax_scale)
    pv_abs, _ = OA.prefill_gqa(kvq_synth.f64(inp.q), khat, np.abs(vhat), inp.kv_lens, inp.softmax_scale)
    kp, vp, lens = _gpu_planes(inp, "fp8", per_head=True)
    assert kp.scale.numel() == 2
    out, lse = gpu_prefill(inp, kp, vp, lens)
    _check(out, lse, o_ref, lse_ref, "prefill fp8 per-head", pv_abs, _nkeys(inp))


@pytest.mark.parametrize("fmt,bs", [("nvfp4", 64), ("nvfp4", 256), ("fp8", 128)])
def test_prefill_paged_matches_contiguous(fmt, bs):
    """Paged planes (permuted blocks, table entries past a request's length
    pointing at 0xFF blocks) give bit-identical outputs."""
    announce(f"prefill paged {fmt} bs={bs}")
    inp = kvq_synth.prefill(2, 8, 2, 128, [900, 333], 160, outliers=True)
    kp, vp, lens = _gpu_planes(inp, fmt)
    ref, ref_lse = gpu_prefill(inp, kp, vp, lens)
    kpp, bt = page_plane(kp, bs, 11, inp.kv_lens)
    vpp, bt2 = page_plane(vp, bs, 11, inp.kv_lens)
    assert torch.equal(bt, bt2)
    got, lse = gpu_prefill(inp, kpp, vpp, lens, block_table=bt)
    assert torch.equal(got, ref) and torch.equal(lse, ref_lse)


def test_prefill_strided_views():
    """q and out as strided views ([B, Hq, Sq, D] storage seen as
    [B, Sq, Hq, D]): the strides go through the ABI unchanged."""
    announce("prefill strided views")
    inp = kvq_synth.prefill(2, 8, 2, 128, [250, 300], 70)
    kp, vp, lens = _gpu_planes(inp, "nvfp4")
    ref, ref_lse = gpu_prefill(inp, kp, vp, lens)
    q_t = inp.q.to(DEV).transpose(1, 2).contiguous().transpose(1, 2)   # [B, Sq, Hq, D] view of [B, Hq, Sq, D]
    k_ = K()
    out_t = torch.zeros(2, 8, 70, 128, dtype=torch.bfloat16, device=DEV).transpose(1, 2)
    lse = torch.empty(2, 70, 8, dtype=torch.float32, device=DEV)
    args = k_.make_prefill_args(q_t, kp, vp, lens, out_t, max_kv_len=inp.Lmax, softmax_scale=inp.softmax_scale,
                                lse_out=lse)
    k_.attn_prefill(args)
    torch.cuda.synchronize()
    assert torch.equal(out_t, ref) and torch.equal(lse, ref_lse)


def test_prefill_one_token_chunk_equals_decode():
    """A one-token chunk is a decode step at position kv_len - 1: the output
    matches attn_decode's within the two kernels' rounding (both are gated
    against the oracle elsewhere; here the two HIP paths agree to 2 bf16 ulp,
    and the log-sum-exp within the prefill's f16 denominator, L_F16 plus
    2^-25 per key)."""
    announce("prefill one-token chunk vs decode")
    k_ = K()
    inp = kvq_synth.prefill(2, 32, 8, 128, [1024, 777], 1)
    kp, vp, lens = _gpu_planes(inp, "nvfp4")
    out, lse = gpu_prefill(inp, kp, vp, lens, out_dtype=torch.float32)
    q = inp.q[:, 0].to(DEV).contiguous()
    part_o = torch.empty(2 * 32 * 64 * 128, dtype=torch.float32, device=DEV)
    part_lse = torch.empty(2 * 32 * 64, dtype=torch.float32, device=DEV)
    args = k_.make_decode_args(q, kp, vp, lens, max_kv_len=inp.Lmax, softmax_scale=inp.softmax_scale, num_splits=1,
                               part_o=part_o, part_lse=part_lse)
    dec = torch.empty(2, 32, 128, dtype=torch.float32, device=DEV)
    dlse = torch.empty(2, 32, dtype=torch.float32, device=DEV)
    used = k_.attn_decode_splitkv(args)
    k_.attn_decode_combine(part_o, part_lse, 2, 32, 128, used, dec, lse_out=dlse)
    torch.cuda.synchronize()
    assert torch.allclose(out[:, 0], dec, rtol=2e-3, atol=2e-3)
    assert torch.allclose(lse[:, 0], dlse, rtol=1e-5, atol=1e-5 + L_F16 + 1024 * 2.0 ** -25)


def test_prefill_empty_and_zero_length():
    """Sq = 0 launches nothing; requests with kv_len = 0 give 0 and -inf."""
    announce("prefill empty chunk / empty request")
    k_ = K()
    inp = kvq_synth.prefill(2, 8, 2, 128, [0, 100], 40)
    khat, vhat = _oracle_cache(inp, "nvfp4")
    o_ref, lse_ref = OA.prefill_gqa(kvq_synth.f64(inp.q), khat, vhat, inp.kv_lens, inp.softmax_scale)
    pv_abs, _ = OA.prefill_gqa(kvq_synth.f64(inp.q), khat, np.abs(vhat), inp.kv_lens, inp.softmax_scale)
    kp, vp, lens = _gpu_planes(inp, "nvfp4")
    out, lse = gpu_prefill(inp, kp, vp, lens)
    _check(out, lse, o_ref, lse_ref, "prefill kv_len 0", pv_abs, _nkeys(inp))
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    q0 = torch.empty(2, 0, 8, 128, dtype=torch.bfloat16, device=DEV)
    o0 = torch.empty(2, 0, 8, 128, dtype=torch.bfloat16, device=DEV)
    k_.attn_prefill(k_.make_prefill_args(q0, kp, vp, lens, o0, max_kv_len=inp.Lmax))


# ---------------------------------------------------------------- full size
BENCH_B, BENCH_HQ, BENCH_HKV, BENCH_L, BENCH_SQ = 2, 32, 8, 32768, 1024


def test_prefill_bench_shape_sampled():
    """The bench workload: GQA 4:1 NVFP4 32K cache (the decode metric's
    cache, kvq_synth.gqa(32768)), a 1024-token chunk per request, in the
    launch bench.py times; 48 sampled (request, query, head) rows against the
    oracle, each as decode of the cache truncated at the query's position
    (the reduction the oracle's prefill is pinned to)."""
    announce("prefill bench shape, sampled rows")
    from gpu_helpers import oracle_gqa
    cache = kvq_synth.gqa(BENCH_L)
    q = kvq_synth.prefill_queries(BENCH_B, BENCH_SQ, BENCH_HQ, 128)
    inp = kvq_synth.PrefillInputs(q=q, k=cache.k, v=cache.v, kv_lens=cache.kv_lens,
                                  softmax_scale=cache.softmax_scale)
    kp, vp, _, _, lens = gpu_pack(cache, "nvfp4")
    out, lse = gpu_prefill(inp, kp, vp, lens, out_dtype=torch.float32)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    _, _, _, khat, vhat = oracle_gqa(("nvfp4", "gqa", BENCH_L))
    rng = np.random.default_rng(5)
    G = BENCH_HQ // BENCH_HKV
    for n in range(48):
        b = int(rng.integers(BENCH_B))
        i = int(rng.integers(BENCH_SQ)) if n % 4 else (0 if n % 8 == 0 else BENCH_SQ - 1)
        h = int(rng.integers(BENCH_HQ))
        pos = BENCH_L - BENCH_SQ + i
        qv = kvq_synth.f64(q[b, i, h])[None, None, None]
        o1, l1 = OA.prefill_gqa(qv, khat[b:b + 1, h // G:h // G + 1], vhat[b:b + 1, h // G:h // G + 1],
                                np.array([pos + 1]), inp.softmax_scale)
        pv, _ = OA.prefill_gqa(qv, khat[b:b + 1, h // G:h // G + 1], np.abs(vhat[b:b + 1, h // G:h // G + 1]),
                               np.array([pos + 1]), inp.softmax_scale)
        got = out[b, i, h].cpu().double().numpy()
        bound = 1e-5 * (1.0 + np.abs(o1[0, 0, 0])) + W_F16 * pv[0, 0, 0]
        assert np.all(np.abs(got - o1[0, 0, 0]) <= bound), f"row (b={b}, i={i}, h={h})"
        assert abs(float(lse[b, i, h]) - l1[0, 0, 0]) <= 1e-5 * (1 + abs(l1[0, 0, 0])) + L_F16 + (pos + 1) * 2.0 ** -25, \
            f"lse (b={b}, i={i}, h={h})"


# ---------------------------------------------------------------- FP8 queries
def _quantize_chunk(q, per_head):
    """The chunk's queries packed by the library's FP8 packer, viewed as
    [B * Sq, Hq, 1, D] (one scale, or one per query head)."""
    k_ = K()
    B, Sq, Hq, D = q.shape
    q4 = q.contiguous().view(B * Sq, Hq, 1, D)
    qp = k_.kvq_pack_fp8(q4, k_.kvq_amax(q4, per_head=per_head))
    return qp.codes.view(B, Sq, Hq, D), qp.scale


def _oracle_query(q, per_head):
    """Oracle FP8 quantization of the chunk (codes, scales, dequantized)."""
    B, Sq, Hq, D = q.shape
    codes, scales, qhat = OQ.fp8_quantize_query(kvq_synth.f64(q).reshape(B * Sq, Hq, D), per_head)
    return codes.reshape(B, Sq, Hq, D), scales, qhat.reshape(B, Sq, Hq, D)


# the FP8 matrix core's accumulation error per score, as a fraction of
# sum_k |q_k k_k| (measured on the device by test_gpu_fp8_mfma.py)
EPS_FP8_DOT = 2.0 ** -10


def _fp8_score_eps(qhat, khat, kv_lens, softmax_scale):
    """Per query row (b, i, h): EPS_FP8_DOT * softmax_scale * the largest
    sum_k |q_k| |K_tk| over the keys the row sees (natural-log units)."""
    B, Sq, Hq, _ = qhat.shape
    G = Hq // khat.shape[1]
    eps = np.zeros((B, Sq, Hq))
    for b in range(B):
        L = int(kv_lens[b])
        if L == 0:
            continue
        pos = L - Sq + np.arange(Sq)
        for h in range(Hq):
            m = np.abs(qhat[b, :, h]) @ np.abs(khat[b, h // G, :L]).T          # [Sq, L]
            m = np.where(np.arange(L)[None, :] <= pos[:, None], m, 0.0)
            eps[b, :, h] = EPS_FP8_DOT * softmax_scale * m.max(axis=1)
    return eps


def gpu_prefill_q8(inp, kp, vp, lens, q8, q_scale, out_dtype=torch.float32, block_table=None):
    k_ = K()
    out = torch.full(tuple(q8.shape), float("nan"), dtype=out_dtype, device=DEV)
    lse = torch.full(tuple(q8.shape[:3]), float("nan"), dtype=torch.float32, device=DEV)
    args = k_.make_prefill_args(q8, kp, vp, lens, out, max_kv_len=inp.Lmax, softmax_scale=inp.softmax_scale,
                                lse_out=lse, block_table=block_table, q_scale=q_scale)
    k_.attn_prefill(args)
    torch.cuda.synchronize()
    return out, lse


Q8_CASES = [
    # (name, kv fmt, B, Hq, Hkv, kv_lens, Sq, per-head query scale, per-head kv scale)
    ("fp8cache_gqa4", "fp8", 2, 8, 2, (700, 69), 96, False, False),
    ("fp8cache_gqa8_perhead", "fp8", 2, 16, 2, (300, 1000), 200, True, True),
    ("fp8cache_mha_whole", "fp8", 1, 2, 2, (200,), 200, True, False),
    ("fp8cache_gqa4_longer_than_cache", "fp8", 2, 8, 2, (130, 64), 100, False, True),
    ("nvfp4cache_gqa4", "nvfp4", 2, 8, 2, (300, 1000), 200, False, False),
    ("nvfp4cache_gqa2_whole_perhead", "nvfp4", 1, 8, 4, (513,), 513, True, False),
]


@pytest.mark.parametrize("case", Q8_CASES, ids=[c[0] for c in Q8_CASES])
def test_prefill_fp8_query_matches_oracle(case):
    """FP8 query codes and scales bit-exact against the oracle's packing;
    the prefill over them against the oracle's prefill with the dequantized
    query.  NVFP4 cache: the codes are converted to f16 (exact) and the
    bf16-query gates hold as they are.  FP8 cache: Q.K^T runs on the FP8
    matrix cores, and the gates add the effect of their accumulation error
    (at most EPS_FP8_DOT sum_k |q_k k_k| per score)."""
    name, fmt, B, Hq, Hkv, lens, Sq, qh, kvh = case
    announce(f"prefill fp8 query {case}")
    inp = kvq_synth.prefill(B, Hq, Hkv, 128, list(lens), Sq, outliers=True)
    q8, q_scale = _quantize_chunk(inp.q.to(DEV), qh)
    oc, osc, qhat = _oracle_query(inp.q, qh)
    torch.cuda.synchronize()
    assert np.array_equal(q8.cpu().numpy(), oc)
    assert np.array_equal(q_scale.cpu().numpy().astype(np.float64), osc)
    khat, vhat = _oracle_cache(inp, fmt, per_head=kvh)
    o_ref, lse_ref = OA.prefill_gqa(qhat, khat, vhat, inp.kv_lens, inp.softmax_scale)
    pv_abs, _ = OA.prefill_gqa(qhat, khat, np.abs(vhat), inp.kv_lens, inp.softmax_scale)
    kp, vp, klens = _gpu_planes(inp, fmt, per_head=kvh)
    eps = _fp8_score_eps(qhat, khat, inp.kv_lens, inp.softmax_scale) if fmt == "fp8" else None
    out32, lse32 = gpu_prefill_q8(inp, kp, vp, klens, q8, q_scale)
    _check(out32, lse32, o_ref, lse_ref, f"prefill fp8 query {name} f32", pv_abs, _nkeys(inp), eps)
    out, lse = gpu_prefill_q8(inp, kp, vp, klens, q8, q_scale, out_dtype=torch.bfloat16)
    _check(out, lse, o_ref, lse_ref, f"prefill fp8 query {name} bf16", pv_abs, _nkeys(inp), eps)
    assert torch.equal(out32.to(torch.bfloat16), out)


@pytest.mark.parametrize("fmt", ["fp8", "nvfp4"])
def test_prefill_fp8_query_paged_matches_contiguous(fmt):
    announce(f"prefill fp8 query paged {fmt}")
    inp = kvq_synth.prefill(2, 8, 2, 128, [900, 333], 160, outliers=True)
    kp, vp, lens = _gpu_planes(inp, fmt)
    q8, q_scale = _quantize_chunk(inp.q.to(DEV), True)
    ref, ref_lse = gpu_prefill_q8(inp, kp, vp, lens, q8, q_scale)
    kpp, bt = page_plane(kp, 128, 11, inp.kv_lens)
    vpp, _ = page_plane(vp, 128, 11, inp.kv_lens)
    got, lse = gpu_prefill_q8(inp, kpp, vpp, lens, q8, q_scale, block_table=bt)
    assert torch.equal(got, ref) and torch.equal(lse, ref_lse)


def test_prefill_fp8_query_bench_shape_sampled():
    """The FP8 variant of the bench workload (the 32K GQA 4:1 cache packed in
    FP8, the 1024-token chunk as FP8 codes with one scale): 24 sampled rows
    against the oracle, each as the truncated-cache reduction, with the FP8
    matrix cores' score-error term."""
    announce("prefill fp8 query bench shape, sampled rows")
    cache = kvq_synth.gqa(BENCH_L)
    q = kvq_synth.prefill_queries(BENCH_B, BENCH_SQ, BENCH_HQ, 128)
    inp = kvq_synth.PrefillInputs(q=q, k=cache.k, v=cache.v, kv_lens=cache.kv_lens,
                                  softmax_scale=cache.softmax_scale)
    kp, vp, _, _, lens = gpu_pack(cache, "fp8")
    q8, q_scale = _quantize_chunk(q.to(DEV), False)
    out, lse = gpu_prefill_q8(inp, kp, vp, lens, q8, q_scale)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    oc, _, qhat = _oracle_query(q, False)
    assert np.array_equal(q8.cpu().numpy(), oc)
    from gpu_helpers import oracle_gqa
    _, _, _, khat, vhat = oracle_gqa(("fp8", "gqa", BENCH_L))
    rng = np.random.default_rng(9)
    G = BENCH_HQ // BENCH_HKV
    for n in range(24):
        b, i, h = int(rng.integers(BENCH_B)), int(rng.integers(BENCH_SQ)), int(rng.integers(BENCH_HQ))
        pos = BENCH_L - BENCH_SQ + i
        qv = qhat[b, i, h][None, None, None]
        kh, vh = khat[b:b + 1, h // G:h // G + 1], vhat[b:b + 1, h // G:h // G + 1]
        o1, l1 = OA.prefill_gqa(qv, kh, vh, np.array([pos + 1]), inp.softmax_scale)
        pv, _ = OA.prefill_gqa(qv, kh, np.abs(vh), np.array([pos + 1]), inp.softmax_scale)
        eps = EPS_FP8_DOT * inp.softmax_scale * float((np.abs(kh[0, 0, :pos + 1]) @ np.abs(qhat[b, i, h])).max())
        got = out[b, i, h].cpu().double().numpy()
        bound = 1e-5 * (1.0 + np.abs(o1[0, 0, 0])) + (W_F16 * np.exp(2 * eps) + np.expm1(2 * eps)) * pv[0, 0, 0]
        assert np.all(np.abs(got - o1[0, 0, 0]) <= bound), f"row (b={b}, i={i}, h={h})"
        assert abs(float(lse[b, i, h]) - l1[0, 0, 0]) <= 1e-5 * (1 + abs(l1[0, 0, 0])) + L_F16 + (pos + 1) * 2.0 ** -25 + eps, \
            f"lse (b={b}, i={i}, h={h})"
