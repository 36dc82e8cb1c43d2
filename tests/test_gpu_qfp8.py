"""GPU parity for FP8 queries (the QKV-FP8 schemes): the query batch is
calibrated and packed by the same kernels as the KV planes (viewed as
[B, Hq, 1, D]), bit-exact against the oracle, and the decode over FP8
query codes (scale per tensor or per query head) is checked against the
oracle's attention with the dequantized query, within the same output gates
as the bf16-query path."""
import numpy as np
import pytest
import torch

import kvq_synth
from gpu_helpers import DEV, K, announce, assert_bf16_output, gpu_decode, gpu_pack, make_inputs, oracle_gqa
from oracle import attention as OA
from oracle import quant as OQ

pytestmark = pytest.mark.gpu


def _quantize_query(q, per_head):
    k_ = K()
    B, Hq, D = q.shape
    q4 = q.contiguous().view(B, Hq, 1, D)
    amax = k_.kvq_amax(q4, per_head=per_head)
    qp = k_.kvq_pack_fp8(q4, amax)
    return qp.codes.view(B, Hq, D), qp.scale


@pytest.mark.parametrize("per_head", [False, True])
@pytest.mark.parametrize("key", [("nvfp4", "gqa", 1024), ("nvfp4", "custom", 2, 16, 2, 128, (300, 77), "bf16")])
def test_query_pack_bit_exact(key, per_head):
    announce(f"fp8 query pack {key} per_head={per_head}")
    inp = make_inputs(key)
    codes, scale = _quantize_query(inp.q.to(DEV), per_head)
    torch.cuda.synchronize()
    oc, osc, _ = OQ.fp8_quantize_query(kvq_synth.f64(inp.q), per_head)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(scale.cpu().numpy().astype(np.float64), osc)


CASES = [
    # (key, kv format, v_layout, splits, fused, per_head)
    (("nvfp4", "gqa", 1024), "nvfp4", 1, 3, False, False),
    (("nvfp4", "gqa", 1024), "nvfp4", 1, 0, True, True),
    (("fp8", "fp8", 64), "fp8", 1, 2, False, False),
    (("fp8", "fp8", 64), "fp8", 1, 0, True, True),
    (("nvfp4", "mha", 1024, 2, 16), "nvfp4", 1, 2, False, True),                       # G = 1
    (("nvfp4", "custom", 2, 16, 2, 128, (300, 77), "bf16"), "nvfp4", 1, 4, False, True),  # G = 8
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0][0]}-{c[0][1]}-v{c[2]}-s{c[3]}-f{int(c[4])}-h{int(c[5])}")
def test_decode_fp8_query(case):
    key, fmt, v_layout, s, fused, per_head = case
    announce(f"fp8 query decode {case}")
    k_ = K()
    inp = make_inputs(key)
    kp, vp, _, _, lens = gpu_pack(inp, fmt, v_layout)
    q8, q_scale = _quantize_query(inp.q.to(DEV), per_head)
    B, Hq, D = inp.B, inp.Hq, inp.D
    part_o = torch.empty(B * Hq * 64 * D, dtype=torch.float32, device=DEV)
    part_lse = torch.empty(B * Hq * 64, dtype=torch.float32, device=DEV)
    args = k_.make_decode_args(q8, kp, vp, lens, max_kv_len=inp.Lmax, softmax_scale=inp.softmax_scale,
                               num_splits=s, part_o=part_o, part_lse=part_lse, q_scale=q_scale)
    out = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    if fused:
        counters = torch.zeros(B * inp.Hkv, dtype=torch.int32, device=DEV)
        k_.attn_decode(args, out, counters=counters)
    else:
        used = k_.attn_decode_splitkv(args)
        k_.attn_decode_combine(part_o, part_lse, B, Hq, D, used, out)
    torch.cuda.synchronize()
    _, _, qhat = OQ.fp8_quantize_query(kvq_synth.f64(inp.q), per_head)
    _, _, _, khat, vhat = oracle_gqa(key)
    o_ref, _ = OA.decode_gqa(qhat, khat, vhat, inp.kv_lens, inp.softmax_scale)
    assert_bf16_output(out, o_ref, f"fp8 query {case}")


# ---------------------------------------------------------------- FP8 queries with FP8 probabilities
PS = float(np.float32(1.0 / 448.0))
EPS = 2e-5


def _fp8p_reference(qhat, khat, vhat, inp, ps):
    """The oracle's FP8-P decode with the dequantized query, and the
    near-boundary allowance of the FP8-P gate (tokens whose P / prob_scale
    lies within a relative 2e-5 of an E4M3 rounding boundary may take the
    neighbouring code: each adds |code step| * prob_scale * |V_t|)."""
    from oracle import formats as OF
    P = OA.gqa_probs(qhat, khat, inp.kv_lens, inp.softmax_scale)
    o = OA.decode_gqa_fp8p(qhat, khat, vhat, inp.kv_lens, inp.softmax_scale, ps)
    r = P / ps
    step = np.abs(OF.e4m3_round(r * (1 + EPS)) - OF.e4m3_round(r * (1 - EPS))) * ps
    va = np.repeat(np.abs(vhat), inp.Hq // inp.Hkv, axis=1)
    flip = np.einsum("bht,bhtd->bhd", step, va)
    mass = np.einsum("bht,bhtd->bhd", OF.e4m3_round(r) * ps, va)
    return o, flip, mass


FP8P_CASES = [
    # (key, kv format, splits, per-head query scale)
    (("fp8", "fp8", 64), "fp8", 3, False),
    (("nvfp4", "custom", 3, 8, 2, 128, (0, 1, 300), "bf16"), "nvfp4", 4, True),
    (("nvfp4", "custom", 2, 16, 1, 128, (700, 33), "bf16"), "nvfp4", 0, False),   # G = 16, auto splits
]


@pytest.mark.parametrize("case", FP8P_CASES, ids=lambda c: f"{c[0][0]}-{c[0][1]}-s{c[2]}-h{int(c[3])}")
def test_decode_fp8_query_fp8_probabilities(case):
    """FP8 query codes (per tensor or per head) with FP8-quantized
    probabilities: pass 1 forms the scores from the codes, pass 2 the
    quantized P . V; against the oracle's FP8-P decode with the dequantized
    query, within the FP8-P gate (fp32 output: 1e-5 (1 + |o|) + 2^-16
    sum_t P~_t |V_t| + the near-boundary allowance)."""
    key, fmt, s, per_head = case
    announce(f"fp8 query + fp8p {case}")
    inp = make_inputs(key)
    kp, vp, _, _, lens = gpu_pack(inp, fmt)
    q8, q_scale = _quantize_query(inp.q.to(DEV), per_head)
    out, used, lse = gpu_decode(inp, kp, vp, lens, s, out_dtype=torch.float32, with_lse=True, prob_scale=PS,
                                q=q8, q_scale=q_scale)
    _, _, qhat = OQ.fp8_quantize_query(kvq_synth.f64(inp.q), per_head)
    _, _, _, khat, vhat = oracle_gqa(key)
    o_ref, flip, mass = _fp8p_reference(qhat, khat, vhat, inp, PS)
    g = out.cpu().double().numpy()
    bad = np.abs(g - o_ref) > 1e-5 * (1 + np.abs(o_ref)) + 2.0 ** -16 * mass + flip
    assert not bad.any(), f"{case}: {bad.sum()} outputs off; max abs {np.abs(g - o_ref).max():.3g}"
    _, lse_ref = OA.decode_gqa(qhat, khat, vhat, inp.kv_lens, inp.softmax_scale)
    l = lse.cpu().double().numpy()
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(l), fin)
    assert np.all(np.abs(l[fin] - lse_ref[fin]) <= 1e-5 * (1 + np.abs(lse_ref[fin])))
