"""GPU parity of the FP8-probability decode (normalized softmax P quantized to
E4M3 with a probability scale, o = sum_t P~_t V_t, not renormalized) against
the fp64 oracle.

Gate.  The kernel forms P in fp32 (scores summed in fp32, exp2 of the
difference to the log-sum-exp), so P carries a relative error of a few 1e-6
against the oracle's fp64 P; where P / prob_scale lies that close to an E4M3
rounding boundary the two sides may pick neighbouring codes.  Such tokens are
found from the oracle alone (the code of r(1 - eps) differs from the code of
r(1 + eps), eps = 2e-5) and each adds |code step| * prob_scale * |V_t| to the
bound of the outputs it feeds.  Otherwise P~ enters the P.V product exactly
(E4M3 values are f16 values), so the fp32 bound is 1e-5 (1 + |o|) +
2^-16 sum_t P~_t |V_t| (fp32 accumulation and the split rescaling); bf16
output: max(2e-3, 1 bf16 ulp) + the flip allowance, cosine >= 0.9999.
"""
import dataclasses
import functools

import numpy as np
import pytest
import torch

import kvq_synth
from oracle import attention as OA
from oracle import formats as OF

from gpu_helpers import DEV, K, announce, err_report, gpu_decode, gpu_pack, make_inputs, oracle_gqa

pytestmark = pytest.mark.gpu

EPS = 2e-5
PS = float(np.float32(1.0 / 448.0))   # the pages' probability scale, as the fp32 the kernel receives


@functools.lru_cache(maxsize=16)
def _oracle(key, ps):
    inp = make_inputs(key)
    _, _, lse, khat, vhat = oracle_gqa(key)
    q = kvq_synth.f64(inp.q)
    P = OA.gqa_probs(q, khat, inp.kv_lens, inp.softmax_scale)
    o = OA.decode_gqa_fp8p(q, khat, vhat, inp.kv_lens, inp.softmax_scale, ps)
    r = P / ps
    pq = OF.e4m3_round(r) * ps
    step = np.abs(OF.e4m3_round(r * (1 + EPS)) - OF.e4m3_round(r * (1 - EPS))) * ps
    G = inp.Hq // inp.Hkv
    va = np.repeat(np.abs(vhat), G, axis=1)           # [B, Hq, L, D]
    flip = np.einsum("bht,bhtd->bhd", step, va)
    mass = np.einsum("bht,bhtd->bhd", pq, va)
    announce(f"  oracle fp8p {key}: {int((step > 0).sum())} near-boundary probabilities")
    return o, lse, flip, mass


def _check(out, lse, key, ps, label):
    o_ref, lse_ref, flip, mass = _oracle(key, ps)
    g = out.detach().float().cpu().double().numpy()
    if out.dtype == torch.float32:
        tol = 1e-5 * (1 + np.abs(o_ref)) + 2.0 ** -16 * mass + flip
    else:
        tol = np.maximum(2e-3, OF.bf16_ulp(o_ref)) + flip
    bad = np.abs(g - o_ref) > tol
    mae, mre, cos = err_report(g, o_ref)
    assert not bad.any(), f"{label}: {bad.sum()} outputs off; max abs {mae:.3g}"
    assert cos >= 0.9999, f"{label}: cosine {cos}"
    if lse is not None:
        l = lse.cpu().double().numpy()
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(l), fin)
        assert np.all(np.abs(l[fin] - lse_ref[fin]) <= 1e-5 * (1 + np.abs(lse_ref[fin])))
        assert np.all(g[~fin] == 0)
    announce(f"  {label}: max abs {mae:.2e} cos {cos:.6f}")


@pytest.mark.parametrize("s", [1, 3, 0])
def test_fp8p_fp8_ragged(s):
    """The FP8 ragged configuration (B=64, Hq=32, Hkv=8, D=128, kv_len ~ U{512..4096})."""
    key = ("fp8", "fp8", 64)
    announce(f"fp8p fp8 ragged s={s}")
    inp = make_inputs(key)
    kp, vp, _, _, lens = gpu_pack(inp, "fp8")
    out, used, lse = gpu_decode(inp, kp, vp, lens, s, out_dtype=torch.float32, with_lse=True, prob_scale=PS)
    _check(out, lse, key, PS, f"fp8p fp32 s={used}")
    outb, _, _ = gpu_decode(inp, kp, vp, lens, s, prob_scale=PS)
    _check(outb, None, key, PS, f"fp8p bf16 s={used}")


CASES = [
    # (fmt, B, Hq, Hkv, D, lens, q dtype, s)
    ("nvfp4", 3, 8, 2, 128, (0, 1, 300), "bf16", 4),     # empty request, one token, ragged tail
    ("nvfp4", 2, 16, 1, 128, (700, 33), "bf16", 3),      # G = 16
    ("fp8", 2, 16, 2, 64, (129, 64), "bf16", 2),         # G = 8, D = 64
    ("nvfp4", 2, 4, 4, 64, (200, 31), "f32", 5),         # G = 1, fp32 queries
    ("fp8", 1, 8, 4, 128, (1000,), "f32", 1),            # G = 2, fp32 queries, one split
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}B{c[1]}Hq{c[2]}Hkv{c[3]}D{c[4]}L{c[5]}{c[6]}s{c[7]}")
def test_fp8p_shapes(case):
    fmt, B, Hq, Hkv, D, lens, dt, s = case
    key = (fmt, "custom", B, Hq, Hkv, D, lens, dt)
    announce(f"fp8p {case}")
    inp = make_inputs(key)
    kp, vp, _, _, lens_d = gpu_pack(inp, fmt)
    out, used, lse = gpu_decode(inp, kp, vp, lens_d, s, out_dtype=torch.float32, with_lse=True, prob_scale=PS)
    _check(out, lse, key, PS, f"fp8p {case}")


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_fp8p_token4_v_and_fused_entry(fmt):
    """TOKEN4 V plane, through both entry points (same partials, same combine)."""
    key = (fmt, "custom", 2, 8, 2, 128, (517, 90), "bf16")
    announce(f"fp8p token4 {fmt}")
    inp = make_inputs(key)
    k_ = K()
    kp, vp, _, _, lens_d = gpu_pack(inp, fmt, v_layout=k_.KVQ_PLANE_TOKEN4)
    a, used, la = gpu_decode(inp, kp, vp, lens_d, 3, out_dtype=torch.float32, with_lse=True, prob_scale=PS)
    b, _, lb = gpu_decode(inp, kp, vp, lens_d, 3, out_dtype=torch.float32, with_lse=True, prob_scale=PS, fused=True)
    assert torch.equal(a, b) and torch.equal(la, lb)
    _check(a, la, key, PS, f"fp8p token4 {fmt}")


def test_fp8p_saturating_scale():
    """prob_scale = 1/1024: P / prob_scale exceeds 448 for the dominant
    tokens, which saturate to 448 (P~ = 0.4375)."""
    ps = float(np.float32(1.0 / 1024.0))
    key = ("nvfp4", "custom", 2, 8, 2, 128, (40, 300), "bf16")
    announce("fp8p saturating prob_scale")
    inp = make_inputs(key)
    kp, vp, _, _, lens_d = gpu_pack(inp, "nvfp4")
    out, used, lse = gpu_decode(inp, kp, vp, lens_d, 2, out_dtype=torch.float32, with_lse=True, prob_scale=ps)
    _check(out, lse, key, ps, "fp8p saturating")


def test_fp8p_equal_scores_closed_form():
    """q = 0: every score is 0, P = 1/3 for L = 3, 448/3 = 149.33 -> E4M3 144,
    so o = 144 * prob_scale * (V_0 + V_1 + V_2) for every head (closed form,
    with the oracle's dequantized V)."""
    key = ("fp8", "custom", 1, 4, 1, 64, (3,), "bf16")
    inp = make_inputs(key)
    _, _, _, _, vhat = oracle_gqa(key)
    inp0 = dataclasses.replace(inp, q=torch.zeros_like(inp.q))
    kp, vp, _, _, lens_d = gpu_pack(inp0, "fp8")
    out, _, _ = gpu_decode(inp0, kp, vp, lens_d, 1, out_dtype=torch.float32, prob_scale=PS)
    expect = 144.0 * PS * vhat[0, 0, :3].sum(axis=0)
    g = out.cpu().double().numpy()[0]
    assert np.all(np.abs(g - expect[None, :]) <= 1e-6 * (1 + np.abs(expect[None, :])))
