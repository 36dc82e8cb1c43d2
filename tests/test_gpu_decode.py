"""GPU parity of the split-KV decode + combine against the fp64 oracle.

Tolerances: fp32 path (tiny config, fp32 Q and output) max abs error 1e-5;
bf16 output per element |o - o_ref| <= max(2e-3, 1 bf16 ulp(o_ref)) and
cosine >= 0.9999 (2e-3 alone is below bf16's half-ulp once |o| >= 0.5, which
the x20 outlier channels reach).  The fp32 output of the same kernels is also
held to a per-element bound derived from the arithmetic (gpu_helpers.
fp32_bound): exact f16 products with fp32 accumulation, P rounded once to f16
on the bf16-query path (2^-11 * sum_t P_t |V_t|) or split hi + lo on the
fp32-query path, plus 1e-5 (1 + |o|) for the fp32 roundings.
"""
import math

import numpy as np
import pytest
import torch

import kvq_synth
from oracle import attention as OA
from oracle import formats as OF
from oracle import quant as OQ

from gpu_helpers import (DEV, K, announce, assert_bf16_output, err_report, fp32_bound, gpu_decode, gpu_pack,
                         make_inputs, oracle_gqa, oracle_pv_abs)

pytestmark = pytest.mark.gpu


def _fp32_close(got, ref, label, key):
    g = got.detach().cpu().double().numpy()
    bound = fp32_bound(key, ref)
    bad = np.abs(g - ref) > bound
    assert not bad.any(), f"{label}: {bad.sum()} fp32 outputs off; max abs {np.abs(g - ref).max():.3g}"


@pytest.mark.parametrize("s", [1, 2])
def test_tiny_fp32_path(s):
    key = ("nvfp4", "tiny")
    announce(f"decode tiny s={s}")
    inp = make_inputs(key)
    packed, o_ref, lse_ref, _, _ = oracle_gqa(key)
    kp, vp, _, _, lens = gpu_pack(inp, "nvfp4")
    out, used, lse = gpu_decode(inp, kp, vp, lens, s, out_dtype=torch.float32, with_lse=True)
    assert used == s
    err = np.abs(out.cpu().double().numpy() - o_ref).max()
    assert err <= 1e-5, f"max abs err {err}"
    assert np.abs(lse.cpu().double().numpy() - lse_ref).max() <= 1e-5


GQA_CASES = [(L, s) for L in (1024, 8192, 32768) for s in (1, 2, 4, 8, 0)]


@pytest.mark.parametrize("L,s", GQA_CASES, ids=lambda v: str(v))
def test_gqa_nvfp4(L, s):
    key = ("nvfp4", "gqa", L)
    announce(f"decode gqa L={L} s={s}")
    inp = make_inputs(key)
    _, o_ref, _, _, _ = oracle_gqa(key)
    kp, vp, _, _, lens = gpu_pack(inp, "nvfp4")
    out, used, _ = gpu_decode(inp, kp, vp, lens, s)
    mae, mre, cos = assert_bf16_output(out, o_ref, f"gqa L={L} s={used}")
    out32, _, _ = gpu_decode(inp, kp, vp, lens, s, out_dtype=torch.float32)
    _fp32_close(out32, o_ref, f"gqa fp32 L={L} s={used}", key)
    announce(f"  s={used}: max abs {mae:.2e} max rel {mre:.2e} cos {cos:.6f}")


MHA_CASES = ([(L, 2, 16, s) for L in (1024, 8192) for s in (1, 2, 4, 8, 0)] +
             [(32768, B, H, s) for (B, H) in ((2, 16), (1, 32)) for s in (1, 8, 0)])


@pytest.mark.parametrize("L,B,H,s", MHA_CASES, ids=lambda v: str(v))
def test_mha_nvfp4(L, B, H, s):
    key = ("nvfp4", "mha", L, B, H)
    announce(f"decode mha L={L} B={B} H={H} s={s}")
    inp = make_inputs(key)
    _, o_ref, _, _, _ = oracle_gqa(key)
    kp, vp, _, _, lens = gpu_pack(inp, "nvfp4")
    out, used, _ = gpu_decode(inp, kp, vp, lens, s)
    assert_bf16_output(out, o_ref, f"mha L={L} s={used}")


@pytest.mark.parametrize("s", [1, 3, 0])
def test_fp8_ragged(s):
    key = ("fp8", "fp8", 64)
    announce(f"decode fp8 ragged s={s}")
    inp = make_inputs(key)
    _, o_ref, _, _, _ = oracle_gqa(key)
    kp, vp, _, _, lens = gpu_pack(inp, "fp8")
    out, used, _ = gpu_decode(inp, kp, vp, lens, s)
    assert_bf16_output(out, o_ref, f"fp8 s={used}")
    out32, _, _ = gpu_decode(inp, kp, vp, lens, s, out_dtype=torch.float32)
    _fp32_close(out32, o_ref, f"fp8 fp32 s={used}", key)


EDGE = [
    # (B, Hq, Hkv, D, lens, q dtype, s)
    (3, 8, 2, 128, (0, 1, 77), "bf16", 4),        # empty request, single token, ragged tail
    (2, 16, 1, 128, (300, 5), "bf16", 8),         # G = 16, splits past the end
    (2, 16, 2, 64, (129, 64), "bf16", 2),         # G = 8, D = 64
    (1, 4, 2, 128, (1000,), "bf16", 64),          # G = 2, s = 64
    (2, 4, 4, 64, (33, 200), "f32", 3),           # G = 1 fp32 queries
    (1, 32, 8, 128, (4097,), "f32", 5),           # fp32 queries, odd length
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: f"B{c[0]}Hq{c[1]}Hkv{c[2]}D{c[3]}L{c[4]}{c[5]}s{c[6]}")
@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_edge_cases(case, fmt):
    B, Hq, Hkv, D, lens, dt, s = case
    key = (fmt, "custom", B, Hq, Hkv, D, lens, dt)
    announce(f"decode edge {fmt} {case}")
    inp = make_inputs(key)
    _, o_ref, lse_ref, _, _ = oracle_gqa(key)
    kp, vp, _, _, lens_d = gpu_pack(inp, fmt)
    out, used, lse = gpu_decode(inp, kp, vp, lens_d, s, out_dtype=torch.float32, with_lse=True)
    _fp32_close(out, o_ref, f"edge {case}", key)
    l = lse.cpu().double().numpy()
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(l), fin)
    assert np.all(np.abs(l[fin] - lse_ref[fin]) <= 1e-5 * (1 + np.abs(lse_ref[fin])))
    assert np.all(out.cpu().numpy()[~fin] == 0)


def test_deterministic_and_split_invariant():
    key = ("nvfp4", "gqa", 8192)
    announce("decode determinism / split invariance")
    inp = make_inputs(key)
    kp, vp, _, _, lens = gpu_pack(inp, "nvfp4")
    a, _, _ = gpu_decode(inp, kp, vp, lens, 8, out_dtype=torch.float32)
    b, _, _ = gpu_decode(inp, kp, vp, lens, 8, out_dtype=torch.float32)
    assert torch.equal(a, b)
    c, _, _ = gpu_decode(inp, kp, vp, lens, 1, out_dtype=torch.float32)
    # s = 8 and s = 1 round P to f16 against different running maxima: each
    # is within the fp32 bound of the oracle, so they differ by at most twice it
    _, o_ref, _, _, _ = oracle_gqa(key)
    bound = 2 * fp32_bound(key, o_ref)
    assert np.all(np.abs((a - c).cpu().double().numpy()) <= bound)


def test_combine_against_oracle():
    announce("combine vs oracle")
    rng = np.random.default_rng(5)
    B, Hq, s, Dv = 3, 5, 7, 96
    po = rng.standard_normal((B, Hq, s, Dv)).astype(np.float32)
    pl = (rng.standard_normal((B, Hq, s)) * 5).astype(np.float32)
    pl[0, 0, :] = -np.inf            # all splits empty
    pl[1, 2, ::2] = -np.inf          # some empty
    ref_o, ref_l = OA.combine(po.astype(np.float64), pl.astype(np.float64))
    out = torch.empty(B, Hq, Dv, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    K().attn_decode_combine(torch.from_numpy(po).to(DEV), torch.from_numpy(pl).to(DEV), B, Hq, Dv, s, out,
                            lse_out=lse)
    torch.cuda.synchronize()
    o = out.cpu().double().numpy()
    assert np.all(np.abs(o - ref_o) <= 1e-5 * (1 + np.abs(ref_o)))
    l = lse.cpu().double().numpy()
    assert np.isneginf(l[0, 0]) and np.all(o[0, 0] == 0)
    fin = np.isfinite(ref_l)
    assert np.all(np.abs(l[fin] - ref_l[fin]) <= 1e-5 * (1 + np.abs(ref_l[fin])))


def test_fp8_output_codes():
    """FP8 output (code = E4M3(o / out_scale)): codes equal the oracle's except
    where o_ref / out_scale lies within the fp32 error bound (divided by
    out_scale) of an E4M3 midpoint, where the two sides may round apart."""
    key = ("nvfp4", "gqa", 1024)
    announce("decode fp8 output")
    inp = make_inputs(key)
    _, o_ref, _, _, _ = oracle_gqa(key)
    kp, vp, _, _, lens = gpu_pack(inp, "nvfp4")
    out_scale = float(OF.fp32_round(np.abs(o_ref).max() / 448.0))
    osc = torch.tensor([out_scale], dtype=torch.float32, device=DEV)
    codes, _, _ = gpu_decode(inp, kp, vp, lens, 4, out_dtype=torch.uint8, out_scale=osc)
    want = OA.fp8_output(o_ref, out_scale)
    got = codes.cpu().numpy()
    diff = got != want
    r = np.abs(o_ref / out_scale)
    pos = OF.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    band = fp32_bound(key, o_ref) / out_scale
    near = np.min(np.abs(r[..., None] - mids), axis=-1) <= band
    assert not (diff & ~near).any(), f"{(diff & ~near).sum()} FP8 output codes differ away from a midpoint"
    assert np.all(np.abs(OF.e4m3_decode(got[diff]).astype(np.float64) - OF.e4m3_decode(want[diff])) <=
                  np.abs(OF.e4m3_decode(want[diff])) * 0.125 + 2 ** -9)


FUSED_CASES = [("nvfp4", "gqa", 32768, 0), ("nvfp4", "gqa", 1024, 1), ("nvfp4", "gqa", 8192, 7),
               ("nvfp4", "mha", 8192, 2, 16, 4), ("fp8", "fp8", 64, 0)]


@pytest.mark.parametrize("case", FUSED_CASES, ids=str)
def test_fused_single_launch(case):
    """attn_decode (split + combine in one launch) against the oracle, and
    bit-identical to the two-launch path."""
    key, s = case[:-1], case[-1]
    fmt = key[0]
    announce(f"decode fused {key} s={s}")
    inp = make_inputs(key)
    _, o_ref, lse_ref, _, _ = oracle_gqa(key)
    kp, vp, _, _, lens = gpu_pack(inp, fmt)
    out, used, lse = gpu_decode(inp, kp, vp, lens, s, out_dtype=torch.float32, with_lse=True, fused=True)
    _fp32_close(out, o_ref, f"fused {key} s={used}", key)
    fin = np.isfinite(lse_ref)
    assert np.all(np.abs(lse.cpu().double().numpy()[fin] - lse_ref[fin]) <= 1e-5 * (1 + np.abs(lse_ref[fin])))
    out2, _, _ = gpu_decode(inp, kp, vp, lens, s, out_dtype=torch.float32)
    assert torch.equal(out, out2)
    outb, _, _ = gpu_decode(inp, kp, vp, lens, s, out_dtype=torch.bfloat16, fused=True)
    assert_bf16_output(outb, o_ref, f"fused bf16 {key}")


T4_CASES = [("nvfp4", "gqa", 32768, 0), ("nvfp4", "gqa", 32768, 8), ("nvfp4", "gqa", 8192, 3),
            ("nvfp4", "gqa", 1024, 1), ("nvfp4", "mha", 8192, 2, 16, 0), ("fp8", "fp8", 64, 0),
            ("nvfp4", "custom", 3, 8, 2, 128, (0, 1, 77), "bf16", 4),
            ("nvfp4", "custom", 2, 16, 1, 128, (300, 5), "bf16", 8),
            ("fp8", "custom", 1, 32, 8, 128, (4097,), "f32", 5),
            ("nvfp4", "custom", 1, 4, 2, 128, (1000,), "bf16", 64)]


@pytest.mark.parametrize("case", T4_CASES, ids=str)
@pytest.mark.parametrize("fused", [False, True])
def test_token4_v_layout(case, fused):
    """V planes in the TOKEN4 layout (padding rows hold 0xFF bytes, i.e. NaN
    scales, which must never reach the output)."""
    key, s = case[:-1], case[-1]
    fmt = key[0]
    announce(f"decode token4 {key} s={s} fused={fused}")
    inp = make_inputs(key)
    _, o_ref, lse_ref, _, _ = oracle_gqa(key)
    kp, vp, _, _, lens = gpu_pack(inp, fmt, v_layout=K().KVQ_PLANE_TOKEN4)
    out, used, lse = gpu_decode(inp, kp, vp, lens, s, out_dtype=torch.float32, with_lse=True, fused=fused)
    _fp32_close(out, o_ref, f"token4 {key} s={used}", key)
    # the padding tokens of the last group and of the planes never reach the
    # output: zero padding instead of 0xFF bytes gives identical bits
    kp2, vp2, _, _, _ = gpu_pack(inp, fmt, v_layout=K().KVQ_PLANE_TOKEN4, fill=0)
    out2, _, _ = gpu_decode(inp, kp2, vp2, lens, s, out_dtype=torch.float32, fused=fused)
    assert torch.equal(out, out2), "the padding bytes of TOKEN4 planes must not change the result"
