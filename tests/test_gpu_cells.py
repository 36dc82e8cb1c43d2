"""GPU parity for configuration cells and edge cases beyond the main sweeps:

* FP8 output codes on the FP8 ragged B = 64 configuration, with exact and
  with FP8-quantized probabilities (codes equal the oracle's E4M3(o / out_scale)
  except inside the error band around an E4M3 midpoint);
* an all-zero K / V cache (amax = 0: tensor scale 1, scale bytes 0, codes 0;
  the scores are all zero, so the output is the mean of V over the request);
* values above the calibrated amax (a stale static scale): the pack kernels,
  the batched append and the append fused into the decode saturate exactly
  as the oracle does (block scale 448, E2M1 code 6, E4M3 code 448).
"""
import numpy as np
import pytest
import torch

import kvq_synth
from oracle import attention as OA
from oracle import formats as OF
from oracle import quant as OQ

from gpu_helpers import DEV, K, announce, fp32_bound, gpu_decode, gpu_pack, make_inputs, oracle_gqa

pytestmark = pytest.mark.gpu

PS = float(np.float32(1.0 / 448.0))


def _codes_match(got, o_ref, out_scale, band, label):
    """got must be the E4M3 rounding of some value within `band` of
    o_ref / out_scale: between the codes of v - band and v + band (equal to
    the oracle's code wherever no rounding midpoint lies within the band)."""
    v = o_ref / out_scale
    g = OF.e4m3_decode(got).astype(np.float64)
    lo, hi = OF.e4m3_round(v - band), OF.e4m3_round(v + band)
    bad = (g < lo) | (g > hi)
    assert not bad.any(), f"{label}: {int(bad.sum())} FP8 output codes outside the rounding band"
    diff = got != OA.fp8_output(o_ref, out_scale)
    announce(f"  {label}: {int(diff.sum())} of {diff.size} codes differ from the oracle's, all inside the band")


@pytest.mark.parametrize("s", [0, 3])
def test_fp8_output_on_fp8_ragged(s):
    key = ("fp8", "fp8", 64)
    announce(f"fp8 output, fp8 ragged, s={s}")
    inp = make_inputs(key)
    _, o_ref, _, _, _ = oracle_gqa(key)
    kp, vp, _, _, lens = gpu_pack(inp, "fp8")
    out_scale = float(OF.fp32_round(np.abs(o_ref).max() / 448.0))
    osc = torch.tensor([out_scale], dtype=torch.float32, device=DEV)
    codes, _, _ = gpu_decode(inp, kp, vp, lens, s, out_dtype=torch.uint8, out_scale=osc)
    _codes_match(codes.cpu().numpy(), o_ref, out_scale, fp32_bound(key, o_ref) / out_scale, "fp8 out")
    fused, _, _ = gpu_decode(inp, kp, vp, lens, s, out_dtype=torch.uint8, out_scale=osc, fused=True)
    assert torch.equal(fused, codes), "fused and two-launch FP8 output codes differ"


def test_fp8_output_with_fp8_probabilities_on_fp8_ragged():
    key = ("fp8", "fp8", 64)
    announce("fp8 output + fp8 probabilities, fp8 ragged")
    inp = make_inputs(key)
    _, _, _, khat, vhat = oracle_gqa(key)
    q = kvq_synth.f64(inp.q)
    o_ref = OA.decode_gqa_fp8p(q, khat, vhat, inp.kv_lens, inp.softmax_scale, PS)
    # the error band of the FP8-P output (as in the FP8-P parity tests): fp32
    # accumulation plus a code step of P~ at probabilities near an E4M3 boundary
    P = OA.gqa_probs(q, khat, inp.kv_lens, inp.softmax_scale)
    r = P / PS
    step = np.abs(OF.e4m3_round(r * (1 + 2e-5)) - OF.e4m3_round(r * (1 - 2e-5))) * PS
    G = inp.Hq // inp.Hkv
    va = np.repeat(np.abs(vhat), G, axis=1)
    flip = np.einsum("bht,bhtd->bhd", step, va)
    mass = np.einsum("bht,bhtd->bhd", OF.e4m3_round(r) * PS, va)
    tol = 1e-5 * (1 + np.abs(o_ref)) + 2.0 ** -16 * mass + flip
    out_scale = float(OF.fp32_round(np.abs(o_ref).max() / 448.0))
    osc = torch.tensor([out_scale], dtype=torch.float32, device=DEV)
    kp, vp, _, _, lens = gpu_pack(inp, "fp8")
    codes, _, _ = gpu_decode(inp, kp, vp, lens, 0, out_dtype=torch.uint8, out_scale=osc, prob_scale=PS)
    _codes_match(codes.cpu().numpy(), o_ref, out_scale, tol / out_scale, "fp8 out + fp8p")


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("zero_v", [False, True])
def test_all_zero_cache(fmt, zero_v):
    """K all zero (and V too, or random): amax 0 gives tensor scale 1 (the
    pages' default KV scale), every scale byte and code 0; the scores are 0,
    so o = mean of V over the request (0 for a zero V) and lse = ln L."""
    announce(f"all-zero cache {fmt} zero_v={zero_v}")
    base = kvq_synth.gqa_inputs(2, 8, 2, 128, None, kv_lens=[100, 37], config="gqa", salt=11, Lmax=100)
    k0 = torch.zeros_like(base.k)
    v0 = torch.zeros_like(base.v) if zero_v else base.v
    inp = type(base)(q=base.q, k=k0, v=v0, kv_lens=base.kv_lens, softmax_scale=base.softmax_scale)
    kp, vp, ka, va, lens = gpu_pack(inp, fmt)
    torch.cuda.synchronize()
    assert float(ka.item()) == 0.0
    if fmt == "nvfp4":
        assert float(kp.tensor_scale.item()) == 1.0
        assert int(kp.codes[:, :, :100].to(torch.int32).sum().item()) == 0
        assert int(kp.scales[:, :, :100].to(torch.int32).sum().item()) == 0
    else:
        assert float(kp.scale.item()) == 1.0 and int(kp.codes[:, :, :100].to(torch.int32).sum().item()) == 0
    kf, vf = kvq_synth.f64(inp.k), kvq_synth.f64(inp.v)
    if fmt == "nvfp4":
        vc, vs, vst = OQ.nvfp4_pack(vf, OQ.amax(vf, inp.kv_lens))
        vhat = OQ.nvfp4_unpack(vc, vs, vst)
        kc, ks, kst = OQ.nvfp4_pack(kf, OQ.amax(kf, inp.kv_lens))
        assert kst == 1.0 and not kc.any() and not ks.any()
        khat = OQ.nvfp4_unpack(kc, ks, kst)
    else:
        vc, vst = OQ.fp8_pack(vf, OQ.amax(vf, inp.kv_lens))
        vhat = OQ.fp8_unpack(vc, vst)
        kc, kst = OQ.fp8_pack(kf, OQ.amax(kf, inp.kv_lens))
        assert kst == 1.0 and not kc.any()
        khat = OQ.fp8_unpack(kc, kst)
    o_ref, lse_ref = OA.decode_gqa(kvq_synth.f64(inp.q), khat, vhat, inp.kv_lens, inp.softmax_scale)
    for b, Lb in enumerate(inp.kv_lens):   # closed form: uniform weights
        np.testing.assert_allclose(o_ref[b], np.repeat(vhat[b, :, :Lb].mean(axis=1), 4, axis=0), atol=1e-12)
        np.testing.assert_allclose(lse_ref[b], np.log(Lb), rtol=1e-15)
    out, _, lse = gpu_decode(inp, kp, vp, lens, 3, out_dtype=torch.float32, with_lse=True)
    g = out.cpu().double().numpy()
    assert np.all(np.abs(g - o_ref) <= 1e-5 * (1 + np.abs(o_ref)) + 2.0 ** -11 * np.abs(o_ref).max())
    assert np.all(np.abs(lse.cpu().double().numpy() - lse_ref) <= 1e-5 * np.abs(lse_ref))
    if zero_v:
        assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_pack_saturates_above_calibrated_amax(fmt):
    """Rows packed with an amax below their own max |x| (stale static scale):
    NVFP4 block scales clamp at 448 and codes at 6, FP8 codes at 448, bit for
    bit as the oracle's saturating encoders."""
    announce(f"pack saturation {fmt}")
    inp = kvq_synth.gqa_inputs(1, 4, 2, 128, 64, config="gqa", salt=12, dtype=torch.float32)
    x = inp.k * 3.0   # (rounded to fp32; the same tensor feeds both sides)
    k_ = K()
    xd = x.to(DEV)
    stale = torch.tensor([float(inp.k.abs().max())], dtype=torch.float32, device=DEV)
    xf = kvq_synth.f64(x)
    if fmt == "nvfp4":
        p = k_.kvq_pack_nvfp4(xd, stale)
        torch.cuda.synchronize()
        codes, scales, st = OQ.nvfp4_pack(xf, float(stale.item()))
        assert np.array_equal(p.codes.cpu().numpy(), codes) and np.array_equal(p.scales.cpu().numpy(), scales)
        assert (scales == 0x7E).any(), "some block scale must saturate at 448"
        assert ((codes & 0x7) == 7).any() or ((codes >> 4 & 0x7) == 7).any()
    else:
        p = k_.kvq_pack_fp8(xd, stale)
        torch.cuda.synchronize()
        codes, sc = OQ.fp8_pack(xf, float(stale.item()))
        assert np.array_equal(p.codes.cpu().numpy(), codes)
        assert ((codes & 0x7F) == 0x7E).any(), "some code must saturate at 448"


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("fused_decode", [False, True])
def test_append_saturates_with_stale_scale(fmt, fused_decode):
    """The new token's rows, 3x beyond the amax the planes' scales came from:
    the batched append and the append fused into the decode write the same
    saturated bytes as the oracle's encoders."""
    announce(f"append saturation {fmt} fused_decode={fused_decode}")
    k_ = K()
    key = ("nvfp4", "gqa", 1024) if fmt == "nvfp4" else ("fp8", "fp8", 64)
    inp = make_inputs(key)
    B, Hkv, D = inp.B, inp.Hkv, inp.D
    kp, vp, ka, va, lens = gpu_pack(inp, fmt)
    lens_np = inp.kv_lens.astype(np.int64)
    new_k = (torch.stack([inp.k[b, :, lens_np[b] - 1] for b in range(B)]) * 3.0).contiguous()
    new_v = (torch.stack([inp.v[b, :, lens_np[b] - 1] for b in range(B)]) * 3.0).contiguous()
    nk, nv = new_k.to(DEV), new_v.to(DEV)
    if fused_decode:
        part_o = torch.empty(B * inp.Hq * 64 * D, dtype=torch.float32, device=DEV)
        part_lse = torch.empty(B * inp.Hq * 64, dtype=torch.float32, device=DEV)
        args = k_.make_decode_args(inp.q.to(DEV), kp, vp, lens, max_kv_len=inp.Lmax, softmax_scale=inp.softmax_scale,
                                   num_splits=2, part_o=part_o, part_lse=part_lse, new_k=nk, new_v=nv)
        used = k_.attn_decode_splitkv(args)
        out = torch.empty(B, inp.Hq, D, dtype=torch.float32, device=DEV)
        k_.attn_decode_combine(part_o, part_lse, B, inp.Hq, D, used, out)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
    else:
        pos = torch.from_numpy((lens_np - 1).astype(np.int32)).to(DEV)
        k_.kvq_pack_batch([(nk.view(B, Hkv, 1, D), ka, kp, pos), (nv.view(B, Hkv, 1, D), va, vp, pos)])
        torch.cuda.synchronize()
    amk, amv = float(ka.item()), float(va.item())
    for plane, x, am, is_v in ((kp, new_k, amk, False), (vp, new_v, amv, True)):
        xf = kvq_synth.f64(x)[:, :, None, :]   # [B, Hkv, 1, D]
        for b in range(B):
            t = int(lens_np[b] - 1)
            if fmt == "nvfp4":
                codes, scales, _ = OQ.nvfp4_pack(xf[b:b + 1], am)
                got_c, got_s = _row_nvfp4(plane, b, t, is_v)
                assert np.array_equal(got_c, codes[0, :, 0]) and np.array_equal(got_s, scales[0, :, 0])
            else:
                codes, _ = OQ.fp8_pack(xf[b:b + 1], am)
                assert np.array_equal(_row_fp8(plane, b, t, is_v), codes[0, :, 0])


def _row_nvfp4(plane, b, t, token4):
    """Row t of request b (all kv heads) as row-layout bytes: codes [H, 64], scales [H, 8]."""
    c = plane.codes[b].cpu().numpy()    # [H, L, 64]
    s = plane.scales[b].cpu().numpy()   # [H, L, 8]
    if not token4:
        return c[:, t], s[:, t]
    q, j = t // 4, t % 4
    grp = c[:, 4 * q:4 * q + 4].reshape(c.shape[0], -1)          # 256 bytes: element x of token j -> nibble (j&1) of byte 2x + (j>>1)
    nib = (grp[:, 2 * np.arange(128) + (j >> 1)] >> (4 * (j & 1))) & 0xF
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    sg = s[:, 4 * q:4 * q + 4].reshape(s.shape[0], -1)           # 32 bytes: block b of token j -> byte 4b + j
    return codes, sg[:, 4 * np.arange(8) + j]


def _row_fp8(plane, b, t, token4):
    c = plane.codes[b].cpu().numpy()    # [H, L, 128]
    if not token4:
        return c[:, t]
    q, j = t // 4, t % 4
    grp = c[:, 4 * q:4 * q + 4].reshape(c.shape[0], -1)          # element x of token j -> byte 4x + j
    return grp[:, 4 * np.arange(128) + j]
