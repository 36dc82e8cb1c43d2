"""GPU parity for FP8 with one scale per kv head (the attn_head strategy of
compressed-tensors PR #436): per-head amax and packing bit-exact against the
oracle, decode (split, fused, FP8 probabilities) within the output gates of
the per-tensor path."""
import numpy as np
import pytest
import torch

import kvq_synth
from oracle import attention as OA
from oracle import formats as OF
from oracle import quant as OQ

from gpu_helpers import DEV, K, announce, assert_bf16_output, empty_plane, gpu_decode, to_token4

pytestmark = pytest.mark.gpu


def _inputs():
    """Ragged FP8 workload, 8 requests, K and V heads scaled by 2^(h - 4)
    (exact in bf16) so that the eight per-head scales differ by up to 128x."""
    inp = kvq_synth.fp8_ragged(B=8, lo=100, hi=700)
    f = (2.0 ** (torch.arange(inp.Hkv, dtype=torch.float32) - 4)).view(1, -1, 1, 1)
    inp.k = (inp.k.float() * f).to(inp.k.dtype)
    inp.v = (inp.v.float() * f.flip(1)).to(inp.v.dtype)
    return inp


_CACHE = {}


def _oracle(inp):
    if "o" not in _CACHE:
        kf, vf = kvq_synth.f64(inp.k), kvq_synth.f64(inp.v)
        ka, va = OQ.amax_heads(kf, inp.kv_lens), OQ.amax_heads(vf, inp.kv_lens)
        kc, ks = OQ.fp8_pack_heads(kf, ka)
        vc, vs = OQ.fp8_pack_heads(vf, va)
        khat, vhat = OQ.fp8_unpack_heads(kc, ks), OQ.fp8_unpack_heads(vc, vs)
        q64 = kvq_synth.f64(inp.q)
        o, lse = OA.decode_gqa(q64, khat, vhat, inp.kv_lens, inp.softmax_scale)
        pv_abs, _ = OA.decode_gqa(q64, khat, np.abs(vhat), inp.kv_lens, inp.softmax_scale)
        _CACHE.update(ka=ka, va=va, kc=kc, ks=ks, vc=vc, vs=vs, o=o, lse=lse, pv_abs=pv_abs)
    return _CACHE


def _pack(inp, v_layout):
    k_ = K()
    k, v = inp.k.to(DEV), inp.v.to(DEV)
    lens = torch.from_numpy(inp.kv_lens).to(DEV)
    ka, va = k_.kvq_amax(k, lens, per_head=True), k_.kvq_amax(v, lens, per_head=True)
    B, H, L, D = v.shape
    Lp = (L + 3) // 4 * 4
    kp = empty_plane("fp8", (B, H, Lp), D, k_.KVQ_PLANE_ROWS)
    kp.scale = torch.empty(H, dtype=torch.float32, device=DEV)
    k_.kvq_pack_fp8(k, ka, out=kp)
    vp = empty_plane("fp8", (B, H, Lp), D, v_layout)
    vp.scale = torch.empty(H, dtype=torch.float32, device=DEV)
    k_.kvq_pack_fp8(v, va, out=vp)
    torch.cuda.synchronize()
    return kp, vp, ka, va, lens


def test_amax_heads_exact():
    announce("fp8 heads amax")
    inp = _inputs()
    ref = _oracle(inp)
    k_ = K()
    lens = torch.from_numpy(inp.kv_lens).to(DEV)
    for x, want in ((inp.k, ref["ka"]), (inp.v, ref["va"])):
        got = k_.kvq_amax(x.to(DEV), lens, per_head=True).cpu().double().numpy()
        assert np.array_equal(got, want)
    # accumulate: max-merge into the values already there
    out = torch.full((inp.Hkv,), 3.0, dtype=torch.float32, device=DEV)
    k_.kvq_amax(inp.k.to(DEV), lens, out=out, accumulate=True, per_head=True)
    assert np.array_equal(out.cpu().double().numpy(), np.maximum(ref["ka"], 3.0))


@pytest.mark.parametrize("v_layout", [0, 1], ids=["rows", "token4"])
def test_pack_heads_bit_exact(v_layout):
    announce(f"fp8 heads pack v_layout={v_layout}")
    inp = _inputs()
    ref = _oracle(inp)
    kp, vp, _, _, _ = _pack(inp, v_layout)
    L = inp.Lmax
    assert np.array_equal(kp.scale.cpu().double().numpy(), ref["ks"])
    assert np.array_equal(vp.scale.cpu().double().numpy(), ref["vs"])
    kc = kp.codes.cpu().numpy()[:, :, :L]
    valid = np.arange(L)[None, :] < inp.kv_lens[:, None]
    sel = np.broadcast_to(valid[:, None, :, None], kc.shape)
    assert np.array_equal(kc[sel], ref["kc"][sel])
    vc = vp.codes.cpu().numpy()
    if v_layout == 1:
        Lp = vc.shape[2]
        want = np.zeros(ref["vc"].shape[:2] + (Lp, ref["vc"].shape[3]), np.uint8)
        want[:, :, :L] = ref["vc"]
        want = to_token4(want, "fp8")
        # compare the groups fully inside every request (the packer writes all rows of x)
        assert np.array_equal(vc[:, :, : L // 4 * 4], want[:, :, : L // 4 * 4])
    else:
        assert np.array_equal(vc[:, :, :L][sel], ref["vc"][sel])


def test_append_heads_batch():
    """Quantize-on-append with per-head scales: the new token's K and V rows
    go into existing planes at position dst_pos in one launch."""
    announce("fp8 heads append")
    inp = _inputs()
    ref = _oracle(inp)
    k_ = K()
    kp, vp, ka, va, lens = _pack(inp, 1)
    pos = torch.from_numpy(np.maximum(inp.kv_lens - 1, 0)).to(DEV)
    rows = torch.arange(inp.B)
    pos_c = pos.cpu()
    newk = inp.k[rows, :, pos_c].unsqueeze(2).contiguous().to(DEV)
    newv = inp.v[rows, :, pos_c].unsqueeze(2).contiguous().to(DEV)
    kp2 = K().FP8Plane(torch.zeros_like(kp.codes), torch.empty_like(kp.scale), kp.layout)
    vp2 = K().FP8Plane(torch.zeros_like(vp.codes), torch.empty_like(vp.scale), vp.layout)
    k_.kvq_pack_batch([(newk, ka, kp2, pos), (newv, va, vp2, pos)])
    torch.cuda.synchronize()
    kc2, vc2 = kp2.codes.cpu().numpy(), vp2.codes.cpu().numpy()
    for b in range(inp.B):
        if inp.kv_lens[b] == 0:
            continue
        t = int(pos_c[b])
        assert np.array_equal(kc2[b, :, t], ref["kc"][b, :, t])
        g, j = t // 4, t % 4          # TOKEN4: element x of token j at byte 4x + j of the group row
        vrow = vc2[b, :, 4 * g: 4 * g + 4].reshape(inp.Hkv, -1)
        assert np.array_equal(vrow[:, j::4][:, : inp.D], ref["vc"][b, :, t])


@pytest.mark.parametrize("mode", ["split3", "auto", "fused", "fp8p"])
def test_decode_heads(mode):
    announce(f"fp8 heads decode {mode}")
    inp = _inputs()
    ref = _oracle(inp)
    kp, vp, _, _, lens = _pack(inp, 1)
    s = 3 if mode in ("split3", "fp8p") else 0
    if mode == "fp8p":
        # the gate of the per-tensor FP8-P tests: P~ codes may differ only where
        # P / prob_scale lies within 2e-5 (relative) of an E4M3 boundary, each
        # such token adding one code step times |V_t| to the bound
        PS = float(np.float32(1.0 / 448.0))
        khat, vhat = OQ.fp8_unpack_heads(ref["kc"], ref["ks"]), OQ.fp8_unpack_heads(ref["vc"], ref["vs"])
        q = kvq_synth.f64(inp.q)
        want = OA.decode_gqa_fp8p(q, khat, vhat, inp.kv_lens, inp.softmax_scale, PS)
        r = OA.gqa_probs(q, khat, inp.kv_lens, inp.softmax_scale) / PS
        step = np.abs(OF.e4m3_round(r * (1 + 2e-5)) - OF.e4m3_round(r * (1 - 2e-5))) * PS
        va = np.repeat(np.abs(vhat), inp.Hq // inp.Hkv, axis=1)
        flip = np.einsum("bht,bhtd->bhd", step, va)
        mass = np.einsum("bht,bhtd->bhd", OF.e4m3_round(r) * PS, va)
        out, _, _ = gpu_decode(inp, kp, vp, lens, s, out_dtype=torch.float32, prob_scale=PS)
        g = out.cpu().double().numpy()
        bound = 1e-5 * (1 + np.abs(want)) + 2.0 ** -16 * mass + flip
        assert (np.abs(g - want) <= bound).all(), f"max abs {np.abs(g - want).max():.3g}"
        return
    out, used, _ = gpu_decode(inp, kp, vp, lens, s, fused=(mode == "fused"))
    assert_bf16_output(out, ref["o"], f"fp8 heads {mode} s={used}")
    out32, _, lse = gpu_decode(inp, kp, vp, lens, s, out_dtype=torch.float32, with_lse=True,
                               fused=(mode == "fused"))
    g = out32.cpu().double().numpy()
    bound = 1e-5 * (1.0 + np.abs(ref["o"])) + 2.0 ** -11 * ref["pv_abs"]
    assert (np.abs(g - ref["o"]) <= bound).all(), f"max abs {np.abs(g - ref['o']).max():.3g}"
    fin = np.isfinite(ref["lse"])
    l = lse.cpu().double().numpy()
    assert np.array_equal(np.isfinite(l), fin)
    assert np.abs(l[fin] - ref["lse"][fin]).max() < 1e-4


def test_per_head_amax_must_match_heads():
    """A per-head amax needs one value per kv head."""
    k_ = K()
    with pytest.raises(ValueError):
        k_.kvq_pack_fp8(torch.zeros(1, 3, 4, 16, dtype=torch.bfloat16, device=DEV),
                        torch.ones(2, dtype=torch.float32, device=DEV))
