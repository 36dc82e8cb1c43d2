"""GPU parity: amax, NVFP4 / FP8 pack and unpack are bit-exact against the
oracle (the pages fix the formats; every decision is exact-real on both
sides)."""
import numpy as np
import pytest
import torch

import kvq_synth
from oracle import formats as OF
from oracle import quant as OQ

from gpu_helpers import DEV, K, announce, empty_plane, nibbles, to_token4

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("cfg", [("tiny",), ("gqa", 1024), ("mha", 1024)], ids=str)
def test_amax_and_nvfp4_pack_bit_exact(cfg):
    announce(f"pack nvfp4 {cfg}")
    inp = kvq_synth.tiny() if cfg[0] == "tiny" else (kvq_synth.gqa(cfg[1]) if cfg[0] == "gqa" else kvq_synth.mha(cfg[1]))
    for x in (inp.k, inp.v):
        xd = x.to(DEV)
        amax = K().kvq_amax(xd)
        xf = kvq_synth.f64(x)
        ref_amax = OQ.amax(xf)
        assert float(amax.item()) == ref_amax
        p = K().kvq_pack_nvfp4(xd, amax)
        c, s, st = OQ.nvfp4_pack(xf, ref_amax)
        torch.cuda.synchronize()
        assert float(p.tensor_scale.item()) == st
        assert np.array_equal(_np(p.scales), s)
        assert np.array_equal(_np(p.codes), c)
        # unpack: fp32(e * s_hat * s_t), one rounding
        u = K().kvq_unpack_nvfp4(p)
        assert np.array_equal(_np(u).astype(np.float64), OF.fp32_round(OQ.nvfp4_unpack(c, s, st)))


def test_amax_masks_ragged_padding():
    announce("amax ragged")
    inp = kvq_synth.fp8_ragged(B=8, lo=100, hi=700)
    lens = torch.from_numpy(inp.kv_lens).to(DEV)
    xd = inp.k.to(DEV)
    xd[:, :, -1, 0] = 1e4     # padding beyond every length (max len < 700 = Lmax) ... unless a request has len 700
    got = float(K().kvq_amax(xd, lens).item())
    ref = OQ.amax(kvq_synth.f64(xd.cpu()), inp.kv_lens)
    assert got == ref
    # accumulate = max-merge into an existing value
    out = torch.full((1,), 1e6, dtype=torch.float32, device=DEV)
    K().kvq_amax(xd, lens, out=out, accumulate=True)
    assert float(out.item()) == 1e6


@pytest.mark.parametrize("case", ["f32_flat", "bf16_strided", "bf16_misaligned", "bf16_d20"])
def test_amax_layouts(case):
    """amax over rows read as one flat run (contiguous, 16-byte aligned, d %
    8 == 0) and through the general row walk (strided rows, an unaligned
    base, d not a multiple of 8), with ragged lengths; exact against the
    oracle's max."""
    announce(f"amax layout {case}")
    g = torch.Generator().manual_seed(11)
    B, H, L = 3, 2, 37
    lens_np = np.array([37, 5, 0], dtype=np.int32)
    if case == "f32_flat":
        x = torch.randn(B, H, L, 64, generator=g, dtype=torch.float32) * 3
    elif case == "bf16_strided":
        x = (torch.randn(B, H, L, 80, generator=g) * 3).to(torch.bfloat16)[..., 8:72]
    elif case == "bf16_misaligned":
        flat = (torch.randn(B * H * L * 64 + 1, generator=g) * 3).to(torch.bfloat16)
        x = flat[1:].view(B, H, L, 64)
    else:
        x = (torch.randn(B, H, L, 20, generator=g) * 3).to(torch.bfloat16)
    x[0, 1, 36, 3] = -50.0                   # the maximum of a full-length request
    x[1, 0, 20, 2] = 1e4                     # past request 1's length: excluded
    xd = x.to(DEV)
    if case == "bf16_strided":
        xd = torch.empty(B, H, L, 80, dtype=torch.bfloat16, device=DEV)[..., 8:72]
        xd.copy_(x)
    elif case == "bf16_misaligned":
        fd = torch.empty(B * H * L * 64 + 1, dtype=torch.bfloat16, device=DEV)
        xd = fd[1:].view(B, H, L, 64)
        xd.copy_(x)
    lens = torch.from_numpy(lens_np).to(DEV)
    got = float(K().kvq_amax(xd, lens).item())
    assert got == OQ.amax(kvq_synth.f64(x), lens_np) == 50.0
    big = float(x[1, 0, 20, 2].abs())
    assert float(K().kvq_amax(xd).item()) == OQ.amax(kvq_synth.f64(x)) == big


def _adversarial_rows():
    """Rows that sit on every E2M1 / E4M3 decision boundary, plus zeros, -0,
    subnormal block scales and saturation; one 2688-scaled anchor fixes s_t."""
    rows = []
    s_t = 1.0
    for s_hat in [1.0, 0.875, 2.0 ** -7, 3 * 2.0 ** -9, 2.0 ** -9, 448.0, 13 * 2.0 ** -8, 1.5]:
        d = s_hat * s_t
        for mid in [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]:
            for x in [mid * d, np.nextafter(np.float32(mid * d), np.float32(0)),
                      np.nextafter(np.float32(mid * d), np.float32(1e9))]:
                r = np.zeros(16, np.float32)
                r[0] = 6 * d
                r[1] = x
                r[2] = -x
                r[3] = -0.0
                rows.append(r)
    # block-scale boundaries: bamax / 6 exactly at and around E4M3 midpoints
    pos = OF.e4m3_decode(np.arange(0x7F))
    for a, b in zip(pos[:-1], pos[1:]):
        m = np.float32((a + b) / 2 * 6)
        for x in (m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))):
            r = np.zeros(16, np.float32)
            r[5] = x
            r[6] = x / 3
            rows.append(r)
    z = np.zeros(16, np.float32); z[7] = -0.0
    rows.append(z)
    big = np.zeros(16, np.float32); big[0] = 2688.0; big[1] = -2000.0; big[2] = 2e-6
    rows.append(big)
    return np.stack(rows)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_nvfp4_pack_adversarial(dt):
    announce(f"pack nvfp4 adversarial {dt}")
    x = torch.from_numpy(_adversarial_rows()).to(dt)
    x = x.reshape(-1, 64) if x.shape[0] % 4 == 0 else x
    xf = kvq_synth.f64(x)
    amax_val = np.float32(2688.0)
    amax = torch.tensor([amax_val], device=DEV)
    p = K().kvq_pack_nvfp4(x.to(DEV), amax)
    c, s, st = OQ.nvfp4_pack(xf, amax_val)
    torch.cuda.synchronize()
    assert np.array_equal(_np(p.scales), s)
    assert np.array_equal(_np(p.codes), c)


def test_nvfp4_golden_blocks_on_gpu():
    announce("pack nvfp4 golden")
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_blocks.txt")
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        head, xs, sc, codes = [p.strip() for p in line.split("|")]
        amax = float(head.split("amax=")[1])
        x = torch.tensor([[float(v) for v in xs.split()]], dtype=torch.float32, device=DEV)
        p = K().kvq_pack_nvfp4(x, torch.tensor([amax], device=DEV))
        torch.cuda.synchronize()
        assert int(p.scales[0, 0].item()) == int(sc, 16), head
        assert [int(b) for b in _np(p.codes[0])] == [int(v, 16) for v in codes.split()], head


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_fp8_pack_bit_exact(dt):
    announce(f"pack fp8 {dt}")
    inp = kvq_synth.fp8_ragged(B=4, lo=64, hi=300)
    x = inp.k.to(dt)
    extra = torch.from_numpy(np.concatenate([
        np.ldexp(np.arange(1, 300, dtype=np.float64), -12), [1.0625, 1.1875, 2 ** -10, 3 * 2 ** -10, -0.0, 464.0, 470.0]
    ]).astype(np.float32)).to(dt)
    x.view(-1)[:extra.numel()] = extra
    xd = x.to(DEV)
    amax = K().kvq_amax(xd)
    p = K().kvq_pack_fp8(xd, amax)
    xf = kvq_synth.f64(x)
    c, sc = OQ.fp8_pack(xf, OQ.amax(xf))
    torch.cuda.synchronize()
    assert float(p.scale.item()) == sc
    assert np.array_equal(_np(p.codes), c)
    u = K().kvq_unpack_fp8(p)
    assert np.array_equal(_np(u).astype(np.float64), OF.fp32_round(OQ.fp8_unpack(c, sc)))


def _fp8_adversarial_values(amax_val):
    """Every E4M3 rounding midpoint (times the scale amax/448) and its two
    float32 neighbours, plus saturation, zeros and -0, both signs."""
    scale = np.float32(np.float32(amax_val) / np.float32(448.0))
    pos = OF.e4m3_decode(np.arange(0x7F))
    vals = [0.0, -0.0, 448.0 * scale, 500.0 * scale, 1e30]
    for a, b in zip(pos[:-1], pos[1:]):
        m = np.float32((a + b) / 2 * np.float64(scale))
        vals += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))]
    v = np.asarray(vals, np.float32)
    return np.concatenate([v, -v])


@pytest.mark.parametrize("amax_val,d", [(448.0, 16), (224.0, 16), (672.0, 16), (0.3, 16), (448.0, 20)])
def test_fp8_pack_adversarial(amax_val, d):
    """The adversarial values (every decision boundary): exact ties go to the
    even code; the GPU codes equal the oracle's bit for bit (d = 20: rows of a
    whole 16-element run and a 4-element one)."""
    announce(f"pack fp8 adversarial amax={amax_val} d={d}")
    v = _fp8_adversarial_values(amax_val)
    v = np.concatenate([v, np.zeros((-len(v)) % d, np.float32)]).reshape(-1, d)
    x = torch.from_numpy(v)
    amax = torch.tensor([np.float32(amax_val)], device=DEV)
    p = K().kvq_pack_fp8(x.to(DEV), amax)
    c, sc = OQ.fp8_pack(kvq_synth.f64(x), np.float32(amax_val))
    torch.cuda.synchronize()
    assert float(p.scale.item()) == sc
    assert np.array_equal(_np(p.codes), c)


@pytest.mark.parametrize("case", [("nvfp4", 64, torch.float32), ("nvfp4", 64, torch.bfloat16),
                                  ("fp8", 16, torch.float32), ("fp8", 20, torch.float32), ("fp8", 16, torch.bfloat16)],
                         ids=str)
def test_token4_pack_adversarial(case):
    """The adversarial rows packed into a TOKEN4 plane (whole 4-token groups:
    the per-element decisions of the group paths; d = 20 takes the FP8
    4-element path) equal the oracle's codes in that layout, bit for bit."""
    fmt, d, dt = case
    announce(f"pack {fmt} token4 adversarial d={d} {dt}")
    if fmt == "nvfp4":
        v, amax_val = _adversarial_rows().reshape(-1), np.float32(2688.0)
    else:
        v, amax_val = _fp8_adversarial_values(448.0), np.float32(448.0)
    per = 4 * d   # four tokens of d elements
    v = np.concatenate([v, np.zeros((-len(v)) % per, np.float32)]).reshape(1, 1, -1, d)
    x = torch.from_numpy(v).to(dt)
    L = x.shape[2]
    plane = empty_plane(fmt, (1, 1, L), d, K().KVQ_PLANE_TOKEN4, fill=0)
    amax = torch.tensor([amax_val], device=DEV)
    xf = kvq_synth.f64(x)
    if fmt == "nvfp4":
        K().kvq_pack_nvfp4(x.to(DEV), amax, out=plane)
        c, sc, _ = OQ.nvfp4_pack(xf, float(amax_val))
        torch.cuda.synchronize()
        assert np.array_equal(_np(plane.scales), to_token4(sc, "scales"))
        assert np.array_equal(_np(plane.codes), to_token4(nibbles(c), "nvfp4"))
    else:
        K().kvq_pack_fp8(x.to(DEV), amax, out=plane)
        c, _ = OQ.fp8_pack(xf, float(amax_val))
        torch.cuda.synchronize()
        assert np.array_equal(_np(plane.codes), to_token4(c, "fp8"))


def test_append_with_dst_pos():
    announce("pack append dst_pos")
    B, H, Lmax, D = 3, 2, 40, 128
    cache = K().NVFP4Plane(torch.zeros(B, H, Lmax, D // 2, dtype=torch.uint8, device=DEV),
                           torch.zeros(B, H, Lmax, D // 16, dtype=torch.uint8, device=DEV),
                           torch.zeros(1, device=DEV))
    new = torch.randn(B, H, 1, D, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    pos = torch.tensor([5, 0, 39], dtype=torch.int32, device=DEV)
    amax = torch.tensor([20.0], device=DEV)
    K().kvq_pack_nvfp4(new.to(DEV), amax, out=cache, dst_pos=pos)
    c, s, st = OQ.nvfp4_pack(kvq_synth.f64(new), 20.0)
    torch.cuda.synchronize()
    cc, cs = _np(cache.codes), _np(cache.scales)
    for b, p in enumerate([5, 0, 39]):
        assert np.array_equal(cc[b, :, p], c[b, :, 0])
        assert np.array_equal(cs[b, :, p], s[b, :, 0])
        mask = np.ones(Lmax, bool); mask[p] = False
        assert not cc[b, :, mask].any()


def test_full_size_gqa32k_sampled_rows():
    """The bench workload's cache (B=2, Hkv=8, 32K, D=128 with outliers):
    codes and scales of sampled rows (plus the amax row) bit-exact."""
    announce("pack nvfp4 gqa-32k sampled")
    inp = kvq_synth.gqa(32768)
    for x in (inp.k, inp.v):
        xd = x.to(DEV)
        amax = K().kvq_amax(xd)
        p = K().kvq_pack_nvfp4(xd, amax)
        flat = x.reshape(-1, 128)
        rng = np.random.default_rng(0)
        rows = rng.choice(flat.shape[0], 4096, replace=False)
        am_row = int(torch.argmax(flat.float().abs().max(dim=1).values))
        rows = np.unique(np.append(rows, am_row))
        xf = kvq_synth.f64(flat[torch.from_numpy(rows)])
        ref_amax = float(np.float32(amax.item()))
        assert ref_amax == OQ.amax(kvq_synth.f64(flat[am_row:am_row + 1]))
        c, s, st = OQ.nvfp4_pack(xf, ref_amax)
        torch.cuda.synchronize()
        gc = _np(p.codes.reshape(-1, 64))[rows]
        gs = _np(p.scales.reshape(-1, 8))[rows]
        assert np.array_equal(gs, s)
        assert np.array_equal(gc, c)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_token4_layout_pack_unpack(fmt):
    """TOKEN4 planes hold exactly the oracle's codes in the element-major
    interleaved order; padding rows keep their bytes; unpack reads the
    layout back; an append into a partly filled group keeps the neighbours."""
    announce(f"pack {fmt} token4")
    inp = kvq_synth.gqa_inputs(2, 8, 2, 128, None, kv_lens=[37, 61], config="gqa", salt=11, outliers=True)
    x = inp.v
    B, H, L, D = x.shape
    Lp = (L + 3) // 4 * 4
    xd = x.to(DEV)
    amax = K().kvq_amax(xd)
    plane = empty_plane(fmt, (B, H, Lp), D, K().KVQ_PLANE_TOKEN4, fill=0xAB)
    xf = kvq_synth.f64(x)
    pad_c = np.full((B, H, Lp - L, D), 0xAB, np.uint8)  # FP8 padding bytes
    if fmt == "nvfp4":
        K().kvq_pack_nvfp4(xd, amax, out=plane)
        c, sc, st = OQ.nvfp4_pack(xf, float(amax.item()))
        # untouched 0xAB bytes read as nibble 0xB for even tokens of a group
        # (low nibble) and 0xA for odd ones
        pad_n = np.where((np.arange(L, Lp) % 2 == 0)[:, None], 0xB, 0xA).astype(np.uint8)
        pad_n = np.broadcast_to(pad_n, (B, H, Lp - L, D))
        c_full = np.concatenate([nibbles(c), pad_n], axis=2)
        s_full = np.concatenate([sc, np.full((B, H, Lp - L, D // 16), 0xAB, np.uint8)], axis=2)
        torch.cuda.synchronize()
        assert np.array_equal(_np(plane.scales), to_token4(s_full, "scales"))
        assert np.array_equal(_np(plane.codes), to_token4(c_full, "nvfp4"))
        u = K().kvq_unpack_nvfp4(plane)
        ref = OF.fp32_round(OQ.nvfp4_unpack(c, sc, st))
    else:
        K().kvq_pack_fp8(xd, amax, out=plane)
        c, sc = OQ.fp8_pack(xf, float(amax.item()))
        c_full = np.concatenate([c, pad_c], axis=2)
        torch.cuda.synchronize()
        assert np.array_equal(_np(plane.codes), to_token4(c_full, "fp8"))
        u = K().kvq_unpack_fp8(plane)
        ref = OF.fp32_round(OQ.fp8_unpack(c, sc))
    torch.cuda.synchronize()
    assert np.array_equal(_np(u)[:, :, :L].astype(np.float64), ref)
    # append one token per request into the last, partly filled group: the
    # other tokens of that group must keep their bytes
    before = _np(u).copy()
    new = torch.randn(B, H, 1, D, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    pos = torch.tensor([L, L - 2], dtype=torch.int32, device=DEV)
    if fmt == "nvfp4":
        K().kvq_pack_nvfp4(new.to(DEV), amax, out=plane, dst_pos=pos)
        nc, ns, _ = OQ.nvfp4_pack(kvq_synth.f64(new), float(amax.item()))
        nref = OF.fp32_round(OQ.nvfp4_unpack(nc, ns, st))
        u2 = K().kvq_unpack_nvfp4(plane)
    else:
        K().kvq_pack_fp8(new.to(DEV), amax, out=plane, dst_pos=pos)
        nc, _ = OQ.fp8_pack(kvq_synth.f64(new), float(amax.item()))
        nref = OF.fp32_round(OQ.fp8_unpack(nc, sc))
        u2 = K().kvq_unpack_fp8(plane)
    torch.cuda.synchronize()
    u2 = _np(u2)
    for b_, p_ in enumerate([L, L - 2]):
        assert np.array_equal(u2[b_, :, p_].astype(np.float64), nref[b_, :, 0])
        keep = [t for t in range(L) if t != p_]
        assert np.array_equal(u2[b_][:, keep], before[b_][:, keep])


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_pack_batch_matches_single_calls(fmt):
    """One batched launch (K rows into a ROWS plane, V rows into a TOKEN4
    plane, with per-request positions) writes the same bytes as two
    single-plane calls, and those bytes are the oracle's."""
    announce(f"pack batch {fmt}")
    inp = kvq_synth.gqa_inputs(2, 8, 2, 128, None, kv_lens=[30, 45], config="gqa", salt=13, outliers=True)
    B, H, L, D = inp.k.shape
    Lp = (L + 3) // 4 * 4
    k, v = inp.k.to(DEV), inp.v.to(DEV)
    ka, va = K().kvq_amax(k), K().kvq_amax(v)
    pos = torch.tensor([3, 0], dtype=torch.int32, device=DEV)
    Lt = Lp + 4
    pack = K().kvq_pack_nvfp4 if fmt == "nvfp4" else K().kvq_pack_fp8
    a_k = empty_plane(fmt, (B, H, Lt), D, K().KVQ_PLANE_ROWS, fill=0x5A)
    a_v = empty_plane(fmt, (B, H, Lt), D, K().KVQ_PLANE_TOKEN4, fill=0x5A)
    b_k = empty_plane(fmt, (B, H, Lt), D, K().KVQ_PLANE_ROWS, fill=0x5A)
    b_v = empty_plane(fmt, (B, H, Lt), D, K().KVQ_PLANE_TOKEN4, fill=0x5A)
    pack(k, ka, out=a_k, dst_pos=pos)
    pack(v, va, out=a_v, dst_pos=pos)
    K().kvq_pack_batch([(k, ka, b_k, pos), (v, va, b_v, pos)])
    torch.cuda.synchronize()
    for a_, b_ in ((a_k, b_k), (a_v, b_v)):
        assert torch.equal(a_.codes, b_.codes)
        if fmt == "nvfp4":
            assert torch.equal(a_.scales, b_.scales)
            assert torch.equal(a_.tensor_scale, b_.tensor_scale)
        else:
            assert torch.equal(a_.scale, b_.scale)
    # and the K plane holds the oracle's codes at rows pos[b] + t
    kf = kvq_synth.f64(inp.k)
    if fmt == "nvfp4":
        c, sc, _ = OQ.nvfp4_pack(kf, float(ka.item()))
        got_c, got_s = _np(b_k.codes), _np(b_k.scales)
        for b_, p_ in enumerate([3, 0]):
            assert np.array_equal(got_c[b_, :, p_:p_ + L], c[b_])
            assert np.array_equal(got_s[b_, :, p_:p_ + L], sc[b_])
    else:
        c, _ = OQ.fp8_pack(kf, float(ka.item()))
        got_c = _np(b_k.codes)
        for b_, p_ in enumerate([3, 0]):
            assert np.array_equal(got_c[b_, :, p_:p_ + L], c[b_])
