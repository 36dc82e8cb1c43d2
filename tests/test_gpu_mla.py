"""GPU parity of the MLA latent-cache decode (NVFP4 latent 512 + bf16 rope 64,
16 heads) against the fp64 oracle.

The latent is packed on the GPU (bit-exact with the oracle, asserted here
too), the oracle dequantizes its own packing and runs exact MLA attention.
Gates: bf16 output per element |o - o_ref| <= max(2e-3, 1 bf16 ulp) and
cosine >= 0.9999; fp32 output per element <= 1e-5 (1 + |o|) +
2^-11 * sum_t P_t |c_hat_t| (P enters the P.V contraction as one f16 value;
scores and products are exact f16 / bf16 products summed in fp32).
"""
import functools

import numpy as np
import pytest
import torch

import kvq_synth
from oracle import attention as OA
from oracle import quant as OQ

from gpu_helpers import DEV, K, announce, assert_bf16_output

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


@functools.lru_cache(maxsize=8)
def _case(B, lens, salt):
    inp = kvq_synth.mla(L=max(lens), B=B, salt=salt, kv_lens=list(lens))
    cf = kvq_synth.f64(inp.c)
    amax = OQ.amax(cf[:, None], inp.kv_lens)   # latent viewed as [B, 1, L, 512]
    codes, scales, st = OQ.nvfp4_pack(cf, amax)
    chat = OQ.nvfp4_unpack(codes, scales, st)
    q_c, q_r, k_r = kvq_synth.f64(inp.q_c), kvq_synth.f64(inp.q_r), kvq_synth.f64(inp.k_r)
    o, lse = OA.decode_mla(q_c, q_r, chat, k_r, inp.kv_lens, inp.softmax_scale)
    o_abs, _ = OA.decode_mla(q_c, q_r, np.abs(chat), k_r, inp.kv_lens, inp.softmax_scale)
    return inp, (codes, scales, st, amax), o, lse, o_abs


def _gpu(inp, s, out_dtype, fused=False):
    k_ = K()
    c = inp.c.to(DEV)
    lens = torch.from_numpy(inp.kv_lens).to(DEV)
    amax = k_.kvq_amax(c.unsqueeze(1), lens)
    plane = k_.kvq_pack_nvfp4(c, amax)                      # codes [B, Lmax, 256], scales [B, Lmax, 32]
    q_c, q_r, k_r = inp.q_c.to(DEV), inp.q_r.to(DEV), inp.k_r.to(DEV)
    B, H, D = q_c.shape
    cap = 64
    part_o = torch.empty(B * H * cap * D, dtype=torch.float32, device=DEV)
    part_lse = torch.empty(B * H * cap, dtype=torch.float32, device=DEV)
    args = k_.make_decode_args(q_c, plane, None, lens, max_kv_len=int(inp.c.shape[1]),
                               softmax_scale=inp.softmax_scale, num_splits=s, part_o=part_o, part_lse=part_lse,
                               q_rope=q_r, k_rope=k_r)
    out = torch.empty(B, H, D, dtype=out_dtype, device=DEV)
    lse = torch.empty(B, H, dtype=torch.float32, device=DEV)
    if fused:
        used = k_.attn_decode(args, out, lse_out=lse)
    else:
        used = k_.attn_decode_splitkv(args)
        k_.attn_decode_combine(part_o, part_lse, B, H, D, used, out, lse_out=lse)
    torch.cuda.synchronize()
    return plane, amax, out, lse, used


def _check_fp32(out, o_ref, o_abs, label):
    g = _np(out).astype(np.float64)
    bound = 1e-5 * (1.0 + np.abs(o_ref)) + 2.0 ** -11 * o_abs
    bad = np.abs(g - o_ref) > bound
    assert not bad.any(), f"{label}: {bad.sum()} outputs off; max abs {np.abs(g - o_ref).max():.3g}"


MLA_CASES = [
    (2, (300, 77), 1), (2, (300, 77), 3), (3, (1000, 64, 65), 0), (2, (513, 1), 8), (4, (2048, 2000, 1500, 129), 4),
]


@pytest.mark.parametrize("B,lens,s", MLA_CASES, ids=lambda v: str(v))
def test_mla_decode(B, lens, s):
    announce(f"mla B={B} lens={lens} s={s}")
    inp, (codes, scales, st, amax), o_ref, lse_ref, o_abs = _case(B, lens, 1)
    plane, amax_g, out32, lse, used = _gpu(inp, s, torch.float32)
    # the latent plane is the oracle's, byte for byte
    assert float(amax_g.item()) == amax
    L = max(lens)
    assert np.array_equal(_np(plane.codes)[:, :L], codes)
    assert np.array_equal(_np(plane.scales)[:, :L], scales)
    _check_fp32(out32, o_ref, o_abs, f"mla s={used}")
    lse_g = _np(lse).astype(np.float64)
    assert np.allclose(lse_g, lse_ref, rtol=0, atol=1e-4)
    _, _, outb, _, _ = _gpu(inp, s, torch.bfloat16)
    assert_bf16_output(outb, o_ref, f"mla bf16 s={used}")


def test_mla_fused_entry_matches_two_launch():
    inp, _, o_ref, _, o_abs = _case(2, (700, 450), 2)
    _, _, a32, alse, _ = _gpu(inp, 5, torch.float32)
    _, _, b32, blse, _ = _gpu(inp, 5, torch.float32, fused=True)
    assert torch.equal(a32, b32) and torch.equal(alse, blse)
    _check_fp32(b32, o_ref, o_abs, "mla fused")


def test_mla_empty_request():
    """kv_len 0 gives output 0 and lse -inf; its neighbour is unaffected."""
    inp, _, o_ref, lse_ref, o_abs = _case(2, (0, 200), 3)
    _, _, out, lse, _ = _gpu(inp, 4, torch.float32)
    o = _np(out)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(_np(lse)[0]))
    _check_fp32(out[1:], o_ref[1:], o_abs[1:], "mla neighbour of empty")


@functools.lru_cache(maxsize=1)
def _full_inputs():
    inp = kvq_synth.mla()   # B=32, L=8192
    cf = kvq_synth.f64(inp.c)
    return inp, cf, OQ.amax(cf[:, None], inp.kv_lens)


@pytest.mark.parametrize("s", [0, 1, 4, 8])
def test_mla_full_config_sampled(s):
    """DeepSeek-V2 per-rank shape, B = 32, kv 8192, explicit and auto splits:
    the GPU output of 8 requests checked against the oracle run on those
    requests alone."""
    announce(f"mla full config s={s}")
    inp, cf, amax = _full_inputs()
    plane, amax_g, out, _, used = _gpu(inp, s, torch.bfloat16)
    assert used >= 1 and (s == 0 or used == s)
    assert float(amax_g.item()) == amax
    for b in range(0, 32, 4) if s else (0, 7, 17, 22, 31):
        codes, scales, st = OQ.nvfp4_pack(cf[b:b + 1], amax)
        assert np.array_equal(_np(plane.codes)[b:b + 1], codes)
        chat = OQ.nvfp4_unpack(codes, scales, st)
        o, _ = OA.decode_mla(kvq_synth.f64(inp.q_c[b:b + 1]), kvq_synth.f64(inp.q_r[b:b + 1]), chat,
                             kvq_synth.f64(inp.k_r[b:b + 1]), inp.kv_lens[b:b + 1], inp.softmax_scale)
        assert_bf16_output(out[b:b + 1], o, f"mla full b={b}")


# ------------------------------------------------------------ paged latent cache
def _page_mla(t, lens, bs, perm_seed):
    """Paged copy of a contiguous per-request plane t [B, Lp, .] (latent codes,
    scales or rope): blocks of bs tokens at physical blocks given by a seeded
    permutation of B * nb + 3 slots.  Blocks that lie wholly at or past a
    request's length point at the spare slots, which (like every unused
    slot) hold 0xFF bytes: NaN E4M3 scales and NaN bf16 rope values, so a
    read through such an entry shows in the output.  Returns (paged plane
    [nphys, bs, .], block table int32 [B, nb])."""
    B, Lp = t.shape[:2]
    nb = (Lp + bs - 1) // bs
    nphys = B * nb + 3
    perm = np.random.default_rng(perm_seed).permutation(nphys)
    table = perm[: B * nb].reshape(B, nb).astype(np.int32)
    spare = perm[B * nb:]
    for b in range(B):
        first_unused = (int(lens[b]) + bs - 1) // bs
        table[b, first_unused:] = spare[np.arange(nb - first_unused) % len(spare)]
    row_shape = tuple(t.shape[2:])
    raw = t.contiguous().view(torch.uint8).reshape(B, Lp, -1)
    out = torch.full((nphys, bs, raw.shape[-1]), 0xFF, dtype=torch.uint8, device=DEV)
    for b in range(B):
        for j in range((int(lens[b]) + bs - 1) // bs):
            n = min(bs, Lp - j * bs)
            out[int(table[b, j]), :n] = raw[b, j * bs: j * bs + n]
    return out.view(t.dtype).reshape((nphys, bs) + row_shape), torch.from_numpy(table).to(DEV)


def _gpu_paged(inp, plane, s, bs, out_dtype=torch.float32, fused=False, perm_seed=7):
    k_ = K()
    lens_np = inp.kv_lens
    lens = torch.from_numpy(lens_np).to(DEV)
    codes, bt = _page_mla(plane.codes, lens_np, bs, perm_seed)
    scales, bt2 = _page_mla(plane.scales, lens_np, bs, perm_seed)
    k_r, bt3 = _page_mla(inp.k_r.to(DEV), lens_np, bs, perm_seed)
    assert torch.equal(bt, bt2) and torch.equal(bt, bt3)
    paged = k_.NVFP4Plane(codes, scales, plane.tensor_scale, plane.layout)
    q_c, q_r = inp.q_c.to(DEV), inp.q_r.to(DEV)
    B, H, D = q_c.shape
    cap = 64
    part_o = torch.empty(B * H * cap * D, dtype=torch.float32, device=DEV)
    part_lse = torch.empty(B * H * cap, dtype=torch.float32, device=DEV)
    args = k_.make_decode_args(q_c, paged, None, lens, max_kv_len=int(inp.c.shape[1]),
                               softmax_scale=inp.softmax_scale, num_splits=s, part_o=part_o, part_lse=part_lse,
                               q_rope=q_r, k_rope=k_r, block_table=bt)
    out = torch.empty(B, H, D, dtype=out_dtype, device=DEV)
    lse = torch.empty(B, H, dtype=torch.float32, device=DEV)
    if fused:
        used = k_.attn_decode(args, out, lse_out=lse)
    else:
        used = k_.attn_decode_splitkv(args)
        k_.attn_decode_combine(part_o, part_lse, B, H, D, used, out, lse_out=lse)
    torch.cuda.synchronize()
    return out, lse, used


# (B, lens, s, block size): chunks that start inside a block (s = 4 over 2048
# tokens with 1024-token blocks), one-block requests, auto splits, a
# one-token request, more than one block per chunk
MLA_PAGED_CASES = [
    (2, (300, 77), 1, 64), (2, (300, 77), 3, 128), (3, (1000, 64, 65), 0, 256),
    (4, (2048, 2000, 1500, 129), 4, 1024), (2, (513, 1), 8, 64), (4, (2048, 2000, 1500, 129), 2, 64),
]


@pytest.mark.parametrize("B,lens,s,bs", MLA_PAGED_CASES, ids=lambda v: str(v))
def test_mla_paged_matches_contiguous(B, lens, s, bs):
    """The latent, scale and rope planes in permuted blocks decode to outputs
    and lse bit-identical to the contiguous planes (same chunking, same
    arithmetic), and within the oracle's fp32 gate."""
    announce(f"mla paged B={B} lens={lens} s={s} bs={bs}")
    inp, _, o_ref, _, o_abs = _case(B, lens, 1)
    plane, _, out_c, lse_c, used_c = _gpu(inp, s, torch.float32)
    out_p, lse_p, used_p = _gpu_paged(inp, plane, s, bs)
    assert used_p == used_c
    assert torch.equal(out_p, out_c) and torch.equal(lse_p, lse_c)
    _check_fp32(out_p, o_ref, o_abs, f"mla paged s={used_p} bs={bs}")


def test_mla_paged_fused_bf16():
    announce("mla paged fused bf16")
    inp, _, o_ref, _, _ = _case(2, (700, 450), 2)
    plane, _, out_c, _, _ = _gpu(inp, 5, torch.bfloat16, fused=True)
    out_p, _, _ = _gpu_paged(inp, plane, 5, 128, out_dtype=torch.bfloat16, fused=True)
    assert torch.equal(out_p, out_c)
    assert_bf16_output(out_p, o_ref, "mla paged fused")


def test_mla_paged_full_config_sampled():
    """B = 32, kv 8192, auto splits, 64-token blocks: bit-identical to the
    contiguous planes over every request."""
    announce("mla paged full config")
    inp = kvq_synth.mla()
    plane, _, out_c, lse_c, used = _gpu(inp, 0, torch.bfloat16)
    out_p, lse_p, used_p = _gpu_paged(inp, plane, 0, 64, out_dtype=torch.bfloat16)
    assert used_p == used
    assert torch.equal(out_p, out_c) and torch.equal(lse_p, lse_c)


def test_mla_paged_rejects_bad_blocks():
    """Block sizes that are not a power of two or not a multiple of the MLA
    tile (64 tokens) are refused before any launch."""
    k_ = K()
    inp, _, _, _, _ = _case(2, (300, 77), 1)
    plane, _, _, _, _ = _gpu(inp, 1, torch.float32)
    for bs in (32, 96):
        with pytest.raises(k_.KvqError):
            _gpu_paged(inp, plane, 2, bs)


# ---------------------------------------------------------------- NVFP4 latent query
QNV_CASES = [(2, (300, 77), 1, False), (3, (1000, 64, 65), 0, False), (2, (513, 1), 8, True)]


@pytest.mark.parametrize("B,lens,s,paged", QNV_CASES, ids=lambda v: str(v))
def test_mla_nvfp4_query(B, lens, s, paged):
    """The latent query q_c quantized to NVFP4 (per-tensor amax over the
    batch's queries, the same quantizer as the latent cache) and decoded from
    its codes: the query codes are bit-exact against the oracle's packing,
    and the output is within the fp32 gate of the oracle's MLA attention with
    the dequantized query (q_r stays bf16).  Paged: the same through a block
    table of 64-token blocks."""
    announce(f"mla nvfp4 query B={B} lens={lens} s={s} paged={paged}")
    k_ = K()
    inp, (codes, scales, st, _), _, _, _ = _case(B, lens, 2)
    # oracle: quantize q_c with its own packing, attention with the dequantized query
    qf = kvq_synth.f64(inp.q_c)
    q_amax = OQ.amax(qf[:, None])                        # [B, 1, H, 512]: every query element counts
    q_codes, q_scales, q_st = OQ.nvfp4_pack(qf, q_amax)
    q_hat = OQ.nvfp4_unpack(q_codes, q_scales, q_st)
    chat = OQ.nvfp4_unpack(codes, scales, st)
    q_r, k_r = kvq_synth.f64(inp.q_r), kvq_synth.f64(inp.k_r)
    o_ref, lse_ref = OA.decode_mla(q_hat, q_r, chat, k_r, inp.kv_lens, inp.softmax_scale)
    o_abs, _ = OA.decode_mla(q_hat, q_r, np.abs(chat), k_r, inp.kv_lens, inp.softmax_scale)
    # GPU: the same two kernels quantize the query
    c = inp.c.to(DEV)
    lens_d = torch.from_numpy(inp.kv_lens).to(DEV)
    plane = k_.kvq_pack_nvfp4(c, k_.kvq_amax(c.unsqueeze(1), lens_d))
    qc = inp.q_c.to(DEV)
    qplane = k_.kvq_pack_nvfp4(qc, k_.kvq_amax(qc.unsqueeze(1)))   # codes [B, H, 256], scales [B, H, 32]
    torch.cuda.synchronize()
    assert np.array_equal(_np(qplane.codes), q_codes)
    assert np.array_equal(_np(qplane.scales), q_scales)
    assert float(qplane.tensor_scale.item()) == np.float32(q_st)
    bt, k_r_d = None, inp.k_r.to(DEV)
    if paged:   # 64-token blocks at permuted physical blocks, 0xFF spares past each request
        codes_p, bt = _page_mla(plane.codes, inp.kv_lens, 64, 5)
        scales_p, bt2 = _page_mla(plane.scales, inp.kv_lens, 64, 5)
        k_r_d, bt3 = _page_mla(k_r_d, inp.kv_lens, 64, 5)
        assert torch.equal(bt, bt2) and torch.equal(bt, bt3)
        plane = k_.NVFP4Plane(codes_p, scales_p, plane.tensor_scale, plane.layout)
    H, D = 16, 512
    cap = 64
    part_o = torch.empty(B * H * cap * D, dtype=torch.float32, device=DEV)
    part_lse = torch.empty(B * H * cap, dtype=torch.float32, device=DEV)
    args = k_.make_decode_args(qplane, plane, None, lens_d, max_kv_len=int(inp.c.shape[1]),
                               softmax_scale=inp.softmax_scale, num_splits=s, part_o=part_o, part_lse=part_lse,
                               q_rope=inp.q_r.to(DEV), k_rope=k_r_d, block_table=bt)
    out = torch.empty(B, H, D, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, H, dtype=torch.float32, device=DEV)
    used = k_.attn_decode_splitkv(args)
    k_.attn_decode_combine(part_o, part_lse, B, H, D, used, out, lse_out=lse)
    torch.cuda.synchronize()
    _check_fp32(out, o_ref, o_abs, f"mla nvfp4 query B={B} lens={lens}")
    fin = np.isfinite(lse_ref)
    assert np.all(np.abs(_np(lse).astype(np.float64)[fin] - lse_ref[fin]) <= 1e-5 * (1 + np.abs(lse_ref[fin])))
