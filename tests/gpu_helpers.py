"""Shared plumbing for the GPU parity tests: run the HIP path through the C ABI
and the oracle on the same seeded inputs.  The oracle side never sees a value
produced by the HIP path."""
import functools
import math

import numpy as np
import torch

import kvq_synth
from oracle import attention as OA
from oracle import formats as OF
from oracle import quant as OQ

DEV = "cuda:0"


def K():
    import quantized_kv_cache_nvfp4_amd as mod
    return mod


def announce(msg):
    print(f"[gpu-test] {msg}", flush=True)


# ---------------------------------------------------------------- oracle side
@functools.lru_cache(maxsize=8)
def oracle_gqa(cfg_key):
    """Oracle packing + dequantization of a GQA config (cached per session)."""
    inp = make_inputs(cfg_key)
    fmt = cfg_key[0]
    announce(f"  oracle pack {cfg_key}")
    kf, vf = kvq_synth.f64(inp.k), kvq_synth.f64(inp.v)
    ka, va = OQ.amax(kf, inp.kv_lens), OQ.amax(vf, inp.kv_lens)
    if fmt == "nvfp4":
        kc, ks, kst = OQ.nvfp4_pack(kf, ka)
        vc, vs, vst = OQ.nvfp4_pack(vf, va)
        khat, vhat = OQ.nvfp4_unpack(kc, ks, kst), OQ.nvfp4_unpack(vc, vs, vst)
        packed = dict(kc=kc, ks=ks, kst=kst, vc=vc, vs=vs, vst=vst, ka=ka, va=va)
    else:
        kc, kst = OQ.fp8_pack(kf, ka)
        vc, vst = OQ.fp8_pack(vf, va)
        khat, vhat = OQ.fp8_unpack(kc, kst), OQ.fp8_unpack(vc, vst)
        packed = dict(kc=kc, kst=kst, vc=vc, vst=vst, ka=ka, va=va)
    q64 = kvq_synth.f64(inp.q)
    announce(f"  oracle attention {cfg_key}")
    o, lse = OA.decode_gqa(q64, khat, vhat, inp.kv_lens, inp.softmax_scale)
    return packed, o, lse, khat, vhat


@functools.lru_cache(maxsize=8)
def oracle_pv_abs(cfg_key):
    """sum_t P_t |V_t| per output element (the oracle's attention with |V|):
    the scale of the error that rounding P to f16 can cause."""
    inp = make_inputs(cfg_key)
    _, _, _, khat, vhat = oracle_gqa(cfg_key)
    o, _ = OA.decode_gqa(kvq_synth.f64(inp.q), khat, np.abs(vhat), inp.kv_lens, inp.softmax_scale)
    return o


def fp32_bound(cfg_key, ref):
    """Per-element bound on |o_gpu - o_ref| for fp32 output.  Scores are
    exact f16 products summed in fp32; P goes to the P.V MFMA as f16 (one
    rounding, <= 2^-11 relative) on the bf16-query path, or as f16 hi + lo
    (<= 2^-22) on the fp32-query path; the rest is fp32 rounding, covered by
    1e-5 (1 + |o|)."""
    inp = make_inputs(cfg_key)
    base = 1e-5 * (1.0 + np.abs(ref))
    if inp.q.dtype == torch.float32:
        return base
    return base + 2.0 ** -11 * oracle_pv_abs(cfg_key)


_INPUT_CACHE = {}


def make_inputs(cfg_key):
    """cfg_key: (fmt, name, *params)."""
    if cfg_key in _INPUT_CACHE:
        return _INPUT_CACHE[cfg_key]
    fmt, name, *p = cfg_key
    if name == "tiny":
        inp = kvq_synth.tiny()
    elif name == "gqa":
        inp = kvq_synth.gqa(p[0])
    elif name == "mha":
        inp = kvq_synth.mha(p[0], B=p[1], H=p[2])
    elif name == "fp8":
        inp = kvq_synth.fp8_ragged(B=p[0])
    elif name == "custom":
        B, Hq, Hkv, D, lens, dt = p
        inp = kvq_synth.gqa_inputs(B, Hq, Hkv, D, None, kv_lens=list(lens), config="gqa", salt=7,
                                   dtype=torch.float32 if dt == "f32" else torch.bfloat16, outliers=False)
    else:
        raise KeyError(name)
    _INPUT_CACHE[cfg_key] = inp
    return inp


# ---------------------------------------------------------------- GPU side
def to_token4(codes, fmt):
    """Byte image of a TOKEN4 plane built from the oracle's per-element codes
    (pure index permutation, no arithmetic).  codes: [..., L, n] with one
    code per element (E2M1 nibble values 0..15 for "nvfp4", E4M3 bytes for
    "fp8" and for "scales", L % 4 == 0).  Inside each group of 4 tokens the
    elements go in order and, per element, the 4 tokens in token order; two
    NVFP4 nibbles share a byte, low nibble first."""
    a = np.asarray(codes, dtype=np.uint8)
    L, n = a.shape[-2], a.shape[-1]
    g = a.reshape(a.shape[:-2] + (L // 4, 4, n))
    g = np.swapaxes(g, -2, -1)                           # [.., q, element, token]
    if fmt == "nvfp4":
        g = (g[..., 0::2] | (g[..., 1::2] << 4)).astype(np.uint8)   # [.., q, element, 2]
    return g.reshape(a.shape[:-2] + (L, -1))


def nibbles(packed):
    """Row-major NVFP4 code bytes [..., n/2] -> per-element nibbles [..., n]."""
    p = np.asarray(packed, np.uint8)
    return np.stack([p & 0xF, p >> 4], -1).reshape(p.shape[:-1] + (-1,))


def empty_plane(fmt, shape_lead, D, layout, fill=0xFF):
    """A V plane of shape [..., L, .] pre-filled with `fill` bytes (0xFF:
    NaN E4M3 scales) so that reading padding rows would be caught."""
    k_ = K()
    if fmt == "nvfp4":
        return k_.NVFP4Plane(torch.full(shape_lead + (D // 2,), fill, dtype=torch.uint8, device=DEV),
                             torch.full(shape_lead + (D // 16,), fill, dtype=torch.uint8, device=DEV),
                             torch.empty(1, dtype=torch.float32, device=DEV), layout)
    return k_.FP8Plane(torch.full(shape_lead + (D,), fill, dtype=torch.uint8, device=DEV),
                       torch.empty(1, dtype=torch.float32, device=DEV), layout)


def gpu_pack(inp, fmt, v_layout=None, fill=0xFF):
    """K in the row layout; V in v_layout, by default the one the decode
    kernel reads at this head_dim (TOKEN4 at 128, rows at 64; TOKEN4 planes
    are padded to a multiple of 4 tokens and the padding holds 0xFF bytes)."""
    k_ = K()
    if v_layout is None:
        v_layout = k_.KVQ_PLANE_TOKEN4 if inp.D == 128 else k_.KVQ_PLANE_ROWS
    k, v = inp.k.to(DEV), inp.v.to(DEV)
    lens = torch.from_numpy(inp.kv_lens).to(DEV)
    ka, va = k_.kvq_amax(k, lens), k_.kvq_amax(v, lens)
    pack = k_.kvq_pack_nvfp4 if fmt == "nvfp4" else k_.kvq_pack_fp8
    if v_layout == k_.KVQ_PLANE_ROWS:
        kp = pack(k, ka)
        vp = pack(v, va)
    else:
        # both planes padded to a multiple of 4 tokens (shared strides)
        B, H, L, D = v.shape
        Lp = (L + 3) // 4 * 4
        kp = empty_plane(fmt, (B, H, Lp), D, k_.KVQ_PLANE_ROWS, fill)
        pack(k, ka, out=kp)
        vp = empty_plane(fmt, (B, H, Lp), D, v_layout, fill)
        pack(v, va, out=vp)
    return kp, vp, ka, va, lens


def page_plane(plane, bs, perm_seed, lens=None):
    """Paged copy of a contiguous plane [B, H, Lp, .] (codes and, for NVFP4,
    scales): blocks of bs tokens at physical blocks given by a seeded
    permutation of B * nb + 3 slots; returns (paged plane, block table).
    With lens (host ints [B]) the table entries of blocks that lie wholly at
    or past a request's length point at the spare slots, which hold 0xFF
    bytes (NaN E4M3 scales): the decode may read those entries but must not
    use them, and a read through one would show in the output."""
    k_ = K()
    B, H, Lp = plane.codes.shape[:3]
    nb = (Lp + bs - 1) // bs
    nphys = B * nb + 3
    full = np.random.default_rng(perm_seed).permutation(nphys)
    perm = full[: B * nb].reshape(B, nb).astype(np.int32)
    used = [nb] * B
    if lens is not None:
        spare = full[B * nb:]
        for b in range(B):
            used[b] = (int(lens[b]) + bs - 1) // bs
            perm[b, used[b]:] = spare[np.arange(nb - used[b]) % len(spare)]

    def pg(t):
        out = torch.full((nphys, H, bs) + tuple(t.shape[3:]), 0xFF, dtype=t.dtype, device=DEV)
        for b in range(B):
            for j in range(used[b]):
                n = min(bs, Lp - j * bs)
                out[int(perm[b, j]), :, :n] = t[b, :, j * bs: j * bs + n]
        return out

    if isinstance(plane, k_.NVFP4Plane):
        paged = k_.NVFP4Plane(pg(plane.codes), pg(plane.scales), plane.tensor_scale, plane.layout)
    else:
        paged = k_.FP8Plane(pg(plane.codes), plane.scale, plane.layout)
    return paged, torch.from_numpy(perm).to(DEV)


def gpu_decode(inp, kp, vp, lens, s, out_dtype=torch.bfloat16, out_scale=None, with_lse=False, fused=False,
               prob_scale=None, block_table=None, q=None, q_scale=None):
    """prob_scale: None for exact probabilities, else the FP8-P path;
    block_table: paged planes kp / vp (None: contiguous); q / q_scale: a
    query other than inp.q (e.g. FP8 codes with their scale)."""
    k_ = K()
    B, Hq, D = inp.B, inp.Hq, inp.D
    cap = 64
    part_o = torch.empty(B * Hq * cap * D, dtype=torch.float32, device=DEV)
    part_lse = torch.empty(B * Hq * cap, dtype=torch.float32, device=DEV)
    q = inp.q.to(DEV) if q is None else q
    fp8p = {}
    if prob_scale is not None:
        n = k_.kvq_fp8p_scratch_floats(B, Hq, cap, inp.Lmax)
        # NaN-filled: a score read that pass 1 did not write would show up
        fp8p = dict(quantize_p=True, prob_scale=prob_scale,
                    p_scratch=torch.full((max(n, 4),), float("nan"), dtype=torch.float32, device=DEV))
    args = k_.make_decode_args(q, kp, vp, lens, max_kv_len=inp.Lmax, softmax_scale=inp.softmax_scale,
                               num_splits=s, part_o=part_o, part_lse=part_lse, block_table=block_table,
                               q_scale=q_scale, **fp8p)
    out = torch.empty(B, Hq, D, dtype=out_dtype, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV) if with_lse else None
    if fused:
        counters = torch.zeros(B * inp.Hkv, dtype=torch.int32, device=DEV)
        used = k_.attn_decode(args, out, out_scale=out_scale, lse_out=lse, counters=counters)
        torch.cuda.synchronize()
        assert int(counters.abs().sum().item()) == 0, "fused decode must leave its counters at zero"
    else:
        used = k_.attn_decode_splitkv(args)
        k_.attn_decode_combine(part_o, part_lse, B, Hq, D, used, out, out_scale=out_scale, lse_out=lse)
    torch.cuda.synchronize()
    return out, used, lse


# ---------------------------------------------------------------- metrics
def err_report(got, ref):
    """The pages' three columns: max abs error, max rel error, cosine."""
    g = np.asarray(got, np.float64).ravel()
    r = np.asarray(ref, np.float64).ravel()
    ae = np.abs(g - r)
    rel = ae / np.maximum(np.abs(r), 1e-30)
    cos = float(g @ r / max(np.linalg.norm(g) * np.linalg.norm(r), 1e-300))
    return float(ae.max()), float(rel.max()), cos


def assert_bf16_output(got_bf16, ref, label=""):
    """Per element |o - o_ref| <= max(2e-3, 1 bf16 ulp(o_ref)) and cosine >= 0.9999."""
    g = got_bf16.float().cpu().double().numpy()
    tol = np.maximum(2e-3, OF.bf16_ulp(ref))
    bad = np.abs(g - ref) > tol
    mae, mre, cos = err_report(g, ref)
    assert not bad.any(), f"{label}: {bad.sum()} elements out of tolerance; max abs {mae:.3g}"
    assert cos >= 0.9999, f"{label}: cosine {cos}"
    return mae, mre, cos
