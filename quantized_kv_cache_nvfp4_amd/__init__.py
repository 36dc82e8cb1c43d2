"""Quantized KV-cache attention decode for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``include/kvq.h`` (libkvq.so): each
function here has the C entry point's name, takes torch tensors, and only
marshals pointers, strides and the current HIP stream.  Every step of the
path runs in the HIP kernels; nothing is computed here.

Packed planes are plain uint8 tensors:
  NVFP4: codes [..., D/2] (element 2j in the low nibble of byte j),
         scales [..., D/16] (E4M3 bits), tensor scale float32 [1]
  FP8:   codes [..., D] (E4M3 bits), scale float32 [1]
"""
import ctypes
import math
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import (KVQ_OK, KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_ALIGN, KVQ_ERR_WORKSPACE, KVQ_ERR_HIP,
                   KVQ_BF16, KVQ_F16, KVQ_F32, KVQ_FP8E4M3, KVQ_LAYOUT_GQA, KVQ_LAYOUT_MLA, KVQ_NVFP4,
                   KVQ_PLANE_ROWS, KVQ_PLANE_TOKEN4, KvqError, KvqDecodeArgs, KvqPrefillArgs, KvqRows, check)

__all__ = [
    "kvq_amax", "kvq_pack_nvfp4", "kvq_pack_fp8", "kvq_unpack_nvfp4", "kvq_unpack_fp8",
    "attn_decode_splitkv", "attn_decode_combine", "attn_decode", "attn_decode_noalloc", "kvq_auto_num_splits", "kvq_device_cu_count",
    "kvq_fp8p_scratch_floats", "kvq_decode_workspace_bytes", "decode_workspace", "kvq_last_error", "kvq_version", "NVFP4Plane", "FP8Plane", "KvqError",
    "KVQ_F32", "KVQ_BF16", "KVQ_F16", "KVQ_FP8E4M3", "KVQ_NVFP4", "KVQ_LAYOUT_GQA", "KVQ_LAYOUT_MLA",
    "KVQ_PLANE_ROWS", "KVQ_PLANE_TOKEN4", "make_decode_args", "make_prefill_args", "attn_prefill",
    "KVQ_OK", "KVQ_ERR_ARG", "KVQ_ERR_UNSUPPORTED", "KVQ_ERR_ALIGN", "KVQ_ERR_WORKSPACE", "KVQ_ERR_HIP",
]

_DT = {torch.float32: KVQ_F32, torch.bfloat16: KVQ_BF16, torch.float16: KVQ_F16}


@dataclass
class NVFP4Plane:
    """An NVFP4-packed tensor: codes [..., D/2], scales [..., D/16], s_t [1];
    layout KVQ_PLANE_ROWS or KVQ_PLANE_TOKEN4 (byte order inside groups of 4
    tokens; the tensor shapes are the same)."""
    codes: torch.Tensor
    scales: torch.Tensor
    tensor_scale: torch.Tensor
    layout: int = KVQ_PLANE_ROWS

    @property
    def d(self):
        return self.codes.shape[-1] * 2


@dataclass
class FP8Plane:
    """An FP8 E4M3 tensor: codes [..., D], scale [1] (per tensor) or [Hkv]
    (one per kv head, the attn_head strategy), layout."""
    codes: torch.Tensor
    scale: torch.Tensor
    layout: int = KVQ_PLANE_ROWS

    @property
    def d(self):
        return self.codes.shape[-1]


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _rows(t: torch.Tensor, row_elems: int = None) -> KvqRows:
    """Rows of the last dim of t (up to 3 leading dims).  With row_elems set
    (packed planes) the strides are converted to plane rows."""
    if t.dim() < 1 or t.dim() > 4:
        raise ValueError("tensors must have 1 to 4 dims")
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError("the last dim must be contiguous")
    lead = list(t.shape[:-1])
    strides = list(t.stride()[:-1])
    while len(lead) < 3:
        lead.insert(0, 1)
        strides.insert(0, 0)
    if row_elems is not None:
        for s in strides:
            if s % row_elems:
                raise ValueError("packed plane strides must be whole rows")
        strides = [s // row_elems for s in strides]
    return KvqRows(*lead, *strides)


def kvq_last_error() -> str:
    return _lib.lib().kvq_last_error().decode()


def kvq_version() -> int:
    return _lib.lib().kvq_version()


def kvq_amax(x: torch.Tensor, kv_lens: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
             accumulate: bool = False, per_head: bool = False, stream=None) -> torch.Tensor:
    """Max |x| over rows [..., d]; rows with i2 >= kv_lens[i0] skipped.
    Returns a float32 [1] device tensor, or with per_head one value per
    index of the second-to-last-but-one dim (the kv heads of [B, Hkv, L, d])."""
    rows = _rows(x)
    if out is None:
        out = torch.zeros(rows.n1 if per_head else 1, dtype=torch.float32, device=x.device)
    fn = _lib.lib().kvq_amax_heads if per_head else _lib.lib().kvq_amax
    check(fn(_ptr(x), _DT[x.dtype], rows, x.shape[-1], _ptr(kv_lens), _ptr(out), int(accumulate), _stream(stream)))
    return out


def kvq_pack_nvfp4(x: torch.Tensor, amax: torch.Tensor, out: Optional[NVFP4Plane] = None,
                   dst_pos: Optional[torch.Tensor] = None, layout: int = KVQ_PLANE_ROWS,
                   stream=None) -> NVFP4Plane:
    """Pack rows of x ([..., D], D % 16 == 0) to NVFP4.  With ``out`` given,
    x's rows go to out's rows (offset by dst_pos[i0] along i2 if given) in
    out's layout."""
    d = x.shape[-1]
    if out is None:
        shp = tuple(x.shape[:-1])
        out = NVFP4Plane(torch.empty(shp + (d // 2,), dtype=torch.uint8, device=x.device),
                         torch.empty(shp + (d // 16,), dtype=torch.uint8, device=x.device),
                         torch.empty(1, dtype=torch.float32, device=x.device), layout)
    dst = _rows(out.codes, d // 2)
    sdst = _rows(out.scales, d // 16)
    if (dst.s0, dst.s1, dst.s2) != (sdst.s0, sdst.s1, sdst.s2):
        raise ValueError("code and scale planes must share their row layout")
    xr = _rows(x)
    check(_lib.lib().kvq_pack_nvfp4(_ptr(x), _DT[x.dtype], xr, d, _ptr(amax), _ptr(out.codes), _ptr(out.scales),
                                    dst, out.layout, _ptr(dst_pos), _ptr(out.tensor_scale), _stream(stream)))
    return out


def kvq_pack_fp8(x: torch.Tensor, amax: torch.Tensor, out: Optional[FP8Plane] = None,
                 dst_pos: Optional[torch.Tensor] = None, layout: int = KVQ_PLANE_ROWS, stream=None) -> FP8Plane:
    """Pack rows of x ([..., D]) to FP8 E4M3: one scale per tensor, or one per
    kv head when amax holds one value per head (kvq_amax(..., per_head=True))."""
    d = x.shape[-1]
    xr = _rows(x)
    per_head = amax.numel() > 1
    if per_head and amax.numel() != xr.n1:
        raise ValueError(f"per-head amax must have {xr.n1} entries (got {amax.numel()})")
    if out is None:
        out = FP8Plane(torch.empty(tuple(x.shape), dtype=torch.uint8, device=x.device),
                       torch.empty(amax.numel(), dtype=torch.float32, device=x.device), layout)
    dst = _rows(out.codes, d)
    fn = _lib.lib().kvq_pack_fp8_heads if per_head else _lib.lib().kvq_pack_fp8
    check(fn(_ptr(x), _DT[x.dtype], xr, d, _ptr(amax), _ptr(out.codes), dst, out.layout, _ptr(dst_pos),
             _ptr(out.scale), _stream(stream)))
    return out


def kvq_pack_batch(jobs, stream=None):
    """Pack several planes in one launch.  jobs: sequence of
    (x, amax, plane, dst_pos) with plane an NVFP4Plane (all of them) or an
    FP8Plane (all of them) already allocated; dst_pos may be None.  Typical
    use: the K and V rows of the new tokens of a decode step."""
    if not 1 <= len(jobs) <= _lib.KVQ_MAX_PACK_JOBS:
        raise ValueError(f"1..{_lib.KVQ_MAX_PACK_JOBS} jobs per call")
    fp4 = isinstance(jobs[0][2], NVFP4Plane)
    arr = (_lib.KvqPackJob * len(jobs))()
    for i, (x, amax, plane, dst_pos) in enumerate(jobs):
        if isinstance(plane, NVFP4Plane) != fp4:
            raise ValueError("all jobs of a batch must have the same format")
        d = x.shape[-1]
        if fp4:
            dst = _rows(plane.codes, d // 2)
            sdst = _rows(plane.scales, d // 16)
            if (dst.s0, dst.s1, dst.s2) != (sdst.s0, sdst.s1, sdst.s2):
                raise ValueError("code and scale planes must share their row layout")
            scales, sout = _ptr(plane.scales), _ptr(plane.tensor_scale)
        else:
            dst, scales, sout = _rows(plane.codes, d), ctypes.c_void_p(0), _ptr(plane.scale)
        per_head = (not fp4) and amax.numel() > 1   # FP8 with one scale per kv head
        arr[i] = _lib.KvqPackJob(_ptr(x), _DT[x.dtype], _rows(x), d, _ptr(amax), _ptr(plane.codes), scales, dst,
                                 plane.layout, _ptr(dst_pos), sout, int(per_head))
    fn = _lib.lib().kvq_pack_nvfp4_batch if fp4 else _lib.lib().kvq_pack_fp8_batch
    check(fn(arr, len(jobs), _stream(stream)))


def kvq_unpack_nvfp4(p: NVFP4Plane, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    d = p.d
    if out is None:
        out = torch.empty(tuple(p.codes.shape[:-1]) + (d,), dtype=torch.float32, device=p.codes.device)
    check(_lib.lib().kvq_unpack_nvfp4(_ptr(p.codes), _ptr(p.scales), _rows(p.codes, d // 2), p.layout, d,
                                      _ptr(p.tensor_scale), _ptr(out), _rows(out), _stream(stream)))
    return out


def kvq_unpack_fp8(p: FP8Plane, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    d = p.d
    if out is None:
        out = torch.empty(tuple(p.codes.shape), dtype=torch.float32, device=p.codes.device)
    check(_lib.lib().kvq_unpack_fp8(_ptr(p.codes), _rows(p.codes, d), p.layout, d, _ptr(p.scale), _ptr(out), _rows(out),
                                    _stream(stream)))
    return out


def kvq_auto_num_splits(num_cus: int, B: int, programs_per_req: int, max_kv_len: int, Dv: int, Hq: int) -> int:
    s = ctypes.c_int32(0)
    check(_lib.lib().kvq_auto_num_splits(num_cus, B, programs_per_req, max_kv_len, Dv, Hq, ctypes.byref(s)))
    return s.value


def kvq_device_cu_count() -> int:
    n = ctypes.c_int32(0)
    check(_lib.lib().kvq_device_cu_count(ctypes.byref(n)))
    return n.value


def kvq_fp8p_scratch_floats(B: int, Hq: int, s: int, max_kv_len: int) -> int:
    return _lib.lib().kvq_fp8p_scratch_floats(B, Hq, s, max_kv_len)


def kvq_decode_workspace_bytes(B: int, Hq: int, Dv: int, s: int) -> int:
    """Bytes of the split partials (part_o plus part_lse) for s splits."""
    return _lib.lib().kvq_decode_workspace_bytes(B, Hq, Dv, s)


def decode_workspace(B: int, Hq: int, Dv: int, s: int, device) -> tuple:
    """(part_o [B*Hq*s*Dv], part_lse [B*Hq*s]) float32 views of one buffer of
    kvq_decode_workspace_bytes(B, Hq, Dv, s) bytes: part_o first, part_lse
    right after it (both 4-byte aligned)."""
    nbytes = kvq_decode_workspace_bytes(B, Hq, Dv, s)
    if nbytes == 0:
        raise ValueError("B, Hq, Dv and s must be positive")
    buf = torch.empty(nbytes // 4, dtype=torch.float32, device=device)
    n_o = B * Hq * s * Dv
    return buf[:n_o], buf[n_o:]


def make_decode_args(q, k, v, kv_lens, *, max_kv_len, softmax_scale=None, num_splits=0, part_o, part_lse,
                     q_rope=None, k_rope=None, quantize_p=False, prob_scale=1.0 / 448.0,
                     p_scratch=None, block_table=None, q_scale=None, new_k=None, new_v=None) -> KvqDecodeArgs:
    """Fill the C decode-argument struct from tensors (no device work).

    GQA: q [B, Hq, D]; k, v NVFP4Plane / FP8Plane with codes [B, Hkv, Lmax, .],
    or, with block_table (int32 [B, max_blocks]), paged planes with codes
    [num_blocks, Hkv, block_size, .] (token t of request b in block
    block_table[b, t // block_size]).
    MLA: q = q_c [B, H, Dc]; k = NVFP4Plane of the latent [B, Lmax, .];
    v = None; q_rope [B, H, Dr] and k_rope [B, Lmax, Dr] bf16; with
    block_table, the latent and rope planes are [num_blocks, block_size, .].
    FP8 query (GQA): q uint8 E4M3 codes [B, Hq, D] with q_scale, a device
    float tensor of 1 (per tensor) or Hq (per query head) entries.
    Fused append (GQA): new_k, new_v [B, Hkv, D] (contiguous bf16 / f16 /
    f32) are the step's new token, packed into row kv_lens[b] - 1 of the
    planes by the decode itself and attended from its fresh codes; the
    split launch then reports one more partial per head.
    """
    a = KvqDecodeArgs()
    mla = v is None
    q_nv = None
    if isinstance(q, NVFP4Plane):   # NVFP4 latent query (MLA): codes [B, Hq, D/2], scales [B, Hq, D/16]
        if not mla:
            raise ValueError("NVFP4 queries are decoded for the MLA layout only")
        q_nv, q = q, q.codes
        if q.dim() != 3 or q_nv.scales.dim() != 3:
            raise ValueError("an NVFP4 query must be [B, Hq, D/2] codes with [B, Hq, D/16] scales")
        qr_c, qr_s = _rows(q, q.shape[-1]), _rows(q_nv.scales, q_nv.scales.shape[-1])
        if (qr_c.s1, qr_c.s2) != (qr_s.s1, qr_s.s2):
            raise ValueError("the NVFP4 query's codes and scales must share their row strides")
    if q.dim() != 3 or (q.shape[-1] > 1 and q.stride(-1) != 1):
        raise ValueError("q must be [B, Hq, D] with a contiguous last dim")
    if q_rope is not None and (q_rope.dim() != 3 or (q_rope.shape[-1] > 1 and q_rope.stride(-1) != 1)):
        raise ValueError("q_rope must be [B, Hq, Drope] with a contiguous last dim")
    fmt = KVQ_NVFP4 if isinstance(k, NVFP4Plane) else KVQ_FP8E4M3
    B, Hq, D = q.shape
    if q_nv is not None:
        D = q_nv.d
    a.kv_format, a.layout = fmt, (KVQ_LAYOUT_MLA if mla else KVQ_LAYOUT_GQA)
    a.B, a.Hq, a.D, a.Dv = B, Hq, D, D
    row_elems = D // 2 if fmt == KVQ_NVFP4 else D
    if mla:
        if k.layout != KVQ_PLANE_ROWS:
            raise ValueError("the MLA latent plane is read in the row layout")
        a.Hkv, a.Drope = 1, (q_rope.shape[-1] if q_rope is not None else 0)
        kr = _rows(k.codes, row_elems)  # [B, Lmax, .] -> n0=1, n1=B, n2=Lmax
        a.kv_sb, a.kv_sh, a.kv_st = kr.s1, 0, kr.s2
        if k_rope is not None:
            rr = _rows(k_rope, k_rope.shape[-1])
            if (rr.s1, rr.s2) != (kr.s1, kr.s2):
                raise ValueError("k_rope must share the latent plane's row layout")
        if block_table is not None:   # paged latent planes [num_blocks, block_size, .]
            if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
                raise ValueError("block_table must be an int32 [B, max_blocks] tensor with contiguous rows")
            a.block_table, a.block_size = _ptr(block_table), int(k.codes.shape[1])
            a.bt_stride, a.kv_sblk, a.kv_sb = block_table.stride(0), kr.s1, 0
        a.q_rope, a.k_rope = _ptr(q_rope), _ptr(k_rope)
        if q_rope is not None:
            a.qr_sb, a.qr_sh = q_rope.stride(0), q_rope.stride(1)
    else:
        a.Hkv = k.codes.shape[1]
        kr = _rows(k.codes, row_elems)
        vr = _rows(v.codes, row_elems)
        if (kr.s0, kr.s1, kr.s2) != (vr.s0, vr.s1, vr.s2):
            raise ValueError("K and V planes must share their row strides")
        if k.layout != KVQ_PLANE_ROWS:
            raise ValueError("K planes are read in the row layout")
        a.kv_sb, a.kv_sh, a.kv_st = kr.s0, kr.s1, kr.s2
        a.Drope = 0
        a.v_layout = v.layout
        if block_table is not None:   # paged planes [num_blocks, Hkv, block_size, .]
            if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
                raise ValueError("block_table must be an int32 [B, max_blocks] tensor with contiguous rows")
            a.block_table, a.block_size = _ptr(block_table), int(k.codes.shape[2])
            a.bt_stride, a.kv_sblk, a.kv_sb = block_table.stride(0), kr.s0, 0
    a.max_kv_len = int(max_kv_len)
    if q_nv is not None:
        qr_c = _rows(q, q.shape[-1])   # query rows: the struct counts them for NVFP4 queries
        a.q_dtype, a.q_scale, a.q_block_scales = KVQ_NVFP4, _ptr(q_nv.tensor_scale), _ptr(q_nv.scales)
        a.q, a.q_sb, a.q_sh = _ptr(q), qr_c.s1, qr_c.s2
    elif q.dtype == torch.uint8:   # FP8 query codes
        if q_scale is None:
            raise ValueError("an FP8 query needs q_scale")
        if q_scale.numel() not in (1, Hq):
            raise ValueError(f"q_scale must have 1 or Hq = {Hq} entries")
        a.q_dtype, a.q_scale, a.q_scale_per_head = KVQ_FP8E4M3, _ptr(q_scale), int(q_scale.numel() > 1)
    else:
        a.q_dtype = _DT[q.dtype]
    if q_nv is None:
        a.q, a.q_sb, a.q_sh = _ptr(q), q.stride(0), q.stride(1)
    if fmt == KVQ_NVFP4:
        a.k_codes, a.k_scales, a.k_scale = _ptr(k.codes), _ptr(k.scales), _ptr(k.tensor_scale)
        if not mla:
            a.v_codes, a.v_scales, a.v_scale = _ptr(v.codes), _ptr(v.scales), _ptr(v.tensor_scale)
        else:
            a.v_scale = _ptr(k.tensor_scale)
    else:
        a.k_codes, a.k_scale = _ptr(k.codes), _ptr(k.scale)
        a.v_codes, a.v_scale = _ptr(v.codes), _ptr(v.scale)
        per_head = k.scale.numel() > 1 or v.scale.numel() > 1   # the attn_head strategy
        if per_head and not (k.scale.numel() == v.scale.numel() == a.Hkv):
            raise ValueError(f"per-head FP8 scales must have Hkv = {a.Hkv} entries for K and V")
        a.kv_scale_per_head = int(per_head)
    a.kv_lens = _ptr(kv_lens)
    if (new_k is None) != (new_v is None):
        raise ValueError("new_k and new_v go together")
    if new_k is not None:
        Hkv = a.Hkv
        for t in (new_k, new_v):
            if tuple(t.shape) != (B, Hkv, D) or not t.is_contiguous() or t.dtype != new_k.dtype:
                raise ValueError(f"new_k / new_v must be contiguous [{B}, {Hkv}, {D}] tensors of one dtype")
        a.new_k, a.new_v, a.new_dtype = _ptr(new_k), _ptr(new_v), _DT[new_k.dtype]
    a.softmax_scale = float(softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(D))
    a.num_splits = int(num_splits)
    a.quantize_p, a.prob_scale = int(bool(quantize_p)), float(prob_scale)
    a.part_o, a.part_lse = _ptr(part_o), _ptr(part_lse)
    a.part_capacity = part_o.numel() // (B * Hq * D) if part_o is not None else 0
    a.p_scratch = _ptr(p_scratch)
    # the struct holds raw device pointers: keep the tensors they point into
    # alive for as long as the struct is (a plane built inline for the call
    # would otherwise be freed, and its memory may be returned to the driver)
    a._keep = (q, k, v, kv_lens, q_rope, k_rope, part_o, part_lse, p_scratch, block_table, q_scale, new_k, new_v,
               q_nv)
    return a


def attn_decode_tile_tokens(Hq: int, Hkv: int) -> int:
    """Tokens per tile of the GQA decode kernel (paged block sizes must be a multiple)."""
    return _lib.lib().attn_decode_tile_tokens(Hq, Hkv)


def attn_decode_splitkv(args: KvqDecodeArgs, stream=None) -> int:
    """Launch the split-KV decode for prepared args; returns the split count."""
    s = ctypes.c_int32(0)
    check(_lib.lib().attn_decode_splitkv(ctypes.byref(args), ctypes.byref(s), _stream(stream)))
    return s.value


def attn_decode_combine(part_o, part_lse, B, Hq, Dv, num_splits, out, out_scale=None, lse_out=None,
                        stream=None):
    """Merge partials into out ([B, Hq, Dv] float32, bfloat16 or uint8 = FP8 codes)."""
    odt = {torch.float32: KVQ_F32, torch.bfloat16: KVQ_BF16, torch.uint8: KVQ_FP8E4M3}[out.dtype]
    check(_lib.lib().attn_decode_combine(_ptr(part_o), _ptr(part_lse), B, Hq, Dv, num_splits, _ptr(out), odt,
                                         _ptr(out_scale), _ptr(lse_out), _stream(stream)))
    return out


def attn_decode(args: KvqDecodeArgs, out, out_scale=None, lse_out=None, counters=None, stream=None) -> int:
    """Split-KV decode and combine in one launch (the last work-group of each
    (request, kv head) merges the partials).  counters: int32 [B * Hkv],
    zero before the first call, left zero by every call.  Returns s."""
    odt = {torch.float32: KVQ_F32, torch.bfloat16: KVQ_BF16, torch.uint8: KVQ_FP8E4M3}[out.dtype]
    s = ctypes.c_int32(0)
    check(_lib.lib().attn_decode(ctypes.byref(args), _ptr(out), odt, _ptr(out_scale), _ptr(lse_out), _ptr(counters),
                                 ctypes.byref(s), _stream(stream)))
    return s.value


def attn_decode_noalloc(args: KvqDecodeArgs, out, out_scale=None, lse_out=None, stream=None) -> int:
    """attn_decode with the partials and merge counters in the library's
    static per-GPU scratch (no allocation, no workspace: the part_o /
    part_lse fields of args are ignored).  Calls that overlap on one GPU
    race.  Returns the number of partials merged per head."""
    odt = {torch.float32: KVQ_F32, torch.bfloat16: KVQ_BF16, torch.uint8: KVQ_FP8E4M3}[out.dtype]
    s = ctypes.c_int32(0)
    check(_lib.lib().attn_decode_noalloc(ctypes.byref(args), _ptr(out), odt, _ptr(out_scale), _ptr(lse_out),
                                         ctypes.byref(s), _stream(stream)))
    return s.value


def make_prefill_args(q, k, v, kv_lens, out, *, max_kv_len, softmax_scale=None, lse_out=None,
                      block_table=None, q_scale=None) -> KvqPrefillArgs:
    """Fill the C prefill-argument struct from tensors (no device work).

    q [B, Sq, Hq, D] bfloat16 (the chunk's queries; last dim contiguous);
    k, v NVFP4Plane / FP8Plane with codes [B, Hkv, Lmax, .] (K rows, V
    TOKEN4), or, with block_table (int32 [B, max_blocks]), paged planes
    [num_blocks, Hkv, block_size, .]; kv_lens int32 [B] (cache length
    including the chunk); out [B, Sq, Hq, D] float32 or bfloat16; lse_out
    float32 [B, Sq, Hq] contiguous or None.  FP8 queries: q uint8 E4M3
    codes [B, Sq, Hq, D] with q_scale, a device float tensor of 1 (per
    tensor) or Hq (per query head) entries.
    """
    if q.dim() != 4 or (q.shape[-1] > 1 and q.stride(-1) != 1):
        raise ValueError("q must be [B, Sq, Hq, D] with a contiguous last dim")
    if out.dim() != 4 or tuple(out.shape) != tuple(q.shape) or (out.shape[-1] > 1 and out.stride(-1) != 1):
        raise ValueError("out must be [B, Sq, Hq, D] like q, with a contiguous last dim")
    q8 = q.dtype == torch.uint8
    if q.dtype != torch.bfloat16 and not q8:
        raise ValueError("q must be bfloat16 or uint8 E4M3 codes")
    if q8 != (q_scale is not None):
        raise ValueError("q_scale goes with FP8 (uint8) queries and only with them")
    if q8 and q_scale.numel() not in (1, q.shape[2]):
        raise ValueError(f"q_scale must have 1 or Hq = {q.shape[2]} entries")
    if lse_out is not None and (tuple(lse_out.shape) != tuple(q.shape[:3]) or not lse_out.is_contiguous()
                                or lse_out.dtype != torch.float32):
        raise ValueError("lse_out must be a contiguous float32 [B, Sq, Hq] tensor")
    if k.layout != KVQ_PLANE_ROWS:
        raise ValueError("K planes are read in the row layout")
    a = KvqPrefillArgs()
    fmt = KVQ_NVFP4 if isinstance(k, NVFP4Plane) else KVQ_FP8E4M3
    B, Sq, Hq, D = q.shape
    a.kv_format, a.B, a.Hq, a.D, a.Sq = fmt, B, Hq, D, Sq
    a.Hkv = k.codes.shape[1]
    row_elems = D // 2 if fmt == KVQ_NVFP4 else D
    kr, vr = _rows(k.codes, row_elems), _rows(v.codes, row_elems)
    if (kr.s0, kr.s1, kr.s2) != (vr.s0, vr.s1, vr.s2):
        raise ValueError("K and V planes must share their row strides")
    if kr.s2 != 1 and kr.n2 > 1:
        raise ValueError("planes must have token stride 1")
    a.kv_sb, a.kv_sh = kr.s0, kr.s1
    a.v_layout = v.layout
    if block_table is not None:   # paged planes [num_blocks, Hkv, block_size, .]
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
            raise ValueError("block_table must be an int32 [B, max_blocks] tensor with contiguous rows")
        a.block_table, a.block_size = _ptr(block_table), int(k.codes.shape[2])
        a.bt_stride, a.kv_sblk, a.kv_sb = block_table.stride(0), kr.s0, 0
    a.max_kv_len = int(max_kv_len)
    a.q, a.q_dtype = _ptr(q), (KVQ_FP8E4M3 if q8 else KVQ_BF16)
    a.q_sb, a.q_st, a.q_sh = q.stride(0), q.stride(1), q.stride(2)
    if q8:
        a.q_scale, a.q_scale_per_head = _ptr(q_scale), int(q_scale.numel() > 1)
    if fmt == KVQ_NVFP4:
        a.k_codes, a.k_scales, a.k_scale = _ptr(k.codes), _ptr(k.scales), _ptr(k.tensor_scale)
        a.v_codes, a.v_scales, a.v_scale = _ptr(v.codes), _ptr(v.scales), _ptr(v.tensor_scale)
    else:
        a.k_codes, a.k_scale = _ptr(k.codes), _ptr(k.scale)
        a.v_codes, a.v_scale = _ptr(v.codes), _ptr(v.scale)
        per_head = k.scale.numel() > 1 or v.scale.numel() > 1
        if per_head and not (k.scale.numel() == v.scale.numel() == a.Hkv):
            raise ValueError(f"per-head FP8 scales must have Hkv = {a.Hkv} entries for K and V")
        a.kv_scale_per_head = int(per_head)
    a.kv_lens = _ptr(kv_lens)
    a.softmax_scale = float(softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(D))
    a.out, a.out_dtype = _ptr(out), {torch.float32: KVQ_F32, torch.bfloat16: KVQ_BF16}[out.dtype]
    a.o_sb, a.o_st, a.o_sh = out.stride(0), out.stride(1), out.stride(2)
    a.lse_out = _ptr(lse_out)
    a._keep = (q, k, v, kv_lens, out, lse_out, block_table, q_scale)
    return a


def attn_prefill(args: KvqPrefillArgs, stream=None):
    """Chunked prefill over the packed cache for prepared args (one launch)."""
    check(_lib.lib().attn_prefill(ctypes.byref(args), _stream(stream)))
