"""Host-side tests of the C ABI: the library loads and exports every function
include/kvq.h declares, the pure-host planning functions, and the argument
validation (every rejected call returns before any HIP call, so these run
without a GPU)."""
import ctypes
import math
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from quantized_kv_cache_nvfp4_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return _lib.lib()


@pytest.fixture(scope="module")
def K():
    import quantized_kv_cache_nvfp4_amd as K
    return K


def test_struct_size_matches_binding(L):
    from quantized_kv_cache_nvfp4_amd import _lib
    assert L.kvq_decode_args_size() == ctypes.sizeof(_lib.KvqDecodeArgs)


def test_exports_every_declared_symbol(L):
    from quantized_kv_cache_nvfp4_amd import _lib
    names = _lib.header_functions()
    assert {"kvq_pack_nvfp4", "kvq_pack_fp8", "attn_decode_splitkv", "attn_decode_combine",
            "kvq_auto_num_splits"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"libkvq.so does not export {n}"
    assert L.kvq_version() >= 100


def test_auto_split_worked_values(K):
    # 256 CUs (MI355X): GQA 4:1, B=2, 8 kv heads, 32K -> one work-group per
    # CU (query group of 4): 256 / 16 = 16 splits
    assert K.kvq_auto_num_splits(256, 2, 8, 32768, 128, 32) == 16
    # the same shape as MHA (query group of 1): two per CU, 2*256/16 = 32
    assert K.kvq_auto_num_splits(256, 2, 8, 32768, 128, 8) == 32
    # short context caps at ceil(L / 256)
    assert K.kvq_auto_num_splits(256, 2, 8, 1024, 128, 32) == 4
    # MHA B=1 H=32 32K: 2*256/32 = 16
    assert K.kvq_auto_num_splits(256, 1, 32, 32768, 128, 32) == 16
    # MHA B=2 H=16: at 32K two per CU (16 splits, 2048-token chunks); at 8K
    # two per CU would leave 512-token chunks, so one per CU: 256/32 = 8
    assert K.kvq_auto_num_splits(256, 2, 16, 32768, 128, 16) == 16
    assert K.kvq_auto_num_splits(256, 2, 16, 8192, 128, 16) == 8
    # large batch: already 512 programs -> 1
    assert K.kvq_auto_num_splits(256, 64, 8, 4096, 128, 32) == 1
    # MLA B=32 (16 heads share the request's latent: one 8-wave work-group
    # per CU): 256/32 = 8 splits; the partial-traffic bound (a third of the
    # KV bytes: 32*8192*576 / (3 * 32*16*513*8)) = 23 does not bind
    assert K.kvq_auto_num_splits(256, 32, 1, 8192, 512, 16) == 8
    # the bound binds for a wide head at B=4, kv 2048: min(256/4 = 64,
    # 2048/256 = 8, floor(4*2048*576 / (3 * 4*16*513*8)) = 5) = 5
    assert K.kvq_auto_num_splits(256, 4, 1, 2048, 512, 16) == 5
    assert K.kvq_auto_num_splits(256, 1, 1, 0, 128, 1) == 1


def test_auto_split_properties(K):
    for cus in (80, 256, 304):
        for B in (1, 2, 8, 64):
            for P in (1, 8, 32):
                for Lm in (1, 100, 1000, 32768, 1 << 20):
                    s = K.kvq_auto_num_splits(cus, B, P, Lm, 128, P * 4)
                    assert 1 <= s <= 64
                    assert s <= max(1, math.ceil(Lm / 256))


def test_auto_split_rejects_bad_args(K):
    with pytest.raises(K.KvqError) as e:
        K.kvq_auto_num_splits(0, 1, 1, 10, 128, 1)
    assert e.value.code == 1


def test_fp8p_scratch_size(K):
    assert K.kvq_fp8p_scratch_floats(2, 4, 3, 100) == 2 * 4 * 100
    assert K.kvq_fp8p_scratch_floats(2, 4, 3, 101) == 2 * 4 * 104
    assert K.kvq_fp8p_scratch_floats(0, 4, 3, 100) == 0


def _rows(n0, n1, n2, s0, s1, s2):
    from quantized_kv_cache_nvfp4_amd._lib import KvqRows
    return KvqRows(n0, n1, n2, s0, s1, s2)


FAKE = ctypes.c_void_p(0x10000)       # never dereferenced: every call below is rejected
FAKE_ODD = ctypes.c_void_p(0x10001)


def test_pack_validation(L, K):
    r = _rows(1, 1, 4, 0, 0, 24)
    R, T4 = K.KVQ_PLANE_ROWS, K.KVQ_PLANE_TOKEN4
    rc = L.kvq_pack_nvfp4(FAKE, K.KVQ_BF16, r, 24, FAKE, FAKE, FAKE, r, R, None, None, None)
    assert rc == 1 and "multiple of 16" in K.kvq_last_error()
    r16 = _rows(1, 1, 4, 0, 0, 16)
    assert L.kvq_pack_nvfp4(FAKE, K.KVQ_BF16, r16, 16, None, FAKE, FAKE, r16, R, None, None, None) == 1
    assert L.kvq_pack_nvfp4(FAKE, K.KVQ_F16, r16, 16, FAKE, FAKE, FAKE, r16, R, None, None, None) == 2
    assert L.kvq_pack_nvfp4(FAKE, K.KVQ_BF16, r16, 16, FAKE, FAKE_ODD, FAKE, r16, R, None, None, None) == 3
    rdiff = _rows(1, 2, 5, 0, 0, 1)
    assert L.kvq_pack_nvfp4(FAKE, K.KVQ_BF16, r16, 16, FAKE, FAKE, FAKE, rdiff, R, None, None, None) == 1
    assert L.kvq_pack_nvfp4(FAKE, K.KVQ_BF16, r16, 16, FAKE, FAKE, FAKE, r16, 9, None, None, None) == 1
    # TOKEN4: token stride must be 1 and lengths / strides multiples of 4
    assert L.kvq_pack_nvfp4(FAKE, K.KVQ_BF16, r16, 16, FAKE, FAKE, FAKE, r16, T4, None, None, None) == 3
    r_t4 = _rows(2, 3, 8, 24, 8, 1)
    r_t4_bad = _rows(2, 3, 6, 18, 6, 1)
    assert L.kvq_pack_nvfp4(FAKE, K.KVQ_BF16, r_t4_bad, 16, FAKE, FAKE, FAKE, r_t4_bad, T4, None, None, None) == 3
    assert L.kvq_pack_fp8(FAKE, K.KVQ_BF16, r_t4, 10, FAKE, FAKE, r_t4, T4, None, None, None) == 1
    assert L.kvq_pack_fp8(FAKE, K.KVQ_BF16, r16, 6, FAKE, FAKE, r16, R, None, None, None) == 1
    assert L.kvq_pack_fp8(FAKE, K.KVQ_F32, _rows(-1, 1, 1, 0, 0, 0), 16, FAKE, FAKE, r16, R, None, None, None) == 1
    assert L.kvq_amax(None, K.KVQ_F32, r16, 16, None, FAKE, 0, None) == 1
    assert L.kvq_amax(FAKE, K.KVQ_F32, r16, 0, None, FAKE, 0, None) == 1
    assert L.kvq_unpack_nvfp4(FAKE, FAKE, r16, R, 20, FAKE, FAKE, r16, None) == 1
    assert L.kvq_unpack_fp8(FAKE, r16, R, 16, None, FAKE, r16, None) == 1


def _good_args(K):
    a = K.KvqDecodeArgs()
    a.kv_format, a.layout = K.KVQ_NVFP4, K.KVQ_LAYOUT_GQA
    a.B, a.Hq, a.Hkv, a.D, a.Dv = 2, 32, 8, 128, 128
    a.max_kv_len = 1024
    a.q, a.q_dtype = FAKE, K.KVQ_BF16
    a.k_codes = a.k_scales = a.k_scale = FAKE
    a.v_codes = a.v_scales = a.v_scale = FAKE
    a.kv_lens = FAKE
    a.kv_sb, a.kv_sh, a.kv_st = 8 * 1024, 1024, 1
    a.v_layout = K.KVQ_PLANE_TOKEN4
    a.softmax_scale = 0.088
    a.num_splits = 4
    a.part_o = a.part_lse = FAKE
    a.part_capacity = 4
    return a


def _decode_rc(L, a):
    s = ctypes.c_int32(0)
    return L.attn_decode_splitkv(ctypes.byref(a), ctypes.byref(s), None)


def test_decode_validation(L, K):
    a = _good_args(K); a.Hq = 30
    assert _decode_rc(L, a) == 1                     # Hq % Hkv
    a = _good_args(K); a.Hq, a.Hkv = 24, 8
    assert _decode_rc(L, a) == 2                     # G = 3 unsupported
    a = _good_args(K); a.D = a.Dv = 96
    assert _decode_rc(L, a) == 2                     # D = 96 unsupported
    a = _good_args(K); a.num_splits = 8
    assert _decode_rc(L, a) == 4                     # exceeds part_capacity
    a = _good_args(K); a.num_splits = 65; a.part_capacity = 100
    assert _decode_rc(L, a) == 1
    a = _good_args(K); a.k_codes = FAKE_ODD
    assert _decode_rc(L, a) == 3
    a = _good_args(K); a.kv_format = 7
    assert _decode_rc(L, a) == 2
    a = _good_args(K); a.softmax_scale = float("nan")
    assert _decode_rc(L, a) == 1
    a = _good_args(K); a.kv_lens = None
    assert _decode_rc(L, a) == 1
    a = _good_args(K); a.layout = K.KVQ_LAYOUT_MLA; a.Hkv = 2; a.Hq = 16
    assert _decode_rc(L, a) == 1                     # MLA needs Hkv == 1
    a = _good_args(K); a.k_scales = None
    assert _decode_rc(L, a) == 1
    a = _good_args(K); a.v_layout = K.KVQ_PLANE_TOKEN4; a.D = a.Dv = 64
    assert _decode_rc(L, a) == 2                     # TOKEN4 V needs D = 128
    a = _good_args(K); a.v_layout = K.KVQ_PLANE_ROWS
    assert _decode_rc(L, a) == 2 and "TOKEN4" in K.kvq_last_error()   # D = 128 V is TOKEN4
    a = _good_args(K); a.v_layout = K.KVQ_PLANE_ROWS; a.D = a.Dv = 64
    a.block_table, a.block_size, a.bt_stride, a.kv_sblk = FAKE, 64, 16, 512
    assert _decode_rc(L, a) == 2 and "paged" in K.kvq_last_error()    # D = 64: contiguous planes only
    a = _good_args(K); a.q_dtype = K.KVQ_F32
    a.block_table, a.block_size, a.bt_stride, a.kv_sblk = FAKE, 64, 16, 512
    assert _decode_rc(L, a) == 2 and "fp32" in K.kvq_last_error()     # fp32 queries: contiguous planes
    a = _good_args(K); a.v_layout = K.KVQ_PLANE_TOKEN4; a.kv_st = 2
    assert _decode_rc(L, a) == 3
    a = _good_args(K); a.v_layout = 5
    assert _decode_rc(L, a) == 1
    a = _good_args(K); a.kv_scale_per_head = 1
    assert _decode_rc(L, a) == 2                     # per-head scales: FP8 only
    a = _good_args(K); a.kv_format = K.KVQ_FP8E4M3; a.k_scales = a.v_scales = None; a.kv_scale_per_head = 2
    assert _decode_rc(L, a) == 2
    assert L.attn_decode_splitkv(None, None, None) == 1


def test_combine_validation(L, K):
    assert L.attn_decode_combine(FAKE, FAKE, 2, 4, 128, 0, FAKE, K.KVQ_F32, None, None, None) == 1
    assert L.attn_decode_combine(FAKE, FAKE, 2, 4, 128, 65, FAKE, K.KVQ_F32, None, None, None) == 1
    assert L.attn_decode_combine(FAKE, FAKE, 2, 4, 128, 2, FAKE, K.KVQ_NVFP4, None, None, None) == 2
    assert L.attn_decode_combine(FAKE, FAKE, 2, 4, 128, 2, FAKE, K.KVQ_FP8E4M3, None, None, None) == 1
    assert L.attn_decode_combine(None, FAKE, 2, 4, 128, 2, FAKE, K.KVQ_F32, None, None, None) == 1
    assert L.attn_decode_combine(FAKE, FAKE, 2, 4, 128, 2, FAKE_ODD, K.KVQ_BF16, None, None, None) == 3


def test_pack_batch_validation(L, K):
    from quantized_kv_cache_nvfp4_amd import _lib
    R = K.KVQ_PLANE_ROWS
    r16 = _rows(1, 1, 4, 0, 0, 16)
    good = _lib.KvqPackJob(FAKE, K.KVQ_BF16, r16, 16, FAKE, FAKE, FAKE, r16, R, None, None)
    arr = (_lib.KvqPackJob * 9)(*([good] * 9))
    assert L.kvq_pack_nvfp4_batch(arr, 0, None) == 1
    assert L.kvq_pack_nvfp4_batch(arr, 9, None) == 1
    assert L.kvq_pack_nvfp4_batch(None, 1, None) == 1
    assert L.kvq_pack_fp8_batch(arr, 0, None) == 1
    # a bad job anywhere in the batch is reported with the single-call code
    bad = _lib.KvqPackJob(FAKE, K.KVQ_BF16, r16, 24, FAKE, FAKE, FAKE, r16, R, None, None)
    arr2 = (_lib.KvqPackJob * 2)(good, bad)
    assert L.kvq_pack_nvfp4_batch(arr2, 2, None) == 1 and "multiple of 16" in K.kvq_last_error()
    odd = _lib.KvqPackJob(FAKE, K.KVQ_BF16, r16, 16, FAKE, FAKE_ODD, FAKE, r16, R, None, None)
    arr3 = (_lib.KvqPackJob * 2)(good, odd)
    assert L.kvq_pack_nvfp4_batch(arr3, 2, None) == 3
    # one scale per kv head is an FP8 option
    ph = _lib.KvqPackJob(FAKE, K.KVQ_BF16, r16, 16, FAKE, FAKE, FAKE, r16, R, None, None, 1)
    assert L.kvq_pack_nvfp4_batch((_lib.KvqPackJob * 1)(ph), 1, None) == 1
    ph2 = _lib.KvqPackJob(FAKE, K.KVQ_BF16, r16, 16, FAKE, FAKE, FAKE, r16, R, None, None, 3)
    assert L.kvq_pack_fp8_batch((_lib.KvqPackJob * 1)(ph2), 1, None) == 1
    assert L.kvq_amax_heads(None, K.KVQ_F32, r16, 16, None, FAKE, 0, None) == 1
    assert L.kvq_pack_fp8_heads(FAKE, K.KVQ_F32, r16, 6, FAKE, FAKE, r16, R, None, None, None) == 1
    # empty jobs are skipped without a launch
    r0 = _rows(1, 1, 0, 0, 0, 16)
    empty = _lib.KvqPackJob(FAKE, K.KVQ_BF16, r0, 16, FAKE, FAKE, FAKE, r16, R, None, None)
    arr4 = (_lib.KvqPackJob * 2)(empty, empty)
    assert L.kvq_pack_nvfp4_batch(arr4, 2, None) == 0


def _mla_args(K):
    a = K.KvqDecodeArgs()
    a.kv_format, a.layout = K.KVQ_NVFP4, K.KVQ_LAYOUT_MLA
    a.B, a.Hq, a.Hkv, a.D, a.Dv, a.Drope = 2, 16, 1, 512, 512, 64
    a.max_kv_len = 1024
    a.q, a.q_dtype, a.q_sb, a.q_sh = FAKE, K.KVQ_BF16, 16 * 512, 512
    a.q_rope, a.qr_sb, a.qr_sh = FAKE, 16 * 64, 64
    a.k_codes = a.k_scales = a.k_scale = a.k_rope = FAKE
    a.kv_lens = FAKE
    a.kv_sb, a.kv_sh, a.kv_st = 1024, 0, 1
    a.softmax_scale = 0.072
    a.num_splits = 4
    a.part_o = a.part_lse = FAKE
    a.part_capacity = 4
    return a


def test_mla_paged_validation(L, K):
    """Paged latent planes: power-of-two block sizes that are multiples of the
    MLA tile (64 tokens), a table row covering max_kv_len, kv_sblk >= 0, a
    4-byte aligned table, at most 510 blocks per split."""
    def paged(bs=64, stride=16):
        a = _mla_args(K)
        a.block_table, a.block_size, a.bt_stride, a.kv_sblk, a.kv_sb = FAKE, bs, stride, bs, 0
        return a
    assert _decode_rc(L, paged(bs=32, stride=32)) == 1       # below the tile
    assert _decode_rc(L, paged(bs=192, stride=6)) == 1       # a multiple of the tile, not a power of two
    assert _decode_rc(L, paged(bs=0)) == 1
    assert _decode_rc(L, paged(stride=15)) == 1              # table row shorter than ceil(1024 / 64)
    a = paged(); a.kv_sblk = -1
    assert _decode_rc(L, a) == 1
    a = paged(); a.block_table = FAKE_ODD
    assert _decode_rc(L, a) == 3
    a = paged(stride=600); a.max_kv_len = 600 * 64; a.num_splits = 1
    assert _decode_rc(L, a) == 1                             # one split over 600 blocks
    a = paged(); a.kv_format = K.KVQ_FP8E4M3
    assert _decode_rc(L, a) == 2                             # NVFP4 latent only


def test_mla_validation(L, K):
    a = _mla_args(K); a.Hq = 8
    assert _decode_rc(L, a) == 2                     # 16 heads only
    a = _mla_args(K); a.Drope = 32
    assert _decode_rc(L, a) == 2
    a = _mla_args(K); a.q_dtype = K.KVQ_F32
    assert _decode_rc(L, a) == 2
    a = _mla_args(K); a.kv_format = K.KVQ_FP8E4M3
    assert _decode_rc(L, a) == 2
    a = _mla_args(K); a.k_rope = None
    assert _decode_rc(L, a) == 1
    a = _mla_args(K); a.q_sh = 500
    assert _decode_rc(L, a) == 3
    a = _mla_args(K); a.kv_st = 0
    assert _decode_rc(L, a) == 1


def test_nvfp4_query_validation(L, K):
    """NVFP4 latent queries: MLA layout only, with block scales and a tensor
    scale, 16-byte aligned codes and 4-byte aligned scales; the rows of a
    query count query rows (no element-stride rule)."""
    def nv(**kw):
        a = _mla_args(K)
        a.q_dtype, a.q_block_scales, a.q_scale, a.q_sb, a.q_sh = K.KVQ_NVFP4, FAKE, FAKE, 16, 1
        for k_, v_ in kw.items():
            setattr(a, k_, v_)
        return a
    assert _decode_rc(L, nv(q_block_scales=None)) == 1
    assert _decode_rc(L, nv(q_scale=None)) == 1
    assert _decode_rc(L, nv(q=FAKE_ODD)) == 3
    assert _decode_rc(L, nv(q_block_scales=FAKE_ODD)) == 3
    assert _decode_rc(L, nv(q_sb=-1)) == 1
    a = _good_args(K)
    a.q_dtype, a.q_block_scales, a.q_scale = K.KVQ_NVFP4, FAKE, FAKE
    assert _decode_rc(L, a) == 2                     # GQA layout: not implemented
    assert L.kvq_decode_args_size() == ctypes.sizeof(K.KvqDecodeArgs)


def test_decode_args_keep_their_tensors(K):
    """The decode-argument struct holds raw pointers: the tensors behind them
    (planes built inline for the call included) must live as long as it does,
    or a later kernel reads memory the allocator may have handed back."""
    import gc
    import weakref
    import torch
    B, Hkv, Hq, D, bs, nb = 1, 2, 8, 128, 64, 3
    q = torch.zeros(B, Hq, D, dtype=torch.bfloat16)
    lens = torch.full((B,), bs * nb, dtype=torch.int32)

    def plane():
        return K.NVFP4Plane(torch.zeros(B * nb, Hkv, bs, D // 2, dtype=torch.uint8),
                            torch.zeros(B * nb, Hkv, bs, D // 16, dtype=torch.uint8),
                            torch.ones(1), K.KVQ_PLANE_ROWS)

    part_o = torch.empty(B * Hq * 4 * D)
    part_lse = torch.empty(B * Hq * 4)
    bt = torch.arange(B * nb, dtype=torch.int32).view(B, nb)
    a = K.make_decode_args(q, plane(), plane(), lens, max_kv_len=bs * nb, num_splits=1, part_o=part_o,
                           part_lse=part_lse, block_table=bt)
    kc = weakref.ref(a._keep[1].codes)
    gc.collect()
    assert kc() is not None and kc().data_ptr() == a.k_codes
    del a
    gc.collect()
    assert kc() is None


def test_paged_decode_validation(L, K):
    """Paged caches: block sizes must be powers of two and multiples of the
    decode tile (64 tokens at G = 4); the table must cover max_kv_len."""
    def paged(bs=64, stride=16):
        a = _good_args(K)
        a.block_table, a.block_size, a.bt_stride, a.kv_sblk, a.kv_sb = FAKE, bs, stride, 8 * bs, 0
        a.kv_sh = bs
        return a
    assert K.attn_decode_tile_tokens(32, 8) == 64
    assert _decode_rc(L, paged(bs=32, stride=32)) == 1       # below the tile
    assert _decode_rc(L, paged(bs=192, stride=6)) == 1       # a multiple of the tile, not a power of two
    assert _decode_rc(L, paged(bs=0)) == 1
    assert _decode_rc(L, paged(stride=15)) == 1              # table row shorter than ceil(1024 / 64)
    a = paged(); a.kv_sblk = -1
    assert _decode_rc(L, a) == 1
    a = paged(); a.block_table = FAKE_ODD
    assert _decode_rc(L, a) == 3
    a = paged(); a.quantize_p, a.prob_scale, a.p_scratch = 1, 1.0 / 448.0, FAKE; a.block_size = 32
    assert _decode_rc(L, a) == 1                             # FP8-P: the same block-size rule
    a = paged(); a.v_layout = K.KVQ_PLANE_TOKEN4; a.kv_sblk = 8 * 64 + 2
    assert _decode_rc(L, a) == 3


def test_fp8_query_validation(L, K):
    """FP8 queries: GQA layout only, a scale pointer, 8-byte aligned rows."""
    def q8():
        a = _good_args(K)
        a.q_dtype, a.q_scale = K.KVQ_FP8E4M3, FAKE
        return a
    a = q8(); a.q_scale = None
    assert _decode_rc(L, a) == 1
    a = q8(); a.q_scale_per_head = 2
    assert _decode_rc(L, a) == 1
    a = q8(); a.q_scale = FAKE_ODD
    assert _decode_rc(L, a) == 3
    a = q8(); a.q = ctypes.c_void_p(0x10004)
    assert _decode_rc(L, a) == 3
    a = q8(); a.q_sh = 12
    assert _decode_rc(L, a) == 3
    a = q8(); a.layout = K.KVQ_LAYOUT_MLA; a.Hkv = 1; a.Hq = 16
    assert _decode_rc(L, a) == 2
    # FP8 queries with FP8 probabilities pass the query checks and meet the FP8-P ones
    a = q8(); a.quantize_p, a.prob_scale, a.p_scratch = 1, 1.0 / 448.0, None
    assert _decode_rc(L, a) == 1
    a = _good_args(K); a.q_dtype = K.KVQ_F16
    assert _decode_rc(L, a) == 2


def test_fused_append_validation(L, K):
    """Fused append: both rows, GQA layout, exact probabilities, a known row
    dtype, one more partial per head than splits (at most 64)."""
    def app():
        a = _good_args(K)
        a.new_k = a.new_v = FAKE
        a.new_dtype = K.KVQ_BF16
        a.num_splits, a.part_capacity = 3, 4
        return a
    a = app(); a.new_v = None
    assert _decode_rc(L, a) == 1
    a = app(); a.new_dtype = K.KVQ_FP8E4M3
    assert _decode_rc(L, a) == 2
    a = app(); a.num_splits = 4
    assert _decode_rc(L, a) == 4                     # 5 partials, capacity 4
    a = app(); a.num_splits, a.part_capacity = 64, 100
    assert _decode_rc(L, a) == 1
    a = app(); a.quantize_p, a.prob_scale, a.p_scratch = 1, 1.0 / 448.0, FAKE
    assert _decode_rc(L, a) == 2
    a = app(); a.new_k = FAKE_ODD
    assert _decode_rc(L, a) == 3
    a = app(); a.layout = K.KVQ_LAYOUT_MLA; a.Hkv = 1; a.Hq = 16
    assert _decode_rc(L, a) == 2
    a = app(); a.q_dtype = K.KVQ_F32
    assert _decode_rc(L, a) == 2                     # bf16 queries only


def test_query_alignment_validation(L, K):
    """bf16 / fp32 query rows are read with 16-byte loads: the base must be
    16-byte aligned and q_sb, q_sh whole 16-byte units (8 bf16, 4 fp32)."""
    a = _good_args(K); a.q = ctypes.c_void_p(0x10002)         # offset by one bf16 element
    assert _decode_rc(L, a) == 3 and "16-byte" in K.kvq_last_error()
    a = _good_args(K); a.q_sh = 129
    assert _decode_rc(L, a) == 3
    a = _good_args(K); a.q_sb = 4
    assert _decode_rc(L, a) == 3
    a = _good_args(K); a.q_dtype = K.KVQ_F32; a.q_sh = 4; a.q_sb = 4 * 32
    a.num_splits = 65; a.part_capacity = 100                 # passes the query checks, fails on s
    assert _decode_rc(L, a) == 1 and "num_splits" in K.kvq_last_error()
    a = _good_args(K); a.q_dtype = K.KVQ_F32; a.q_sh = 6
    assert _decode_rc(L, a) == 3


def test_mla_single_split_still_needs_partials(L, K):
    """The MLA path always writes partials and runs the combine, also through
    attn_decode with one split."""
    a = _mla_args(K); a.num_splits = 1; a.part_o = None
    s = ctypes.c_int32(0)
    rc = L.attn_decode(ctypes.byref(a), FAKE, K.KVQ_BF16, None, None, None, ctypes.byref(s), None)
    assert rc == 1 and "part_o" in K.kvq_last_error()
    a = _mla_args(K); a.num_splits = 1; a.part_capacity = 0
    rc = L.attn_decode(ctypes.byref(a), FAKE, K.KVQ_BF16, None, None, None, ctypes.byref(s), None)
    assert rc == 4
    a = _mla_args(K); a.num_splits = 1; a.part_lse = FAKE_ODD
    rc = L.attn_decode(ctypes.byref(a), FAKE, K.KVQ_BF16, None, None, None, ctypes.byref(s), None)
    assert rc == 3


def test_decode_workspace_bytes(K):
    # part_o [B][Hq][s][Dv] + part_lse [B][Hq][s], float32
    assert K.kvq_decode_workspace_bytes(2, 32, 128, 16) == 2 * 32 * 16 * 129 * 4
    assert K.kvq_decode_workspace_bytes(32, 16, 512, 16) == 32 * 16 * 16 * 513 * 4
    assert K.kvq_decode_workspace_bytes(0, 32, 128, 16) == 0
    assert K.kvq_decode_workspace_bytes(2, 32, 128, 0) == 0
    import torch
    po, pl = K.decode_workspace(2, 4, 8, 3, "cpu")
    assert po.numel() == 2 * 4 * 3 * 8 and pl.numel() == 2 * 4 * 3
    assert pl.data_ptr() == po.data_ptr() + po.numel() * 4


def test_binding_rejects_unreadable_views(K):
    """The binding refuses query views whose last dim is strided and MLA
    latent planes that are not in the row layout (the kernels read neither)."""
    import torch
    B, H, Dc, Dr, Lm = 1, 16, 512, 64, 64
    lens = torch.full((B,), Lm, dtype=torch.int32)
    lat = K.NVFP4Plane(torch.zeros(B, Lm, Dc // 2, dtype=torch.uint8), torch.zeros(B, Lm, Dc // 16, dtype=torch.uint8),
                       torch.ones(1), K.KVQ_PLANE_ROWS)
    q_c = torch.zeros(B, H, Dc, dtype=torch.bfloat16)
    q_r = torch.zeros(B, H, Dr, dtype=torch.bfloat16)
    k_r = torch.zeros(B, Lm, Dr, dtype=torch.bfloat16)
    po, pl = K.decode_workspace(B, H, Dc, 4, "cpu")
    K.make_decode_args(q_c, lat, None, lens, max_kv_len=Lm, num_splits=4, part_o=po, part_lse=pl, q_rope=q_r,
                       k_rope=k_r)
    with pytest.raises(ValueError):
        K.make_decode_args(torch.zeros(B, Dc, H, dtype=torch.bfloat16).transpose(1, 2), lat, None, lens,
                           max_kv_len=Lm, num_splits=4, part_o=po, part_lse=pl, q_rope=q_r, k_rope=k_r)
    with pytest.raises(ValueError):
        K.make_decode_args(q_c, lat, None, lens, max_kv_len=Lm, num_splits=4, part_o=po, part_lse=pl,
                           q_rope=torch.zeros(B, Dr, H, dtype=torch.bfloat16).transpose(1, 2), k_rope=k_r)
    lat4 = K.NVFP4Plane(lat.codes, lat.scales, lat.tensor_scale, K.KVQ_PLANE_TOKEN4)
    with pytest.raises(ValueError):
        K.make_decode_args(q_c, lat4, None, lens, max_kv_len=Lm, num_splits=4, part_o=po, part_lse=pl, q_rope=q_r,
                           k_rope=k_r)


def test_prefill_struct_size_matches_binding(L):
    from quantized_kv_cache_nvfp4_amd import _lib
    assert L.kvq_prefill_args_size() == ctypes.sizeof(_lib.KvqPrefillArgs)
    assert "attn_prefill" in _lib.header_functions()


def _prefill_args(K):
    a = K.KvqPrefillArgs()
    a.kv_format = K.KVQ_NVFP4
    a.B, a.Hq, a.Hkv, a.D, a.Sq = 2, 32, 8, 128, 64
    a.max_kv_len = 1024
    a.q, a.q_dtype = FAKE, K.KVQ_BF16
    a.q_sb, a.q_st, a.q_sh = 64 * 32 * 128, 32 * 128, 128
    a.k_codes = a.k_scales = a.k_scale = FAKE
    a.v_codes = a.v_scales = a.v_scale = FAKE
    a.v_layout = K.KVQ_PLANE_TOKEN4
    a.kv_sb, a.kv_sh = 8 * 1024, 1024
    a.kv_lens = FAKE
    a.softmax_scale = 0.088
    a.out, a.out_dtype = FAKE, K.KVQ_BF16
    a.o_sb, a.o_st, a.o_sh = 64 * 32 * 128, 32 * 128, 128
    return a


def test_prefill_validation(L, K):
    """Every case breaks one rule and must be refused before any launch."""
    rc = lambda a: L.attn_prefill(ctypes.byref(a), None)   # noqa: E731
    cases = [
        (lambda a: setattr(a, "kv_format", 7), K.KVQ_ERR_UNSUPPORTED),
        (lambda a: setattr(a, "Hq", 30), K.KVQ_ERR_ARG),                      # Hq % Hkv
        (lambda a: (setattr(a, "Hq", 128)), K.KVQ_ERR_UNSUPPORTED),           # G = 16
        (lambda a: (setattr(a, "Hq", 24)), K.KVQ_ERR_UNSUPPORTED),            # G = 3
        (lambda a: setattr(a, "D", 64), K.KVQ_ERR_UNSUPPORTED),
        (lambda a: setattr(a, "Sq", -1), K.KVQ_ERR_ARG),
        (lambda a: setattr(a, "max_kv_len", -1), K.KVQ_ERR_ARG),
        (lambda a: setattr(a, "q", None), K.KVQ_ERR_ARG),
        (lambda a: setattr(a, "v_codes", None), K.KVQ_ERR_ARG),
        (lambda a: setattr(a, "kv_lens", None), K.KVQ_ERR_ARG),
        (lambda a: setattr(a, "out", None), K.KVQ_ERR_ARG),
        (lambda a: setattr(a, "v_scales", None), K.KVQ_ERR_ARG),               # NVFP4 needs scales
        (lambda a: setattr(a, "q_dtype", K.KVQ_F32), K.KVQ_ERR_UNSUPPORTED),
        (lambda a: setattr(a, "v_layout", K.KVQ_PLANE_ROWS), K.KVQ_ERR_UNSUPPORTED),
        (lambda a: setattr(a, "kv_scale_per_head", 1), K.KVQ_ERR_UNSUPPORTED),  # NVFP4
        (lambda a: setattr(a, "softmax_scale", 0.0), K.KVQ_ERR_ARG),
        (lambda a: setattr(a, "softmax_scale", float("inf")), K.KVQ_ERR_ARG),
        (lambda a: setattr(a, "out_dtype", K.KVQ_FP8E4M3), K.KVQ_ERR_UNSUPPORTED),
        (lambda a: setattr(a, "q", FAKE_ODD), K.KVQ_ERR_ALIGN),
        (lambda a: setattr(a, "q_st", 100), K.KVQ_ERR_ALIGN),
        (lambda a: setattr(a, "k_codes", FAKE_ODD), K.KVQ_ERR_ALIGN),
        (lambda a: setattr(a, "o_sh", 130), K.KVQ_ERR_ALIGN),
        (lambda a: setattr(a, "kv_sh", 1022), K.KVQ_ERR_ALIGN),                 # TOKEN4 groups
        (lambda a: setattr(a, "kv_sb", -4), K.KVQ_ERR_ARG),
        (lambda a: (setattr(a, "block_table", FAKE), setattr(a, "block_size", 32), setattr(a, "bt_stride", 64)),
         K.KVQ_ERR_ARG),                                                         # below the 64-token tile
        (lambda a: (setattr(a, "block_table", FAKE), setattr(a, "block_size", 96), setattr(a, "bt_stride", 64)),
         K.KVQ_ERR_ARG),                                                         # not a power of two
        (lambda a: (setattr(a, "block_table", FAKE), setattr(a, "block_size", 64), setattr(a, "bt_stride", 8)),
         K.KVQ_ERR_ARG),                                                         # table too short
        (lambda a: (setattr(a, "block_table", FAKE), setattr(a, "block_size", 64), setattr(a, "bt_stride", 16),
                    setattr(a, "kv_sblk", 6)), K.KVQ_ERR_ALIGN),
        # FP8 queries: a scale is required, per-head flag 0/1, 8-byte codes, aligned scale
        (lambda a: setattr(a, "q_dtype", K.KVQ_FP8E4M3), K.KVQ_ERR_ARG),
        (lambda a: (setattr(a, "q_dtype", K.KVQ_FP8E4M3), setattr(a, "q_scale", FAKE),
                    setattr(a, "q_scale_per_head", 2)), K.KVQ_ERR_ARG),
        (lambda a: (setattr(a, "q_dtype", K.KVQ_FP8E4M3), setattr(a, "q_scale", FAKE),
                    setattr(a, "q", FAKE_ODD)), K.KVQ_ERR_ALIGN),
        (lambda a: (setattr(a, "q_dtype", K.KVQ_FP8E4M3), setattr(a, "q_scale", FAKE_ODD)), K.KVQ_ERR_ALIGN),
        (lambda a: (setattr(a, "q_dtype", K.KVQ_FP8E4M3), setattr(a, "q_scale", FAKE),
                    setattr(a, "q_sh", 12)), K.KVQ_ERR_ALIGN),
    ]
    for i, (mutate, want) in enumerate(cases):
        a = _prefill_args(K)
        mutate(a)
        got = rc(a)
        assert got == want, f"case {i}: got {got}, want {want} ({L.kvq_last_error().decode()})"
        assert L.kvq_last_error().decode() != ""
    assert L.attn_prefill(None, None) == K.KVQ_ERR_ARG
    # an empty chunk is valid and launches nothing
    a = _prefill_args(K)
    a.Sq = 0
    assert rc(a) == K.KVQ_OK
