"""ctypes view of libkvq.so: structs and function prototypes of include/kvq.h.

Loading fails loudly when the library has not been built; there is no
fallback path of any kind.
"""
import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "kvq.h")

KVQ_OK, KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_ALIGN, KVQ_ERR_WORKSPACE, KVQ_ERR_HIP = range(6)
KVQ_F32, KVQ_BF16, KVQ_F16, KVQ_FP8E4M3, KVQ_NVFP4 = range(5)
KVQ_LAYOUT_GQA, KVQ_LAYOUT_MLA = 0, 1
KVQ_PLANE_ROWS, KVQ_PLANE_TOKEN4 = 0, 1


class KvqRows(ctypes.Structure):
    _fields_ = [("n0", ctypes.c_int64), ("n1", ctypes.c_int64), ("n2", ctypes.c_int64),
                ("s0", ctypes.c_int64), ("s1", ctypes.c_int64), ("s2", ctypes.c_int64)]


class KvqPackJob(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("x_dtype", ctypes.c_int32), ("x_rows", KvqRows), ("d", ctypes.c_int32),
                ("amax", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("dst_rows", KvqRows), ("dst_layout", ctypes.c_int32), ("dst_pos", ctypes.c_void_p),
                ("scale_out", ctypes.c_void_p), ("scale_per_head", ctypes.c_int32)]


KVQ_MAX_PACK_JOBS = 8
KVQ_NOALLOC_SCRATCH_BYTES = 24 << 20


class KvqDecodeArgs(ctypes.Structure):
    _fields_ = [
        ("kv_format", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32), ("Dv", ctypes.c_int32), ("Drope", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("q_dtype", ctypes.c_int32),
        ("q_sb", ctypes.c_int64), ("q_sh", ctypes.c_int64),
        ("q_rope", ctypes.c_void_p), ("qr_sb", ctypes.c_int64), ("qr_sh", ctypes.c_int64),
        ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("v_layout", ctypes.c_int32),
        ("k_rope", ctypes.c_void_p),
        ("kv_sb", ctypes.c_int64), ("kv_sh", ctypes.c_int64), ("kv_st", ctypes.c_int64),
        ("kv_lens", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float),
        ("num_splits", ctypes.c_int32),
        ("quantize_p", ctypes.c_int32), ("prob_scale", ctypes.c_float),
        ("part_o", ctypes.c_void_p), ("part_lse", ctypes.c_void_p),
        ("part_capacity", ctypes.c_int32),
        ("p_scratch", ctypes.c_void_p),
        ("kv_scale_per_head", ctypes.c_int32),
        ("block_table", ctypes.c_void_p), ("block_size", ctypes.c_int32),
        ("bt_stride", ctypes.c_int64), ("kv_sblk", ctypes.c_int64),
        ("q_scale", ctypes.c_void_p), ("q_scale_per_head", ctypes.c_int32),
        ("new_k", ctypes.c_void_p), ("new_v", ctypes.c_void_p), ("new_dtype", ctypes.c_int32),
        ("q_block_scales", ctypes.c_void_p),
    ]


class KvqPrefillArgs(ctypes.Structure):
    _fields_ = [
        ("kv_format", ctypes.c_int32),
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("Sq", ctypes.c_int32), ("max_kv_len", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("q_dtype", ctypes.c_int32),
        ("q_sb", ctypes.c_int64), ("q_st", ctypes.c_int64), ("q_sh", ctypes.c_int64),
        ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("v_layout", ctypes.c_int32), ("kv_scale_per_head", ctypes.c_int32),
        ("kv_sb", ctypes.c_int64), ("kv_sh", ctypes.c_int64),
        ("kv_lens", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float),
        ("block_table", ctypes.c_void_p), ("block_size", ctypes.c_int32),
        ("bt_stride", ctypes.c_int64), ("kv_sblk", ctypes.c_int64),
        ("out", ctypes.c_void_p), ("out_dtype", ctypes.c_int32),
        ("o_sb", ctypes.c_int64), ("o_st", ctypes.c_int64), ("o_sh", ctypes.c_int64),
        ("lse_out", ctypes.c_void_p),
        ("q_scale", ctypes.c_void_p), ("q_scale_per_head", ctypes.c_int32),
    ]


_VP, _I32, _I64, _F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_PROTOS = {
    "kvq_last_error": (ctypes.c_char_p, []),
    "kvq_version": (_I32, []),
    "kvq_decode_args_size": (ctypes.c_size_t, []),
    "kvq_amax": (ctypes.c_int, [_VP, _I32, KvqRows, _I32, _VP, _VP, _I32, _VP]),
    "kvq_amax_heads": (ctypes.c_int, [_VP, _I32, KvqRows, _I32, _VP, _VP, _I32, _VP]),
    "kvq_pack_nvfp4": (ctypes.c_int, [_VP, _I32, KvqRows, _I32, _VP, _VP, _VP, KvqRows, _I32, _VP, _VP, _VP]),
    "kvq_pack_fp8": (ctypes.c_int, [_VP, _I32, KvqRows, _I32, _VP, _VP, KvqRows, _I32, _VP, _VP, _VP]),
    "kvq_pack_fp8_heads": (ctypes.c_int, [_VP, _I32, KvqRows, _I32, _VP, _VP, KvqRows, _I32, _VP, _VP, _VP]),
    "kvq_pack_nvfp4_batch": (ctypes.c_int, [ctypes.POINTER(KvqPackJob), _I32, _VP]),
    "kvq_pack_fp8_batch": (ctypes.c_int, [ctypes.POINTER(KvqPackJob), _I32, _VP]),
    "kvq_unpack_nvfp4": (ctypes.c_int, [_VP, _VP, KvqRows, _I32, _I32, _VP, _VP, KvqRows, _VP]),
    "kvq_unpack_fp8": (ctypes.c_int, [_VP, KvqRows, _I32, _I32, _VP, _VP, KvqRows, _VP]),
    "attn_decode_splitkv": (ctypes.c_int, [ctypes.POINTER(KvqDecodeArgs), ctypes.POINTER(_I32), _VP]),
    "attn_decode_combine": (ctypes.c_int, [_VP, _VP, _I32, _I32, _I32, _I32, _VP, _I32, _VP, _VP, _VP]),
    "attn_decode": (ctypes.c_int, [ctypes.POINTER(KvqDecodeArgs), _VP, _I32, _VP, _VP, _VP, ctypes.POINTER(_I32), _VP]),
    "attn_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(KvqDecodeArgs), _VP, _I32, _VP, _VP, ctypes.POINTER(_I32), _VP]),
    "kvq_auto_num_splits": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(_I32)]),
    "kvq_device_cu_count": (ctypes.c_int, [ctypes.POINTER(_I32)]),
    "kvq_fp8p_scratch_floats": (ctypes.c_size_t, [_I32, _I32, _I32, _I32]),
    "kvq_decode_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32]),
    "attn_decode_tile_tokens": (_I32, [_I32, _I32]),
    "kvq_prefill_args_size": (ctypes.c_size_t, []),
    "attn_prefill": (ctypes.c_int, [ctypes.POINTER(KvqPrefillArgs), _VP]),
}

_lib = None


def header_functions():
    """Names of the functions include/kvq.h declares."""
    with open(HEADER) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def lib():
    """The loaded library (raises if libkvq.so has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m quantized_kv_cache_nvfp4_amd.build` "
                "(or __graft_entry__.build()); there is no non-HIP fallback")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if L.kvq_decode_args_size() != ctypes.sizeof(KvqDecodeArgs):
            raise RuntimeError("libkvq.so and this binding disagree on kvq_decode_args; rebuild the library")
        if L.kvq_prefill_args_size() != ctypes.sizeof(KvqPrefillArgs):
            raise RuntimeError("libkvq.so and this binding disagree on kvq_prefill_args; rebuild the library")
        _lib = L
    return _lib


class KvqError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"kvq error {code}: {msg}")
        self.code = code


def check(rc):
    if rc != KVQ_OK:
        raise KvqError(rc, lib().kvq_last_error().decode())
    return rc
