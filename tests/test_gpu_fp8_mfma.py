"""The FP8 matrix core's accumulation error, measured on the device through
the probe library (kvq_probe_mfma_fp8): the constant that the FP8-query
prefill's tolerance rests on.

gfx950's FP8 E4M3 16x16x32 MFMA forms its 32 products exactly but adds them
at less than fp32 precision when their magnitudes spread widely: measured
on uniformly random codes (the widest spread E4M3 allows) the error reaches
about 2^-11.6 of sum |p| for one instruction and 2^-12.7 of the total for
four chained ones (the prefill's head_dim of 128), and products within a
narrow magnitude range add exactly.  The prefill tests allow each score an
error of EPS_FP8_DOT * sum_k |q_k k_k|, EPS_FP8_DOT = 2^-10; this test
checks that bound on the matrix core itself, with the operand layout the
prefill kernel uses (lane l: row l % 16, elements 8 (l / 16) .. + 7)."""
import ctypes
import os

import numpy as np
import pytest

from oracle import formats as OF

EPS_FP8_DOT = 2.0 ** -10


def _probe_lib():
    from quantized_kv_cache_nvfp4_amd import build as kbuild
    if not os.path.exists(kbuild.PROBE_LIB_PATH):
        pytest.fail(f"{kbuild.PROBE_LIB_PATH} missing: build the package first")
    lib = ctypes.CDLL(kbuild.PROBE_LIB_PATH)
    lib.kvq_probe_mfma_fp8.restype = ctypes.c_int
    lib.kvq_probe_mfma_fp8.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p]
    return lib


def test_probe_library_exports():
    lib = _probe_lib()
    assert all(hasattr(lib, n) for n in ("kvq_probe_read", "kvq_probe_read_chunks", "kvq_probe_read_nt",
                                        "kvq_probe_read_chunks_nt", "kvq_probe_mfma_fp8"))
    # argument checks run on the host: nothing is launched
    assert lib.kvq_probe_mfma_fp8(None, None, 4, 4, None, None) == 1
    fake = ctypes.c_void_p(0x10000)
    assert lib.kvq_probe_mfma_fp8(fake, fake, 6, 4, fake, None) == 1    # n % chain
    assert lib.kvq_probe_mfma_fp8(fake, fake, 4, 3, fake, None) == 1    # chain
    assert lib.kvq_probe_mfma_fp8(ctypes.c_void_p(0x10004), fake, 4, 4, fake, None) == 1   # alignment


def _codes(rng, n, narrow):
    """n tiles of 512 random E4M3 codes (no NaN); narrow: exponent fields
    5..8 only (products within a factor 2^8 of each other)."""
    c = rng.integers(0, 256, size=(n, 512), dtype=np.int64)
    c = np.where((c & 0x7F) == 0x7F, c ^ 0x01, c)
    if narrow:
        c = (c & 0x87) | ((rng.integers(0, 4, size=c.shape) + 5) << 3)
    return c.astype(np.uint8)


def _exact(a, b, chain):
    """Exact (fp64) chained products and sum |p| in the probe's layout."""
    def mat(t, transpose):   # tile bytes -> [16][32] (A) or [32][16] (B)
        v = OF.e4m3_decode(t.reshape(-1, 4, 16, 8))            # [n, k/8, row, k%8]
        m = v.transpose(0, 2, 1, 3).reshape(-1, 16, 32)         # [n, row, k]
        return m.transpose(0, 2, 1) if transpose else m
    A, Bm = mat(a, False), mat(b, True)
    n = a.shape[0]
    prod = A[:, :, :, None] * Bm[:, None, :, :]                  # [n, i, k, m]
    s = prod.sum(axis=2).reshape(n // chain, chain, 16, 16).sum(axis=1)
    sa = np.abs(prod).sum(axis=2).reshape(n // chain, chain, 16, 16).sum(axis=1)
    return s, sa


@pytest.mark.gpu
@pytest.mark.parametrize("chain", [1, 4])
def test_fp8_mfma_accumulation_bound(chain):
    import torch
    lib = _probe_lib()
    rng = np.random.default_rng(17 + chain)
    n = 1024
    for narrow in (False, True):
        a, b = _codes(rng, n, narrow), _codes(rng, n, narrow)
        da, db = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
        c = torch.empty(n // chain, 16, 16, dtype=torch.float32, device="cuda")
        rc = lib.kvq_probe_mfma_fp8(ctypes.c_void_p(da.data_ptr()), ctypes.c_void_p(db.data_ptr()), n, chain,
                                    ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == 0
        torch.cuda.synchronize()
        got = c.cpu().double().numpy()
        s, sa = _exact(a, b, chain)
        err = np.abs(got - s)
        worst = float((err / np.maximum(sa, 1e-300)).max())
        print(f"chain {chain} narrow={narrow}: max |err| / sum|p| = {worst:.3e}")
        assert np.all(err <= EPS_FP8_DOT * sa), f"chain {chain}: {worst:.3e} of sum |p| exceeds 2^-10"
        if narrow:   # products within 2^8 of each other: the sum is exact up to fp32 rounding
            assert np.all(err <= 2.0 ** -23 * np.abs(s) + 2.0 ** -40), f"chain {chain}: narrow-range sums inexact"
