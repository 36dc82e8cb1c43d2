"""GPU parity for paged caches (block tables): the same packed bytes laid out
in randomly permuted blocks must decode to bit-identical outputs as the
contiguous planes (same chunking, same arithmetic), and within the output
gates of the oracle's attention over the logical cache.  Unused blocks hold
0xFF bytes (NaN E4M3 scales), so a read through a wrong table entry shows."""
import numpy as np
import pytest
import torch

from gpu_helpers import (DEV, K, announce, assert_bf16_output, gpu_decode, gpu_pack, make_inputs, oracle_gqa,
                         page_plane as _page)

pytestmark = pytest.mark.gpu


def _decode(inp, kp, vp, lens, s, block_table=None, fused=False, out_dtype=torch.bfloat16):
    k_ = K()
    B, Hq, D = inp.B, inp.Hq, inp.D
    part_o = torch.empty(B * Hq * 64 * D, dtype=torch.float32, device=DEV)
    part_lse = torch.empty(B * Hq * 64, dtype=torch.float32, device=DEV)
    args = k_.make_decode_args(inp.q.to(DEV), kp, vp, lens, max_kv_len=inp.Lmax, softmax_scale=inp.softmax_scale,
                               num_splits=s, part_o=part_o, part_lse=part_lse, block_table=block_table)
    out = torch.empty(B, Hq, D, dtype=out_dtype, device=DEV)
    if fused:
        counters = torch.zeros(B * inp.Hkv, dtype=torch.int32, device=DEV)
        k_.attn_decode(args, out, counters=counters)
    else:
        used = k_.attn_decode_splitkv(args)
        k_.attn_decode_combine(part_o, part_lse, B, Hq, D, used, out)
    torch.cuda.synchronize()
    return out


CASES = [
    # (key, v_layout, block_size, splits, fused)
    (("nvfp4", "gqa", 1024), 1, 64, 3, False),
    (("nvfp4", "gqa", 1024), 1, 256, 0, False),
    (("nvfp4", "gqa", 1024), 1, 128, 1, True),
    (("nvfp4", "gqa", 1024), 1, 64, 5, True),
    (("fp8", "fp8", 64), 1, 64, 1, False),
    (("nvfp4", "mha", 1024, 2, 16), 1, 256, 2, False),                        # G = 1: tile 256
    (("nvfp4", "custom", 2, 16, 2, 128, (300, 77), "bf16"), 1, 32, 4, False),  # G = 8: tile 32
    # one split over long requests: more than 64 tiles per wave, so the
    # register windows of tile rows are refilled from the LDS table
    (("nvfp4", "custom", 2, 8, 1, 128, (9000, 8300), "bf16"), 1, 32, 1, False),   # G = 8: 71 tiles per wave
    (("nvfp4", "custom", 1, 32, 8, 128, (20000,), "bf16"), 1, 64, 1, True),       # G = 4: 79 tiles per wave
    # the GQA 4:1 32K cache in the launch configuration bench.py times
    # (auto splits, TOKEN4 V, 64-token blocks), two launches and fused
    (("nvfp4", "gqa", 32768), 1, 64, 0, False),
    (("nvfp4", "gqa", 32768), 1, 64, 0, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0][0]}-{c[0][1]}-v{c[1]}-bs{c[2]}-s{c[3]}-f{int(c[4])}")
def test_paged_matches_contiguous(case):
    key, v_layout, bs, s, fused = case
    fmt = key[0]
    announce(f"paged {case}")
    inp = make_inputs(key)
    kp, vp, _, _, lens = gpu_pack(inp, fmt, v_layout)
    ref = _decode(inp, kp, vp, lens, s, fused=fused)
    kpp, bt = _page(kp, bs, 1, inp.kv_lens)
    vpp, bt2 = _page(vp, bs, 1, inp.kv_lens)
    assert torch.equal(bt, bt2)
    got = _decode(inp, kpp, vpp, lens, s, block_table=bt, fused=fused)
    assert torch.equal(got, ref), "paged and contiguous planes must decode to identical bits"
    _, o_ref, _, _, _ = oracle_gqa(key)
    assert_bf16_output(got, o_ref, f"paged {case}")


def test_paged_rejects_small_blocks():
    """The block size must be a multiple of the decode tile (64 tokens at G = 4)."""
    k_ = K()
    key = ("nvfp4", "gqa", 1024)
    inp = make_inputs(key)
    kp, vp, _, _, lens = gpu_pack(inp, "nvfp4", 1)
    assert k_.attn_decode_tile_tokens(32, 8) == 64
    kpp, bt = _page(kp, 32, 2)
    vpp, _ = _page(vp, 32, 2)
    with pytest.raises(k_.KvqError):
        _decode(inp, kpp, vpp, lens, 2, block_table=bt)


FP8P_CASES = [
    # (key, v_layout, block_size, splits, fused)
    (("nvfp4", "gqa", 1024), 1, 64, 3, False),
    (("nvfp4", "gqa", 1024), 1, 128, 0, True),
    (("fp8", "fp8", 64), 1, 64, 2, False),
    (("nvfp4", "custom", 2, 16, 2, 128, (300, 77), "bf16"), 1, 32, 4, False),   # G = 8: tile 32
    (("nvfp4", "custom", 2, 8, 1, 128, (9000, 8300), "bf16"), 1, 32, 1, False),   # windows refilled
]


@pytest.mark.parametrize("case", FP8P_CASES, ids=lambda c: f"{c[0][0]}-{c[0][1]}-v{c[1]}-bs{c[2]}-s{c[3]}-f{int(c[4])}")
def test_paged_fp8p_matches_contiguous(case):
    """FP8-quantized probabilities over paged planes: both passes address the
    blocks through the table, so output and lse are bit-identical to the
    contiguous planes' FP8-P decode (itself checked against the oracle)."""
    key, v_layout, bs, s, fused = case
    fmt = key[0]
    announce(f"paged fp8p {case}")
    inp = make_inputs(key)
    kp, vp, _, _, lens = gpu_pack(inp, fmt, v_layout)
    ps = float(np.float32(1.0 / 448.0))
    ref, used, ref_lse = gpu_decode(inp, kp, vp, lens, s, out_dtype=torch.float32, with_lse=True, fused=fused,
                                    prob_scale=ps)
    kpp, bt = _page(kp, bs, 4, inp.kv_lens)
    vpp, bt2 = _page(vp, bs, 4, inp.kv_lens)
    assert torch.equal(bt, bt2)
    got, used_p, lse = gpu_decode(inp, kpp, vpp, lens, s, out_dtype=torch.float32, with_lse=True, fused=fused,
                                  prob_scale=ps, block_table=bt)
    assert used_p == used
    assert torch.isfinite(got).all()
    assert torch.equal(got, ref) and torch.equal(lse, ref_lse), "paged FP8-P must match the contiguous planes"
