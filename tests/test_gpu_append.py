"""GPU parity for the decode step with the new token's append fused in: the
decode packs the token's K and V rows into row kv_lens[b] - 1 of the planes
itself (bytes identical to the pack kernels' with the same amax, checked over
the whole planes) and attends to it from its fresh codes (output within the
oracle's gates over the full cache).  The planes start with that row holding
other values (packed from -K, -V), so a step that skipped the write, wrote
the wrong row or read the stale row shows."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, K, announce, assert_bf16_output, gpu_pack, make_inputs, oracle_gqa, page_plane

pytestmark = pytest.mark.gpu


def _planes_equal(p, q):
    if isinstance(p, K().NVFP4Plane):
        return torch.equal(p.codes, q.codes) and torch.equal(p.scales, q.scales)
    return torch.equal(p.codes, q.codes)


def _clone(p):
    k_ = K()
    if isinstance(p, k_.NVFP4Plane):
        return k_.NVFP4Plane(p.codes.clone(), p.scales.clone(), p.tensor_scale.clone(), p.layout)
    return k_.FP8Plane(p.codes.clone(), p.scale.clone(), p.layout)


FP8_KEY = ("fp8", "custom", 3, 32, 8, 128, (200, 513, 64), "bf16")   # ragged, FP8 planes

CASES = [
    # (key, format, v_layout, splits, fused, paged block size or 0, per-head FP8 scales)
    (("nvfp4", "gqa", 1024), "nvfp4", 1, 3, False, 0, False),
    (("nvfp4", "gqa", 1024), "nvfp4", 1, 0, True, 0, False),
    (("nvfp4", "gqa", 1024), "nvfp4", 1, 4, True, 0, False),
    (("nvfp4", "gqa", 1024), "nvfp4", 1, 2, True, 64, False),
    (FP8_KEY, "fp8", 1, 2, False, 0, False),
    (FP8_KEY, "fp8", 1, 0, True, 0, True),
    (FP8_KEY, "fp8", 1, 1, True, 64, True),
    (("nvfp4", "mha", 1024, 2, 16), "nvfp4", 1, 2, False, 0, False),                        # G = 1
    (("nvfp4", "custom", 2, 16, 2, 128, (1, 130), "bf16"), "nvfp4", 1, 2, True, 0, False),  # G = 8, a 1-token request
    (("nvfp4", "custom", 2, 16, 2, 128, (1, 130), "bf16"), "nvfp4", 1, 1, False, 64, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0][0]}-{c[0][1]}-v{c[2]}-s{c[3]}-f{int(c[4])}-p{c[5]}-h{int(c[6])}")
def test_decode_with_fused_append(case):
    key, fmt, v_layout, s, fused, bs, per_head = case
    announce(f"fused append {case}")
    k_ = K()
    inp = make_inputs(key)
    B, Hq, Hkv, D = inp.B, inp.Hq, inp.Hkv, inp.D
    lens_np = inp.kv_lens.astype(np.int64)
    k, v = inp.k.to(DEV), inp.v.to(DEV)
    lens = torch.from_numpy(inp.kv_lens).to(DEV)
    Lp = (k.shape[2] + 3) // 4 * 4   # planes padded to whole 4-token groups
    kn, vn = k.clone(), v.clone()     # the stale row: -K, -V at the new token
    for b in range(B):
        kn[b, :, lens_np[b] - 1] *= -1
        vn[b, :, lens_np[b] - 1] *= -1
    if per_head:
        ka, va = k_.kvq_amax(k, lens, per_head=True), k_.kvq_amax(v, lens, per_head=True)

        def plane(x, amax, layout):
            p_ = k_.FP8Plane(torch.full((B, Hkv, Lp, D), 0xFF, dtype=torch.uint8, device=DEV),
                             torch.empty(Hkv, dtype=torch.float32, device=DEV), layout)
            k_.kvq_pack_fp8(x, amax, out=p_)
            return p_
        ref_k, ref_v = plane(k, ka, 0), plane(v, va, v_layout)
        st_k, st_v = plane(kn, ka, 0), plane(vn, va, v_layout)
    else:
        ref_k, ref_v, ka, va, _ = gpu_pack(inp, fmt, v_layout)
        st_k, st_v = _clone(ref_k), _clone(ref_v)
        pack = k_.kvq_pack_nvfp4 if fmt == "nvfp4" else k_.kvq_pack_fp8
        pack(kn, ka, out=st_k)
        pack(vn, va, out=st_v)
    torch.cuda.synchronize()
    assert not _planes_equal(st_k, ref_k) and not _planes_equal(st_v, ref_v)
    new_k = torch.stack([k[b, :, lens_np[b] - 1] for b in range(B)]).contiguous()
    new_v = torch.stack([v[b, :, lens_np[b] - 1] for b in range(B)]).contiguous()
    bt = None
    if bs:
        st_k, bt = page_plane(st_k, bs, 5, lens_np)
        st_v, _ = page_plane(st_v, bs, 5, lens_np)
        ref_k, _ = page_plane(ref_k, bs, 5, lens_np)
        ref_v, _ = page_plane(ref_v, bs, 5, lens_np)
    part_o = torch.empty(B * Hq * 64 * D, dtype=torch.float32, device=DEV)
    part_lse = torch.empty(B * Hq * 64, dtype=torch.float32, device=DEV)
    args = k_.make_decode_args(inp.q.to(DEV), st_k, st_v, lens, max_kv_len=inp.Lmax, softmax_scale=inp.softmax_scale,
                               num_splits=s, part_o=part_o, part_lse=part_lse, block_table=bt, new_k=new_k, new_v=new_v)
    out = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    if fused:
        counters = torch.zeros(B * Hkv, dtype=torch.int32, device=DEV)
        used = k_.attn_decode(args, out, counters=counters)
        torch.cuda.synchronize()
        assert int(counters.abs().sum().item()) == 0
    else:
        used = k_.attn_decode_splitkv(args)
        k_.attn_decode_combine(part_o, part_lse, B, Hq, D, used, out)
    torch.cuda.synchronize()
    if s > 0:
        assert used == s + 1
    assert _planes_equal(st_k, ref_k), "the appended K row must match the pack kernel's bytes"
    assert _planes_equal(st_v, ref_v), "the appended V row must match the pack kernel's bytes"
    if per_head:
        from oracle import attention as OA
        from oracle import quant as OQ
        import kvq_synth
        kf, vf = kvq_synth.f64(inp.k), kvq_synth.f64(inp.v)
        kc, ks = OQ.fp8_pack_heads(kf, OQ.amax_heads(kf, inp.kv_lens))
        vc, vs = OQ.fp8_pack_heads(vf, OQ.amax_heads(vf, inp.kv_lens))
        o_ref, _ = OA.decode_gqa(kvq_synth.f64(inp.q), OQ.fp8_unpack_heads(kc, ks), OQ.fp8_unpack_heads(vc, vs),
                                 inp.kv_lens, inp.softmax_scale)
    else:
        _, o_ref, _, _, _ = oracle_gqa(key)
    assert_bf16_output(out, o_ref, f"fused append {case}")
