"""attn_decode_noalloc (the entry point that allocates nothing: its partials and
merge counters live in the library's static per-GPU scratch array) against
attn_decode with a caller-owned workspace: same kernels, so the outputs and
log-sum-exps are bit-identical.  Two calls in a row per layout, the second on
a smaller input; the limits are refused before anything is launched."""
import pytest
import torch

import kvq_synth

from gpu_helpers import DEV, K, announce, gpu_pack, make_inputs

pytestmark = pytest.mark.gpu


def _gqa_pair(key, s):
    k_ = K()
    inp = make_inputs(key)
    kp, vp, _, _, lens = gpu_pack(inp, "nvfp4")
    B, Hq, D = inp.B, inp.Hq, inp.D
    po, pl = k_.decode_workspace(B, Hq, D, 64, DEV)
    args = k_.make_decode_args(inp.q.to(DEV), kp, vp, lens, max_kv_len=inp.Lmax, softmax_scale=inp.softmax_scale,
                               num_splits=s, part_o=po, part_lse=pl)
    ref = torch.empty(B, Hq, D, dtype=torch.float32, device=DEV)
    ref_lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    counters = torch.zeros(B * inp.Hkv, dtype=torch.int32, device=DEV)
    used_ref = k_.attn_decode(args, ref, lse_out=ref_lse, counters=counters)
    # the same arguments without any workspace
    args_na = k_.make_decode_args(inp.q.to(DEV), kp, vp, lens, max_kv_len=inp.Lmax, softmax_scale=inp.softmax_scale,
                                  num_splits=s, part_o=None, part_lse=None)
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    used = k_.attn_decode_noalloc(args_na, out, lse_out=lse)
    torch.cuda.synchronize()
    return ref, ref_lse, used_ref, out, lse, used


@pytest.mark.parametrize("order", ["large_then_small", "twice"])
def test_noalloc_matches_attn_decode_gqa(order):
    keys = [(("nvfp4", "gqa", 8192), 0), (("nvfp4", "custom", 1, 8, 2, 128, (300,), "bf16"), 3)]
    if order == "twice":
        keys = [keys[0], keys[0]]
    for key, s in keys:
        announce(f"noalloc gqa {key} s={s}")
        ref, ref_lse, used_ref, out, lse, used = _gqa_pair(key, s)
        assert used == used_ref
        assert torch.equal(out, ref), f"{key}: no-alloc output differs from attn_decode"
        assert torch.equal(lse, ref_lse)


def _mla(B, lens, s, noalloc):
    k_ = K()
    inp = kvq_synth.mla(L=max(lens), B=B, kv_lens=list(lens), salt=2)
    c = inp.c.to(DEV)
    lens_d = torch.from_numpy(inp.kv_lens).to(DEV)
    plane = k_.kvq_pack_nvfp4(c, k_.kvq_amax(c.unsqueeze(1), lens_d))
    H, D = inp.q_c.shape[1], inp.q_c.shape[2]
    po, pl = (None, None) if noalloc else k_.decode_workspace(B, H, D, 64, DEV)
    args = k_.make_decode_args(inp.q_c.to(DEV), plane, None, lens_d, max_kv_len=int(inp.c.shape[1]),
                               softmax_scale=inp.softmax_scale, num_splits=s, part_o=po, part_lse=pl,
                               q_rope=inp.q_r.to(DEV), k_rope=inp.k_r.to(DEV))
    out = torch.empty(B, H, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, H, dtype=torch.float32, device=DEV)
    used = k_.attn_decode_noalloc(args, out, lse_out=lse) if noalloc else k_.attn_decode(args, out, lse_out=lse)
    torch.cuda.synchronize()
    return out, lse, used


def test_noalloc_matches_attn_decode_mla():
    for B, lens, s in ((4, (2048, 2000, 1500, 129), 0), (2, (300, 77), 3)):
        announce(f"noalloc mla B={B} lens={lens} s={s}")
        ref, ref_lse, u0 = _mla(B, lens, s, False)
        out, lse, u1 = _mla(B, lens, s, True)
        assert u0 == u1
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse)


def test_noalloc_limits():
    k_ = K()
    key = ("nvfp4", "gqa", 1024)
    inp = make_inputs(key)
    kp, vp, _, _, lens = gpu_pack(inp, "nvfp4")
    out = torch.empty(inp.B, inp.Hq, inp.D, dtype=torch.float32, device=DEV)
    args = k_.make_decode_args(inp.q.to(DEV), kp, vp, lens, max_kv_len=inp.Lmax, softmax_scale=inp.softmax_scale,
                               num_splits=2, part_o=None, part_lse=None, quantize_p=True,
                               p_scratch=torch.empty(4, device=DEV))
    with pytest.raises(k_.KvqError) as e:
        k_.attn_decode_noalloc(args, out)
    assert e.value.code == 2
    # partials beyond the scratch: B = 16, 256 query heads, 64 splits of 65 floats (68 MB)
    Hq, Dv, s = 256, 64, 64
    assert k_.kvq_decode_workspace_bytes(16, Hq, Dv, s) > k_._lib.KVQ_NOALLOC_SCRATCH_BYTES
    inp2 = kvq_synth.gqa_inputs(16, Hq, Hq // 4, Dv, 256, config="gqa", salt=4)
    kp2, vp2, _, _, lens2 = gpu_pack(inp2, "nvfp4")
    args2 = k_.make_decode_args(inp2.q.to(DEV), kp2, vp2, lens2, max_kv_len=inp2.Lmax,
                                softmax_scale=inp2.softmax_scale, num_splits=s, part_o=None, part_lse=None)
    out2 = torch.empty(16, Hq, Dv, dtype=torch.float32, device=DEV)
    with pytest.raises(k_.KvqError) as e:
        k_.attn_decode_noalloc(args2, out2)
    assert e.value.code == 4 and "scratch" in str(e.value)
