"""Seeded synthetic inputs for quantized-KV decode, shared by tests and bench.

This module holds no part of the method's arithmetic: it only draws Gaussian
tensors, plants outlier channels, picks ragged lengths and rounds the draws to
the storage dtype (bf16 via torch's own cast).  The oracle and the HIP path are
then fed the very same arrays.

Shapes follow the workloads on the pages: the GQA 4:1 / MHA split-KV
accuracy table of Model-Optimizer PR #1832 (batch 2, head_dim 128, 32 query
heads over 8 kv heads, or 16 / 16), the Llama-3.1-8B attention shape of the
llm-compressor KV-cache recipe (32 query heads, 8 kv heads, head_dim 128) and
the DeepSeek-V2 per-rank MLA shape of Model-Optimizer PR #714 (16 heads,
latent rank 512, rope width 64).  They stand in for the pages' evaluation
sets (GSM8K, aa-lcr, ultrachat calibration), which are not used.

Recipe (one ``SeedSequence(20261202 + config_id).spawn(6)`` per config, with
streams q, k, v, outliers_k, outliers_v, kv_lens):
  * values ~ N(0, 1) drawn in float32, then rounded to the storage dtype;
  * "outliers": per kv head, 4 distinct channels (drawn without replacement,
    separately for K and V, fixed over batch and tokens) are multiplied by 20
    in float32 before the rounding;
  * ragged lengths: kv_len_b ~ U{lo..hi} inclusive.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

BASE_SEED = 20261202

CONFIG_IDS = {"tiny": 1, "gqa": 2, "mha": 3, "fp8": 4, "mla": 5, "prefill": 6}


def _streams(config_id, salt=0):
    ss = np.random.SeedSequence([BASE_SEED + config_id, salt])
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(6)]


def _to_dtype(x32: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t if dtype == torch.float32 else t.to(dtype)


def _plant_outliers(x32, rng, n_ch=4, factor=20.0):
    """x32: [B, H, L, D] float32, modified in place: per head h, n_ch distinct
    channels scaled by factor."""
    H, D = x32.shape[1], x32.shape[-1]
    chans = np.stack([rng.choice(D, size=n_ch, replace=False) for _ in range(H)])
    for h in range(H):
        x32[:, h, :, chans[h]] *= np.float32(factor)
    return chans


@dataclass
class GQAInputs:
    """Decode inputs for the GQA / MHA layout (head-major cache)."""
    q: torch.Tensor            # [B, Hq, D]
    k: torch.Tensor            # [B, Hkv, Lmax, D]
    v: torch.Tensor            # [B, Hkv, Lmax, D]
    kv_lens: np.ndarray        # [B] int32
    softmax_scale: float
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def Hq(self):
        return self.q.shape[1]

    @property
    def Hkv(self):
        return self.k.shape[1]

    @property
    def D(self):
        return self.q.shape[2]

    @property
    def Lmax(self):
        return self.k.shape[2]


@dataclass
class MLAInputs:
    """Decode inputs for the MLA latent layout."""
    q_c: torch.Tensor          # [B, H, 512]
    q_r: torch.Tensor          # [B, H, 64]
    c: torch.Tensor            # [B, Lmax, 512]
    k_r: torch.Tensor          # [B, Lmax, 64]
    kv_lens: np.ndarray
    softmax_scale: float
    name: str = ""


def gqa_inputs(B, Hq, Hkv, D, L, *, dtype=torch.bfloat16, q_dtype=None, outliers=False,
               kv_lens=None, config="gqa", salt=0, Lmax=None) -> GQAInputs:
    """Gaussian GQA/MHA decode inputs.  ``L`` is the kv length of every
    request unless ``kv_lens`` is given; ``Lmax`` pads the cache."""
    rq, rk, rv, rok, rov, rl = _streams(CONFIG_IDS[config], salt)
    if kv_lens is None:
        kv_lens = np.full(B, L, dtype=np.int32)
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    Lmax = int(Lmax if Lmax is not None else max(int(kv_lens.max()), 1))
    q32 = rq.standard_normal((B, Hq, D), dtype=np.float32)
    k32 = rk.standard_normal((B, Hkv, Lmax, D), dtype=np.float32)
    v32 = rv.standard_normal((B, Hkv, Lmax, D), dtype=np.float32)
    meta = {}
    if outliers:
        meta["k_outlier_channels"] = _plant_outliers(k32, rok)
        meta["v_outlier_channels"] = _plant_outliers(v32, rov)
    q_dtype = dtype if q_dtype is None else q_dtype
    return GQAInputs(q=_to_dtype(q32, q_dtype), k=_to_dtype(k32, dtype), v=_to_dtype(v32, dtype),
                     kv_lens=kv_lens, softmax_scale=float(np.float32(1.0 / np.sqrt(D))),
                     name=f"{config}_B{B}_Hq{Hq}_Hkv{Hkv}_D{D}_L{Lmax}", meta=meta)


def tiny(salt=0) -> GQAInputs:
    """B=1, Hq=4, Hkv=1, D=64, kv_len=256, Q/K/V float32 N(0,1)."""
    return gqa_inputs(1, 4, 1, 64, 256, dtype=torch.float32, config="tiny", salt=salt)


def gqa(L, salt=0) -> GQAInputs:
    """B=2, Hq=32, Hkv=8, D=128, bf16, 4 outlier channels x20 per kv head."""
    return gqa_inputs(2, 32, 8, 128, L, outliers=True, config="gqa", salt=salt)


def mha(L, B=2, H=16, salt=0) -> GQAInputs:
    """MHA: Hq = Hkv = H, D=128, bf16."""
    return gqa_inputs(B, H, H, 128, L, config="mha", salt=salt)


def ragged_lens(B, lo, hi, salt=0, config="fp8"):
    rl = _streams(CONFIG_IDS[config], salt)[5]
    return rl.integers(lo, hi + 1, size=B).astype(np.int32)


def fp8_ragged(B=64, lo=512, hi=4096, salt=0) -> GQAInputs:
    """Llama-3-8B attention shape, ragged kv_len ~ U{lo..hi}, bf16 inputs."""
    lens = ragged_lens(B, lo, hi, salt)
    return gqa_inputs(B, 32, 8, 128, None, kv_lens=lens, config="fp8", salt=salt, Lmax=hi)


def mla(L=8192, B=32, H=16, Dc=512, Dr=64, salt=0, kv_lens=None) -> MLAInputs:
    """DeepSeek-V2 per-rank MLA: 16 heads, latent 512 (to be NVFP4), rope 64
    (bf16), softmax scale 1/sqrt(128 + 64)."""
    rq, rk, rv, _, _, _ = _streams(CONFIG_IDS["mla"], salt)
    if kv_lens is None:
        kv_lens = np.full(B, L, dtype=np.int32)
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    Lmax = max(int(kv_lens.max()), 1)
    q_c = rq.standard_normal((B, H, Dc), dtype=np.float32)
    q_r = rq.standard_normal((B, H, Dr), dtype=np.float32)
    c = rk.standard_normal((B, Lmax, Dc), dtype=np.float32)
    k_r = rv.standard_normal((B, Lmax, Dr), dtype=np.float32)
    bf = torch.bfloat16
    return MLAInputs(q_c=_to_dtype(q_c, bf), q_r=_to_dtype(q_r, bf), c=_to_dtype(c, bf),
                     k_r=_to_dtype(k_r, bf), kv_lens=kv_lens,
                     softmax_scale=float(np.float32(1.0 / np.sqrt(192.0))),
                     name=f"mla_B{B}_H{H}_L{Lmax}")


@dataclass
class PrefillInputs:
    """Chunked-prefill inputs: a chunk of Sq query tokens per request over a
    cache whose last Sq rows are the chunk's own keys and values."""
    q: torch.Tensor            # [B, Sq, Hq, D]
    k: torch.Tensor            # [B, Hkv, Lmax, D]
    v: torch.Tensor            # [B, Hkv, Lmax, D]
    kv_lens: np.ndarray        # [B] int32, cache length including the chunk
    softmax_scale: float
    name: str = ""

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def Sq(self):
        return self.q.shape[1]

    @property
    def Hq(self):
        return self.q.shape[2]

    @property
    def Hkv(self):
        return self.k.shape[1]

    @property
    def D(self):
        return self.q.shape[3]

    @property
    def Lmax(self):
        return self.k.shape[2]


def prefill_queries(B, Sq, Hq, D, salt=0, dtype=torch.bfloat16) -> torch.Tensor:
    """A chunk of Sq query tokens per request, N(0, 1) rounded to dtype
    (the prefill config's own stream)."""
    rq = _streams(CONFIG_IDS["prefill"], salt)[0]
    return _to_dtype(rq.standard_normal((B, Sq, Hq, D), dtype=np.float32), dtype)


def prefill(B, Hq, Hkv, D, kv_lens, Sq, *, salt=0, outliers=False, Lmax=None) -> PrefillInputs:
    """Gaussian chunked-prefill inputs (bf16): cache K/V drawn as
    gqa_inputs draws them (optionally with the 4 x20 outlier channels per kv
    head) from the prefill config's streams, queries [B, Sq, Hq, D]."""
    cache = gqa_inputs(B, Hq, Hkv, D, None, kv_lens=kv_lens, config="prefill", salt=salt, outliers=outliers,
                       Lmax=Lmax)
    q = prefill_queries(B, Sq, Hq, D, salt=salt + 1000)
    return PrefillInputs(q=q, k=cache.k, v=cache.v, kv_lens=cache.kv_lens, softmax_scale=cache.softmax_scale,
                         name=f"prefill_B{B}_Sq{Sq}_Hq{Hq}_Hkv{Hkv}_D{D}_L{cache.Lmax}")


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a float32 / bf16 CPU tensor."""
    return t.detach().to("cpu", torch.float64).numpy()
