"""CPU oracle for quantized-KV-cache attention decode (NVFP4 / FP8 E4M3).

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
reference that the HIP path is checked against.  Only the test suite, the
smoke check in ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The HIP library never links, imports or calls it,
and it shares no code, table or constant with the HIP library.

Everything here is NumPy in float64 (exact where the pages' formats allow it),
written from the format and method descriptions on these pages:

* Model-Optimizer PR #714 ("KV cache quantization for MLAAttention in vLLM
  fakequant"), Testing section: the NVFP4 quantizer dump
  ``(2, 1) bit fake block_sizes={-1: 16, 'type': 'dynamic',
  'scale_bits': (4, 3)}, amax=..., calibrator=MaxCalibrator`` on
  ``kv_c_bmm_quantizer`` of ``QuantMLAAttention``.
* compressed-tensors PR #436 / llm-compressor attention quantization,
  the ``kv_cache_scheme`` JSON (8-bit float, tensor strategy, symmetric,
  min-max observer, static).
* vLLM PR #15734 (FP8 FA output via an output scale; FP8 quantization of
  softmax(QK^T) inside the FA loop via a probability scale).
* Model-Optimizer PR #1832 ("Add quant+sparse attention for vLLM serving"),
  Testing section: the split-KV decode description (s contiguous chunks per
  (request, head), partial softmax with running max, denominator and
  weighted V; the per-split results are merged by a separate step).

Modules:
  formats    E2M1 / E4M3 / bf16 / fp32 encoders and decoders
  quant      amax calibration, NVFP4 and FP8 pack / unpack
  attention  exact softmax decode attention (GQA/MHA and MLA latent), split
             emulation, combine, FP8 probabilities, FP8 output
"""
