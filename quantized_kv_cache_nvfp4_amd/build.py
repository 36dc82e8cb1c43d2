"""Build libkvq.so (the HIP kernels + C ABI) in-tree for gfx950.

Usage: ``python -m quantized_kv_cache_nvfp4_amd.build`` or ``build()``.
Every source is compiled with hipcc for gfx950 only; the shared library is
written next to this file, where the Python binding loads it.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libkvq.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "quant_kernels.hip", "decode_gqa.hip", "decode_gqa_nvfp4_d128.hip", "decode_gqa_nvfp4_d64.hip",
           "decode_gqa_fp8_d128.hip", "decode_gqa_fp8_d64.hip", "decode_mla.hip", "combine.hip",
           "prefill_gqa.hip"]
# measurement probes (the benchmark's streaming-read ceiling, the FP8 matrix
# core's accumulation error): their own small library, not part of the C ABI
PROBE_SOURCES = ["probe_read.hip", "probe_mfma8.hip"]
PROBE_LIB_PATH = os.path.join(HERE, "libkvq_probe.so")

ARCH = "gfx950"


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-I", os.path.join(ROOT, "include"),
        # packed fp32 VALU ops are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    ]


# per-source flags: the prefill kernel's softmax takes row maxima of MFMA
# results, which hold no NaN; without NaN semantics fmax needs no quieting
# of its operands (one VALU instruction per maximum instead of two)
FILE_FLAGS = {"prefill_gqa.hip": ["-fno-honor-nans"]}


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *_flags(), *FILE_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose=False) -> str:
    """Compile every HIP source for gfx950 and link libkvq.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB_PATH, verbose)
    _link(objs[len(SOURCES):], PROBE_LIB_PATH, verbose)
    return LIB_PATH


def _link(objs, path, verbose):
    tmp = path + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, path)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
