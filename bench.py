"""Benchmark: NVFP4-KV split-KV decode step on one MI355X.

Default workload: GQA 4:1 decode, B=2, Hq=32, Hkv=8, head_dim=128,
kv_len=32768 (the split-KV accuracy table shape of Model-Optimizer PR #1832),
K/V ~ N(0,1) with 4 outlier channels x20 per kv head, bf16, packed to NVFP4;
bf16 output; softmax scale 1/sqrt(128).

One step = one layer's decode over the packed cache: split-KV decode over
the whole cache and the combine of the partials, either fused (attn_decode:
the last work-group of each (request, kv head) merges the partials) or in two
launches (attn_decode_splitkv + attn_decode_combine); both are timed and
`value` is the faster.  Beside it: the quantize-on-append of the new token
(its own launch, and folded into the decode launch), the same decode over
64-token paged copies of the cache, and the split kernel alone (the roofline
entry).  Calibration (kvq_amax) and the bulk packing run before the timed
region and are timed on their own.

Timing: the 256 MB Infinity Cache would hold one 75.5 MB cache, so every step
reads a different copy from a rotation of >= 1 GiB of identical caches (as
successive layers would).  `--warmup W` eager steps run first; then each
variant is captured as a HIP graph of exactly `--steps K` steps and replayed
once untimed and once timed.  The timed replay is bracketed by device
synchronizations; HIP events recorded on the replay stream around it give
the time of exactly K steps (a short device-side spin is queued before the
first event so that the host's submission of the graph is not timed).

Other modes: --workload mha | mla | fp8 (the other configurations), --sweep
(decode step over s in {1,2,4,8,16,32,auto} x kv {1K,8K,32K}, GQA 4:1 and
MHA, in the layout of the pages' split-KV latency table), --read-probe (a
plain 16-byte-load streaming read of the GQA cache's size: the practical read
ceiling), --copy-probe (a device copy of known size, to scale the HBM
traffic counters).

Prints one JSON line.  ``--gpus N`` with N > 1 exits: this build runs on one
GPU.
"""
import argparse
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/decode step + achieved HBM GB/s, NVFP4-KV split-KV decode B=2 GQA4:1 32K"
HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0                     # MI355X dense f16 / bf16 matrix peak (no sparsity)
B, HQ, HKV, D, L = 2, 32, 8, 128, 32768
BYTES_PER_TOKEN_HEAD = 2 * (D // 2 + D // 16)   # K and V: codes + E4M3 scales = 144 B
SPIN_CYCLES = 4_000_000                          # device spin before a timed replay (~1-2 ms)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="steps per timed graph (exactly)")
    ap.add_argument("--warmup", type=int, default=10, help="untimed eager steps before capture")
    ap.add_argument("--splits", type=int, default=0, help="<= 0: auto")
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--workload", choices=["gqa32k", "mha", "mla", "fp8", "prefill"], default="gqa32k",
                    help="gqa32k: the metric's configuration (default); mha: B=2, Hq=Hkv=16, D=128, kv 32768 "
                         "(plus the split-starved B=1, H=32 case); mla: DeepSeek-V2 per-rank MLA, B=32, 16 heads, "
                         "NVFP4 latent 512 + bf16 rope 64, kv 8192; fp8: per-tensor FP8 KV, B=64, Hq=32, Hkv=8, "
                         "D=128, ragged kv_len ~ U{512..4096}, with and without FP8 probabilities; prefill: "
                         "chunked prefill of a 1024-token chunk per request over the GQA 4:1 B=2 32K cache "
                         "(MFMA-bound)")
    ap.add_argument("--sweep", action="store_true",
                    help="decode step over split counts x kv lengths for GQA 4:1 and MHA (table + JSON)")
    ap.add_argument("--read-probe", action="store_true",
                    help="streaming-read ceiling: a plain 16-byte-load read of the GQA cache's size")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device copy of the cache's size (counter calibration under rocprofv3)")
    ap.add_argument("--source-hash", choices=["gqa", "mla", "fp8"],
                    help="print the hash of a decode kernel's sources (the key of its committed traffic counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ traffic
CSRC = os.path.join(ROOT, "quantized_kv_cache_nvfp4_amd", "csrc")
TRAFFIC = {   # committed counter summaries and the kernel sources they were taken from (launch + instantiation)
    "gqa": (os.path.join(ROOT, "profiles", "k_decode_gqa_nvfp4_b2_hq32_hkv8_d128_kv32k_traffic.txt"),
            (os.path.join(CSRC, "decode_gqa.hip"), os.path.join(CSRC, "decode_gqa_nvfp4_d128.hip"))),
    "mla": (os.path.join(ROOT, "profiles", "k_decode_mla_nvfp4_b32_h16_c512_r64_kv8k_traffic.txt"),
            (os.path.join(CSRC, "decode_mla.hip"),)),
    "fp8": (os.path.join(ROOT, "profiles", "k_decode_gqa_fp8_b64_hq32_hkv8_d128_ragged_traffic.txt"),
            (os.path.join(CSRC, "decode_gqa.hip"), os.path.join(CSRC, "decode_gqa_fp8_d128.hip"))),
}


def source_closure(paths):
    """The kernel sources and every file they include with #include "..."
    (recursively), sorted: what the compiled kernel depends on here."""
    seen, todo = set(), [os.path.abspath(p) for p in paths]
    while todo:
        p = todo.pop()
        if p in seen or not os.path.exists(p):
            continue
        seen.add(p)
        for inc in re.findall(r'^\s*#\s*include\s+"([^"]+)"', open(p).read(), flags=re.M):
            todo.append(os.path.abspath(os.path.join(os.path.dirname(p), inc)))
    return sorted(seen)


def source_hash(which):
    import hashlib
    h = hashlib.sha256()
    for p in source_closure(TRAFFIC[which][1]):
        h.update(os.path.relpath(p, ROOT).encode() + b"\0" + open(p, "rb").read() + b"\0")
    return h.hexdigest()


def measured_traffic(which="gqa"):
    """HBM bytes per launch of the split kernel from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE scaled by a plain copy of known size),
    or None when the kernel source or a header it includes changed since the
    counters were taken."""
    path = TRAFFIC[which][0]
    try:
        kv = dict(line.split(":", 1) for line in open(path).read().splitlines() if ":" in line)
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel_sources_sha256") != source_hash(which):
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ timing
class Timer:
    """Graphs of exactly `steps` steps over `n_copies` rotating cache copies
    (step i reads copy i mod n_copies), timed with HIP events on the replay
    stream."""

    def __init__(self, torch, n_copies, steps):
        self.torch, self.n_copies, self.steps = torch, n_copies, steps

    def capture(self, fn):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            fn(0)   # eager once on the capture stream
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(self.steps):
                fn(i % self.n_copies)
        torch.cuda.synchronize()
        return g

    def _spin(self):
        try:
            self.torch.cuda._sleep(SPIN_CYCLES)
        except Exception:   # no device spin available: the submission is then inside the timed span
            pass

    def time(self, g):
        """ms per step: one untimed replay, then one timed replay of the
        graph's `steps` steps."""
        torch = self.torch
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        self._spin()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / self.steps

    def run(self, fn):
        return self.time(self.capture(fn))


def n_rotation(args, per_copy):
    return max(2, math.ceil(args.rotate_gib * (1 << 30) / per_copy))


# ------------------------------------------------------------------ CPU oracle
def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([1] + [int(p.get("num_threads", 1)) for p in threadpool_info()])
    except Exception:
        return 1


def _cores():
    return len(os.sched_getaffinity(0))


def _cpu_entry(t_s, sample):
    return {"value": t_s * 1e6, "unit": "us/step", "cores": _cores(), "blas_threads": _blas_threads(),
            "kind": "oracle", "sample": sample}


def cpu_baseline_gqa(inp, reps, heads=None):
    """The oracle, untouched, timed on this host: per decode step it
    dequantizes the packed cache and runs exact fp64 attention.  Sample:
    `reps` steps over `heads` kv heads of every request (all when None),
    scaled to the whole cache by the kv-head count; the oracle's one-off
    packing is not timed."""
    import numpy as np
    import kvq_synth
    from oracle import attention as OA
    from oracle import quant as OQ
    Hkv = inp.Hkv
    h = Hkv if heads is None else min(heads, Hkv)
    G = inp.Hq // Hkv
    log(f"oracle: packing {h} of {Hkv} kv heads once (untimed)")
    kf, vf = kvq_synth.f64(inp.k[:, :h]), kvq_synth.f64(inp.v[:, :h])
    ka, va = OQ.amax(kf), OQ.amax(vf)
    kc, ks, kst = OQ.nvfp4_pack(kf, ka)
    vc, vs, vst = OQ.nvfp4_pack(vf, va)
    q = kvq_synth.f64(inp.q[:, :h * G])
    times = []
    for r in range(reps):
        log(f"oracle step {r + 1}/{reps}")
        t0 = time.perf_counter()
        khat, vhat = OQ.nvfp4_unpack(kc, ks, kst), OQ.nvfp4_unpack(vc, vs, vst)
        OA.decode_gqa(q, khat, vhat, inp.kv_lens, inp.softmax_scale)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times)) * Hkv / h
    return _cpu_entry(t, f"{reps} decode steps over {h} of {Hkv} kv heads (B={inp.B}, {inp.Lmax} tokens): fp64 "
                         f"dequantize + exact attention, median scaled by {Hkv}/{h}; numpy elementwise "
                         f"single-threaded, BLAS threads {_blas_threads()}")


def cpu_baseline_mla(inp, reps, n_req=4):
    """The oracle timed on this host for the MLA step, on a bounded sample:
    `n_req` of the B requests (fp64 dequantize of their latent + exact MLA
    attention), scaled to the whole batch by the request count."""
    import numpy as np
    import kvq_synth
    from oracle import attention as OA
    from oracle import quant as OQ
    Bm = inp.q_c.shape[0]
    cf = kvq_synth.f64(inp.c[:n_req])
    amax = OQ.amax(cf[:, None], inp.kv_lens[:n_req])   # the sample's own scale (timing only; untimed)
    codes, scales, st = OQ.nvfp4_pack(cf, amax)
    q_c, q_r, k_r = (kvq_synth.f64(t[:n_req]) for t in (inp.q_c, inp.q_r, inp.k_r))
    times = []
    for r in range(reps):
        t0 = time.perf_counter()
        chat = OQ.nvfp4_unpack(codes, scales, st)
        OA.decode_mla(q_c, q_r, chat, k_r, inp.kv_lens[:n_req], inp.softmax_scale)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times)) * Bm / n_req
    return _cpu_entry(t, f"{n_req} of {Bm} requests x {reps} reps (fp64 dequantize of their latent + exact MLA "
                         f"attention), median scaled by {Bm}/{n_req}")


def cpu_baseline_fp8(inp, reps, n_req=3, prob_scale=None):
    """The oracle timed on this host for the FP8 ragged step, on a bounded
    sample: the first `n_req` requests (fp64 dequantize of their K/V + exact
    attention, or FP8-P attention), scaled to the batch by token count."""
    import numpy as np
    import kvq_synth
    from oracle import attention as OA
    from oracle import quant as OQ
    lens = inp.kv_lens
    kf, vf = kvq_synth.f64(inp.k[:n_req]), kvq_synth.f64(inp.v[:n_req])
    ka, va = OQ.amax(kf, lens[:n_req]), OQ.amax(vf, lens[:n_req])   # the sample's own scales (timing only; untimed)
    kc, ks = OQ.fp8_pack(kf, ka)
    vc, vs = OQ.fp8_pack(vf, va)
    q = kvq_synth.f64(inp.q[:n_req])
    times = []
    for r in range(reps):
        t0 = time.perf_counter()
        khat, vhat = OQ.fp8_unpack(kc, ks), OQ.fp8_unpack(vc, vs)
        if prob_scale is None:
            OA.decode_gqa(q, khat, vhat, lens[:n_req], inp.softmax_scale)
        else:
            OA.decode_gqa_fp8p(q, khat, vhat, lens[:n_req], inp.softmax_scale, prob_scale)
        times.append(time.perf_counter() - t0)
    scale = float(lens.sum()) / float(lens[:n_req].sum())
    t = float(np.median(times)) * scale
    return _cpu_entry(t, f"first {n_req} of {len(lens)} requests x {reps} reps (fp64 dequantize + exact attention"
                         f"{'' if prob_scale is None else ' with FP8 probabilities'}), median scaled by the token "
                         f"count ratio {scale:.2f}")


def eager_timer(torch, fn, reps=5):
    """Average time of fn() over `reps` back-to-back calls (HIP events on the
    current stream, after one warm-up call), in microseconds."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def base_record(metric, value_us, steps, warmup, dtype, config):
    return {"metric": metric, "value": round(value_us, 3), "unit": "us/step", "n_gpus": 1, "steps": steps,
            "warmup": warmup, "ms_per_step": round(value_us * 1e-3, 6), "higher_is_better": False,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": config}


def roofline(algo_bytes, kernel_us, kernel, traffic):
    achieved = algo_bytes / (kernel_us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": kernel,
            "kernel_us_mean": round(kernel_us, 3), "algorithmic_bytes": algo_bytes}


# ------------------------------------------------------------------ probes
def copy_probe():
    """A plain device-to-device copy of the cache's size (75,497,472 B read
    and written per launch), 20 launches: the reference for scaling the
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = B * HKV * L * BYTES_PER_TOKEN_HEAD
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(20):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 20}), flush=True)


def read_probe(args):
    """Streaming-read ceiling: kvq_probe_read (16-byte loads, 8 in flight
    per thread, nothing written) over a rotation of >= 1 GiB of buffers of the
    GQA cache's size (75,497,472 B), one buffer per launch, K launches per
    graph, for several launch shapes; reports the best as the practical read
    ceiling of the decode kernel's traffic."""
    import ctypes
    import torch
    from quantized_kv_cache_nvfp4_amd import build as kbuild
    if not os.path.exists(kbuild.PROBE_LIB_PATH):
        raise RuntimeError(f"{kbuild.PROBE_LIB_PATH} missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(kbuild.PROBE_LIB_PATH)
    for name in ("kvq_probe_read", "kvq_probe_read_nt"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p]
    for name in ("kvq_probe_read_chunks", "kvq_probe_read_chunks_nt"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n = B * HKV * L * BYTES_PER_TOKEN_HEAD
    n_copies = n_rotation(args, n)
    bufs = [torch.randint(0, 255, (n,), dtype=torch.uint8, device=dev) for _ in range(n_copies)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    tm = Timer(torch, n_copies, args.steps)
    # plain loads and loads with the non-temporal hint (the hint the NVFP4
    # decode planes are read with)
    res, chunks = {"": {}, "_nt": {}}, {"": {}, "_nt": {}}
    for sfx in ("", "_nt"):
        fread = getattr(lib, "kvq_probe_read" + sfx)
        for grid in (256, 512, 1024, 2048, 4096, 8192):
            def fn(i, grid=grid, fread=fread):
                rc = fread(ctypes.c_void_p(bufs[i].data_ptr()), n, grid, ctypes.c_void_p(sink.data_ptr()),
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
                if rc != 0:
                    raise RuntimeError(f"kvq_probe_read{sfx} failed ({rc})")
            us = tm.run(fn) * 1e3
            res[sfx][grid] = us
            log(f"read probe{sfx} grid {grid}: {us:.3f} us/launch, {n / us / 1e3:.1f} GB/s")
        # the decode kernels' launch shape: one 256-thread work-group per CU,
        # each reading one contiguous chunk (as the split-KV work-groups do),
        # with the chunk streamed as 1, 2 or 4 side-by-side parts
        fchunk = getattr(lib, "kvq_probe_read_chunks" + sfx)
        for grid, fronts in ((256, 1), (256, 2), (256, 4), (512, 1)):
            def fc(i, grid=grid, fronts=fronts, fchunk=fchunk):
                rc = fchunk(ctypes.c_void_p(bufs[i].data_ptr()), n, grid, fronts, ctypes.c_void_p(sink.data_ptr()),
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
                if rc != 0:
                    raise RuntimeError(f"kvq_probe_read_chunks{sfx} failed ({rc})")
            cu = tm.run(fc) * 1e3
            chunks[sfx][f"grid{grid}_fronts{fronts}"] = round(cu, 3)
            log(f"chunked read{sfx} grid {grid} fronts {fronts}: {cu:.3f} us/launch, {n / cu / 1e3:.1f} GB/s")
    # the ceiling: the fastest plain read over both load policies and every grid
    best_sfx, best = min(((sfx, g) for sfx in res for g in res[sfx]), key=lambda k: res[k[0]][k[1]])
    us = res[best_sfx][best]
    out = {"metric": "streaming-read ceiling (plain 16-byte-load read, graph of back-to-back launches)",
           "value": round(us, 3), "unit": "us/launch", "bytes_per_launch": n, "steps": args.steps,
           "GB/s": round(n / us / 1e3, 1), "frac_of_8TBs": round(n / us / 1e3 / HBM_PEAK_GBPS, 4),
           "best_grid": best, "best_loads": "non-temporal" if best_sfx else "plain", "threads": 256,
           "per_grid_us": {str(k): round(v, 3) for k, v in res[""].items()},
           "per_grid_us_nt": {str(k): round(v, 3) for k, v in res["_nt"].items()},
           "chunked_us": chunks[""], "chunked_us_nt": chunks["_nt"], "rotation_copies": n_copies}
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------ GQA / MHA
def _setup_gqa(K, torch, inp, dev, v_layout=None):
    """Calibrate and pack K / V of a GQA-layout input on the device; returns
    (q, kv_lens, k_amax, v_amax, K plane, V plane, k, v)."""
    v_layout = K.KVQ_PLANE_TOKEN4 if v_layout is None else v_layout
    kv_lens = torch.from_numpy(inp.kv_lens).to(dev)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    k_amax, v_amax = K.kvq_amax(k, kv_lens), K.kvq_amax(v, kv_lens)
    kp = K.kvq_pack_nvfp4(k, k_amax)
    vp = K.kvq_pack_nvfp4(v, v_amax, layout=v_layout)
    return q, kv_lens, k_amax, v_amax, kp, vp, k, v


def _rotation(K, kp0, vp0, n_copies):
    copies = [(kp0, vp0)]
    for _ in range(n_copies - 1):
        copies.append((K.NVFP4Plane(kp0.codes.clone(), kp0.scales.clone(), kp0.tensor_scale.clone(), kp0.layout),
                       K.NVFP4Plane(vp0.codes.clone(), vp0.scales.clone(), vp0.tensor_scale.clone(), vp0.layout)))
    return copies


class GQADecode:
    """Two-launch and fused decode steps over rotating cache copies."""

    def __init__(self, K, torch, inp, q, kv_lens, copies, s, dev, cap_extra=1):
        self.K, self.torch, self.inp, self.copies = K, torch, inp, copies
        Bq, Hq, Dq = inp.B, inp.Hq, inp.D
        self.part_o, self.part_lse = K.decode_workspace(Bq, Hq, Dq, s + cap_extra, dev)
        self.out = torch.empty(Bq, Hq, Dq, dtype=torch.bfloat16, device=dev)
        self.counters = torch.zeros(Bq * inp.Hkv, dtype=torch.int32, device=dev)
        self.q, self.kv_lens, self.s = q, kv_lens, s
        self.args = [self.mk(kc, vc) for kc, vc in copies]

    def mk(self, kc, vc, **kw):
        inp = self.inp
        return self.K.make_decode_args(self.q, kc, vc, self.kv_lens, max_kv_len=inp.Lmax,
                                       softmax_scale=inp.softmax_scale, num_splits=self.s, part_o=self.part_o,
                                       part_lse=self.part_lse, **kw)

    def two_launch(self, a):
        K, inp = self.K, self.inp
        used = K.attn_decode_splitkv(a)
        K.attn_decode_combine(self.part_o, self.part_lse, inp.B, inp.Hq, inp.D, used, self.out)

    def fused(self, a):
        self.K.attn_decode(a, self.out, counters=self.counters)

    def split(self, a):
        self.K.attn_decode_splitkv(a)


def run_gqa(args):
    import torch
    import kvq_synth
    import quantized_kv_cache_nvfp4_amd as K

    K._lib.lib()  # fails loudly if libkvq.so is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating inputs")
    inp = kvq_synth.gqa(L)
    q, kv_lens, k_amax, v_amax, kp0, vp0, k, v = _setup_gqa(K, torch, inp, dev)
    # calibration + bulk pack (outside the decode step; timed on their own)
    kp_t = K.kvq_pack_nvfp4(k, k_amax)
    vp_t = K.kvq_pack_nvfp4(v, v_amax, layout=K.KVQ_PLANE_TOKEN4)
    elems = k.numel()
    prep_us = {"amax_k": eager_timer(torch, lambda: K.kvq_amax(k, kv_lens, out=k_amax)),
               "pack_k_nvfp4_rows": eager_timer(torch, lambda: K.kvq_pack_nvfp4(k, k_amax, out=kp_t)),
               "pack_v_nvfp4_token4": eager_timer(torch, lambda: K.kvq_pack_nvfp4(v, v_amax, out=vp_t))}
    prep_bytes = {"amax_k": elems * 2, "pack_k_nvfp4_rows": elems * 2 + elems * 9 // 16,
                  "pack_v_nvfp4_token4": elems * 2 + elems * 9 // 16}
    del kp_t, vp_t
    new_k = k[:, :, L - 1:L, :].contiguous()
    new_v = v[:, :, L - 1:L, :].contiguous()
    del k, v
    pos = torch.full((B,), L - 1, dtype=torch.int32, device=dev)

    per_copy = sum(t.numel() for t in (kp0.codes, kp0.scales, vp0.codes, vp0.scales))
    assert per_copy == B * HKV * L * BYTES_PER_TOKEN_HEAD
    n_copies = n_rotation(args, per_copy)
    log(f"rotation: {n_copies} cache copies x {per_copy / 1e6:.1f} MB")
    copies = _rotation(K, kp0, vp0, n_copies)
    cus = K.kvq_device_cu_count()
    s = args.splits if args.splits > 0 else K.kvq_auto_num_splits(cus, B, HKV, L, D, HQ)
    dec = GQADecode(K, torch, inp, q, kv_lens, copies, s, dev)

    def append(i):   # quantize-on-append of the new K and V rows: one launch
        kc, vc = copies[i]
        K.kvq_pack_batch([(new_k, k_amax, kc, pos), (new_v, v_amax, vc, pos)])

    # the decode step with the new token's append fused in (the decode packs
    # row L - 1 itself and attends to it from its fresh codes)
    new_k3, new_v3 = new_k.view(B, HKV, D), new_v.view(B, HKV, D)
    aargs = [dec.mk(kc, vc, new_k=new_k3, new_v=new_v3) for kc, vc in copies]

    # the same caches paged: blocks of 64 tokens at permuted physical blocks
    # (one table per copy), decoded through the block table
    PB = 64
    nb = L // PB
    rng = torch.Generator().manual_seed(3)

    def to_paged(plane, perm):
        def pg(t):
            blocks = t.view(B, HKV, nb, PB, t.shape[-1]).permute(0, 2, 1, 3, 4).reshape(B * nb, HKV, PB, t.shape[-1])
            out_ = torch.empty_like(blocks)
            out_[perm] = blocks
            return out_
        return K.NVFP4Plane(pg(plane.codes), pg(plane.scales), plane.tensor_scale, plane.layout)

    pdargs, keep = [], []
    for kc, vc in copies:
        perm = torch.randperm(B * nb, generator=rng).to(dev)
        bt = perm.view(B, nb).to(torch.int32).contiguous()
        pk, pv = to_paged(kc, perm), to_paged(vc, perm)
        pdargs.append(dec.mk(pk, pv, block_table=bt))
        keep.append((pk, pv, bt))
    torch.cuda.synchronize()

    log(f"warm-up: {args.warmup} steps")
    for i in range(args.warmup):
        dec.two_launch(dec.args[i % n_copies])
        dec.fused(dec.args[i % n_copies])
    torch.cuda.synchronize()
    tm = Timer(torch, n_copies, args.steps)
    variants = {
        "decode_two_launch": lambda i: dec.two_launch(dec.args[i]),
        "decode_fused": lambda i: dec.fused(dec.args[i]),
        "split_kernel": lambda i: dec.split(dec.args[i]),
        "append": append,
        "fused": lambda i: (append(i), dec.fused(dec.args[i])),
        "two_launch": lambda i: (append(i), dec.two_launch(dec.args[i])),
        "fused_append_in_decode": lambda i: dec.fused(aargs[i]),
        "two_launch_append_in_split": lambda i: dec.two_launch(aargs[i]),
        "decode_fused_paged64": lambda i: dec.fused(pdargs[i]),
        "split_kernel_paged64": lambda i: dec.split(pdargs[i]),
    }
    log(f"timing {args.steps} steps per variant (graphs of exactly {args.steps} steps)")
    ms = {}
    for name, fn in variants.items():
        ms[name] = tm.run(fn)
        log(f"  {name}: {ms[name] * 1e3:.3f} us/step")
    best = "decode_fused" if ms["decode_fused"] <= ms["decode_two_launch"] else "decode_two_launch"
    assert torch.isfinite(dec.out.float()).all()
    algo_bytes = B * HKV * L * BYTES_PER_TOKEN_HEAD
    step_us = ms[best] * 1e3
    res = base_record(METRIC, step_us, args.steps, args.warmup, "f16 MFMA, fp32 accumulate (NVFP4 KV)",
                      {"workload": "NVFP4-KV split-KV decode, GQA 4:1", "B": B, "Hq": HQ, "Hkv": HKV,
                       "head_dim": D, "kv_len": L, "splits": s, "out_dtype": "bf16", "v_layout": "token4",
                       "rotation_copies": n_copies, "step_path": best})
    res["hbm_gbps_step"] = round(algo_bytes / (step_us * 1e-6) / 1e9, 1)
    res["step_us"] = {k_: round(v_ * 1e3, 3) for k_, v_ in ms.items()}
    res["calibrate_pack"] = {k_: {"us": round(t, 2), "GB/s": round(prep_bytes[k_] / (t * 1e-6) / 1e9, 1)}
                             for k_, t in prep_us.items()}
    res["roofline"] = roofline(algo_bytes, ms["split_kernel"] * 1e3,
                               "k_decode_gqa<NVFP4,G=4,D=128> (split kernel, partials)", measured_traffic("gqa"))
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline_gqa(inp, args.cpu_reps)
    print(json.dumps(res), flush=True)


def _mha_case(args, K, torch, dev, Bm, H, Lm, splits):
    """Decode of the MHA configuration (Hq = Hkv = H): returns (dict of ms per
    step, s, n_copies, algorithmic bytes, inputs)."""
    import kvq_synth
    inp = kvq_synth.mha(Lm, B=Bm, H=H)
    q, kv_lens, _, _, kp0, vp0, k, v = _setup_gqa(K, torch, inp, dev)
    del k, v
    per_copy = sum(t.numel() for t in (kp0.codes, kp0.scales, vp0.codes, vp0.scales))
    n_copies = n_rotation(args, per_copy)
    copies = _rotation(K, kp0, vp0, n_copies)
    s = splits if splits > 0 else K.kvq_auto_num_splits(K.kvq_device_cu_count(), Bm, H, Lm, 128, H)
    dec = GQADecode(K, torch, inp, q, kv_lens, copies, s, dev)
    for i in range(args.warmup):
        dec.two_launch(dec.args[i % n_copies])
        dec.fused(dec.args[i % n_copies])
    torch.cuda.synchronize()
    tm = Timer(torch, n_copies, args.steps)
    ms = {"decode_two_launch": tm.run(lambda i: dec.two_launch(dec.args[i])),
          "decode_fused": tm.run(lambda i: dec.fused(dec.args[i])),
          "split_kernel": tm.run(lambda i: dec.split(dec.args[i]))}
    assert torch.isfinite(dec.out.float()).all()
    return ms, s, n_copies, per_copy, inp


def run_mha(args):
    """MHA decode, B=2, Hq=Hkv=16, D=128, kv 32768 (the metric's line), plus
    the split-starved B=1, Hq=Hkv=32 case at the same length."""
    import torch
    import quantized_kv_cache_nvfp4_amd as K
    K._lib.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("MHA B=2 H=16 kv 32768")
    ms, s, nc, algo, inp = _mha_case(args, K, torch, dev, 2, 16, 32768, args.splits)
    log("MHA B=1 H=32 kv 32768 (split-starved)")
    ms1, s1, _, algo1, _ = _mha_case(args, K, torch, dev, 1, 32, 32768, args.splits)
    best = "decode_fused" if ms["decode_fused"] <= ms["decode_two_launch"] else "decode_two_launch"
    step_us = ms[best] * 1e3
    res = base_record("us/decode step + achieved HBM GB/s, NVFP4-KV split-KV decode B=2 MHA H=16 32K", step_us,
                      args.steps, args.warmup, "f16 MFMA, fp32 accumulate (NVFP4 KV)",
                      {"workload": "NVFP4-KV split-KV decode, MHA", "B": 2, "Hq": 16, "Hkv": 16, "head_dim": 128,
                       "kv_len": 32768, "splits": s, "out_dtype": "bf16", "v_layout": "token4",
                       "rotation_copies": nc, "step_path": best})
    res["hbm_gbps_step"] = round(algo / (step_us * 1e-6) / 1e9, 1)
    res["step_us"] = {k_: round(v_ * 1e3, 3) for k_, v_ in ms.items()}
    best1 = min(ms1, key=lambda k_: ms1[k_] if k_ != "split_kernel" else 1e9)
    res["split_starved_b1_h32"] = {
        "splits": s1, "step_us": {k_: round(v_ * 1e3, 3) for k_, v_ in ms1.items()},
        "step_path": best1, "hbm_gbps_step": round(algo1 / (ms1[best1] * 1e-3) / 1e9, 1),
        "roofline_split_kernel": roofline(algo1, ms1["split_kernel"] * 1e3, "k_decode_gqa<NVFP4,G=1,D=128>", None)}
    res["roofline"] = roofline(algo, ms["split_kernel"] * 1e3, "k_decode_gqa<NVFP4,G=1,D=128> (split kernel, partials)",
                               None)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        res["cpu_baseline"] = cpu_baseline_gqa(inp, args.cpu_reps, heads=2)
    print(json.dumps(res), flush=True)


def run_sweep(args):
    """Decode step (split + combine, two launches) over s in {1, 2, 4, 8, 16,
    32, auto} and kv in {1K, 8K, 32K} for GQA 4:1 (B=2, Hq=32, Hkv=8) and MHA
    (B=2, Hq=Hkv=16): the layout of the pages' split-KV latency table
    (Model-Optimizer PR #1832, Testing).  Prints a markdown table to stderr
    and one JSON line."""
    import torch
    import kvq_synth
    import quantized_kv_cache_nvfp4_amd as K
    K._lib.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cus = K.kvq_device_cu_count()
    split_set = [1, 2, 4, 8, 16, 32]
    table = {}
    for name in ("gqa", "mha"):
        for Lm in (1024, 8192, 32768):
            inp = kvq_synth.gqa(Lm) if name == "gqa" else kvq_synth.mha(Lm)
            q, kv_lens, _, _, kp0, vp0, k, v = _setup_gqa(K, torch, inp, dev)
            del k, v
            per_copy = sum(t.numel() for t in (kp0.codes, kp0.scales, vp0.codes, vp0.scales))
            n_copies = min(n_rotation(args, per_copy), 512)
            copies = _rotation(K, kp0, vp0, n_copies)
            auto = K.kvq_auto_num_splits(cus, inp.B, inp.Hkv, Lm, inp.D, inp.Hq)
            steps = max(args.steps, n_copies)
            tm = Timer(torch, n_copies, steps)
            row = {}
            for sv in split_set + ["auto"]:
                s = auto if sv == "auto" else sv
                dec = GQADecode(K, torch, inp, q, kv_lens, copies, s, dev)
                for i in range(args.warmup):
                    dec.two_launch(dec.args[i % n_copies])
                row[str(sv)] = round(tm.run(lambda i: dec.two_launch(dec.args[i])) * 1e3, 3)
                del dec
            best = min(split_set, key=lambda x: row[str(x)])
            row["auto_s"] = auto
            row["best_s"] = best
            row["auto_over_best"] = round(row["auto"] / row[str(best)], 4)
            table[f"{name}_{Lm}"] = row
            log(f"{name} kv {Lm}: " + ", ".join(f"s={k_}: {v_}" for k_, v_ in row.items()))
            del copies, kp0, vp0
            torch.cuda.empty_cache()
    hdr = "| config | kv | " + " | ".join(f"s={x}" for x in split_set) + " | auto (s) | best s | auto / best |"
    lines = [hdr, "|" + "---|" * (len(split_set) + 5)]
    for key, row in table.items():
        name, Lm = key.split("_")
        lines.append(f"| {'GQA 4:1 B=2 Hq=32' if name == 'gqa' else 'MHA B=2 H=16'} | {Lm} | "
                     + " | ".join(f"{row[str(x)]:.2f}" for x in split_set)
                     + f" | {row['auto']:.2f} ({row['auto_s']}) | {row['best_s']} | {row['auto_over_best']:.3f} |")
    print("\n".join(lines), file=sys.stderr, flush=True)
    print(json.dumps({"metric": "decode step us (split + combine, two launches) by split count",
                      "unit": "us/step", "steps_per_graph": "max(--steps, rotation copies)", "table": table}),
          flush=True)


# ------------------------------------------------------------------ MLA
MLA_B, MLA_H, MLA_DC, MLA_DR, MLA_L = 32, 16, 512, 64, 8192
MLA_BYTES_PER_TOKEN = MLA_DC // 2 + MLA_DC // 16 + 2 * MLA_DR   # 256 + 32 + 128 = 416


def run_mla(args):
    """MLA latent-cache decode: one step = attn_decode_splitkv + combine
    over a rotation of >= 1 GiB of cache copies (109 MB each)."""
    import torch
    import kvq_synth
    import quantized_kv_cache_nvfp4_amd as K

    K._lib.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating MLA inputs")
    inp = kvq_synth.mla(L=MLA_L, B=MLA_B, H=MLA_H, Dc=MLA_DC, Dr=MLA_DR)
    lens = torch.from_numpy(inp.kv_lens).to(dev)
    c = inp.c.to(dev)
    amax = K.kvq_amax(c.unsqueeze(1), lens)
    plane0 = K.kvq_pack_nvfp4(c, amax)
    kr0 = inp.k_r.to(dev)
    del c
    q_c, q_r = inp.q_c.to(dev), inp.q_r.to(dev)
    per_copy = plane0.codes.numel() + plane0.scales.numel() + kr0.numel() * 2
    assert per_copy == MLA_B * MLA_L * MLA_BYTES_PER_TOKEN
    n_copies = n_rotation(args, per_copy)
    log(f"rotation: {n_copies} cache copies x {per_copy / 1e6:.1f} MB")
    copies = [(plane0, kr0)] + [(K.NVFP4Plane(plane0.codes.clone(), plane0.scales.clone(),
                                              plane0.tensor_scale.clone(), plane0.layout), kr0.clone())
                                for _ in range(n_copies - 1)]
    s = args.splits if args.splits > 0 else K.kvq_auto_num_splits(K.kvq_device_cu_count(), MLA_B, 1, MLA_L, MLA_DC,
                                                                   MLA_H)
    part_o, part_lse = K.decode_workspace(MLA_B, MLA_H, MLA_DC, s, dev)
    out = torch.empty(MLA_B, MLA_H, MLA_DC, dtype=torch.bfloat16, device=dev)
    dargs = [K.make_decode_args(q_c, pl, None, lens, max_kv_len=MLA_L, softmax_scale=inp.softmax_scale,
                                num_splits=s, part_o=part_o, part_lse=part_lse, q_rope=q_r, k_rope=kr)
             for pl, kr in copies]

    def step(i):
        used = K.attn_decode_splitkv(dargs[i])
        K.attn_decode_combine(part_o, part_lse, MLA_B, MLA_H, MLA_DC, used, out)

    # the same latent caches paged: blocks of 64 tokens at permuted physical
    # blocks (one table per copy; latent codes, scales and rope share it)
    PB = 64
    nb = MLA_L // PB
    rng = torch.Generator().manual_seed(5)

    def pg(t, perm):
        out_ = torch.empty_like(t).view(MLA_B * nb, PB, t.shape[-1])
        out_[perm] = t.view(MLA_B * nb, PB, t.shape[-1])
        return out_

    pdargs, keep = [], []
    for pl, kr in copies:
        perm = torch.randperm(MLA_B * nb, generator=rng).to(dev)
        bt = perm.view(MLA_B, nb).to(torch.int32).contiguous()
        ppl = K.NVFP4Plane(pg(pl.codes, perm), pg(pl.scales, perm), pl.tensor_scale, pl.layout)
        pkr = pg(kr, perm)
        pdargs.append(K.make_decode_args(q_c, ppl, None, lens, max_kv_len=MLA_L, softmax_scale=inp.softmax_scale,
                                         num_splits=s, part_o=part_o, part_lse=part_lse, q_rope=q_r, k_rope=pkr,
                                         block_table=bt))
        keep.append((ppl, pkr, bt))
    torch.cuda.synchronize()

    def paged_step(i):
        used = K.attn_decode_splitkv(pdargs[i])
        K.attn_decode_combine(part_o, part_lse, MLA_B, MLA_H, MLA_DC, used, out)

    for i in range(args.warmup):
        paged_step(i % n_copies)
    torch.cuda.synchronize()
    out_paged = out.clone()
    for i in range(args.warmup):
        step(i % n_copies)
    torch.cuda.synchronize()
    if args.warmup > 0:
        assert torch.equal(out, out_paged), "paged and contiguous MLA decode differ"
    # the latent query quantized to NVFP4 (per-tensor amax over the batch's
    # queries), decoded from its codes; timed beside: the query's calibration
    # and packing (two launches per step)
    qplane = K.kvq_pack_nvfp4(q_c, K.kvq_amax(q_c.unsqueeze(1)))
    qdargs = [K.make_decode_args(qplane, pl, None, lens, max_kv_len=MLA_L, softmax_scale=inp.softmax_scale,
                                 num_splits=s, part_o=part_o, part_lse=part_lse, q_rope=q_r, k_rope=kr)
              for pl, kr in copies]
    q_amax = torch.empty(1, dtype=torch.float32, device=dev)

    def qnv_step(i):
        used = K.attn_decode_splitkv(qdargs[i])
        K.attn_decode_combine(part_o, part_lse, MLA_B, MLA_H, MLA_DC, used, out)

    def quantize_query(i):
        K.kvq_amax(q_c.unsqueeze(1), out=q_amax)
        K.kvq_pack_nvfp4(q_c, q_amax, out=qplane)

    for i in range(args.warmup):
        qnv_step(i % n_copies)
        quantize_query(i)
    torch.cuda.synchronize()
    tm = Timer(torch, n_copies, args.steps)
    ms_step = tm.run(step)
    ms_split = tm.run(lambda i: K.attn_decode_splitkv(dargs[i]))
    ms_step_pg = tm.run(paged_step)
    ms_split_pg = tm.run(lambda i: K.attn_decode_splitkv(pdargs[i]))
    ms_step_qnv = tm.run(qnv_step)
    ms_split_qnv = tm.run(lambda i: K.attn_decode_splitkv(qdargs[i]))
    ms_qquant = tm.run(quantize_query)
    assert torch.isfinite(out.float()).all()
    algo = MLA_B * MLA_L * MLA_BYTES_PER_TOKEN
    res = base_record("us/decode step + achieved HBM GB/s, NVFP4-latent MLA split-KV decode B=32 H=16 8K",
                      ms_step * 1e3, args.steps, args.warmup, "f16/bf16 MFMA, fp32 accumulate (NVFP4 latent)",
                      {"workload": "MLA latent-cache decode (DeepSeek-V2 per-rank shape)", "B": MLA_B,
                       "heads": MLA_H, "latent": MLA_DC, "rope": MLA_DR, "kv_len": MLA_L, "splits": s,
                       "out_dtype": "bf16", "rotation_copies": n_copies})
    res["hbm_gbps_step"] = round(algo / (ms_step * 1e-3) / 1e9, 1)
    res["step_us"] = {"decode_two_launch": round(ms_step * 1e3, 3), "split_kernel": round(ms_split * 1e3, 3),
                      "decode_two_launch_paged64": round(ms_step_pg * 1e3, 3),
                      "split_kernel_paged64": round(ms_split_pg * 1e3, 3),
                      "decode_two_launch_nvfp4_query": round(ms_step_qnv * 1e3, 3),
                      "split_kernel_nvfp4_query": round(ms_split_qnv * 1e3, 3),
                      "quantize_query_nvfp4": round(ms_qquant * 1e3, 3)}
    res["roofline"] = roofline(algo, ms_split * 1e3, "k_decode_mla (split kernel, partials)", measured_traffic("mla"))
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        res["cpu_baseline"] = cpu_baseline_mla(inp, args.cpu_reps)
    print(json.dumps(res), flush=True)


# ------------------------------------------------------------------ FP8
FP8_B, FP8_LO, FP8_HI = 64, 512, 4096
FP8_BYTES_PER_TOKEN_HEAD = 2 * D   # K and V E4M3 codes


def run_fp8(args):
    """FP8 KV decode over ragged requests: one step = attn_decode_splitkv +
    combine (K rows, V TOKEN4), timed with exact probabilities, with FP8
    probabilities (prob_scale 1/448: two split passes + combine) and with
    FP8 output.  Rotation of >= 1 GiB of cache copies."""
    import torch
    import kvq_synth
    import quantized_kv_cache_nvfp4_amd as K

    K._lib.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating FP8 ragged inputs")
    inp = kvq_synth.fp8_ragged(B=FP8_B, lo=FP8_LO, hi=FP8_HI)
    lens = torch.from_numpy(inp.kv_lens).to(dev)
    k, v = inp.k.to(dev), inp.v.to(dev)
    ka, va = K.kvq_amax(k, lens), K.kvq_amax(v, lens)
    kp0 = K.kvq_pack_fp8(k, ka)
    vp0 = K.kvq_pack_fp8(v, va, layout=K.KVQ_PLANE_TOKEN4)
    # the same cache with one scale per kv head (the attn_head strategy)
    kah, vah = K.kvq_amax(k, lens, per_head=True), K.kvq_amax(v, lens, per_head=True)
    kph = K.kvq_pack_fp8(k, kah)
    vph = K.kvq_pack_fp8(v, vah, layout=K.KVQ_PLANE_TOKEN4)
    elems = k.numel()
    prep_us = {"amax_k": eager_timer(torch, lambda: K.kvq_amax(k, lens, out=ka)),
               "pack_k_fp8_rows": eager_timer(torch, lambda: K.kvq_pack_fp8(k, ka, out=kp0)),
               "pack_v_fp8_token4": eager_timer(torch, lambda: K.kvq_pack_fp8(v, va, out=vp0)),
               "amax_k_per_head": eager_timer(torch, lambda: K.kvq_amax(k, lens, out=kah, per_head=True)),
               "pack_k_fp8_rows_per_head": eager_timer(torch, lambda: K.kvq_pack_fp8(k, kah, out=kph))}
    valid = int(inp.kv_lens.astype("int64").sum()) * inp.Hkv * D   # amax reads the valid rows only
    prep_bytes = {"amax_k": valid * 2, "pack_k_fp8_rows": elems * 3, "pack_v_fp8_token4": elems * 3,
                  "amax_k_per_head": valid * 2, "pack_k_fp8_rows_per_head": elems * 3}
    del k, v
    q = inp.q.to(dev)
    per_copy = kp0.codes.numel() + vp0.codes.numel()
    n_copies = n_rotation(args, per_copy)
    log(f"rotation: {n_copies} cache copies x {per_copy / 1e6:.1f} MB (allocated at kv {FP8_HI})")
    copies = [(kp0, vp0)] + [(K.FP8Plane(kp0.codes.clone(), kp0.scale.clone(), kp0.layout),
                              K.FP8Plane(vp0.codes.clone(), vp0.scale.clone(), vp0.layout))
                             for _ in range(n_copies - 1)]
    Hq, Hkv = inp.Hq, inp.Hkv
    s = args.splits if args.splits > 0 else K.kvq_auto_num_splits(K.kvq_device_cu_count(), FP8_B, Hkv, FP8_HI, D, Hq)
    part_o, part_lse = K.decode_workspace(FP8_B, Hq, D, s, dev)
    scratch = torch.empty(K.kvq_fp8p_scratch_floats(FP8_B, Hq, s, FP8_HI), dtype=torch.float32, device=dev)
    out = torch.empty(FP8_B, Hq, D, dtype=torch.bfloat16, device=dev)
    out8 = torch.empty(FP8_B, Hq, D, dtype=torch.uint8, device=dev)
    out_scale = torch.full((1,), 4.0 / 448.0, dtype=torch.float32, device=dev)   # a given fp32 output scale

    # FP8 query (the QKV-FP8 schemes): the query batch calibrated and packed
    # per tensor by the same kernels, viewed as [B, Hq, 1, D]
    q4 = q.contiguous().view(FP8_B, inp.Hq, 1, D)
    qa = K.kvq_amax(q4)
    qp8 = K.kvq_pack_fp8(q4, qa)
    q8 = qp8.codes.view(FP8_B, inp.Hq, D)

    def mk(kc, vc, fp8p, fp8q=False):
        extra = dict(quantize_p=True, prob_scale=float(1.0 / 448.0), p_scratch=scratch) if fp8p else {}
        if fp8q:
            extra["q_scale"] = qp8.scale
        return K.make_decode_args(q8 if fp8q else q, kc, vc, lens, max_kv_len=FP8_HI, softmax_scale=inp.softmax_scale,
                                  num_splits=s, part_o=part_o, part_lse=part_lse, **extra)

    dargs = [mk(kc, vc, False) for kc, vc in copies]
    pargs = [mk(kc, vc, True) for kc, vc in copies]
    # per-head scales: the same code bytes read through one copy per step
    hcopies = [(kph, vph)] + [(K.FP8Plane(kph.codes.clone(), kph.scale.clone(), kph.layout),
                               K.FP8Plane(vph.codes.clone(), vph.scale.clone(), vph.layout))
                              for _ in range(n_copies - 1)]
    hargs = [mk(kc, vc, False) for kc, vc in hcopies]
    qargs = [mk(kc, vc, False, fp8q=True) for kc, vc in copies]

    def step(i, a, o):
        used = K.attn_decode_splitkv(a[i])
        K.attn_decode_combine(part_o, part_lse, FP8_B, Hq, D, used, o, out_scale=out_scale)

    # the one-launch decode (at one split per request it writes the output
    # directly, no partials and no merge)
    counters = torch.zeros(FP8_B * Hkv, dtype=torch.int32, device=dev)

    def fused(i, a, o):
        K.attn_decode(a[i], o, counters=counters)

    for i in range(args.warmup):
        step(i % n_copies, dargs, out)
        step(i % n_copies, pargs, out)
        fused(i % n_copies, dargs, out)
    torch.cuda.synchronize()
    tm = Timer(torch, n_copies, args.steps)
    ms = {"decode": tm.run(lambda i: step(i, dargs, out)),
          "decode_fused": tm.run(lambda i: fused(i, dargs, out)),
          "decode_fp8_out": tm.run(lambda i: step(i, dargs, out8)),
          "decode_fp8p": tm.run(lambda i: step(i, pargs, out)),
          "decode_per_head_scales": tm.run(lambda i: step(i, hargs, out)),
          "decode_fp8_query": tm.run(lambda i: step(i, qargs, out)),
          # the query's calibration + pack (two kernels and the amax clear), per step
          "quantize_query_fp8": tm.run(lambda i: (K.kvq_amax(q4, out=qa), K.kvq_pack_fp8(q4, qa, out=qp8))),
          "split_kernel": tm.run(lambda i: K.attn_decode_splitkv(dargs[i])),
          "fp8p_passes": tm.run(lambda i: K.attn_decode_splitkv(pargs[i]))}
    assert torch.isfinite(out.float()).all()
    tokens = int(inp.kv_lens.astype("int64").sum())
    algo = tokens * Hkv * FP8_BYTES_PER_TOKEN_HEAD
    algo_p = algo + tokens * Hq * 4 * 2   # + the spilled scores, written once and read once
    best = "decode_fused" if ms["decode_fused"] <= ms["decode"] else "decode"
    res = base_record("us/decode step + achieved HBM GB/s, FP8-KV split-KV decode B=64 GQA4:1 ragged 512..4096",
                      ms[best] * 1e3, args.steps, args.warmup, "f16 MFMA, fp32 accumulate (FP8 E4M3 KV)",
                      {"workload": "FP8 per-tensor KV decode, Llama-3-8B attention shape, ragged", "B": FP8_B,
                       "Hq": Hq, "Hkv": Hkv, "head_dim": D, "kv_len": f"U{{{FP8_LO}..{FP8_HI}}}",
                       "tokens": tokens, "splits": s, "out_dtype": "bf16", "v_layout": "token4",
                       "prob_scale": "1/448", "rotation_copies": n_copies, "step_path": best})
    res["hbm_gbps_step"] = round(algo / (ms[best] * 1e-3) / 1e9, 1)
    res["step_us"] = {k_: round(v_ * 1e3, 3) for k_, v_ in ms.items()}
    res["fp8p_hbm_gbps"] = round(algo_p / (ms["fp8p_passes"] * 1e-3) / 1e9, 1)
    res["calibrate_pack"] = {k_: {"us": round(t, 2), "GB/s": round(prep_bytes[k_] / (t * 1e-6) / 1e9, 1)}
                             for k_, t in prep_us.items()}
    res["roofline"] = roofline(algo, ms["split_kernel"] * 1e3, "k_decode_gqa<FP8,G=4,D=128> (split kernel, partials)",
                               measured_traffic("fp8"))
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        res["cpu_baseline"] = cpu_baseline_fp8(inp, args.cpu_reps)
        res["cpu_baseline_fp8p"] = cpu_baseline_fp8(inp, args.cpu_reps, prob_scale=float(1.0 / 448.0))
    print(json.dumps(res), flush=True)


PREFILL_SQ = 1024


def prefill_flops(kv_lens, Sq, Hq, Dh):
    """Algorithmic flops of a chunked prefill: query i of request b sees
    n = kv_len - Sq + i + 1 keys (causal, clamped at 0); each seen key costs
    2 Dh flops in Q.K^T and 2 Dh in P.V per query head."""
    tot = 0
    for Lb in kv_lens:
        for i in range(Sq):
            tot += max(0, int(Lb) - Sq + i + 1)
    return 4 * Dh * Hq * tot


def cpu_baseline_prefill(inp, q, reps, n_rows=64):
    """The oracle, untouched, timed on this host: per prefill step it
    dequantizes the packed cache and runs exact fp64 causal attention for
    every query row.  Sample: the dequantization of one kv head's K and V
    plus the attention of `n_rows` query tokens (all their heads sharing
    that kv head) at the end of request 0's chunk, scaled to the whole step
    (kv heads x requests for the dequantization, query tokens x kv heads x
    requests for the attention; the sampled tokens see the most keys, so the
    scaling over-estimates by at most Sq / (2 L) = 1.6 %); the oracle's
    one-off packing is not timed."""
    import numpy as np
    import kvq_synth
    from oracle import attention as OA
    from oracle import quant as OQ
    G = inp.Hq // inp.Hkv
    log("oracle: packing one kv head once (untimed)")
    kf, vf = kvq_synth.f64(inp.k[:1, :1]), kvq_synth.f64(inp.v[:1, :1])
    kc, ks, kst = OQ.nvfp4_pack(kf, OQ.amax(kf))
    vc, vs, vst = OQ.nvfp4_pack(vf, OQ.amax(vf))
    Sq = q.shape[1]
    qs = kvq_synth.f64(q[:1, Sq - n_rows:, :G])
    times = []
    for r in range(reps):
        log(f"oracle prefill sample {r + 1}/{reps}")
        t0 = time.perf_counter()
        khat, vhat = OQ.nvfp4_unpack(kc, ks, kst), OQ.nvfp4_unpack(vc, vs, vst)
        t1 = time.perf_counter()
        OA.prefill_gqa(qs, khat, vhat, inp.kv_lens[:1], inp.softmax_scale)
        t2 = time.perf_counter()
        times.append((t1 - t0) * inp.B * inp.Hkv + (t2 - t1) * (Sq / n_rows) * inp.Hkv * inp.B)
    t = float(np.median(times))
    return _cpu_entry(t, f"{reps} samples: dequantize 1 of {inp.B * inp.Hkv} (request, kv head) caches and "
                         f"attend {n_rows} of {Sq} query tokens x {G} heads of request 0 over {inp.Lmax} keys "
                         f"(fp64), median scaled to B={inp.B}, Hkv={inp.Hkv}, Sq={Sq}; numpy elementwise "
                         f"single-threaded, BLAS threads {_blas_threads()}")


def run_prefill(args):
    """Chunked prefill over the GQA 4:1 B=2 32K NVFP4 cache (the decode
    metric's cache): the last 1024 tokens of each request are the chunk, so
    query i sits at position 32768 - 1024 + i.  Both contractions run on
    MFMA (f16 inputs, fp32 accumulate); the roofline is the dense f16 matrix
    peak.  Also timed: the same chunk over the FP8 E4M3 copy of the cache,
    and the chunk's queries as FP8 codes (one scale) over both caches (over
    the FP8 cache Q.K^T runs on the FP8 matrix cores)."""
    import torch
    import kvq_synth
    import quantized_kv_cache_nvfp4_amd as K
    K._lib.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("prefill: GQA 4:1 B=2 32K cache, 1024-token chunk")
    inp = kvq_synth.gqa(L)
    q = kvq_synth.prefill_queries(B, PREFILL_SQ, HQ, D)
    _, kv_lens, k_amax, v_amax, kp0, vp0, k, v = _setup_gqa(K, torch, inp, dev)
    kf0 = K.kvq_pack_fp8(k, k_amax)
    vf0 = K.kvq_pack_fp8(v, v_amax, layout=K.KVQ_PLANE_TOKEN4)
    del k, v
    copies = _rotation(K, kp0, vp0, 2)
    qd = q.to(dev)
    out = torch.empty(B, PREFILL_SQ, HQ, D, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, PREFILL_SQ, HQ, dtype=torch.float32, device=dev)
    args_n = [K.make_prefill_args(qd, kc, vc, kv_lens, out, max_kv_len=L, softmax_scale=inp.softmax_scale,
                                  lse_out=lse) for kc, vc in copies]
    args_f = [K.make_prefill_args(qd, kf0, vf0, kv_lens, out, max_kv_len=L, softmax_scale=inp.softmax_scale,
                                  lse_out=lse)]
    q4 = qd.view(B * PREFILL_SQ, HQ, 1, D)
    qp = K.kvq_pack_fp8(q4, K.kvq_amax(q4))
    q8 = qp.codes.view(B, PREFILL_SQ, HQ, D)
    args_q8 = [K.make_prefill_args(q8, kf0, vf0, kv_lens, out, max_kv_len=L, softmax_scale=inp.softmax_scale,
                                   lse_out=lse, q_scale=qp.scale),
               K.make_prefill_args(q8, copies[0][0], copies[0][1], kv_lens, out, max_kv_len=L,
                                   softmax_scale=inp.softmax_scale, lse_out=lse, q_scale=qp.scale)]
    for i in range(args.warmup):
        K.attn_prefill(args_n[i % 2])
        K.attn_prefill(args_f[0])
        K.attn_prefill(args_q8[0])
        K.attn_prefill(args_q8[1])
    torch.cuda.synchronize()
    tm = Timer(torch, 2, args.steps)
    ms = {"prefill_nvfp4": tm.run(lambda i: K.attn_prefill(args_n[i]))}
    assert torch.isfinite(out.float()).all()
    tm1 = Timer(torch, 1, args.steps)
    ms["prefill_fp8"] = tm1.run(lambda i: K.attn_prefill(args_f[0]))
    ms["prefill_fp8_query_fp8"] = tm1.run(lambda i: K.attn_prefill(args_q8[0]))
    ms["prefill_fp8_query_nvfp4"] = tm1.run(lambda i: K.attn_prefill(args_q8[1]))
    assert torch.isfinite(out.float()).all()
    flops = prefill_flops(inp.kv_lens, PREFILL_SQ, HQ, D)
    step_us = ms["prefill_nvfp4"] * 1e3
    res = base_record("us/prefill step + achieved TFLOP/s, NVFP4-KV chunked prefill B=2 GQA4:1 32K cache, "
                      "1024-token chunk", step_us, args.steps, args.warmup, "f16 MFMA, fp32 accumulate (NVFP4 KV)",
                      {"workload": "NVFP4-KV chunked prefill, GQA 4:1", "B": B, "Hq": HQ, "Hkv": HKV, "head_dim": D,
                       "kv_len": L, "chunk": PREFILL_SQ, "out_dtype": "bf16", "v_layout": "token4",
                       "rotation_copies": 2})
    res["step_us"] = {k_: round(v_ * 1e3, 3) for k_, v_ in ms.items()}
    achieved = flops / (step_us * 1e-6) / 1e12
    res["roofline"] = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
                       "kernel": "k_prefill_gqa<NVFP4,G=4> (one launch per step)", "kernel_us_mean": round(step_us, 3),
                       "algorithmic_flops": flops}
    res["fp8_cache_tflops"] = round(flops / (ms["prefill_fp8"] * 1e-3) / 1e12, 1)
    res["fp8_query_fp8_cache_tflops"] = round(flops / (ms["prefill_fp8_query_fp8"] * 1e-3) / 1e12, 1)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        res["cpu_baseline"] = cpu_baseline_prefill(inp, q, args.cpu_reps)
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.source_hash:
        print(source_hash(args.source_hash))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
    elif args.read_probe:
        read_probe(args)
    elif args.sweep:
        run_sweep(args)
    elif args.workload == "mha":
        run_mha(args)
    elif args.workload == "mla":
        run_mla(args)
    elif args.workload == "fp8":
        run_fp8(args)
    elif args.workload == "prefill":
        run_prefill(args)
    else:
        run_gqa(args)


if __name__ == "__main__":
    main()
