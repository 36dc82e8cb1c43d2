// Streaming-read probe: the practical HBM read ceiling of this device for a
// buffer of the decode cache's size, measured the way the decode kernels
// read (16-byte vector loads, every byte read once, nothing written).  It is
// a measurement aid for the benchmark, built into its own library
// (libkvq_probe.so) and not part of the kvq C ABI.
//
//   kvq_probe_read(p, bytes, grid, sink, stream)
//     p      device buffer, 16-byte aligned; bytes a multiple of 16.
//     grid   work-groups of 256 threads (each thread keeps 8 loads in
//            flight per loop trip).
//     sink   device uint32[1]; written only if the xor of everything read
//            equals a fixed constant, so the loads cannot be dropped and
//            the probe writes (almost surely) nothing.
//   Returns 0, or 1 for bad arguments, 2 for a launch error.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;

__global__ void __launch_bounds__(kThreads) k_read_probe(const uint4* __restrict__ p, uint64_t n16, uint32_t* sink) {
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kThreads;
  uint64_t i = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    uint4 v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) v[k] = p[i + k * stride];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

extern "C" int kvq_probe_read(const void* p, uint64_t bytes, int32_t grid, uint32_t* sink, void* stream) {
  if (p == nullptr || sink == nullptr || bytes % 16 != 0 || grid <= 0 ||
      reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return 1;
  hipLaunchKernelGGL(k_read_probe, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(p), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
