// Measurement helpers, not part of the decode step: the device's memory
// properties and a plain streaming read of a buffer, whose rate is the
// achievable HBM read ceiling the step's memory-bound kernels are compared
// against.
#include <algorithm>
#include <cstdint>

#include "fsa_internal.h"

namespace fsa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeThreads = 256;
constexpr int kRowsPerWave = 16;  // 1 KiB rows (64 lanes x 16 bytes) read by one wave, contiguous
constexpr int kProbeUnroll = 4;   // rows in flight per wave

// Wave w reads rows [16 w, 16 w + 16) of the buffer's whole 1 KiB rows with
// non-temporal loads, four rows in flight; workgroup 0 also reads the last
// partial row.  (Measured over 2 GiB on MI355X, this order beats grid-stride
// loops and longer runs per wave: 7.0 vs 5.5-6.8 TB/s.)  The words are
// folded into one xor per lane, stored only if it equals a fixed value, so
// the loads cannot be dropped and the kernel writes nothing in practice.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ p, size_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const size_t rows = n16 / 64;
  const size_t r0 = ((size_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)) * kRowsPerWave;
  const u32x4* base = p + r0 * 64 + lane;
  uint32_t acc = 0;
  if (r0 + kRowsPerWave <= rows) {
#pragma unroll
    for (int r = 0; r < kRowsPerWave; r += kProbeUnroll) {
      u32x4 v[kProbeUnroll];
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(base + (size_t)(r + u) * 64);
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  } else {
    for (size_t r = r0; r < rows; ++r) {
      const u32x4 v = __builtin_nontemporal_load(p + r * 64 + lane);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  if (blockIdx.x == 0 && rows * 64 + threadIdx.x < n16) {
    const u32x4 v = p[rows * 64 + threadIdx.x];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const size_t n16 = bytes / 16, rows = n16 / 64;
  const size_t waves = (rows + kRowsPerWave - 1) / kRowsPerWave;
  const size_t grid = std::max<size_t>(1, (waves + kProbeThreads / 64 - 1) / (kProbeThreads / 64));
  if (grid > 0x7fffffffu) return hipErrorInvalidValue;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(buf), n16, sink);
  return hipGetLastError();
}

}  // namespace fsa
