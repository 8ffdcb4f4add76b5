// KV-cache side of the path: layout import, token append with incremental
// page metadata, and the full metadata rebuild.
//
// Page metadata is Quest's per-page elementwise minimum and maximum of the
// keys (Quest, Tang et al. ICML 2024, named as the selection rule in the
// paper's analysis page, "Methodology", and the digest's "The Move").  Min and
// max are exact selections, so the kernels work on order-preserving 16-bit
// integer keys of the bf16 bit patterns: no rounding, and the result does not
// depend on the order in which tokens are combined.  A zero is written as +0.
#include "append_core.h"

namespace fsa {
namespace {

// One wave per (pool page, KV head): token-major [S][D] -> K chunk-major
// [D/8][S][8] and V channel-major [D][S].
template <int D>
__global__ __launch_bounds__(64) void import_kv_plain_kernel(const uint16_t* __restrict__ kp,
                                                             const uint16_t* __restrict__ vp,
                                                             uint16_t* __restrict__ kc,
                                                             uint16_t* __restrict__ vc) {
  constexpr int NCH = D / 8;
  const size_t base = (size_t)blockIdx.x * (kPage * D);
  const int lane = threadIdx.x;
#pragma unroll
  for (int i = lane; i < kPage * NCH; i += kWave) {
    const int c = i / kPage, j = i % kPage;  // destination chunk order
    const uint4 v = *reinterpret_cast<const uint4*>(kp + base + (size_t)(j * NCH + c) * 8);
    *reinterpret_cast<uint4*>(kc + base + (size_t)(c * kPage + j) * 8) = v;
  }
#pragma unroll
  for (int c = lane; c < D; c += kWave) {
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t lo = vp[base + (size_t)(2 * j) * D + c];
      const uint32_t hi = vp[base + (size_t)(2 * j + 1) * D + c];
      w[j] = lo | (hi << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(vc + base + (size_t)c * kPage);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// One wave per (sequence, KV head, touched page).
template <int D>
__global__ __launch_bounds__(64) void append_kv_kernel(const AppendArgs A) {
  append_task<D>(A, blockIdx.x, threadIdx.x);
}

// One wave per (sequence, logical page, KV head) over pages in use.
template <int D>
__global__ __launch_bounds__(256) void build_page_meta_kernel(
    const uint16_t* __restrict__ kc, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, uint16_t* __restrict__ meta, int hkv, int max_pages,
    int n_max, int64_t n_waves) {
  constexpr int NCH = D / 8;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= n_waves) return;
  const int g = (int)(w % hkv);
  const int p = (int)((w / hkv) % n_max);
  const int b = (int)(w / ((int64_t)hkv * n_max));
  const int L = min(seq_lens[b], n_max * kPage);
  if (p * kPage >= L) return;
  const int lane = threadIdx.x & 63, slot = lane % kPage;
  const int nvalid = min(kPage, L - p * kPage);
  const size_t blk = (size_t)page_table[(size_t)b * max_pages + p] * hkv + g;
  const uint16_t* ksrc = kc + blk * (kPage * D);
  const int tiles = meta_tiles(max_pages);
  const int unit = b * hkv + g;
#pragma unroll
  for (int it = 0; it < NCH / 4; ++it) {
    const int c = 4 * it + lane / kPage;
    const uint4 kv = *reinterpret_cast<const uint4*>(ksrc + (64 * it + lane) * 8);
    uint32_t mn[8], mx[8];
    chunk_minmax(kv, slot < nvalid, mn, mx);
    if (slot == 0) store_meta_chunk(meta, unit, p, c, tiles, D, mn, mx);
  }
}

}  // namespace

hipError_t launch_import_kv_plain(const uint16_t* k_plain, const uint16_t* v_plain, uint16_t* kc,
                                  uint16_t* vc, int pool, int hkv, int d, hipStream_t stream) {
  const dim3 grid((unsigned)((size_t)pool * hkv));
  if (d == 128)
    hipLaunchKernelGGL(import_kv_plain_kernel<128>, grid, dim3(64), 0, stream, k_plain, v_plain, kc, vc);
  else
    hipLaunchKernelGGL(import_kv_plain_kernel<64>, grid, dim3(64), 0, stream, k_plain, v_plain, kc, vc);
  return hipGetLastError();
}

hipError_t launch_append_kv(int n_new, const uint16_t* k_new, const uint16_t* v_new,
                            const int32_t* page_table, const int32_t* seq_lens,
                            int32_t* seq_lens_out, uint16_t* kc, uint16_t* vc, uint16_t* meta,
                            int batch, int hkv, int d, int max_pages, hipStream_t stream) {
  const AppendArgs a = append_args(n_new, k_new, v_new, page_table, seq_lens, seq_lens_out, kc, vc, meta, hkv,
                                   max_pages);
  const dim3 grid((unsigned)((size_t)batch * hkv * a.touch));
  if (d == 128)
    hipLaunchKernelGGL(append_kv_kernel<128>, grid, dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(append_kv_kernel<64>, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_build_page_meta(const uint16_t* kc, const int32_t* page_table,
                                  const int32_t* seq_lens, uint16_t* meta, int batch, int hkv,
                                  int d, int max_pages, int max_seq_len, hipStream_t stream) {
  const int n_max = (max_seq_len + kPage - 1) / kPage;
  const int64_t n_waves = (int64_t)batch * n_max * hkv;
  const dim3 grid((unsigned)((n_waves + 3) / 4));
  if (d == 128)
    hipLaunchKernelGGL(build_page_meta_kernel<128>, grid, dim3(256), 0, stream, kc, page_table,
                       seq_lens, meta, hkv, max_pages, n_max, n_waves);
  else
    hipLaunchKernelGGL(build_page_meta_kernel<64>, grid, dim3(256), 0, stream, kc, page_table,
                       seq_lens, meta, hkv, max_pages, n_max, n_waves);
  return hipGetLastError();
}

}  // namespace fsa
