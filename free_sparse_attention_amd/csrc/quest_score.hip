// Quest page scores on the matrix cores.
//
// Quest's bound for query head h and page p (Quest, Tang et al. ICML 2024;
// the selection rule named on the paper's analysis page, "Methodology") is
//     U_h(p) = sum_i max(q_hi m_pi, q_hi M_pi).
// Because m <= M elementwise, each term equals q+_hi M_pi + q-_hi m_pi with
// q+ = max(q, 0) and q- = min(q, 0), both exact in bf16.  So the bound is a
// plain contraction over 2D channels between Qx = [q- | q+]  (heads x 2D) and
// the page's metadata row [m | M] (2D values), which is exactly how the
// metadata is stored.  The group score is the maximum over the group's heads.
//
// One v_mfma_f32_16x16x32_bf16 chain per 16-page tile computes
// C[head][page] = sum_k Qx[head][k] Mx[page][k] in fp32 (bf16 products are
// exact in fp32), with the heads of the group on M (zero-padded to 16) and 16
// pages on N.  The matrix cores take the arithmetic off the vector ALUs, which
// a plain per-lane bound would keep busy at about (G + 1) / 2 operations per
// metadata byte -- close to the chip's vector issue rate per HBM byte at G = 8.
//
// Operand loads come straight from HBM: lane (col, gq) of k-step s reads the
// 16 bytes at [64 s + 16 gq, +16) of page col's 2D-value row, so each load
// instruction covers 64 contiguous bytes of 16 pages and two consecutive
// steps cover whole 128-byte lines.
#include "fsa_internal.h"

namespace fsa {
namespace {

constexpr int kMaxTilesPerWave = 8;

__device__ __forceinline__ uint32_t keep_sign(uint32_t w, bool negative) {
  // per 16-bit half: keep it when its sign matches `negative`, else zero it
  const uint32_t s = w & 0x80008000u;
  const uint32_t neg_mask = ((s >> 15) & 1u) * 0xFFFFu | ((s >> 31) * 0xFFFFu) << 16;
  return negative ? (w & neg_mask) : (w & ~neg_mask);
}

template <int D>
__global__ __launch_bounds__(256) void quest_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ meta,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    float* __restrict__ scores, int hq, int hkv, int max_pages, int prefix, int window,
    int tiles_per_wave, int wg_per_unit, int max_seq_len) {
  constexpr int NSTEP = 2 * D / 32;  // k-steps over the 2D metadata values
  const int unit = blockIdx.x / wg_per_unit, wg = blockIdx.x % wg_per_unit;
  const int b = unit / hkv, g = unit % hkv, G = hq / hkv;
  const int L = min(seq_lens[b], max_seq_len);  // lengths beyond the host bound are clamped
  const int Pe = min(prefix, L), Ws = max(0, L - window);
  if (Pe >= Ws) return;
  const int c_lo = Pe / kPage, c_hi = (Ws + kPage - 1) / kPage;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, gq = lane >> 4;
  const int p_first = c_lo + (wg * 4 + wave) * tiles_per_wave * 16;
  if (p_first >= c_hi) return;
  const int n_tiles = min(tiles_per_wave, (c_hi - p_first + 15) / 16);

  // A operand: row `col` = query head col of the group (zero beyond G).
  bf16x8_t a[NSTEP];
  const uint16_t* qrow = q + ((size_t)b * hq + (size_t)g * G + col) * D;
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    const int e0 = 32 * s + 8 * gq;  // channel e0 .. e0+7 of [m | M]
    uint4 r = make_uint4(0, 0, 0, 0);
    if (col < G) r = *reinterpret_cast<const uint4*>(qrow + (e0 % D));
    const bool neg = e0 < D;  // the m half pairs with q-, the M half with q+
    r.x = keep_sign(r.x, neg);
    r.y = keep_sign(r.y, neg);
    r.z = keep_sign(r.z, neg);
    r.w = keep_sign(r.w, neg);
    a[s] = __builtin_bit_cast(bf16x8_t, r);
  }

  // pool pages of this wave's tiles (page col of each tile)
  const int32_t* pt = page_table + (size_t)b * max_pages;
  int phys[kMaxTilesPerWave];
#pragma unroll
  for (int t = 0; t < kMaxTilesPerWave; ++t) {
    const int p = p_first + 16 * t + col;
    phys[t] = (t < n_tiles && p < c_hi) ? pt[p] : -1;
  }

  float* srow = scores + (size_t)unit * max_pages;
#pragma unroll
  for (int t0 = 0; t0 < kMaxTilesPerWave; t0 += 2) {
    if (t0 >= n_tiles) break;
    uint4 buf[2][NSTEP];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ph = phys[t0 + u];
      const uint16_t* row = meta + ((size_t)(ph < 0 ? 0 : ph) * hkv + g) * (2 * D) + 8 * gq;
#pragma unroll
      for (int s = 0; s < NSTEP; ++s)
        buf[u][s] = ph < 0 ? make_uint4(0, 0, 0, 0)
                           : ld_nt(reinterpret_cast<const uint4*>(row + 32 * s));
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NSTEP; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], __builtin_bit_cast(bf16x8_t, buf[u][s]),
                                                      acc, 0, 0, 0);
      // lane holds heads 4 gq .. 4 gq + 3 of page col
      float sc = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * gq + r < G) sc = fmaxf(sc, acc[r]);
      if (G > 4) sc = fmaxf(sc, __shfl_xor(sc, 16));
      if (G > 8) sc = fmaxf(sc, __shfl_xor(sc, 32));
      if (gq == 0 && phys[t0 + u] >= 0) srow[p_first + 16 * (t0 + u) + col] = sc;
    }
  }
}

}  // namespace

hipError_t launch_quest_scores(const uint16_t* q, const uint16_t* meta, const int32_t* page_table,
                               const int32_t* seq_lens, float* scores, int batch, int hq, int hkv,
                               int d, int max_pages, int prefix, int window, int max_seq_len,
                               hipStream_t stream) {
  const int units = batch * hkv;
  const int max_cand = (max_seq_len + kPage - 1) / kPage + 1;
  const int tiles_per_unit = (max_cand + 15) / 16;
  const long total_tiles = (long)units * tiles_per_unit;
  int tpw = 1;  // tiles per wave: enough waves to fill 256 CUs, fewer when there is work to spare
  while (tpw < kMaxTilesPerWave && total_tiles / (2 * tpw) >= 2048) tpw *= 2;
  const int wg_per_unit = (tiles_per_unit + 4 * tpw - 1) / (4 * tpw);
  const dim3 grid((unsigned)((long)units * wg_per_unit));
  if (d == 128)
    hipLaunchKernelGGL(quest_score_kernel<128>, grid, dim3(256), 0, stream, q, meta, page_table,
                       seq_lens, scores, hq, hkv, max_pages, (int)prefix, (int)window, tpw,
                       wg_per_unit, max_seq_len);
  else
    hipLaunchKernelGGL(quest_score_kernel<64>, grid, dim3(256), 0, stream, q, meta, page_table,
                       seq_lens, scores, hq, hkv, max_pages, (int)prefix, (int)window, tpw,
                       wg_per_unit, max_seq_len);
  return hipGetLastError();
}

}  // namespace fsa
