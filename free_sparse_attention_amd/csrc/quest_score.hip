// Quest page scores on the matrix cores.
//
// Quest's bound for query head h and page p (Quest, Tang et al. ICML 2024;
// the selection rule named on the paper's analysis page, "Methodology") is
//     U_h(p) = sum_i max(q_hi m_pi, q_hi M_pi).
// Because m <= M elementwise, each term equals q+_hi M_pi + q-_hi m_pi with
// q+ = max(q, 0) and q- = min(q, 0), both exact in bf16.  So the bound is a
// plain contraction over 2D values between Qx = [q- | q+]  (heads x 2D) and
// the page's metadata [m | M] (2D values).  The group score is the maximum
// over the group's heads.
//
// One v_mfma_f32_16x16x32_bf16 chain per 16-page tile computes
// C[head][page] = sum_k Qx[head][k] Mx[page][k] in fp32 (bf16 products are
// exact in fp32), with the heads of the group on M (zero-padded to 16) and the
// tile's 16 pages on N.  The matrix cores take the arithmetic off the vector
// ALUs, which a plain per-lane bound would keep busy at about (G + 1) / 2
// operations per metadata byte -- close to the chip's vector issue rate per
// HBM byte at G = 8.
//
// The metadata layout (per unit, 16-page tiles of [2D/32][16][32] values) makes
// each MFMA step's B operand one contiguous 1 KiB slab: lane (col, gq) of step
// s reads values 8 gq .. 8 gq + 7 of page col, so every load instruction is
// fully coalesced and no page table is involved.
#include <algorithm>
#include <atomic>

#include "append_core.h"

namespace fsa {
namespace {


__device__ __forceinline__ uint32_t keep_sign(uint32_t w, bool negative) {
  // per 16-bit half: keep it when its sign matches `negative`, else zero it
  const uint32_t s = w & 0x80008000u;
  const uint32_t neg_mask = ((s >> 15) & 1u) * 0xFFFFu | ((s >> 31) * 0xFFFFu) << 16;
  return negative ? (w & neg_mask) : (w & ~neg_mask);
}

// Each wave scores every n-th 16-page tile of one (sequence, KV head) unit,
// n being the unit's wave count, so at any moment the unit's waves together
// read one contiguous stretch of metadata; the grid is sized to four resident
// rounds of waves.  Metadata is loaded one tile ahead of the MFMA chain, with
// the non-temporal hint: it is read once per step and should not displace
// cached data (on MI355X this streams about a quarter faster at 256k tokens
// than plain loads or a contiguous run of tiles per wave).
//
// In the combined append + decode step the same launch also carries the
// append: its tasks (append_core.h) in the first append_blocks workgroups, one
// per wave; the scoring then takes the lengths after the append (seq_lens +
// len_add).  The host uses this only when no page the append touches can be a
// candidate (window >= n_new + 15), so the two roles write and read disjoint
// data; the scores of the touched pages' tiles that are not candidates are
// computed from metadata being rewritten, but never stored.
template <int D, int W>  // W: waves per workgroup
__global__ __launch_bounds__(W * 64) void quest_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ meta,
    const int32_t* __restrict__ seq_lens, float* __restrict__ scores, int hq, int hkv,
    int max_pages, int prefix, int window, int tiles_per_wave, int wg_per_unit, int max_seq_len,
    const AppendArgs ap, int append_blocks, int append_tasks, int len_add, FastDiv by_wg, FastDiv by_hkv, int G) {
  constexpr int NSTEP = 2 * D / 32;  // k-steps over the 2D metadata values
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if ((int)blockIdx.x < append_blocks) {
    const int w = (int)blockIdx.x * W + wave;
    if (w < append_tasks) append_task<D>(ap, w, lane);
    return;
  }
  const int blk = (int)blockIdx.x - append_blocks;
  const int unit = (int)fdiv((uint32_t)blk, by_wg), wg = blk - unit * wg_per_unit;
  const int b = (int)fdiv((uint32_t)unit, by_hkv), g = unit - b * hkv;
  const int col = lane & 15, gq = lane >> 4;
  // Every sequence with candidates has L > prefix, so its candidates start at
  // page prefix / 16 and end at or before the host bound's: the wave's first
  // tile is known before the length arrives and is loaded together with it.
  const int c_lo_h = min(prefix, max_seq_len) / kPage;
  const int c_hi_h = (max(0, max_seq_len - window) + kPage - 1) / kPage;
  const int n_waves = W * wg_per_unit;
  const int t_first = c_lo_h / kMetaTile + wg * W + wave;  // then every n_waves-th tile
  const int t_end_h = max(1, (c_hi_h + kMetaTile - 1) / kMetaTile);

  // A operand: row `col` = query head col of the group (zero beyond G).
  bf16x8_t a[NSTEP];
  const uint16_t* qrow = q + ((size_t)b * hq + (size_t)g * G + min(col, G - 1)) * D;
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    const int e0 = 32 * s + 8 * gq;  // values e0 .. e0+7 of [m | M]
    uint4 r = *reinterpret_cast<const uint4*>(qrow + (e0 % D));
    if (col >= G) r = make_uint4(0, 0, 0, 0);
    const bool neg = e0 < D;  // the m half pairs with q-, the M half with q+
    r.x = keep_sign(r.x, neg);
    r.y = keep_sign(r.y, neg);
    r.z = keep_sign(r.z, neg);
    r.w = keep_sign(r.w, neg);
    a[s] = __builtin_bit_cast(bf16x8_t, r);
  }

  const int tiles = meta_tiles(max_pages);
  const uint16_t* mbase = meta + (size_t)unit * tiles * (NSTEP * kMetaTile * 32) + col * 32 + 8 * gq;
  float* srow = scores + (size_t)unit * max_pages;
  uint4 bufA[NSTEP], bufB[NSTEP];
  {
    // first tile, clamped into the host bound's range (used only if valid below)
    const uint16_t* src = mbase + (size_t)min(t_first, t_end_h - 1) * (NSTEP * kMetaTile * 32);
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) bufA[s] = ld_nt(reinterpret_cast<const uint4*>(src + s * (kMetaTile * 32)));
  }
  const int L = min(seq_lens[b] + len_add, max_seq_len);  // lengths beyond the host bound are clamped
  const int Pe = min(prefix, L), Ws = max(0, L - window);
  if (Pe >= Ws) return;
  const int c_lo = Pe / kPage, c_hi = (Ws + kPage - 1) / kPage;  // c_lo == c_lo_h here
  const int t_end = (c_hi + kMetaTile - 1) / kMetaTile;
  if (t_first >= t_end) return;
  const int n_tiles = min(tiles_per_wave, (t_end - t_first + n_waves - 1) / n_waves);
  // Loads are unconditional (tiles are whole; pages outside the candidates
  // are scored but not stored), so the number of loads in flight is the same
  // on every path and the compiler waits only for the tile about to be reduced.
  auto load = [&](int t, uint4 (&buf)[NSTEP]) {
    const uint16_t* src = mbase + (size_t)(t_first + t * n_waves) * (NSTEP * kMetaTile * 32);
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) buf[s] = ld_nt(reinterpret_cast<const uint4*>(src + s * (kMetaTile * 32)));
  };
  auto compute = [&](int t, const uint4 (&buf)[NSTEP]) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NSTEP; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], __builtin_bit_cast(bf16x8_t, buf[s]), acc, 0, 0, 0);
    // lane holds heads 4 gq .. 4 gq + 3 of page col
    float sc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * gq + r < G) sc = fmaxf(sc, acc[r]);
    if (G > 4) sc = fmaxf(sc, __shfl_xor(sc, 16));
    if (G > 8) sc = fmaxf(sc, __shfl_xor(sc, 32));
    const int p = (t_first + t * n_waves) * kMetaTile + col;
    if (gq == 0 && p >= c_lo && p < c_hi) srow[p] = sc;
  };

  int t = 0;
  for (; t + 2 < n_tiles; t += 2) {
    load(t + 1, bufB);
    compute(t, bufA);
    load(t + 2, bufA);
    compute(t + 1, bufB);
  }
  if (t + 1 < n_tiles) {
    load(t + 1, bufB);
    compute(t, bufA);
    compute(t + 1, bufB);
  } else {
    compute(t, bufA);
  }
}

}  // namespace

hipError_t launch_quest_scores(const uint16_t* q, const uint16_t* meta, const int32_t* seq_lens,
                               float* scores, int batch, int hq, int hkv, int d, int max_pages,
                               int prefix, int window, int max_seq_len, hipStream_t stream,
                               const AppendArgs* append) {
  const int units = batch * hkv;
  const int max_cand = (max_seq_len + kPage - 1) / kPage;
  const int tiles_per_unit = (max_cand + kMetaTile - 1) / kMetaTile + 1;  // a range may straddle one more
  // 8-wave workgroups for batches of many units (the 16-sequence serving
  // batch: 128 units, step 171 -> 169 us), 4-wave ones otherwise (64k and
  // 256k: 4 waves 0.1 and 0.9 us faster)
  const int W = units >= 64 ? 8 : 4;
  const void* kern = d == 128 ? (W == 8 ? reinterpret_cast<const void*>(&quest_score_kernel<128, 8>)
                                        : reinterpret_cast<const void*>(&quest_score_kernel<128, 4>))
                              : (W == 8 ? reinterpret_cast<const void*>(&quest_score_kernel<64, 8>)
                                        : reinterpret_cast<const void*>(&quest_score_kernel<64, 4>));
  static std::atomic<int> resident[2][2];  // per head dim and workgroup size, zero until first queried
  int res = resident[d == 128][W == 8].load(std::memory_order_relaxed);
  if (res == 0) {
    res = resident_blocks_per_cu(kern, W * 64);
    resident[d == 128][W == 8].store(res, std::memory_order_relaxed);
  }
  // four resident rounds of workgroups shared out over the units: workgroups
  // whose tiles lie beyond their sequence's length exit at once and the
  // dispatcher gives their slots to the next ones, which evens out batches of
  // unequal lengths (16 sequences of 18k-261k tokens: step 165.9 -> 158.9 us)
  const int round = 4 * res * device_cu_count();
  const int wg_per_unit_max = (tiles_per_unit + W - 1) / W;
  const int wg_per_unit = std::max(1, std::min(wg_per_unit_max, round / std::max(1, units)));
  const int tpw = (tiles_per_unit + W * wg_per_unit - 1) / (W * wg_per_unit);
  AppendArgs ap{};
  int append_tasks = 0, len_add = 0;
  if (append) {
    ap = *append;
    append_tasks = units * ap.touch;
    len_add = ap.n_new;
  }
  const int append_blocks = (append_tasks + W - 1) / W;
  const dim3 grid((unsigned)((long)append_blocks + (long)units * wg_per_unit));
#define FSA_SCORE(DD, WW)                                                                                       \
  hipLaunchKernelGGL((quest_score_kernel<DD, WW>), grid, dim3(WW * 64), 0, stream, q, meta, seq_lens, scores, hq, \
                     hkv, max_pages, prefix, window, tpw, wg_per_unit, max_seq_len, ap, append_blocks, append_tasks,  \
                     len_add, make_fastdiv((uint32_t)wg_per_unit), make_fastdiv((uint32_t)hkv), hq / hkv)
  if (d == 128) {
    if (W == 8) FSA_SCORE(128, 8); else FSA_SCORE(128, 4);
  } else {
    if (W == 8) FSA_SCORE(64, 8); else FSA_SCORE(64, 4);
  }
#undef FSA_SCORE
  return hipGetLastError();
}

}  // namespace fsa
