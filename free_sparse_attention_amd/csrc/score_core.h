// Quest page scores of one (sequence, KV head) unit on the matrix cores: the
// routine shared by the scoring kernel and the scoring tasks of the one-launch
// decode step.
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
#pragma once

#include "fsa_internal.h"

namespace fsa {

__device__ __forceinline__ uint32_t keep_sign(uint32_t w, bool negative) {
  // per 16-bit half: keep it when its sign matches `negative`, else zero it
  const uint32_t s = w & 0x80008000u;
  const uint32_t neg_mask = ((s >> 15) & 1u) * 0xFFFFu | ((s >> 31) * 0xFFFFu) << 16;
  return negative ? (w & neg_mask) : (w & ~neg_mask);
}

// What the scoring reads and writes (the step's arguments).
struct ScoreArgs {
  const uint16_t* q;
  const uint16_t* meta;
  const int32_t* seq_lens;
  float* scores;
  int hq, hkv, max_pages, prefix, window, max_seq_len, len_add, G;
};

// Wave `wave_id` of the n_waves waves that score unit (b, g) takes every
// n_waves-th 16-page tile, at most tiles_per_wave of them, so at any moment the
// unit's waves together read one contiguous stretch of metadata.  Metadata is
// loaded one tile ahead of the MFMA chain, with the non-temporal hint: it is
// read once per step and should not displace cached data (on MI355X this
// streams about a quarter faster at 256k tokens than plain loads or a
// contiguous run of tiles per wave).  Scores go to scores[unit][p] for the
// candidate pages p; the length is seq_lens[b] + len_add, clamped to
// max_seq_len.  Returns without a store when the wave has no candidate tile.
template <int D>
__device__ __forceinline__ void score_wave(const ScoreArgs& S, int unit, int b, int g, int wave_id, int n_waves,
                                           int tiles_per_wave) {
  constexpr int NSTEP = 2 * D / 32;  // k-steps over the 2D metadata values
  const int lane = threadIdx.x & 63;
  const uint16_t* q = S.q;
  const uint16_t* meta = S.meta;
  float* scores = S.scores;
  const int hq = S.hq, max_pages = S.max_pages, prefix = S.prefix, window = S.window;
  const int max_seq_len = S.max_seq_len, G = S.G;
  const int col = lane & 15, gq = lane >> 4;
  // Every sequence with candidates has L > prefix, so its candidates start at
  // page prefix / 16 and end at or before the host bound's: the wave's first
  // tile is known before the length arrives and is loaded together with it.
  const int c_lo_h = min(prefix, max_seq_len) / kPage;
  const int c_hi_h = (max(0, max_seq_len - window) + kPage - 1) / kPage;
  const int t_first = c_lo_h / kMetaTile + wave_id;  // then every n_waves-th tile
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
  const int L = min(S.seq_lens[b] + S.len_add, max_seq_len);  // lengths beyond the host bound are clamped
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

}  // namespace fsa
