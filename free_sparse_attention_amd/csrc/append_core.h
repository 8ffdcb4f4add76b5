// Token append with incremental page metadata: the per-wave work, shared by
// the stand-alone append kernel and by the scoring launch of the combined
// append + decode step.
//
// Page metadata is Quest's per-page elementwise minimum and maximum of the
// keys (Quest, Tang et al. ICML 2024, named as the selection rule in the
// paper's analysis page, "Methodology", and the digest's "The Move").  Min and
// max are exact selections, so the code works on order-preserving 16-bit
// integer keys of the bf16 bit patterns: no rounding, and the result does not
// depend on the order in which tokens are combined.  A zero is written as +0.
#pragma once

#include "fsa_internal.h"

namespace fsa {

// Min/max keys of the 8 channels held by each lane, reduced over the 16 lanes
// of the same chunk (lanes differ in token slot); `valid` masks slots out.
__device__ __forceinline__ void chunk_minmax(const uint4& kv, bool valid, uint32_t mn[8],
                                             uint32_t mx[8]) {
  const uint32_t w[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t key = bf16_order_key((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    mn[e] = valid ? key : 0xFFFFu;
    mx[e] = valid ? key : 0u;
  }
#pragma unroll
  for (int off = 1; off < kPage; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mn[e] = min(mn[e], (uint32_t)__shfl_xor((int)mn[e], off, kPage));
      mx[e] = max(mx[e], (uint32_t)__shfl_xor((int)mx[e], off, kPage));
    }
  }
}

// Metadata of channel chunk c (channels 8c .. 8c + 7) of logical page p of unit u.
__device__ __forceinline__ uint4* meta_min_chunk(uint16_t* meta, int u, int p, int c, int tiles, int D) {
  return reinterpret_cast<uint4*>(meta + meta_offset(u, p, 8 * c, tiles, D));
}
__device__ __forceinline__ uint4* meta_max_chunk(uint16_t* meta, int u, int p, int c, int tiles, int D) {
  return reinterpret_cast<uint4*>(meta + meta_offset(u, p, D + 8 * c, tiles, D));
}

__device__ __forceinline__ void store_meta_chunk(uint16_t* meta, int u, int p, int c, int tiles, int D,
                                                 const uint32_t mn[8], const uint32_t mx[8]) {
  uint32_t lo[4], hi[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    lo[e >> 1] = bf16_from_order_key(mn[e]) | (bf16_from_order_key(mn[e + 1]) << 16);
    hi[e >> 1] = bf16_from_order_key(mx[e]) | (bf16_from_order_key(mx[e + 1]) << 16);
  }
  *meta_min_chunk(meta, u, p, c, tiles, D) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  *meta_max_chunk(meta, u, p, c, tiles, D) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
}

struct AppendArgs {
  int n_new;                  // tokens appended to every sequence
  const uint16_t* k_new;      // bf16 [B][n_new][Hkv][D]
  const uint16_t* v_new;
  const int32_t* page_table;  // [B][max_pages]
  const int32_t* seq_lens;    // lengths before the append
  int32_t* seq_lens_out;      // or null: lengths after the append
  uint16_t* kc;
  uint16_t* vc;
  uint16_t* meta;
  int hkv, max_pages;
  int touch;  // pages one append can reach: ceil(n_new / 16) + 1
};

inline AppendArgs append_args(int n_new, const uint16_t* k_new, const uint16_t* v_new, const int32_t* page_table,
                              const int32_t* seq_lens, int32_t* seq_lens_out, uint16_t* kc, uint16_t* vc,
                              uint16_t* meta, int hkv, int max_pages) {
  AppendArgs a;
  a.n_new = n_new;
  a.k_new = k_new;
  a.v_new = v_new;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.seq_lens_out = seq_lens_out;
  a.kc = kc;
  a.vc = vc;
  a.meta = meta;
  a.hkv = hkv;
  a.max_pages = max_pages;
  a.touch = (n_new + kPage - 1) / kPage + 1;
  return a;
}

// Append task w = unit * touch + j: the new tokens that land in the unit's
// j-th touched page.  Lane (slot = lane % 16, chunk = 4 * it + lane / 16)
// moves one 16-byte chunk of one new token; 64 lanes.
template <int D>
__device__ __forceinline__ void append_task(const AppendArgs& A, int w, int lane) {
  constexpr int NCH = D / 8;
  const int unit = w / A.touch, j = w % A.touch;
  const int b = unit / A.hkv, g = unit % A.hkv;
  const int L0 = A.seq_lens[b];
  const int slot = lane % kPage;
  const int n_new = A.n_new, max_pages = A.max_pages, hkv = A.hkv;
  // Positions past the page table are dropped, and the length counts only
  // the tokens written (fsa_validate_inputs reports such an overflow).
  const int cap = max_pages * kPage;
  if (A.seq_lens_out != nullptr && g == 0 && j == 0 && lane == 0)
    A.seq_lens_out[b] = L0 + n_new <= cap ? L0 + n_new : max(L0, cap);
  const int p = L0 / kPage + j;
  if (p >= max_pages) return;
  const int t_lo = max(L0, p * kPage), t_hi = min(L0 + n_new, p * kPage + kPage);
  if (t_lo >= t_hi) return;
  const int s0 = t_lo - p * kPage, s1 = t_hi - p * kPage;
  const size_t blk = (size_t)A.page_table[(size_t)b * max_pages + p] * hkv + g;
  const int tiles = meta_tiles(max_pages);
  const bool valid = slot >= s0 && slot < s1;
  const bool merge = slot == 0 && s0 > 0;  // the page already holds tokens: merge with its metadata
  // Every load first (new tokens, old metadata; one round trip beside the
  // page-table entry), every store after: on this target a load wait also
  // waits for earlier stores.
  constexpr int NIT = NCH / 4;
  uint4 kv[NIT], vv[NIT], om[NIT], oM[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int c = 4 * it + lane / kPage;
    kv[it] = vv[it] = om[it] = oM[it] = make_uint4(0, 0, 0, 0);
    if (valid) {
      const size_t src = (((size_t)b * n_new + (p * kPage + slot - L0)) * hkv + g) * D + c * 8;
      kv[it] = *reinterpret_cast<const uint4*>(A.k_new + src);
      vv[it] = *reinterpret_cast<const uint4*>(A.v_new + src);
    }
    if (merge) {
      om[it] = *meta_min_chunk(A.meta, unit, p, c, tiles, D);
      oM[it] = *meta_max_chunk(A.meta, unit, p, c, tiles, D);
    }
  }
  uint16_t* kdst = A.kc + blk * (kPage * D);
  uint16_t* vdst = A.vc + blk * (kPage * D);
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int c = 4 * it + lane / kPage;
    if (valid) {
      *reinterpret_cast<uint4*>(kdst + (c * kPage + slot) * 8) = kv[it];
      const uint32_t w[4] = {vv[it].x, vv[it].y, vv[it].z, vv[it].w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vdst[(c * 8 + e) * kPage + slot] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
    uint32_t mn[8], mx[8];
    chunk_minmax(kv[it], valid, mn, mx);
    if (slot == 0) {
      if (merge) {
        const uint32_t a[4] = {om[it].x, om[it].y, om[it].z, om[it].w};
        const uint32_t z[4] = {oM[it].x, oM[it].y, oM[it].z, oM[it].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          mn[e] = min(mn[e], bf16_order_key((a[e >> 1] >> (16 * (e & 1))) & 0xFFFFu));
          mx[e] = max(mx[e], bf16_order_key((z[e >> 1] >> (16 * (e & 1))) & 0xFFFFu));
        }
      }
      store_meta_chunk(A.meta, unit, p, c, tiles, D, mn, mx);
    }
  }
}

}  // namespace fsa
