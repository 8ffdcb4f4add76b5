// The merge of one query head's partial results of a decode step (the
// split-K combine of flash decoding):
//   o = sum_j 2^(m_j - m) o_j / sum_j 2^(m_j - m) l_j,  m = max_j m_j,
// shared by the combine kernel and by the one-launch step, which merges a
// unit's partials in the workgroup that writes the last of them.  Both run
// the same arithmetic in the same order, so their outputs are identical.
//
// 256 threads per head: thread (part, c) owns float4 column c and merges every
// PARTS-th partial online -- running maximum, rescaled sums -- so each
// partial's (m, l) and column are loaded together in one round trip; the
// PARTS states of a column are then merged through LDS.
#pragma once

#include "fsa_internal.h"

namespace fsa {

constexpr int kCombineThreads = 256;  // threads per head

template <int D>
struct CombineLds {
  static constexpr int NQ = D / 4;                     // float4 columns of one head
  static constexpr int PARTS = kCombineThreads / NQ;  // threads sharing a column
  float m[PARTS][NQ], l[PARTS][NQ];
  float4 acc[PARTS][NQ];
};

// Phase 1, thread t of the head's 256: the strand of partials t / NQ, t / NQ +
// PARTS, ... below n of column t % NQ.  ml and po point at the head's first
// partial (ml: its (m, l) pair, po: its float4 columns); consecutive partials
// are 2 G floats and G NQ float4s apart.
template <int D>
__device__ __forceinline__ void combine_strands(CombineLds<D>& S, const float* ml, const float4* po, int G, int n,
                                                int t) {
  constexpr int NQ = CombineLds<D>::NQ, PARTS = CombineLds<D>::PARTS;
  const int c4 = t % NQ, part = t / NQ;
  const size_t wstride = (size_t)G * NQ;  // float4s between consecutive partials
  po += c4;
  float M = -INFINITY, Lsum = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
  for (int w = part; w < n; w += PARTS) {
    const float m = ml[2 * (size_t)w * G];
    const float l = ml[2 * (size_t)w * G + 1];
    const float4 v = po[(size_t)w * wstride];
    const float Mn = fmaxf(M, m);
    const float ea = M == -INFINITY ? 0.f : exp2f(M - Mn);
    const float eb = m == -INFINITY ? 0.f : exp2f(m - Mn);
    a.x = a.x * ea + v.x * eb;
    a.y = a.y * ea + v.y * eb;
    a.z = a.z * ea + v.z * eb;
    a.w = a.w * ea + v.w * eb;
    Lsum = Lsum * ea + l * eb;
    M = Mn;
  }
  S.m[part][c4] = M;
  S.l[part][c4] = Lsum;
  S.acc[part][c4] = a;
}

// Phase 1 for at most kStrandMax partials per strand (n <= kStrandMax PARTS),
// in two halves so that the loads of several heads can be in flight together:
// strand_load issues a thread's loads (clamped in range; the partials past n
// are loaded but not used), strand_merge merges them into S like
// combine_strands.  The decode step's partials (a few per unit) always take
// this form, in the combine kernel and in the one-launch step alike.
constexpr int kStrandMax = 2;
template <int D>
struct StrandLoads {
  float m[kStrandMax], l[kStrandMax];
  float4 v[kStrandMax];
};
template <int D>
__device__ __forceinline__ void strand_load(StrandLoads<D>& L, const float* ml, const float4* po, int G, int n,
                                            int t) {
  constexpr int NQ = CombineLds<D>::NQ, PARTS = CombineLds<D>::PARTS;
  const int c4 = t % NQ, part = t / NQ;
  const size_t wstride = (size_t)G * NQ;
#pragma unroll
  for (int j = 0; j < kStrandMax; ++j) {
    const int w = min(part + j * PARTS, n - 1);
    L.m[j] = ml[2 * (size_t)w * G];
    L.l[j] = ml[2 * (size_t)w * G + 1];
    L.v[j] = po[(size_t)w * wstride + c4];
  }
}
template <int D>
__device__ __forceinline__ void strand_merge(CombineLds<D>& S, const StrandLoads<D>& L, int n, int t) {
  constexpr int NQ = CombineLds<D>::NQ, PARTS = CombineLds<D>::PARTS;
  const int c4 = t % NQ, part = t / NQ;
  float M = -INFINITY, Lsum = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < kStrandMax; ++j) {
    if (part + j * PARTS >= n) break;
    const float m = L.m[j], l = L.l[j];
    const float4 v = L.v[j];
    const float Mn = fmaxf(M, m);
    const float ea = M == -INFINITY ? 0.f : exp2f(M - Mn);
    const float eb = m == -INFINITY ? 0.f : exp2f(m - Mn);
    a.x = a.x * ea + v.x * eb;
    a.y = a.y * ea + v.y * eb;
    a.z = a.z * ea + v.z * eb;
    a.w = a.w * ea + v.w * eb;
    Lsum = Lsum * ea + l * eb;
    M = Mn;
  }
  S.m[part][c4] = M;
  S.l[part][c4] = Lsum;
  S.acc[part][c4] = a;
}

// Phase 2, after a barrier, by threads t < NQ: column t's strands merged in
// order, normalised and written as bf16 to the head's output row.
template <int D>
__device__ __forceinline__ void combine_write(const CombineLds<D>& S, int t, uint16_t* orow) {
  constexpr int PARTS = CombineLds<D>::PARTS;
  const int c4 = t;
  float Mt = S.m[0][c4];
#pragma unroll
  for (int p = 1; p < PARTS; ++p) Mt = fmaxf(Mt, S.m[p][c4]);
  float Lt = 0.f;
  float4 at = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int p = 0; p < PARTS; ++p) {
    const float mp = S.m[p][c4];
    const float e = mp == -INFINITY ? 0.f : exp2f(mp - Mt);
    const float4 v = S.acc[p][c4];
    at.x += e * v.x;
    at.y += e * v.y;
    at.z += e * v.z;
    at.w += e * v.w;
    Lt += e * S.l[p][c4];
  }
  const float inv = Lt > 0.f ? 1.0f / Lt : 0.f;
  const uint32_t w0 = f32_to_bf16_bits(at.x * inv) | (f32_to_bf16_bits(at.y * inv) << 16);
  const uint32_t w1 = f32_to_bf16_bits(at.z * inv) | (f32_to_bf16_bits(at.w * inv) << 16);
  *reinterpret_cast<uint2*>(orow + 4 * c4) = make_uint2(w0, w1);
}

}  // namespace fsa
