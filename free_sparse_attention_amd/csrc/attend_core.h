// Per-wave flash-decoding over pages of one (sequence, KV head) and the merge
// of a workgroup's waves.  Shared by the split-K attention kernel and by the
// prefix/window attention that runs beside the selection.
//
// Per item (one page, a token range [lo, hi) inside it), one wave computes
//   S^T[token][head] = K[token][:] . q[head][:]     v_mfma_f32_16x16x32_bf16, D/32 steps
//   online softmax over the page's tokens in fp32 (base-2 exponent, scale folded)
//   O^T[d][head]    += V^T[d][token] P^T[token][head] v_mfma_f32_16x16x16_bf16, D/16 tiles
// Heads of the group sit on the N side (zero-padded to 16).  The QK result's
// register layout (lane (col, gq) holds tokens 4 gq .. 4 gq + 3 of head col)
// is exactly the B-operand layout the PV product needs, so P never leaves
// registers.  The cache layouts make every operand load a coalesced read
// straight from HBM: a K page [D/8][16][8] is read as D/32 contiguous 1 KiB
// rows, a V page [D][16] as D/16 contiguous 512-byte rows.
#pragma once

#include "fsa_internal.h"

namespace fsa {

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Running state of one wave: maximum (log2 domain) and sum per head column,
// O^T accumulators.
template <int D>
struct WaveAttn {
  float m, l;
  f32x4_t acc[D / 16];
};

// LDS for merging WAVES waves' states.
template <int D, int WAVES>
struct MergeLds {
  float o[WAVES][D][17];
  float m[WAVES][16], l[WAVES][16];
  float e[WAVES][16];     // weight 2^(m_w - M) of wave w for head h
  float M[16], L[16];     // per head: maximum and weighted sum
};

// B operand of QK for head column col of the group: q[col][32 ks + 8 gq .. +8],
// zero rows beyond G.  q_group points at the group's first query head.
template <int D>
__device__ __forceinline__ void load_q_operand(const uint16_t* q_group, int G, bf16x8_t (&qb)[D / 32]) {
  const int lane = threadIdx.x & 63, col = lane & 15, gq = lane >> 4;
  const uint16_t* qrow = q_group + (size_t)min(col, G - 1) * D;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    uint4 r = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * gq);
    if (col >= G) r = make_uint4(0, 0, 0, 0);
    qb[ks] = __builtin_bit_cast(bf16x8_t, r);
  }
}

// One wave attends its first n items; lane j holds item j's pool page and
// token range.  n must be wave-uniform.  PIPE: two-stage pipeline (the next
// page's loads in flight while the current page is computed); otherwise one
// page at a time with fewer registers.  QLDS (with PIPE): n <= 2, both pages'
// loads in flight together, and the query operand read from LDS
// (q_lds[ks * 64 + lane], the layout of qb) to leave the registers to the
// second page.  head_off/page_stride locate KV head g of a pool page in both
// caches.
template <int D, bool PIPE, bool QLDS = false>
__device__ __forceinline__ void attend_items(const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                                             size_t head_off, size_t page_stride, const bf16x8_t (&qb)[D / 32],
                                             int my_phys, int my_lo, int my_hi, int n, float scale_log2,
                                             WaveAttn<D>& st, const bf16x8_t* q_lds = nullptr) {
  constexpr int NKS = D / 32;  // QK k-steps
  constexpr int NDT = D / 16;  // PV d-tiles
  const int lane = threadIdx.x & 63, col = lane & 15, gq = lane >> 4;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int t = 0; t < NDT; ++t) st.acc[t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  auto load = [&](int j, uint4 (&kr)[NKS], uint2 (&vr)[NDT]) {
    const size_t blk = (size_t)__builtin_amdgcn_readlane(my_phys, j) * page_stride + head_off;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kr[ks] = ld_nt(reinterpret_cast<const uint4*>(kc + blk + (size_t)(64 * ks + lane) * 8));
#pragma unroll
    for (int t = 0; t < NDT; ++t)
      vr[t] = ld_nt(reinterpret_cast<const uint2*>(vc + blk + (size_t)(16 * t + col) * kPage + 4 * gq));
  };
  auto compute = [&](int j, const uint4 (&kr)[NKS], const uint2 (&vr)[NDT]) {
    const int lo = __builtin_amdgcn_readlane(my_lo, j), hi = __builtin_amdgcn_readlane(my_hi, j);
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[ks]),
                                                  QLDS ? q_lds[ks * kWave + lane] : qb[ks], s, 0, 0, 0);
    float x[4], mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = 4 * gq + r;
      x[r] = (tok >= lo && tok < hi) ? s[r] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m, mx);
    const float alpha = exp2f(st.m - m_new);
    // The weights are rounded to bf16 for the P.V product, and the sum l adds
    // the same rounded weights: numerator and denominator use one set of
    // weights, so the output is a convex combination of the values.
    uint32_t pr[4];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = f32_to_bf16_bits(exp2f(x[r] - m_new));
      psum += __uint_as_float(pr[r] << 16);
    }
    st.l = st.l * alpha + psum;
    st.m = m_new;
    const uint32_t p01 = pr[0] | (pr[1] << 16);
    const uint32_t p23 = pr[2] | (pr[3] << 16);
    const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(p01, p23));
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      st.acc[t] *= alpha;
      st.acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, vr[t]), pb, st.acc[t], 0, 0, 0);
    }
  };

  if (PIPE && QLDS) {
    // at most two items: both pages' loads in flight together, the second
    // issued even for one item (page 0 again, then attended as an empty
    // range, which leaves the state unchanged) so that no branch separates
    // the loads from the computation
    if (n > 0) {
      uint4 kA[NKS], kB[NKS];
      uint2 vA[NDT], vB[NDT];
      load(0, kA, vA);
      __builtin_amdgcn_sched_barrier(0);  // issue order = completion order: the first page's wait leaves the second in flight
      load(n > 1 ? 1 : 0, kB, vB);
      __builtin_amdgcn_sched_barrier(0);
      compute(0, kA, vA);
      compute(1, kB, vB);
    }
  } else if (PIPE) {
    // Every trip of the loop issues exactly one page of loads and consumes
    // one, so the number of loads in flight at the loop head is the same on
    // entry and on the back edge and the compiler waits only for the page
    // about to be used; the last one or two pages are peeled.
    uint4 kA[NKS], kB[NKS];
    uint2 vA[NDT], vB[NDT];
    if (n > 0) {
      load(0, kA, vA);
      int j = 0;
      for (; j + 2 < n; j += 2) {
        load(j + 1, kB, vB);
        compute(j, kA, vA);
        load(j + 2, kA, vA);
        compute(j + 1, kB, vB);
      }
      if (j + 1 < n) {
        load(j + 1, kB, vB);
        compute(j, kA, vA);
        compute(j + 1, kB, vB);
      } else {
        compute(j, kA, vA);
      }
    }
  } else {
    uint4 kA[NKS];
    uint2 vA[NDT];
    for (int j = 0; j < n; ++j) {
      load(j, kA, vA);
      compute(j, kA, vA);
    }
  }
  st.l += __shfl_xor(st.l, 16);
  st.l += __shfl_xor(st.l, 32);
}

// Merge the WAVES waves of the workgroup through LDS; then each of the G x D
// values is written either as the bf16 output (direct) or into the partial
// slot (po: [G][D] sums, pml: [G] (max, sum) pairs).  Waves without items
// carry m = -inf.
template <int D, int WAVES>
__device__ __forceinline__ void merge_waves(MergeLds<D, WAVES>& S, const WaveAttn<D>& st, int G, bool direct,
                                            uint16_t* __restrict__ out_rows, float* __restrict__ po,
                                            float* __restrict__ pml) {
  constexpr int NDT = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, col = lane & 15, gq = lane >> 4;
  if (gq == 0) {
    S.m[wave][col] = st.m;
    S.l[wave][col] = st.l;
  }
  if (col < G)  // columns beyond the group's heads are padding (LDS bandwidth bounds this phase)
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) S.o[wave][16 * t + 4 * gq + r][col] = st.acc[t][r];
  __syncthreads();
  // per head: the maximum, the waves' weights and the weighted sum, by wave 0:
  // lane (part, h) takes waves part * WAVES/4 .. +WAVES/4 of head h, and the
  // four parts of a head combine with two lane exchanges
  static_assert(WAVES % 4 == 0, "the weights step splits the waves in four parts");
  if (wave == 0) {
    constexpr int PER = WAVES / 4;
    const int h = lane & 15, part = lane >> 4;
    float mw[PER], lw[PER];  // all reads first, so they are in flight together
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      mw[i] = S.m[part * PER + i][h];
      lw[i] = S.l[part * PER + i][h];
    }
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < PER; ++i) M = fmaxf(M, mw[i]);
    M = fmaxf(M, __shfl_xor(M, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      mw[i] = mw[i] == -INFINITY ? 0.f : exp2f(mw[i] - M);
      l += mw[i] * lw[i];
    }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
#pragma unroll
    for (int i = 0; i < PER; ++i) S.e[part * PER + i][h] = mw[i];
    if (part == 0) {
      S.M[h] = M;
      S.L[h] = l;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += WAVES * kWave) {
    const int h = idx / D, d = idx % D;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) o += S.e[w][h] * S.o[w][d][h];
    if (direct) {
      const float l = S.L[h];
      out_rows[idx] = (uint16_t)f32_to_bf16_bits(l > 0.f ? o / l : 0.f);
    } else {
      po[idx] = o;
      if (d == 0) {
        pml[2 * h] = S.M[h];
        pml[2 * h + 1] = S.L[h];
      }
    }
  }
}

}  // namespace fsa
