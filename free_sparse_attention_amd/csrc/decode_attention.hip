// Split-K flash decoding over the attended pages, with the cross-split
// combine fused into the last workgroup of each (sequence, KV head).
//
// Per work item (one page, a token range [lo, hi) inside it), one wave:
//   S^T[token][head] = K[token][:] . q[head][:]     v_mfma_f32_16x16x32_bf16, D/32 steps
//   online softmax over the page's tokens in fp32 (base-2 exponent, scale folded)
//   O^T[d][head]    += V^T[d][token] P^T[token][head] v_mfma_f32_16x16x16_bf16, D/16 tiles
// Heads of the group sit on the N side (zero-padded to 16).  The QK result's
// register layout (lane (col, gq) holds tokens 4 gq .. 4 gq + 3 of head col)
// is exactly the B-operand layout the PV product needs, so P never leaves
// registers.  The cache layouts make every operand load a coalesced read
// straight from HBM: a K page [D/8][16][8] is read as D/32 contiguous
// 1 KiB rows, a V page [D][16] as D/16 contiguous 512-byte rows.
//
// Four waves per workgroup each walk their own run of items; the workgroup
// merges its waves' (max, sum, accumulator) through LDS, writes one partial,
// and the last workgroup of the unit to finish (agent-scope atomic ticket)
// combines all partials:  o = sum_j 2^(m_j - m) o_j / sum_j 2^(m_j - m) l_j.
#include "fsa_internal.h"

namespace fsa {
namespace {

constexpr int kAttnWaves = 4;
typedef short s16x4_t __attribute__((ext_vector_type(4)));

template <int D, bool DENSE>
__global__ __launch_bounds__(256) void decode_attention_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ work,
    const int32_t* __restrict__ counts, float* __restrict__ part_o, float* __restrict__ part_ml,
    int32_t* __restrict__ counters, uint16_t* __restrict__ out, int hq, int hkv, int max_pages,
    int max_items, int ipw, int wg_per_unit, float scale_log2, int max_seq_len) {
  constexpr int NKS = D / 32;  // QK k-steps
  constexpr int NDT = D / 16;  // PV d-tiles
  __shared__ float sh_o[kAttnWaves][D][17];
  __shared__ float sh_m[kAttnWaves][16], sh_l[kAttnWaves][16];
  __shared__ int sh_last;

  const int unit = blockIdx.x / wg_per_unit, wg = blockIdx.x % wg_per_unit;
  const int b = unit / hkv, g = unit % hkv, G = hq / hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, gq = lane >> 4;
  const int L = min(seq_lens[b], max_seq_len);  // lengths beyond the host bound are clamped
  const int n_items = DENSE ? (L + kPage - 1) / kPage : counts[2 * unit + 1];
  const int per_wg = kAttnWaves * ipw;
  const int n_wg = (n_items + per_wg - 1) / per_wg;
  if (wg >= n_wg) return;
  const int i_begin = wg * per_wg + wave * ipw;
  const int i_end = min(i_begin + ipw, n_items);

  // B operand of QK: q[head col][32 ks + 8 gq .. +8] (zero rows beyond G)
  bf16x8_t qb[NKS];
  const uint16_t* qrow = q + ((size_t)b * hq + (size_t)g * G + col) * D;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    uint4 r = make_uint4(0, 0, 0, 0);
    if (col < G) r = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * gq);
    qb[ks] = __builtin_bit_cast(bf16x8_t, r);
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t acc[NDT];
#pragma unroll
  for (int j = 0; j < NDT; ++j) acc[j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  const int32_t* pt = page_table + (size_t)b * max_pages;
  const int32_t* wl = work + 4 * (size_t)unit * max_items;
  for (int i = i_begin; i < i_end; ++i) {
    int phys, lo, hi;
    if (DENSE) {
      phys = pt[i];
      lo = 0;
      hi = min(kPage, L - i * kPage);
    } else {
      const int4 it = *reinterpret_cast<const int4*>(wl + 4 * (size_t)i);
      phys = it.y;
      lo = it.z;
      hi = it.w;
    }
    const size_t blk = ((size_t)phys * hkv + g) * (kPage * D);
    uint4 kr[NKS];
    uint2 vr[NDT];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kr[ks] = ld_nt(reinterpret_cast<const uint4*>(kc + blk + (size_t)(64 * ks + lane) * 8));
#pragma unroll
    for (int j = 0; j < NDT; ++j)
      vr[j] = ld_nt(reinterpret_cast<const uint2*>(vc + blk + (size_t)(16 * j + col) * kPage + 4 * gq));

    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[ks]), qb[ks], s, 0, 0, 0);

    float x[4], mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = 4 * gq + r;
      x[r] = (tok >= lo && tok < hi) ? s[r] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float p[4], psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = exp2f(x[r] - m_new);
      psum += p[r];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    const uint32_t p01 = f32_to_bf16_bits(p[0]) | (f32_to_bf16_bits(p[1]) << 16);
    const uint32_t p23 = f32_to_bf16_bits(p[2]) | (f32_to_bf16_bits(p[3]) << 16);
    const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(p01, p23));
#pragma unroll
    for (int j = 0; j < NDT; ++j) {
      acc[j] *= alpha;
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, vr[j]), pb,
                                                         acc[j], 0, 0, 0);
    }
  }
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  // ---- merge the workgroup's waves through LDS
  if (gq == 0) {
    sh_m[wave][col] = m_run;
    sh_l[wave][col] = l_run;
  }
#pragma unroll
  for (int j = 0; j < NDT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) sh_o[wave][16 * j + 4 * gq + r][col] = acc[j][r];
  __syncthreads();

  const int nout = G * D;
  const bool single = (n_wg == 1);
  float* po = part_o + ((size_t)unit * wg_per_unit + wg) * G * D;
  float* pml = part_ml + 2 * ((size_t)unit * wg_per_unit + wg) * G;
  for (int idx = threadIdx.x; idx < nout; idx += 256) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, sh_m[w][h]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float e = exp2f(sh_m[w][h] - M);  // waves without items carry m = -inf
      o += e * sh_o[w][d][h];
      l += e * sh_l[w][h];
    }
    if (single) {
      out[((size_t)b * hq + (size_t)g * G + h) * D + d] = (uint16_t)f32_to_bf16_bits(o / l);
    } else {
      po[idx] = o;
      if (d == 0) {
        pml[2 * h] = M;
        pml[2 * h + 1] = l;
      }
    }
  }
  if (single) return;

  // ---- last workgroup of the unit combines the partials
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) sh_last = (atomicAdd(&counters[unit], 1) == n_wg - 1);
  __syncthreads();
  if (!sh_last) return;
  __threadfence();
  const float* po0 = part_o + (size_t)unit * wg_per_unit * G * D;
  const float* pml0 = part_ml + 2 * (size_t)unit * wg_per_unit * G;
  for (int idx = threadIdx.x; idx < nout; idx += 256) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
    for (int w = 0; w < n_wg; ++w) M = fmaxf(M, pml0[2 * ((size_t)w * G + h)]);
    float o = 0.f, l = 0.f;
    for (int w = 0; w < n_wg; ++w) {
      const float e = exp2f(pml0[2 * ((size_t)w * G + h)] - M);
      o += e * po0[(size_t)w * G * D + idx];
      l += e * pml0[2 * ((size_t)w * G + h) + 1];
    }
    out[((size_t)b * hq + (size_t)g * G + h) * D + d] = (uint16_t)f32_to_bf16_bits(o / l);
  }
  if (threadIdx.x == 0) counters[unit] = 0;
}

}  // namespace

AttnPlan plan_attention(int units, int max_items) {
  AttnPlan p;
  const long total = (long)units * max_items;
  int ipw = 1;  // items per wave: at least ~4096 waves in flight, longer runs when work allows
  while (ipw < 8 && total / (2 * ipw) >= 4096) ipw *= 2;
  p.items_per_wave = ipw;
  p.wg_per_unit = (max_items + kAttnWaves * ipw - 1) / (kAttnWaves * ipw);
  return p;
}

hipError_t launch_decode_attention(bool dense, const AttnPlan& plan, const uint16_t* q,
                                   const uint16_t* kc, const uint16_t* vc,
                                   const int32_t* page_table, const int32_t* seq_lens,
                                   const int32_t* work, const int32_t* counts, float* part_o,
                                   float* part_ml, int32_t* counters, uint16_t* out, int batch,
                                   int hq, int hkv, int d, int max_pages, int max_items,
                                   float sm_scale, int max_seq_len, hipStream_t stream) {
  const dim3 grid((unsigned)((long)batch * hkv * plan.wg_per_unit));
  const float scale_log2 = sm_scale * 1.4426950408889634f;
#define FSA_LAUNCH(DD, DN)                                                                        \
  hipLaunchKernelGGL((decode_attention_kernel<DD, DN>), grid, dim3(256), 0, stream, q, kc, vc,   \
                     page_table, seq_lens, work, counts, part_o, part_ml, counters, out, hq, hkv, \
                     max_pages, max_items, plan.items_per_wave, plan.wg_per_unit, scale_log2,     \
                     max_seq_len)
  if (d == 128) {
    if (dense) FSA_LAUNCH(128, true); else FSA_LAUNCH(128, false);
  } else {
    if (dense) FSA_LAUNCH(64, true); else FSA_LAUNCH(64, false);
  }
#undef FSA_LAUNCH
  return hipGetLastError();
}

}  // namespace fsa
