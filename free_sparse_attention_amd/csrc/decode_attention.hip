// Split-K flash decoding over attended pages, then the cross-split combine.
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
// 1 KiB rows, a V page [D][16] as D/16 contiguous 512-byte rows.  Each wave
// walks a run of items with the next page's loads in flight while the current
// page is computed.
//
// Items come either from the selection's work list (prefix, selected and
// window pages; kList) or are every page of the sequence (kDense, the dense
// baseline).  Four waves per workgroup; the workgroup merges its waves' (max,
// sum, accumulator) through LDS and writes one partial into its slot, or the
// output directly when a unit needs a single workgroup.  The combine kernel
// merges a unit's partials:
//   o = sum_j 2^(m_j - m) o_j / sum_j 2^(m_j - m) l_j,  m = max_j m_j.
#include <algorithm>

#include "fsa_internal.h"

namespace fsa {
namespace {

constexpr int kAttnWaves = 4;
constexpr int kMaxItemsPerWave = 64;
typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int wave_bcast(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

template <int D, int MODE>
__global__ __launch_bounds__(256, 3) void decode_attention_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ work,
    float* __restrict__ part_o, float* __restrict__ part_ml,
    uint16_t* __restrict__ out, int hq, int hkv, int max_pages, int max_items, int ipw,
    int wg_per_unit, float scale_log2, int max_seq_len) {
  constexpr int NKS = D / 32;  // QK k-steps
  constexpr int NDT = D / 16;  // PV d-tiles
  __shared__ float sh_o[kAttnWaves][D][17];
  __shared__ float sh_m[kAttnWaves][16], sh_l[kAttnWaves][16];

  const int unit = blockIdx.x / wg_per_unit, wg = blockIdx.x % wg_per_unit;
  const int b = unit / hkv, g = unit % hkv, G = hq / hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, gq = lane >> 4;
  const int per_wg = kAttnWaves * ipw;
  const int i_begin = wg * per_wg + wave * ipw;

  // item descriptors of this wave: lane j holds item i_begin + j.  Dense items
  // are the sequence's pages.  A work list is padded with empty items (lo = hi)
  // to max_items, so its entries are read without first loading the item
  // count; the valid items of a wave are a prefix of its lanes.
  int my_phys = 0, my_lo = 0, my_hi = 0, n, n_wg;
  if (MODE == kDense) {
    const int L = min(seq_lens[b], max_seq_len);  // lengths beyond the host bound are clamped
    const int n_items = (L + kPage - 1) / kPage;
    n_wg = (n_items + per_wg - 1) / per_wg;
    if (wg >= n_wg) return;
    n = max(0, min(ipw, n_items - i_begin));
    if (lane < n) {
      const int i = i_begin + lane;
      my_phys = page_table[(size_t)b * max_pages + i];
      my_hi = min(kPage, L - i * kPage);
    }
  } else {
    n_wg = wg_per_unit;
    if (lane < ipw && i_begin + lane < max_items) {
      const int4 it = *reinterpret_cast<const int4*>(work + 4 * ((size_t)unit * max_items + i_begin + lane));
      my_phys = it.y;
      my_lo = it.z;
      my_hi = it.w;
    }
    n = __popcll(__ballot(my_lo < my_hi));
  }

  // B operand of QK: q[head col][32 ks + 8 gq .. +8] (zero rows beyond G)
  bf16x8_t qb[NKS];
  const uint16_t* qrow = q + ((size_t)b * hq + (size_t)g * G + min(col, G - 1)) * D;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    uint4 r = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * gq);
    if (col >= G) r = make_uint4(0, 0, 0, 0);
    qb[ks] = __builtin_bit_cast(bf16x8_t, r);
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t acc[NDT];
#pragma unroll
  for (int j = 0; j < NDT; ++j) acc[j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  const size_t head_off = (size_t)g * (kPage * D);
  const size_t page_stride = (size_t)hkv * (kPage * D);
  auto load = [&](int j, uint4 (&kr)[NKS], uint2 (&vr)[NDT]) {
    const size_t blk = (size_t)wave_bcast(my_phys, j) * page_stride + head_off;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kr[ks] = ld_nt(reinterpret_cast<const uint4*>(kc + blk + (size_t)(64 * ks + lane) * 8));
#pragma unroll
    for (int t = 0; t < NDT; ++t)
      vr[t] = ld_nt(reinterpret_cast<const uint2*>(vc + blk + (size_t)(16 * t + col) * kPage + 4 * gq));
  };
  auto compute = [&](int j, const uint4 (&kr)[NKS], const uint2 (&vr)[NDT]) {
    const int lo = wave_bcast(my_lo, j), hi = wave_bcast(my_hi, j);
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
    for (int t = 0; t < NDT; ++t) {
      acc[t] *= alpha;
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, vr[t]), pb, acc[t], 0, 0, 0);
    }
  };

  // Two-stage pipeline.  Every trip of the loop issues exactly one page of
  // loads and consumes one, so the number of loads in flight at the loop head
  // is the same on entry and on the back edge and the compiler waits only for
  // the page about to be used; the last one or two pages are peeled.
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
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  // ---- merge the workgroup's waves through LDS
  if (gq == 0) {
    sh_m[wave][col] = m_run;
    sh_l[wave][col] = l_run;
  }
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) sh_o[wave][16 * t + 4 * gq + r][col] = acc[t][r];
  __syncthreads();

  const bool direct = n_wg == 1;
  const size_t slot = (size_t)unit * wg_per_unit + wg;
  float* po = part_o + slot * G * D;
  float* pml = part_ml + 2 * slot * G;
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, sh_m[w][h]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float mw = sh_m[w][h];
      const float e = mw == -INFINITY ? 0.f : exp2f(mw - M);  // waves without items carry m = -inf
      o += e * sh_o[w][d][h];
      l += e * sh_l[w][h];
    }
    if (direct) {
      out[((size_t)b * hq + (size_t)g * G + h) * D + d] = (uint16_t)f32_to_bf16_bits(l > 0.f ? o / l : 0.f);
    } else {
      po[idx] = o;
      if (d == 0) {
        pml[2 * h] = M;
        pml[2 * h + 1] = l;
      }
    }
  }
}

// One workgroup per (sequence, KV head, query head of the group): merges the
// unit's partials for that head.  Units handled by a single workgroup were
// finished by the attention kernel.  Thread (part, c) owns float4 column c and
// merges every PARTS-th partial online -- running maximum, rescaled sums -- so
// each partial's (m, l) and column are loaded together in one round trip; the
// PARTS states of a column are then merged through LDS.
template <int D, int MODE>
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ seq_lens, uint16_t* __restrict__ out, int hq, int hkv, int per_wg, int wg_per_unit, int max_seq_len) {
  constexpr int NQ = D / 4;        // float4 columns of one head
  constexpr int PARTS = 256 / NQ;  // threads sharing a column, each with every PARTS-th partial
  __shared__ float sh_m[PARTS][NQ], sh_l[PARTS][NQ];
  __shared__ float4 sh_acc[PARTS][NQ];
  const int G = hq / hkv;
  const int unit = blockIdx.x / G, h = blockIdx.x % G;
  const int b = unit / hkv, g = unit % hkv;
  // partial slots in use: a work list fills all of them (empty ones carry
  // m = -inf); dense units use as many as their length needs
  int n = wg_per_unit;
  if (MODE == kDense) {
    const int L = min(seq_lens[b], max_seq_len);
    n = ((L + kPage - 1) / kPage + per_wg - 1) / per_wg;
  }
  if (n <= 1) return;  // written directly by the attention kernel
  const int tid = threadIdx.x, c4 = tid % NQ, part = tid / NQ;
  const float* ml = part_ml + 2 * ((size_t)unit * wg_per_unit * G + h);
  const float4* po = reinterpret_cast<const float4*>(part_o + ((size_t)unit * wg_per_unit * G + h) * D) + c4;
  const size_t wstride = (size_t)G * NQ;  // float4s between consecutive partials

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
  sh_m[part][c4] = M;
  sh_l[part][c4] = Lsum;
  sh_acc[part][c4] = a;
  __syncthreads();
  if (part == 0) {
    float Mt = M;
#pragma unroll
    for (int p = 1; p < PARTS; ++p) Mt = fmaxf(Mt, sh_m[p][c4]);
    float Lt = 0.f;
    float4 at = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int p = 0; p < PARTS; ++p) {
      const float mp = sh_m[p][c4];
      const float e = mp == -INFINITY ? 0.f : exp2f(mp - Mt);
      const float4 v = sh_acc[p][c4];
      at.x += e * v.x;
      at.y += e * v.y;
      at.z += e * v.z;
      at.w += e * v.w;
      Lt += e * sh_l[p][c4];
    }
    const float inv = Lt > 0.f ? 1.0f / Lt : 0.f;
    const uint32_t w0 = f32_to_bf16_bits(at.x * inv) | (f32_to_bf16_bits(at.y * inv) << 16);
    const uint32_t w1 = f32_to_bf16_bits(at.z * inv) | (f32_to_bf16_bits(at.w * inv) << 16);
    *reinterpret_cast<uint2*>(out + ((size_t)b * hq + (size_t)g * G + h) * D + 4 * c4) = make_uint2(w0, w1);
  }
}

}  // namespace

AttnPlan plan_attention(int units, int max_items) {
  // one resident round of waves (3 workgroups of 4 waves per CU) shared out
  // over all items; longer runs per wave when there is more work
  static int res = 0;
  if (res == 0)
    res = resident_blocks_per_cu(reinterpret_cast<const void*>(&decode_attention_kernel<128, kList>), 256);
  const long round_waves = (long)res * device_cu_count() * kAttnWaves;
  const long total = (long)units * std::max(1, max_items);
  int ipw = (int)((total + round_waves - 1) / round_waves);
  ipw = max(1, min(kMaxItemsPerWave, ipw));
  // bound the partials per unit (the combine walks them in PARTS strands)
  while ((max_items + kAttnWaves * ipw - 1) / (kAttnWaves * ipw) > kMaxPartials) ++ipw;
  AttnPlan p;
  p.items_per_wave = ipw;
  p.wg_per_unit = std::max(1, (max_items + kAttnWaves * ipw - 1) / (kAttnWaves * ipw));
  return p;
}

hipError_t launch_attention(AttnMode mode, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream) {
  const unsigned units = (unsigned)(a.batch * a.hkv);
  const dim3 grid(units * (unsigned)plan.wg_per_unit);
#define FSA_ATTN(DD, MM)                                                                              \
  do {                                                                                                \
    hipLaunchKernelGGL((decode_attention_kernel<DD, MM>), grid, dim3(256), 0, stream, a.q, a.kc, a.vc,  \
                       a.page_table, a.seq_lens, a.work, a.part_o, a.part_ml, a.out, a.hq,   \
                       a.hkv, a.max_pages, a.max_items, plan.items_per_wave, plan.wg_per_unit,        \
                       a.scale_log2, a.max_seq_len);                                                   \
    if (plan.wg_per_unit > 1)                                                                         \
      hipLaunchKernelGGL((combine_kernel<DD, MM>), dim3((unsigned)(a.batch * a.hq)), dim3(256), 0,     \
                         stream, a.part_o, a.part_ml, a.seq_lens, a.out, a.hq, a.hkv,        \
                         kAttnWaves * plan.items_per_wave, plan.wg_per_unit, a.max_seq_len);           \
  } while (0)
  if (a.d == 128) {
    if (mode == kDense) FSA_ATTN(128, kDense); else FSA_ATTN(128, kList);
  } else {
    if (mode == kDense) FSA_ATTN(64, kDense); else FSA_ATTN(64, kList);
  }
#undef FSA_ATTN
  return hipGetLastError();
}

}  // namespace fsa
