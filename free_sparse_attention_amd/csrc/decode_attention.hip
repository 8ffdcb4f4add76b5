// Split-K flash decoding over attended pages, then the cross-split combine.
//
// Each wave walks a run of items (one page, a token range inside it) with the
// per-wave flash-decoding of attend_core.h, the next page's loads in flight
// while the current page is computed.  Items come either from a work list
// (kList: the selected pages) or are every page of the sequence (kDense, the
// dense baseline).  Four waves per workgroup; the workgroup merges its waves'
// (max, sum, accumulator) through LDS and writes one partial into its slot, or
// the output directly when the unit has a single slot.  The combine kernel
// merges a unit's partials:
//   o = sum_j 2^(m_j - m) o_j / sum_j 2^(m_j - m) l_j,  m = max_j m_j.
// A unit's slots may also hold partials written by other kernels of the step
// (the prefix and window attention beside the selection): slots_per_unit
// counts them all, and this kernel's workgroups start at slot_base.
#include <algorithm>
#include <atomic>

#include "attend_core.h"
#include "combine_core.h"

namespace fsa {
namespace {

constexpr int kAttnWaves = 4;
constexpr int kMaxItemsPerWave = 64;

template <int D, int MODE>
__global__ __launch_bounds__(256, 3) void decode_attention_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ work,
    float* __restrict__ part_o, float* __restrict__ part_ml,
    uint16_t* __restrict__ out, int hq, int hkv, int max_pages, int max_items, int ipw,
    int wg_per_unit, int slots_per_unit, int slot_base, float scale_log2, int max_seq_len, FastDiv by_wg,
    FastDiv by_hkv, int G) {
  __shared__ MergeLds<D, kAttnWaves> S;
  poison_lds(&S, sizeof(S));

  const int unit = (int)fdiv(blockIdx.x, by_wg), wg = (int)blockIdx.x - unit * wg_per_unit;
  const int b = (int)fdiv((uint32_t)unit, by_hkv), g = unit - b * hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int per_wg = kAttnWaves * ipw;
  const int i_begin = wg * per_wg + wave * ipw;

  // item descriptors of this wave: lane j holds item i_begin + j.  Dense items
  // are the sequence's pages.  A work list is padded with empty items (lo = hi)
  // to max_items, so its entries are read without first loading the item
  // count; the valid items of a wave are a prefix of its lanes.
  int my_phys = 0, my_lo = 0, my_hi = 0, n;
  bool direct;
  if (MODE == kDense) {
    const int L = min(seq_lens[b], max_seq_len);  // lengths beyond the host bound are clamped
    const int n_items = (L + kPage - 1) / kPage;
    const int n_wg = (n_items + per_wg - 1) / per_wg;
    if (wg >= n_wg) return;
    direct = n_wg == 1;
    n = max(0, min(ipw, n_items - i_begin));
    if (lane < n) {
      const int i = i_begin + lane;
      my_phys = page_table[(size_t)b * max_pages + i];
      my_hi = min(kPage, L - i * kPage);
    }
  } else {
    direct = slots_per_unit == 1;
    if (lane < ipw && i_begin + lane < max_items) {
      const int4 it = *reinterpret_cast<const int4*>(work + 4 * ((size_t)unit * max_items + i_begin + lane));
      my_phys = it.y;
      my_lo = it.z;
      my_hi = it.w;
    }
    n = __popcll(__ballot(my_lo < my_hi));
  }

  bf16x8_t qb[D / 32];
  load_q_operand<D>(q + ((size_t)b * hq + (size_t)g * G) * D, G, qb);
  WaveAttn<D> st;
  attend_items<D, true>(kc, vc, (size_t)g * (kPage * D), (size_t)hkv * (kPage * D), qb, my_phys, my_lo, my_hi, n,
                        scale_log2, st);
  const size_t slot = (size_t)unit * slots_per_unit + slot_base + wg;
  merge_waves<D, kAttnWaves>(S, st, G, direct, out + ((size_t)b * hq + (size_t)g * G) * D, part_o + slot * G * D,
                             part_ml + 2 * slot * G);
}

// The combine of the decode step: one 256-thread workgroup per (unit, query
// head) merges the unit's partials (combine_core.h); for the dense baseline,
// units whose attention fitted one workgroup were written directly and are
// skipped.
template <int D, int MODE>
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ seq_lens, uint16_t* __restrict__ out, int hq, int hkv, int per_wg, int slots_per_unit,
    int max_seq_len, FastDiv by_g, FastDiv by_hkv) {
  __shared__ CombineLds<D> S;
  poison_lds(&S, sizeof(S));
  const int G = (int)by_g.d;
  const int unit = (int)fdiv(blockIdx.x, by_g), h = (int)blockIdx.x - unit * G;
  const int b = (int)fdiv((uint32_t)unit, by_hkv), g = unit - b * hkv;
  // partial slots in use: all of them for the decode step's partials (empty
  // ones carry m = -inf); dense units use as many as their length needs
  int n = slots_per_unit;
  if (MODE == kDense) {
    const int L = min(seq_lens[b], max_seq_len);
    n = ((L + kPage - 1) / kPage + per_wg - 1) / per_wg;
  }
  if (MODE == kDense && n <= 1) return;  // written directly by the attention kernel
  const size_t first = (size_t)unit * slots_per_unit * G + h;  // the head's first partial
  const float* ml = part_ml + 2 * first;
  const float4* po = reinterpret_cast<const float4*>(part_o + first * D);
  if (n <= kStrandMax * CombineLds<D>::PARTS) {  // all loads in flight at once
    StrandLoads<D> L;
    strand_load<D>(L, ml, po, G, n, (int)threadIdx.x);
    strand_merge<D>(S, L, n, (int)threadIdx.x);
  } else {
    combine_strands<D>(S, ml, po, G, n, (int)threadIdx.x);
  }
  __syncthreads();
  if ((int)threadIdx.x < CombineLds<D>::NQ)
    combine_write<D>(S, (int)threadIdx.x, out + ((size_t)b * hq + (size_t)g * G + h) * D);
}

}  // namespace

AttnPlan plan_attention(int units, int max_items) {
  // one resident round of waves (3 workgroups of 4 waves per CU) shared out
  // over all items; longer runs per wave when there is more work
  static std::atomic<int> cached{0};
  int res = cached.load(std::memory_order_relaxed);
  if (res == 0) {
    res = resident_blocks_per_cu(reinterpret_cast<const void*>(&decode_attention_kernel<128, kList>), 256);
    cached.store(res, std::memory_order_relaxed);
  }
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

hipError_t launch_combine(const AttnArgs& a, int slots, hipStream_t stream) {
  if (a.d == 128)
    hipLaunchKernelGGL((combine_kernel<128, kList>), dim3((unsigned)(a.batch * a.hq)), dim3(256), 0, stream, a.part_o,
                       a.part_ml, a.seq_lens, a.out, a.hq, a.hkv, 1, slots, a.max_seq_len,
                       make_fastdiv((uint32_t)(a.hq / a.hkv)), make_fastdiv((uint32_t)a.hkv));
  else
    hipLaunchKernelGGL((combine_kernel<64, kList>), dim3((unsigned)(a.batch * a.hq)), dim3(256), 0, stream, a.part_o,
                       a.part_ml, a.seq_lens, a.out, a.hq, a.hkv, 1, slots, a.max_seq_len,
                       make_fastdiv((uint32_t)(a.hq / a.hkv)), make_fastdiv((uint32_t)a.hkv));
  return hipGetLastError();
}

hipError_t launch_attention(AttnMode mode, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream,
                            LaunchFilter* filter) {
  const unsigned units = (unsigned)(a.batch * a.hkv);
  const dim3 grid(units * (unsigned)plan.wg_per_unit);
  const int slots = a.slots_per_unit > 0 ? a.slots_per_unit : plan.wg_per_unit;
  const int base = a.slots_per_unit > 0 ? a.slot_base : 0;
#define FSA_ATTN(DD, MM)                                                                                  \
  do {                                                                                                    \
    if (!filter || filter->take())                                                                        \
      hipLaunchKernelGGL((decode_attention_kernel<DD, MM>), grid, dim3(256), 0, stream, a.q, a.kc, a.vc, \
                         a.page_table, a.seq_lens, a.work, a.part_o, a.part_ml, a.out, a.hq, a.hkv,       \
                         a.max_pages, a.max_items, plan.items_per_wave, plan.wg_per_unit, slots, base,    \
                         a.scale_log2, a.max_seq_len, make_fastdiv((uint32_t)plan.wg_per_unit),            \
                         make_fastdiv((uint32_t)a.hkv), a.hq / a.hkv);                                    \
    if (slots > 1 && (!filter || filter->take()))                                                         \
      hipLaunchKernelGGL((combine_kernel<DD, MM>), dim3((unsigned)(a.batch * a.hq)), dim3(256), 0, stream, \
                         a.part_o, a.part_ml, a.seq_lens, a.out, a.hq, a.hkv,                             \
                         kAttnWaves * plan.items_per_wave, slots, a.max_seq_len,                          \
                         make_fastdiv((uint32_t)(a.hq / a.hkv)), make_fastdiv((uint32_t)a.hkv));          \
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
