// Top-k page selection (select_core.h), stand-alone and as part of the decode
// step.
//
// Stand-alone: one 1024-thread workgroup per (sequence, KV head) selects and
// writes the full work list (prefix, selected and window items).
//
// In the decode step the selection occupies a CU for a few microseconds and
// needs little memory bandwidth, while the prefix and window pages -- attended
// whatever the selection decides -- are known from the sequence length alone.
// So the selection launch also carries 1024-thread workgroups that attend the
// prefix and window pages on the other CUs (16 waves, each walking a few pages
// with the flash-decoding of attend_core.h, merged through LDS into one
// partial per workgroup).  The selected pages are attended
//   * wide plan: by the selection workgroups themselves -- sel_rep replicas
//     per unit each run the (deterministic) selection and attend their own
//     slice of the selected items; the replicas of a unit share one XCD and
//     may prefetch pages already known to be taken into its L2;
//   * narrow plan: by the split-K attention kernel launched next, from the
//     selected items one selection workgroup per unit writes.
// The combine merges all partials of a unit.
#include <algorithm>

#include "attend_core.h"
#include "select_core.h"

namespace fsa {
namespace {

template <int COLS>
__global__ __launch_bounds__(kSelThreads) void select_pages_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, int32_t* __restrict__ sel_pages,
    int32_t* __restrict__ work, int32_t* __restrict__ counts, int hkv, int max_pages, int prefix,
    int window, int budget, int max_items, int max_seq_len) {
  __shared__ SelectLds S;
  const int unit = blockIdx.x, b = unit / hkv;
  SelectJob J;
  J.scores = scores + (size_t)unit * max_pages;
  J.pt = page_table + (size_t)b * max_pages;
  J.seq_len = seq_lens + b;
  J.pf_kc = nullptr;
  J.max_seq_len = max_seq_len;
  J.prefix = prefix;
  J.window = window;
  J.budget = budget;
  J.max_items = max_items;
  J.work = work ? work + 4 * (size_t)unit * max_items : nullptr;
  J.sel = sel_pages ? sel_pages + (size_t)unit * budget : nullptr;
  J.counts = counts ? counts + 2 * unit : nullptr;
  J.sel_work = nullptr;
  J.sel_items = 0;
  select_unit<COLS>(S, J);
}

// Item i of a unit's prefix/window list for a sequence of length L: prefix
// page i for i < n_pre, else window page w_first + i - n_pre.  Returns false
// (and an empty range) past the end.
__device__ __forceinline__ bool prefix_window_item(int i, int L, int prefix, int window, int& p, int& lo, int& hi) {
  const int Pe = min(prefix, L), Ws = max(0, L - window);
  const int n_pre = (Pe + kPage - 1) / kPage;
  const int w0 = max(Ws, Pe);
  const int w_first = w0 / kPage, n_pages = (L + kPage - 1) / kPage;
  const int n_win = (L > w0) ? n_pages - w_first : 0;
  p = 0;
  lo = hi = 0;
  if (i < 0 || i >= n_pre + n_win) return false;
  if (i < n_pre) {
    p = i;
    hi = min(kPage, Pe - p * kPage);
  } else {
    p = w_first + i - n_pre;
    lo = max(p * kPage, w0) - p * kPage;
    hi = min(p * kPage + kPage, L) - p * kPage;
  }
  return true;
}

// Narrow plan, prefix/window role: attention over the prefix and window pages
// of one unit.  Wave w of workgroup wg takes items (16 wg + w) ipw + [0, ipw).
template <int D>
__device__ __forceinline__ void prefix_window_attend(MergeLds<D, kSelWaves>& S, const StepArgs& A, int unit,
                                                     int wg) {
  const int b = unit / A.hkv, g = unit % A.hkv, G = A.hq / A.hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane < A.pw_ipw ? (wg * kSelWaves + wave) * A.pw_ipw + lane : -1;
  const int32_t* pt = A.page_table + (size_t)b * A.max_pages;
  // The page-table entry is loaded for the item the host-side length bound
  // implies, together with the length itself and q; it is loaded again only
  // where the actual length moves the item to another page.
  int p_guess, lo, hi;
  prefix_window_item(i, A.max_seq_len, A.prefix, A.window, p_guess, lo, hi);
  int my_phys = pt[p_guess];
  bf16x8_t qb[D / 32];
  load_q_operand<D>(A.q + ((size_t)b * A.hq + (size_t)g * G) * D, G, qb);
  const int L = min(A.seq_lens[b], A.max_seq_len);
  int p, my_lo, my_hi;
  prefix_window_item(i, L, A.prefix, A.window, p, my_lo, my_hi);
  if (my_lo < my_hi && p != p_guess) my_phys = pt[p];
  const int n = __popcll(__ballot(my_lo < my_hi));  // a prefix of the wave's lanes
  WaveAttn<D> st;
  attend_items<D, false>(A.kc, A.vc, (size_t)g * (kPage * D), (size_t)A.hkv * (kPage * D), qb, my_phys, my_lo,
                         my_hi, n, A.scale_log2, st);
  const size_t slot = (size_t)unit * A.slots_per_unit + wg;
  merge_waves<D, kSelWaves>(S, st, G, false, nullptr, A.part_o + slot * G * D, A.part_ml + 2 * slot * G);
}

__device__ __forceinline__ SelectJob step_job(const StepArgs& A, int unit) {
  const int b = unit / A.hkv;
  SelectJob J;
  J.scores = A.scores + (size_t)unit * A.max_pages;
  J.pt = A.page_table + (size_t)b * A.max_pages;
  J.seq_len = A.seq_lens + b;
  J.pf_kc = nullptr;
  J.max_seq_len = A.max_seq_len;
  J.prefix = A.prefix;
  J.window = A.window;
  J.budget = A.budget;
  J.max_items = 0;
  J.work = nullptr;
  J.sel = A.sel_pages ? A.sel_pages + (size_t)unit * A.budget : nullptr;
  J.counts = nullptr;
  J.sel_work = nullptr;
  J.sel_items = 0;
  J.slice = nullptr;
  J.slice_lo = J.slice_cap = 0;
  return J;
}

// Wide plan, selection role: the sel_rep workgroups of a unit each run the
// unit's selection (deterministic, so the replicas agree) and then attend
// their own slice of the selected pages, in output-slot order: replica r takes
// selected items [r per, (r + 1) per), at most two per wave.  Running the
// selection redundantly on otherwise idle CUs costs nothing on the critical
// path and spares a launch and a round trip for a work list.
template <int COLS, int D>
__device__ __forceinline__ void select_and_attend(SelectLds& SL, MergeLds<D, kSelWaves>& SM, int4* slice,
                                                  const StepArgs& A, int unit, int r) {
  const int b = unit / A.hkv, g = unit % A.hkv, G = A.hq / A.hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the query operand is loaded first, so that waiting for it later does not
  // wait for the selection's prefetch loads (loads complete in order)
  bf16x8_t qb[D / 32];
  constexpr bool kCanPrefetch = COLS <= 8;  // beyond, the early query operand costs registers
  if (kCanPrefetch) load_q_operand<D>(A.q + ((size_t)b * A.hq + (size_t)g * G) * D, G, qb);
  SelectJob J = step_job(A, unit);
  J.slice = slice;
  J.slice_lo = r * A.per;
  J.slice_cap = A.per;
  if (kCanPrefetch && A.prefetch) {  // the unit's replicas share an L2: each warms its share of the taken pages
    J.pf_kc = A.kc;
    J.pf_vc = A.vc;
    J.pf_head_off = (size_t)g * (kPage * D);
    J.pf_page_stride = (size_t)A.hkv * (kPage * D);
    J.pf_lines = kPage * D * 2 / 128;
    J.pf_rep = A.sel_rep;
    J.pf_r = r;
  }
  const SelectResult R = select_unit<COLS>(SL, J);
  __syncthreads();  // the slice is complete
  const int ipw = (A.per + kSelWaves - 1) / kSelWaves;
  const int local = wave * ipw + lane;
  int my_phys = 0, my_lo = 0, my_hi = 0;
  if (lane < ipw && local < A.per && r * A.per + local < R.k) {
    const int4 it = slice[local];
    my_phys = it.y;
    my_lo = it.z;
    my_hi = it.w;
  }
  __syncthreads();  // every read of the selection's LDS precedes the merge that reuses it
  const int n = __popcll(__ballot(my_lo < my_hi));  // a prefix of the wave's lanes
  if (!kCanPrefetch) load_q_operand<D>(A.q + ((size_t)b * A.hq + (size_t)g * G) * D, G, qb);
  WaveAttn<D> st;
  attend_items<D, false>(A.kc, A.vc, (size_t)g * (kPage * D), (size_t)A.hkv * (kPage * D), qb, my_phys, my_lo,
                         my_hi, n, A.scale_log2, st);
  // the prefetch words are used here, after the attention's own loads
  asm volatile("" ::"v"(R.pf[0]), "v"(R.pf[1]), "v"(R.pf[2]), "v"(R.pf[3]));
  const size_t slot = (size_t)unit * A.slots_per_unit + A.pw_wg + r;
  merge_waves<D, kSelWaves>(SM, st, G, false, nullptr, A.part_o + slot * G * D, A.part_ml + 2 * slot * G);
}

// Workgroups, in launch order: sel_blocks selection workgroups (sel_rep per
// unit in the wide plan, one per unit in the narrow plan), then pw_wg
// prefix/window workgroups per unit.  Workgroup i runs on XCD i % 8 (the
// dispatcher deals workgroups round-robin over the XCDs); when xcd_grouped is
// set, i = 8 (m sel_rep + r) + x is replica r of unit 8 m + x, so all replicas
// of a unit share one XCD's L2: its scores and page-table row are fetched from
// memory once, not once per replica (ids of absent units exit at once).
template <int COLS, int D>
__global__ __launch_bounds__(kSelThreads) void select_attend_kernel(const StepArgs A) {
  __shared__ union {
    SelectLds sel;
    MergeLds<D, kSelWaves> att;
  } U;
  __shared__ int4 slice[kSliceMax];
  const int units = A.batch * A.hkv;
  const int i = blockIdx.x;
  if (i < A.sel_blocks) {
    if (A.sel_rep > 0) {
      int unit = i / A.sel_rep, r = i % A.sel_rep;
      if (A.xcd_grouped) {
        const int k = i / kXcds;
        unit = i % kXcds + kXcds * (k / A.sel_rep);
        r = k % A.sel_rep;
        if (unit >= units) return;
      }
      select_and_attend<COLS, D>(U.sel, U.att, slice, A, unit, r);
    } else {
      // narrow plan: the selected items go to the work list of the split-K
      // attention kernel
      SelectJob J = step_job(A, blockIdx.x);
      J.sel_work = A.sel_work + 4 * (size_t)blockIdx.x * A.sel_items;
      J.sel_items = A.sel_items;
      select_unit<COLS>(U.sel, J);
    }
  } else {
    const int w = i - A.sel_blocks;
    prefix_window_attend<D>(U.att, A, w / A.pw_wg, w % A.pw_wg);
  }
}

}  // namespace

int select_max_candidates() { return kSelMaxPages; }
int select_columns(int max_seq_len) { return select_cols(max_seq_len); }

hipError_t launch_select_pages(const float* scores, const int32_t* page_table,
                               const int32_t* seq_lens, int32_t* sel_pages, int32_t* work,
                               int32_t* counts, int batch, int hkv, int max_pages, int prefix,
                               int window, int budget, int max_items, int max_seq_len,
                               hipStream_t stream) {
#define FSA_SEL(C)                                                                                   \
  hipLaunchKernelGGL(select_pages_kernel<C>, dim3((unsigned)(batch * hkv)), dim3(kSelThreads), 0,   \
                     stream, scores, page_table, seq_lens, sel_pages, work, counts, hkv, max_pages, \
                     prefix, window, budget, max_items, max_seq_len)
  switch (select_cols(max_seq_len)) {
    case 1: FSA_SEL(1); break;
    case 2: FSA_SEL(2); break;
    case 4: FSA_SEL(4); break;
    case 8: FSA_SEL(8); break;
    case 16: FSA_SEL(16); break;
    default: FSA_SEL(32); break;
  }
#undef FSA_SEL
  return hipGetLastError();
}

PwPlan plan_prefix_window(int units, int pw_cus, int prefix, int window, int max_seq_len) {
  const int n_max = (max_seq_len + kPage - 1) / kPage;
  const int pre = std::min((prefix + kPage - 1) / kPage, n_max);
  const int win = std::min((window + kPage - 1) / kPage + 1, n_max);
  PwPlan p;
  p.max_items = std::min(pre + win, n_max);
  if (p.max_items == 0) {
    p.ipw = 1;
    p.wg_per_unit = 0;
    return p;
  }
  // one workgroup per CU at a time (the launch's LDS); pw_cus CUs' worth of workgroups
  const long waves = (long)std::max(1, pw_cus) * kSelWaves;
  const long need = (long)units * p.max_items;
  p.ipw = (int)std::max<long>(1, std::min<long>(kWave, (need + waves - 1) / waves));
  p.wg_per_unit = (p.max_items + kSelWaves * p.ipw - 1) / (kSelWaves * p.ipw);
  return p;
}

StepPlan plan_step(int units, int head_dim, int prefix, int window, int budget, int max_seq_len) {
  const int n_max = (max_seq_len + kPage - 1) / kPage;
  const int cus = device_cu_count();
  StepPlan p;
  p.sel_items = std::max(1, std::min(budget, n_max));
  // Wide when the selection replicas fit on half the CUs with one, else two,
  // selected pages per wave (one page at a time: a two-stage pipeline does not
  // fit beside the selection in 128 registers); the prefix/window workgroups
  // take the other CUs.
  p.sel_rep = 0;
  p.per = 0;
  for (int ipw = 1; ipw <= 2 && p.sel_rep == 0; ++ipw) {
    const int per = ipw * kSelWaves;
    const int rep = (p.sel_items + per - 1) / per;
    if ((long)units * rep <= cus / 2) {
      p.sel_rep = rep;
      p.per = (p.sel_items + rep - 1) / rep;
    }
  }
  const int busy = units * std::max(1, p.sel_rep);
  // Wide plan: the prefix/window workgroups fill the CUs beside the replicas.
  // Narrow plan: two rounds of them over every CU; the first take the
  // CUs beside the selection, the rest the selection's CUs as they free up,
  // so that each wave walks fewer pages (one page in flight per wave).
  p.pw = plan_prefix_window(units, p.sel_rep > 0 ? cus - busy : 2 * cus, prefix, window, max_seq_len);
  // a unit's replicas on one XCD when every XCD's share stays within half its CUs
  const int per_xcd = (units + kXcds - 1) / kXcds * p.sel_rep;
  p.xcd_grouped = p.sel_rep > 0 && per_xcd <= cus / kXcds / 2;
  p.sel_blocks = p.xcd_grouped ? kXcds * per_xcd : busy;
  // prefetch of known-taken pages into the shared L2 while it holds them
  // comfortably: the K and V blocks of one XCD's units' selections within
  // half of its 4 MiB
  const long xcd_bytes = (long)((units + kXcds - 1) / kXcds) * p.sel_items * 2 * kPage * head_dim * 2;
  p.prefetch = p.xcd_grouped && xcd_bytes <= (2l << 20);
  return p;
}

hipError_t launch_select_attend(const StepArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)(a.sel_blocks + a.batch * a.hkv * a.pw_wg);
#define FSA_SA(C, DD) hipLaunchKernelGGL((select_attend_kernel<C, DD>), dim3(grid), dim3(kSelThreads), 0, stream, a)
#define FSA_SA_D(C)         \
  do {                      \
    if (a.d == 128)         \
      FSA_SA(C, 128);       \
    else                    \
      FSA_SA(C, 64);        \
  } while (0)
  switch (select_cols(a.max_seq_len)) {
    case 1: FSA_SA_D(1); break;
    case 2: FSA_SA_D(2); break;
    case 4: FSA_SA_D(4); break;
    case 8: FSA_SA_D(8); break;
    case 16: FSA_SA_D(16); break;
    default: FSA_SA_D(32); break;
  }
#undef FSA_SA_D
#undef FSA_SA
  return hipGetLastError();
}

}  // namespace fsa
