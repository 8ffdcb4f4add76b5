// Top-k page selection (select_core.h), stand-alone and as part of the decode
// step.
//
// Stand-alone: one 1024-thread workgroup per (sequence, KV head) selects and
// writes the full work list (prefix, selected and window items).
//
// In the decode step the selection occupies one CU per (sequence, KV head)
// for a few microseconds and needs little memory bandwidth, while the prefix
// and window pages -- attended whatever the selection decides -- are known
// from the sequence length alone.  So the same launch carries further
// 1024-thread workgroups that attend the prefix and window pages on the other
// CUs (16 waves, each walking a few pages with the flash-decoding of
// attend_core.h, merged through LDS into one partial per workgroup).  The
// selection then writes only the selected items, which the split-K attention
// kernel attends next; the combine merges both kinds of partials.
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
  J.minmax = nullptr;
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

// Prefix and window pages of a sequence of length L.
__device__ __forceinline__ int prefix_window_count(int L, int prefix, int window) {
  const int Pe = min(prefix, L), Ws = max(0, L - window);
  const int w0 = max(Ws, Pe);
  const int n_win = (L > w0) ? (L + kPage - 1) / kPage - w0 / kPage : 0;
  return (Pe + kPage - 1) / kPage + n_win;
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
  J.minmax = nullptr;
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
  J.slice_after_pw = false;
  return J;
}

// Wide plan: the sel_rep workgroups of a unit share out the unit's item list
// -- its prefix pages, its window pages, then its selected pages in output-slot
// order -- workgroup r taking items [r per, (r + 1) per).  A workgroup whose
// items are all prefix or window pages attends them at once, its loads
// overlapping the selection of the others; every other workgroup runs the
// unit's selection (deterministic, so the replicas agree) and then attends its
// share.  Running the selection redundantly on otherwise idle CUs costs
// nothing on the critical path and spares a launch and a round trip for a work
// list.  Whether a workgroup needs the selection is decided from the host-side
// length bound; a shorter sequence only moves work between the two kinds.
template <int COLS, int D>
__device__ __forceinline__ void select_and_attend(SelectLds& SL, MergeLds<D, kSelWaves>& SM, int4* slice,
                                                  const StepArgs& A, int unit, int r) {
  const int b = unit / A.hkv, g = unit % A.hkv, G = A.hq / A.hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ipw = (A.per + kSelWaves - 1) / kSelWaves;
  const int local = wave * ipw + lane;
  const int i = (lane < ipw && local < A.per) ? r * A.per + local : -1;
  const int32_t* pt = A.page_table + (size_t)b * A.max_pages;
  int my_phys = 0, my_lo = 0, my_hi = 0;
  int p, lo, hi;
  const int n_pw_h = prefix_window_count(A.max_seq_len, A.prefix, A.window);
  bool done = false;
  if ((r + 1) * A.per <= n_pw_h) {
    // prefix/window items only (by the host bound): page-table entries are
    // loaded for the bound's items together with the length
    int p_guess;
    prefix_window_item(i, A.max_seq_len, A.prefix, A.window, p_guess, lo, hi);
    my_phys = pt[p_guess];
    const int L = min(A.seq_lens[b], A.max_seq_len);
    if ((r + 1) * A.per <= prefix_window_count(L, A.prefix, A.window)) {
      prefix_window_item(i, L, A.prefix, A.window, p, my_lo, my_hi);
      if (my_lo < my_hi && p != p_guess) my_phys = pt[p];
      done = true;
    }
  }
  if (!done) {
    SelectJob J = step_job(A, unit);
    // the last replica always selects (its items reach past every prefix and
    // window page): it reports the selected pages
    if (r != A.sel_rep - 1) J.sel = nullptr;
    J.slice = slice;
    J.slice_lo = r * A.per;
    J.slice_cap = A.per;
    J.slice_after_pw = true;
    const SelectResult R = select_unit<COLS>(SL, J);
    __syncthreads();  // the slice is complete
    my_phys = my_lo = my_hi = 0;
    const int n_pw = prefix_window_count(R.L, A.prefix, A.window);
    if (i >= 0 && i < n_pw + R.k) {
      if (i >= n_pw) {
        const int4 it = slice[local];
        my_phys = it.y;
        my_lo = it.z;
        my_hi = it.w;
      } else if (prefix_window_item(i, R.L, A.prefix, A.window, p, my_lo, my_hi)) {
        my_phys = SL.sphys[p];
      }
    }
    __syncthreads();  // every read of the selection's LDS precedes the merge that reuses it
  }
  const int n = __popcll(__ballot(my_lo < my_hi));  // a prefix of the wave's lanes
  bf16x8_t qb[D / 32];
  load_q_operand<D>(A.q + ((size_t)b * A.hq + (size_t)g * G) * D, G, qb);
  WaveAttn<D> st;
  attend_items<D, false>(A.kc, A.vc, (size_t)g * (kPage * D), (size_t)A.hkv * (kPage * D), qb, my_phys, my_lo,
                         my_hi, n, A.scale_log2, st);
  const size_t slot = (size_t)unit * A.slots_per_unit + r;
  merge_waves<D, kSelWaves>(SM, st, G, false, nullptr, A.part_o + slot * G * D, A.part_ml + 2 * slot * G);
}

template <int COLS, int D>
__global__ __launch_bounds__(kSelThreads) void select_attend_kernel(const StepArgs A) {
  __shared__ union {
    SelectLds sel;
    MergeLds<D, kSelWaves> att;
  } U;
  __shared__ int4 slice[kSliceMax];
  const int units = A.batch * A.hkv;
  if (A.sel_rep > 0) {
    select_and_attend<COLS, D>(U.sel, U.att, slice, A, blockIdx.x / A.sel_rep, blockIdx.x % A.sel_rep);
  } else if ((int)blockIdx.x < units) {
    // narrow plan, selection role: the selected items go to the work list of
    // the split-K attention kernel
    SelectJob J = step_job(A, blockIdx.x);
    J.sel_work = A.sel_work + 4 * (size_t)blockIdx.x * A.sel_items;
    J.sel_items = A.sel_items;
    select_unit<COLS>(U.sel, J);
  } else {
    const int w = blockIdx.x - units;
    prefix_window_attend<D>(U.att, A, w / A.pw_wg, w % A.pw_wg);
  }
}

}  // namespace

int select_max_candidates() { return kSelMaxPages; }

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

PwPlan plan_prefix_window(int units, int busy_cus, int prefix, int window, int max_seq_len) {
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
  // one workgroup per CU (the launch's LDS), on the CUs beside the selection's
  const long waves = (long)std::max(1, device_cu_count() - busy_cus) * kSelWaves;
  const long need = (long)units * p.max_items;
  p.ipw = (int)std::max<long>(1, std::min<long>(kWave, (need + waves - 1) / waves));
  p.wg_per_unit = (p.max_items + kSelWaves * p.ipw - 1) / (kSelWaves * p.ipw);
  return p;
}

StepPlan plan_step(int units, int prefix, int window, int budget, int max_seq_len) {
  const int n_max = (max_seq_len + kPage - 1) / kPage;
  const int pre = std::min((prefix + kPage - 1) / kPage, n_max);
  const int win = std::min((window + kPage - 1) / kPage + 1, n_max);
  StepPlan p;
  p.sel_items = std::max(1, std::min(budget, n_max));
  // wide: one selection replica per CU, each attending at most 2 items per wave
  // (one page at a time: a two-stage pipeline does not fit beside the
  // selection in 128 registers, and a third page costs more than the
  // narrow plan's extra launch)
  const int rep = device_cu_count() / std::max(1, units);
  const int items = p.sel_items + pre + win;
  if (rep >= 1) {
    const int per = (items + rep - 1) / rep;
    if (per <= 2 * kSelWaves && per <= kSliceMax) {
      p.sel_rep = rep;
      p.per = per;
      p.pw = PwPlan{0, 1, 0};
      return p;
    }
  }
  p.sel_rep = 0;
  p.per = 0;
  p.pw = plan_prefix_window(units, units, prefix, window, max_seq_len);
  return p;
}

hipError_t launch_select_attend(const StepArgs& a, hipStream_t stream) {
  const unsigned grid =
      (unsigned)(a.batch * a.hkv * (a.sel_rep > 0 ? a.sel_rep : 1 + a.pw_wg));
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
