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
#include <atomic>
#include <mutex>

#include "attend_core.h"
#include "combine_core.h"
#include "score_core.h"
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
  poison_lds(&S, sizeof(S));
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
  const int b = (int)fdiv((uint32_t)unit, A.by_hkv), g = unit - b * A.hkv, G = A.G;
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
  const int b = (int)fdiv((uint32_t)unit, A.by_hkv);
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
// their own slice of the selected pages, in the selection's item order:
// replica r takes selected items [r per, (r + 1) per), at most two per wave.  Running the
// selection redundantly on otherwise idle CUs costs nothing on the critical
// path and spares a launch and a round trip for a work list.  Up to 8 pages
// per thread the query operand is loaded into registers with the selection's
// first loads and a wave attends one page at a time (the registers left
// beside the prefetch words); from 16 pages per thread, where each wave may
// have two pages, the first D/32 waves copy the operand straight into LDS with
// the selection's first loads and both pages are in flight together.
template <int COLS, int D>
__device__ __forceinline__ void select_and_attend(SelectLds& SL, MergeLds<D, kSelWaves>& SM, int4* slice,
                                                  bf16x8_t* q_lds, const StepArgs& A, int unit, int r) {
  const int b = (int)fdiv((uint32_t)unit, A.by_hkv), g = unit - b * A.hkv, G = A.G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the query operand is loaded first, so that waiting for it later does not
  // wait for the selection's prefetch loads (loads complete in order)
  bf16x8_t qb[D / 32];
  constexpr bool kCanPrefetch = COLS <= 8;  // beyond, the early query operand costs registers
  if (kCanPrefetch) load_q_operand<D>(A.q + ((size_t)b * A.hq + (size_t)g * G) * D, G, qb);
  if (!kCanPrefetch && wave < D / 32) {  // k-step `wave` of the operand straight to LDS; padding columns
    // repeat head G - 1 (their results are never written)
    const int col = lane & 15, gq = lane >> 4;
    const uint16_t* src = A.q + ((size_t)b * A.hq + (size_t)g * G + min(col, G - 1)) * D + 32 * wave + 8 * gq;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(q_lds + wave * kWave), 16, 0, 0);
  }
  SelectJob J = step_job(A, unit);
  J.slice = slice;
  J.slice_lo = r * A.per;
  J.slice_cap = A.per;
  if (r != 0) J.sel = nullptr;  // the selected pages, when asked for, are written by replica 0
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
  poison_lds(&SM, sizeof(SM));
  const int n = __popcll(__ballot(my_lo < my_hi));  // a prefix of the wave's lanes
  WaveAttn<D> st;
  if constexpr (kCanPrefetch)
    attend_items<D, false>(A.kc, A.vc, (size_t)g * (kPage * D), (size_t)A.hkv * (kPage * D), qb, my_phys, my_lo,
                           my_hi, n, A.scale_log2, st);
  else
    attend_items<D, true, true>(A.kc, A.vc, (size_t)g * (kPage * D), (size_t)A.hkv * (kPage * D), qb, my_phys,
                                my_lo, my_hi, n, A.scale_log2, st, q_lds);
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
  __shared__ bf16x8_t q_lds[D / 32 * kWave];
  poison_lds(&U, sizeof(U));
  poison_lds(slice, sizeof(slice));
  poison_lds(q_lds, sizeof(q_lds));
  const int units = A.batch * A.hkv;
  const int i = blockIdx.x;
  if (i < A.sel_blocks) {
    if (A.sel_rep > 0) {
      int unit = (int)fdiv((uint32_t)i, A.by_rep), r = i - unit * A.sel_rep;
      if (A.xcd_grouped) {
        const int k = i / kXcds;
        const int kq = (int)fdiv((uint32_t)k, A.by_rep);
        unit = i % kXcds + kXcds * kq;
        r = k - kq * A.sel_rep;
        if (unit >= units) return;
      }
      select_and_attend<COLS, D>(U.sel, U.att, slice, q_lds, A, unit, r);
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
    const int pu = (int)fdiv((uint32_t)w, A.by_pw);
    prefix_window_attend<D>(U.att, A, pu, w - pu * A.pw_wg);
  }
}

// ---------------------------------------------------------------- one-launch step
// The separate launches pay a launch boundary between scoring and selection
// and another before the combine.  The one-launch step runs the whole step as
// tasks of one launch:
//   * each 1024-thread workgroup takes the next task from the queue of the
//     XCD it runs on (the XCC_ID hardware register) and runs it; the grid
//     holds eight times the longest queue (the dispatcher deals workgroups
//     to the XCDs in turn), one workgroup per CU at a time (LDS);
//   * XCD x serves units x, x + 8, ...; its queue holds the scoring tasks of
//     its units (n_score per unit, 16 waves each with a share of the unit's
//     16-page tiles; together at most one per CU of the XCD), then their
//     selection replicas, then their prefix/window tasks;
//   * a scoring task stores its scores, waits until the stores have
//     completed (they are then in the XCD's L2, which every CU of the XCD
//     reads), then adds one to its unit's score counter; a selection replica
//     waits until that counter reaches n_score;
//   * every selection and prefix/window task writes one partial the same way
//     and adds one to its unit's partial counter; the task that brings it to
//     the unit's slot count merges the unit's partials into the output with
//     the combine's arithmetic (combine_core.h), so no combine launch is
//     needed and the output is bit-identical to the separate launches';
//   * every wait is on tasks earlier in the same queue, which were taken by
//     workgroups already running that wait on nothing themselves, so the
//     waits end whatever the order and number of resident workgroups.  One
//     task per workgroup also keeps the roles' per-lane values out of a loop,
//     where the compiler would hoist and spill them;
//   * the counters are device-scope atomics in a slot of library memory (one
//     slot per step in flight); the last workgroup to leave zeroes them for
//     the slot's next step.
// A wait is bounded: after about a second it is counted in the slot's stall
// word (one_launch_stalls) and given up, so a broken assumption shows up as a
// wrong result and a count, never as a hang.  Tasks left in a queue (an XCD
// given fewer workgroups than its queue holds) are counted the same way by
// the last workgroup.
// On MI355X this form measured no faster than the separate launches from 4k
// to 512k tokens (within half a microsecond at the shortest and longest
// lengths, up to 2 us slower in between), so it is off unless asked for: a handoff
// through device memory (stores completed, a device-scope atomic, a poll)
// costs about as much as the launch boundary it replaces, the merge of the
// partials takes about as long as the combine launch, and scoring with each
// unit on one XCD ends later than scoring spread over every XCD, since the
// XCDs stream at different rates.
struct alignas(256) SyncWord {
  uint32_t v;
  uint32_t pad[63];
};
struct SyncSlot {
  SyncWord claim[kXcds];           // tasks taken from each XCD's queue
  SyncWord scored[kOneMaxUnits];   // scoring tasks finished, per unit
  SyncWord arrived[kOneMaxUnits];  // partials written, per unit
  SyncWord finished;               // workgroups of the launch that have left
  SyncWord stalls;                 // waits given up (never reset)
};
// Zero when the library is loaded; every one-launch step leaves its slot zero.
__device__ SyncSlot g_sync[kSyncSlots];

constexpr uint32_t kMaxPolls = 1u << 22;  // ~1 s of polling

__device__ __forceinline__ uint32_t this_xcd() {
  return (uint32_t)__builtin_amdgcn_s_getreg((15 << 11) | 20) & 0xFu;  // HW_REG_XCC_ID, bits 0..15
}
__device__ __forceinline__ uint32_t sync_add(SyncWord& w, uint32_t v) {
  return __hip_atomic_fetch_add(&w.v, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t sync_load(SyncWord& w) {
  return __hip_atomic_load(&w.v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sync_store(SyncWord& w, uint32_t v) {
  __hip_atomic_store(&w.v, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Units x, x + 8, ... below `units` (none for an XCD id the plan does not know).
__device__ __forceinline__ int xcd_units(uint32_t x, int units) {
  return x < (uint32_t)kXcds && (int)x < units ? (units - 1 - (int)x) / kXcds + 1 : 0;
}
// The workgroup's stores have completed (so they are in the XCD's L2) before
// thread 0 adds `v` to `w`; returns the old value to every thread.
__device__ __forceinline__ uint32_t publish(SyncWord& w, uint32_t v, uint32_t* s_word) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) *s_word = sync_add(w, v);
  __syncthreads();
  return *s_word;
}

// The unit's partials merged into its G output rows (combine_core.h): 256
// threads per head, four heads side by side, each thread taking heads grp,
// grp + 4, ... (G <= kOneMaxG) with all of their loads in flight at once.
constexpr int kOneMaxG = 16;
template <int D>
__device__ __forceinline__ void merge_unit(CombineLds<D> (&S)[kOneMaxG], const StepArgs& A, int unit) {
  const int b = (int)fdiv((uint32_t)unit, A.by_hkv), g = unit - b * A.hkv, G = A.G, n = A.slots_per_unit;
  const int grp = threadIdx.x / kCombineThreads, t = threadIdx.x % kCombineThreads;
  constexpr int HPT = kOneMaxG / 4;  // heads per thread, at most
  StrandLoads<D> L[HPT];
#pragma unroll
  for (int i = 0; i < HPT; ++i) {
    const int h = grp + 4 * i;
    const size_t first = (size_t)unit * n * G + h;  // the head's first partial
    if (h < G)
      strand_load<D>(L[i], A.part_ml + 2 * first, reinterpret_cast<const float4*>(A.part_o + first * D), G, n, t);
  }
#pragma unroll
  for (int i = 0; i < HPT; ++i)
    if (grp + 4 * i < G) strand_merge<D>(S[grp + 4 * i], L[i], n, t);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < HPT; ++i) {
    const int h = grp + 4 * i;
    if (h < G && t < CombineLds<D>::NQ)
      combine_write<D>(S[h], t, A.out + ((size_t)b * A.hq + (size_t)g * G + h) * D);
  }
}

template <int COLS, int D>
__global__ __launch_bounds__(kSelThreads) void one_launch_step_kernel(const StepArgs A, const OneLaunchArgs O) {
  __shared__ union {
    SelectLds sel;
    MergeLds<D, kSelWaves> att;
    CombineLds<D> comb[kOneMaxG];
  } U;
  __shared__ int4 slice[kSliceMax];
  __shared__ bf16x8_t q_lds[D / 32 * kWave];
  __shared__ uint32_t s_word;
  poison_lds(&U, sizeof(U));
  poison_lds(slice, sizeof(slice));
  poison_lds(q_lds, sizeof(q_lds));
  SyncSlot& S = *static_cast<SyncSlot*>(O.sync);
  const int wave = threadIdx.x >> 6;
  const uint32_t x = this_xcd();
  const int nu = xcd_units(x, O.units);
  const int n_sc = nu * O.n_score;           // scoring tasks
  const int n_sel = n_sc + nu * A.sel_rep;  // + selection replicas
  const int n_tasks = n_sel + nu * A.pw_wg;  // + prefix/window tasks
  if (threadIdx.x == 0) s_word = nu > 0 ? sync_add(S.claim[x], 1u) : (uint32_t)n_tasks;
  __syncthreads();
  const int t = (int)s_word;
  if (t < n_sc) {
    const int k = (int)fdiv((uint32_t)t, O.by_score), r = t - k * O.n_score;
    const int unit = (int)x + kXcds * k;
    const int b = (int)fdiv((uint32_t)unit, A.by_hkv), g = unit - b * A.hkv;
    const ScoreArgs SA{A.q, O.meta, A.seq_lens, const_cast<float*>(A.scores), A.hq, A.hkv, A.max_pages,
                       A.prefix, A.window, A.max_seq_len, 0, A.G};
    score_wave<D>(SA, unit, b, g, r * kSelWaves + wave, O.n_score * kSelWaves, O.score_tpw);
    publish(S.scored[unit], 1u, &s_word);
  } else if (t < n_tasks) {
    int unit;
    if (t < n_sel) {
      const int k = (int)fdiv((uint32_t)(t - n_sc), A.by_rep), r = t - n_sc - k * A.sel_rep;
      unit = (int)x + kXcds * k;
      if (threadIdx.x == 0) {
        uint32_t polls = 0;
        while (sync_load(S.scored[unit]) < (uint32_t)O.n_score) {
          __builtin_amdgcn_s_sleep(1);
          if (++polls == kMaxPolls) {
            sync_add(S.stalls, 1u);
            break;
          }
        }
      }
      __syncthreads();
      select_and_attend<COLS, D>(U.sel, U.att, slice, q_lds, A, unit, r);
    } else {
      const int w = t - n_sel;
      const int k = (int)fdiv((uint32_t)w, A.by_pw);
      unit = (int)x + kXcds * k;
      prefix_window_attend<D>(U.att, A, unit, w - k * A.pw_wg);
    }
    // the task that writes the unit's last partial merges them all (the
    // partials are in this XCD's L2; this CU has read none of them before)
    if (publish(S.arrived[unit], 1u, &s_word) == (uint32_t)A.slots_per_unit - 1) {
      poison_lds(&U, sizeof(U));
      merge_unit<D>(U.comb, A, unit);
    }
  }
  // Leaving: `finished` counts workgroups in its low 16 bits and tasks run in
  // its high bits.  The last workgroup checks that every task ran (an XCD
  // given fewer workgroups than its queue holds leaves some undone) and zeroes
  // the slot for its next step, one word per thread.
  if (threadIdx.x == 0) {
    const uint32_t add = 1u + (t < n_tasks ? 1u << 16 : 0u);
    const uint32_t now = sync_add(S.finished, add) + add;
    s_word = (now & 0xFFFFu) == gridDim.x ? now >> 16 : 0xFFFFFFFFu;
  }
  __syncthreads();
  const uint32_t ran = s_word;
  if (ran != 0xFFFFFFFFu) {
    const int i = threadIdx.x;
    if (i == 0 && ran != (uint32_t)(O.units * (O.n_score + A.sel_rep + A.pw_wg))) sync_add(S.stalls, 1u);
    if (i < kXcds) sync_store(S.claim[i], 0u);
    if (i < O.units) {
      sync_store(S.scored[i], 0u);
      sync_store(S.arrived[i], 0u);
    }
    if (i == 0) sync_store(S.finished, 0u);
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
  // Not clamped to n_max: when the prefix ends and the window starts on the
  // same page, that page is one prefix item and one window item, so a
  // sequence can need n_pages + 1 items.
  p.max_items = pre + win;
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
  // selected pages per wave; the prefix/window workgroups take the other CUs.
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
  // half of its 4 MiB, and at most 8 pages per selection thread (beyond, the
  // registers go to the keys and the second selected page)
  const long xcd_bytes = (long)((units + kXcds - 1) / kXcds) * p.sel_items * 2 * kPage * head_dim * 2;
  p.prefetch = p.xcd_grouped && xcd_bytes <= (2l << 20) && select_cols(max_seq_len) <= 8;
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

bool plan_one_launch(const StepPlan& p, int units, int head_dim, int G, int prefix, int window, int max_seq_len,
                     int mode, OneLaunchArgs* o) {
  const int cus = device_cu_count();
  if (mode == 0 || p.sel_rep <= 0 || units > kOneMaxUnits || cus != kXcds * 32) return false;
  // the in-launch merge: every head's partials loaded at once
  const int parts = kCombineThreads / (head_dim / 4);
  if (G > kOneMaxG || p.sel_rep + p.pw.wg_per_unit > kStrandMax * parts) return false;
  // automatic: only when every XCD serves as many units as the others (each
  // unit's metadata is streamed by its own XCD)
  if (mode == 1 && units % kXcds != 0) return false;
  // candidate tiles at the host bound (as the scoring wave counts them); the
  // scoring tasks of an XCD take one round of its 32 CUs at most (smaller
  // tasks in more rounds measured slower, and so did scoring spread over all
  // XCDs with the scores passed on through device-scope atomics)
  const int c_lo = std::min(prefix, max_seq_len) / kPage;
  const int c_hi = (std::max(0, max_seq_len - window) + kPage - 1) / kPage;
  const int tiles = std::max(1, (c_hi + kMetaTile - 1) / kMetaTile - c_lo / kMetaTile);
  const int per_xcd = (units + kXcds - 1) / kXcds;
  o->units = units;
  o->n_score = std::max(1, std::min((tiles + kSelWaves - 1) / kSelWaves, 32 / per_xcd));
  o->score_tpw = (tiles + kSelWaves * o->n_score - 1) / (kSelWaves * o->n_score);
  // the kernel counts its workgroups in 16 bits
  if ((long)kXcds * per_xcd * (o->n_score + p.sel_rep + p.pw.wg_per_unit) >= 0x10000) return false;
  o->by_score = make_fastdiv((uint32_t)o->n_score);
  return true;
}

namespace {
constexpr int kMaxSyncDevices = 64;
std::mutex g_sync_mu;
SyncSlot* g_sync_ptr[kMaxSyncDevices] = {};
std::atomic<unsigned> g_sync_next{0};
}  // namespace

hipError_t one_launch_slot(void** slot) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxSyncDevices) return hipErrorInvalidDevice;
  SyncSlot* base = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_sync_mu);
    if (!g_sync_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_sync));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_sync_ptr[dev] = static_cast<SyncSlot*>(p);
    }
    base = g_sync_ptr[dev];
  }
  *slot = base + g_sync_next.fetch_add(1, std::memory_order_relaxed) % kSyncSlots;
  return hipSuccess;
}

hipError_t one_launch_stalls(long long* n) {
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_sync));
  if (e != hipSuccess) return e;
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return e;
  long long sum = 0;
  for (int i = 0; i < kSyncSlots; ++i) {
    uint32_t v = 0;
    e = hipMemcpy(&v, &static_cast<SyncSlot*>(p)[i].stalls.v, sizeof(v), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return e;
    sum += v;
  }
  *n = sum;
  return hipSuccess;
}

hipError_t launch_one_step(const StepArgs& a, const OneLaunchArgs& o, hipStream_t stream) {
  // one task per workgroup: eight times the longest XCD queue
  const int per_xcd = (o.units + kXcds - 1) / kXcds * (o.n_score + a.sel_rep + a.pw_wg);
  const unsigned grid = (unsigned)(kXcds * per_xcd);
#define FSA_ONE(C, DD) \
  hipLaunchKernelGGL((one_launch_step_kernel<C, DD>), dim3(grid), dim3(kSelThreads), 0, stream, a, o)
#define FSA_ONE_D(C)        \
  do {                      \
    if (a.d == 128)         \
      FSA_ONE(C, 128);      \
    else                    \
      FSA_ONE(C, 64);       \
  } while (0)
  switch (select_cols(a.max_seq_len)) {
    case 1: FSA_ONE_D(1); break;
    case 2: FSA_ONE_D(2); break;
    case 4: FSA_ONE_D(4); break;
    case 8: FSA_ONE_D(8); break;
    case 16: FSA_ONE_D(16); break;
    default: FSA_ONE_D(32); break;
  }
#undef FSA_ONE_D
#undef FSA_ONE
  return hipGetLastError();
}

}  // namespace fsa
