// Exact top-k page selection of one (sequence, KV head) by a 1024-thread
// workgroup, and the merge of the selection with the pinned prefix and the
// sliding window into a work list.  Used by the stand-alone selection kernel
// and by the selection launch of the decode step.
//
// The paper (Abstract; analysis page "Methodology"; digest "The Move") keeps
// a fixed budget of query-aware top-k pages next to the prefix and the
// window.  Steps:
//   1. thread t owns logical pages t, t + 1024, ... below n_max (from the
//      host-side length bound): it loads their scores and page-table entries
//      together with the sequence length (one memory round trip) and turns
//      the scores into order-preserving 32-bit keys kept in registers; the
//      page-table entries are loaded straight into LDS.  On this CU every instruction of the 1024
//      threads costs 16 wave issue slots, so each page is touched by as few
//      instructions as possible;
//   2. the k-th largest candidate key is found exactly by most-significant-
//      digit radix select: digits start right below the bits that the
//      smallest and the largest candidate key share, 10 bits at a time (1024
//      LDS bins, double-buffered so a pass costs two barriers; 10-bit digits
//      conflict less in the LDS atomics than 11-bit ones and still resolve
//      the threshold in two passes at 64k-256k tokens); one wave scans
//      the bins for the digit holding the k-th key, and the search stops once
//      that digit's bin holds exactly the number of keys still needed;
//   3. the taken pages go to the attention (a replica's slice, or the list
//      the split-K launch reads) in (wave, lane, column) order: a lane's
//      own taken count, one wave scan and one barrier place them.  Only when
//      equal keys straddle the threshold is a first barrier and word scan
//      spent on ranking the tied pages (the lower page id wins);
//   4. outputs that must list pages in ascending order (the selected pages,
//      the stand-alone work list) use per-wave ballots of "taken" as
//      page-ordered 64-bit words (page t + 1024 j is bit t % 64 of word
//      16 j + t / 64); every wave scans the words' popcounts itself, so the
//      slot of a taken page is a word prefix plus a popcount within its word.
//      Prefix and window items, whose places depend only on the length and
//      the budget, are written last.
// The attended set is the disjoint union of three token ranges -- prefix
// [0, Pe), the middle tokens [Pe, Ws) of selected pages and the window
// [max(Ws, Pe), L) -- so no token appears twice and no sort or dedup pass is
// needed.  The list is padded with empty items up to its fixed length.
#pragma once

#include "fsa_internal.h"

namespace fsa {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelCols = 32;  // pages per thread: up to 32768 (512k tokens)
constexpr int kSelMaxPages = kSelThreads * kSelCols;
constexpr int kSelDigitBits = 10;
constexpr int kSelBins = 1 << kSelDigitBits;
static_assert(kSelBins / kWave % 8 == 0, "the bin scan sums each lane's bins in pairs of 16-byte reads");

// s_waitcnt immediate for vmcnt(0) with the other counters left alone
constexpr int kWaitVmcnt0 = 0x0F70;

struct SelectLds {
  int32_t sphys[kSelMaxPages];  // page-table entries of pages [0, n_max)
  uint32_t hist[2][kSelBins + kWave];  // bins, then one discard slot per lane
  __attribute__((aligned(16))) uint32_t cnt[2][kSelCols * kSelWaves];  // per-word popcounts
  uint32_t mm[2 * kSelWaves];
  uint32_t wtot[kSelWaves];  // taken pages per wave (items in wave order)
  uint32_t s_prefix, s_need, s_done;
};

// Pages per thread for lengths up to max_seq_len, rounded up to a power of two.
__host__ __device__ inline int select_cols(int max_seq_len) {
  const int n = (max_seq_len + kPage - 1) / kPage;
  int c = 1;
  while (c * kSelThreads < n) c *= 2;
  return c;
}

struct SelectJob {  // every optional field defaults to null / zero
  const float* scores = nullptr;     // the unit's scores, logical page p at [p]
  const int32_t* pt = nullptr;       // the sequence's page-table row
  const int32_t* seq_len = nullptr;  // the sequence's length (device)
  int max_seq_len = 0;
  int prefix = 0, window = 0, budget = 0, max_items = 0;
  int32_t* work = nullptr;    // the unit's work list, or null
  int32_t* sel = nullptr;     // the unit's selected pages, or null
  int32_t* counts = nullptr;  // the unit's (k, items), or null
  int32_t* sel_work = nullptr;  // or null: the selected items alone, (page, pool page, lo, hi) at [o],
  int sel_items = 0;            // padded with empty items up to sel_items
  int4* slice = nullptr;        // or null: selected items [slice_lo, slice_lo + slice_cap), in the
  int slice_lo = 0, slice_cap = 0;  // attention's item order, go to slice[o - slice_lo] (typically LDS)
  // or null: after the first radix pass, pull into L2 the K and V blocks of
  // some pages already known to be taken (this workgroup's share of them)
  const uint16_t* pf_kc = nullptr;
  const uint16_t* pf_vc = nullptr;
  size_t pf_head_off = 0, pf_page_stride = 0;
  int pf_lines = 0;  // 128-byte lines in one page's K block (and in its V block): head_dim / 4
  int pf_rep = 1, pf_r = 0;
};

constexpr int kPrefetch = 4;  // prefetched pages per wave at most

__device__ __forceinline__ void put_item(int32_t* work, int idx, int p, int phys, int lo, int hi) {
  *reinterpret_cast<int4*>(work + 4 * (size_t)idx) = make_int4(p, phys, lo, hi);
}

// Lanes below this one with their bit set in the wave-uniform mask m.
__device__ __forceinline__ uint32_t lanes_below(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Word prefix sums, in page order, of cnt[0 .. nwords) (nwords a multiple of
// 16).  Returns a per-lane value P such that lane 2 j + wave / 8 of P holds the
// sum of the words before word 16 j + wave.
__device__ __forceinline__ uint32_t wave_word_prefix(const uint32_t* cnt, int nwords, int wave, int lane) {
  uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
  if (8 * lane < nwords) {
    a = *reinterpret_cast<const uint4*>(cnt + 8 * lane);
    b = *reinterpret_cast<const uint4*>(cnt + 8 * lane + 4);
  }
  const uint32_t c[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  const uint32_t s = (c[0] + c[1]) + (c[2] + c[3]) + ((c[4] + c[5]) + (c[6] + c[7]));
  uint32_t pre = wave_incl_sum(s) - s;
  const int r = wave & 7;
#pragma unroll
  for (int i = 0; i < 7; ++i) pre += (i < r) ? c[i] : 0u;
  return pre;
}

// Pages already known to be taken (candidates whose shifted key lies above
// the threshold digit, or in it when that digit is taken whole) have their K
// and V blocks requested into L2.  The pages are split over the pf_rep
// workgroups by lane (lane mod pf_rep == pf_r); each such lane offers its first
// known-taken page, and the wave fetches the first kPrefetch pages offered,
// one load instruction per page: one lane per 128-byte line of the page's K
// block and of its V block (D / 4 lines each).  The loaded words are returned so
// that the caller keeps them live (and so waits for them) only where it waits
// for later loads anyway.
template <int COLS>
__device__ __forceinline__ void prefetch_taken(const SelectLds& S, const SelectJob& J, const uint32_t (&key)[COLS],
                                               uint32_t cand, int shift, uint32_t kprefix, bool done, int tid,
                                               int lane, uint32_t (&pf)[kPrefetch]) {
  uint32_t taken = 0;  // bit j: page tid + 1024 j is known to be taken
#pragma unroll
  for (int j = 0; j < COLS; ++j) {
    const uint32_t d = key[j] >> shift;
    taken |= (uint32_t)(d > kprefix || (done && d == kprefix)) << j;
  }
  taken &= cand;
  if (lane % J.pf_rep != J.pf_r) taken = 0;
  const int j0 = taken ? __builtin_ctz(taken) : 0;
  const int phys = S.sphys[tid + kSelThreads * j0];
  unsigned long long m = __ballot(taken != 0);
  // lanes [0, nl) touch the K block's lines, [nl, 2 nl) the V block's, the rest nothing
  const int nl = J.pf_lines;
  const bool toucher = lane < 2 * nl;
  const uint16_t* base = (lane < nl ? J.pf_kc : J.pf_vc) + J.pf_head_off + (size_t)(lane & (nl - 1)) * 64;
#pragma unroll
  for (int i = 0; i < kPrefetch; ++i) {
    if (m) {
      const int pp = __builtin_amdgcn_readlane(phys, __builtin_ctzll(m));
      m &= m - 1;
      if (toucher) pf[i] = *reinterpret_cast<const uint32_t*>(base + (size_t)pp * J.pf_page_stride);
    }
  }
}

// COLS: pages per thread, a power of two with 1024 COLS >= ceil(max_seq_len / 16)
// (a compile-time trip count: the per-page loops carry no guards).
// What the selection leaves its caller: k, the number of selected pages, and
// L, the sequence length (clamped to the host bound).
struct SelectResult {
  int k, L;
  uint32_t pf[kPrefetch];  // words loaded by the prefetch (keep live until later loads are waited for)
};

// After the call, S.sphys[p] holds page_table[b][p] for p < n_max.
template <int COLS>
__device__ __forceinline__ SelectResult select_unit(SelectLds& S, const SelectJob& J) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_max = (J.max_seq_len + kPage - 1) / kPage;  // pages any sequence can have

  // ---- 1. scores, page-table entries and the length in one round trip
  // (page-table entries go straight to LDS: sphys[tid + 1024 j])
  const int L_in = *J.seq_len;
  uint32_t key[COLS];
#pragma unroll
  for (int j = 0; j < COLS; ++j) {
    const uint32_t off = 4u * (uint32_t)min(tid + kSelThreads * j, n_max - 1);  // byte offset: base + 32-bit VGPR
    key[j] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(J.scores) + off);
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(reinterpret_cast<const char*>(J.pt) + off),
        (__attribute__((address_space(3))) void*)(S.sphys + kSelThreads * j + kWave * wave), 4, 0, 0);
  }
  // Every load is issued before anything waits for one: while loads into LDS
  // are pending the compiler can only wait for all loads, so a key used
  // between two of them would cost a second round trip.
  __builtin_amdgcn_sched_barrier(0);
  // One explicit wait for all of it, on every path, so that the compiler
  // knows no load into LDS is pending afterwards and adds no waits before
  // later LDS accesses (which would also wait for the prefetch below).
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  const int L = min(L_in, J.max_seq_len);  // lengths beyond the host bound are clamped
  const int Pe = min(J.prefix, L), Ws = max(0, L - J.window);
  const int c_lo = Pe / kPage;
  const int c_hi = (Pe < Ws) ? (Ws + kPage - 1) / kPage : c_lo;  // candidates: pages [c_lo, c_hi)
  const int C = c_hi - c_lo;
  const int k = min(J.budget, C);
  const bool radix = k > 0 && k < C;  // otherwise every candidate is taken (k = C) or none is
  const int n_pre = (Pe + kPage - 1) / kPage;
  const int w0 = max(Ws, Pe);
  const int w_first = w0 / kPage, n_pages = (L + kPage - 1) / kPage;
  const int n_win = (L > w0) ? n_pages - w_first : 0;
  const int n_items = n_pre + k + n_win;

  uint32_t cand = 0;  // bit j: page tid + 1024 j is a candidate
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < COLS; ++j) {
    const bool c = (uint32_t)(tid + kSelThreads * j - c_lo) < (uint32_t)C;
    cand |= (uint32_t)c << j;
    key[j] = f32_order_key(__uint_as_float(key[j]));
    kmin = c ? min(kmin, key[j]) : kmin;
    kmax = c ? max(kmax, key[j]) : kmax;
  }

  // ---- 2. exact k-th largest key: keys >> shift compared with kprefix, `need` ties to take
  uint32_t kprefix = 0, need = 0;
  int shift = 0;
  uint32_t pf[kPrefetch] = {0u, 0u, 0u, 0u};
  bool done = false;  // the threshold's bin holds exactly the keys still needed
  if (radix) {
    need = (uint32_t)k;
    for (int i = tid; i < kSelBins; i += kSelThreads) S.hist[0][i] = 0;
    kmin = wave_min(kmin);
    kmax = wave_max(kmax);
    if (lane == 0) {
      S.mm[2 * wave] = kmin;
      S.mm[2 * wave + 1] = kmax;
    }
    __syncthreads();
    const uint32_t gmin = wave_min(lane < kSelWaves ? S.mm[2 * lane] : 0xFFFFFFFFu);
    const uint32_t gmax = wave_max(lane < kSelWaves ? S.mm[2 * lane + 1] : 0u);
    if (gmin == gmax) {
      kprefix = gmin;  // every candidate ties: the lowest ids win
    } else {
      int top = 31 - __clz(gmin ^ gmax);                 // highest bit where candidates differ
      kprefix = (uint32_t)((uint64_t)gmax >> (top + 1));  // shared by every candidate
      for (int pass = 0;; ++pass) {
        uint32_t* h = S.hist[pass & 1];
        uint32_t* h_next = S.hist[(pass + 1) & 1];
        const int width = min(kSelDigitBits, top + 1);
        shift = top + 1 - width;
        const uint32_t above = shift + width;  // <= 32: the bits above the digit
#pragma unroll
        for (int j = 0; j < COLS; ++j) {
          // bit-field extracts: the key's bits above the digit (none when
          // above == 32) and the digit itself, one instruction each
          const uint32_t hi = __builtin_amdgcn_ubfe(key[j], above, 32u - above);
          const uint32_t digit = __builtin_amdgcn_ubfe(key[j], (uint32_t)shift, (uint32_t)width);
          // every lane adds: pages outside the digit's range go to the lane's discard
          // slot, so the loop has no per-page branch
          const bool in = ((cand >> j) & 1u) && hi == kprefix;
          atomicAdd(&h[in ? digit : kSelBins + lane], 1u);
        }
        for (int i = tid; i < kSelBins; i += kSelThreads) h_next[i] = 0;  // for the next pass
        __syncthreads();
        if (wave == 0) {
          // lane l owns the PER_LANE digits below kSelBins - PER_LANE l (largest first)
          constexpr int PER_LANE = kSelBins / kWave;
          const uint4* hv = reinterpret_cast<const uint4*>(h + kSelBins - PER_LANE * (lane + 1));
          uint32_t part[PER_LANE / 4];
#pragma unroll
          for (int v = 0; v < PER_LANE / 4; ++v) {
            const uint4 x = hv[v];
            part[v] = (x.x + x.y) + (x.z + x.w);
          }
          uint32_t s = 0;
#pragma unroll
          for (int v = 0; v < PER_LANE / 4; v += 2) s += part[v] + part[v + 1];
          const uint32_t incl = wave_incl_sum(s);
          const int f = __ffsll((long long)__ballot(incl >= need)) - 1;  // first lane reaching `need`
          const uint32_t before = (uint32_t)__builtin_amdgcn_readlane((int)(incl - s), f);
          // the wave scans lane f's PER_LANE digits (the lanes from PER_LANE on carry zeros)
          const uint32_t digit = (uint32_t)(kSelBins - 1 - PER_LANE * f - (lane & (PER_LANE - 1)));
          const uint32_t c = (lane < PER_LANE) ? h[digit] : 0u;
          const uint32_t ic = wave_incl_sum(c);
          const unsigned long long hit = __ballot(lane < PER_LANE && before + ic >= need);
          if (lane == __ffsll((long long)hit) - 1) {
            const uint32_t cum = before + ic - c;
            S.s_prefix = (kprefix << width) | digit;
            S.s_need = need - cum;
            S.s_done = (c == need - cum);
          }
        }
        __syncthreads();
        kprefix = S.s_prefix;
        need = S.s_need;
        done = S.s_done;
        if (pass == 0 && J.pf_kc) {
          prefetch_taken<COLS>(S, J, key, cand, shift, kprefix, done, tid, lane, pf);
        }
        if (done || shift == 0) break;
        top = shift - 1;
      }
    }
  }

  // ---- 3. taken pages: bit j of `mine` marks page tid + 1024 j
  constexpr int nwords = COLS * kSelWaves;
  uint32_t tie_take = 0;  // bit j: this lane's tied page of column j is taken
  if (radix && !done) {
    // equal keys straddle the threshold: rank the tied pages in page order
    uint32_t wc = 0;  // lane j: tied pages of column j in this wave
#pragma unroll
    for (int j = 0; j < COLS; ++j) {
      const unsigned long long ge = __ballot(((cand >> j) & 1u) && (key[j] >> shift) == kprefix);
      wc = lane == j ? (uint32_t)__popcll(ge) : wc;
    }
    if (lane < COLS) S.cnt[0][lane * kSelWaves + wave] = wc;
    __syncthreads();
    const uint32_t P = wave_word_prefix(S.cnt[0], nwords, wave, lane);
#pragma unroll
    for (int j = 0; j < COLS; ++j) {
      const bool tied = ((cand >> j) & 1u) && (key[j] >> shift) == kprefix;
      const unsigned long long ge = __ballot(tied);
      const uint32_t rank = (uint32_t)__builtin_amdgcn_readlane((int)P, 2 * j + (wave >> 3)) + lanes_below(ge);
      tie_take |= (uint32_t)(tied && rank < need) << j;
    }
  }
  // one uniform branch, then a lean per-page test
  uint32_t mine = 0;
  if (!radix) {
    mine = k == C ? cand : 0u;
  } else if (done) {  // the threshold digit's bin is taken whole
#pragma unroll
    for (int j = 0; j < COLS; ++j) mine |= (uint32_t)((key[j] >> shift) >= kprefix) << j;
    mine &= cand;
  } else {  // keys above the threshold, and the tied pages ranked in
#pragma unroll
    for (int j = 0; j < COLS; ++j) mine |= (uint32_t)((key[j] >> shift) > kprefix) << j;
    mine = (mine | tie_take) & cand;
  }

  // ---- 4. items for the attention (a slice of them, or the selected-item
  // list of the split-K launch) in (wave, lane, column) order.  Any fixed
  // order serves the attention, and this one needs only the lane's own
  // taken count, one wave scan and one barrier: item o of lane l of wave w
  // is its i-th taken page, o = (taken pages of waves < w) + (of lanes < l
  // in w) + i.  Page order (step 5) costs a ballot per column.
  const int e_lo = J.slice ? J.slice_lo : 0;  // items this call emits: the slice's, or all
  const int e_hi = J.slice ? J.slice_lo + J.slice_cap : 0x7FFFFFFF;
  if (J.slice || J.sel_work) {
    const uint32_t cnt = (uint32_t)__popc(mine);
    const uint32_t incl = wave_incl_sum(cnt);
    if (lane == kWave - 1) S.wtot[wave] = incl;
    __syncthreads();
    const uint32_t wt = lane < kSelWaves ? S.wtot[lane] : 0u;
    const int base = __builtin_amdgcn_readlane((int)(wave_incl_sum(wt) - wt), wave);
    int o = base + (int)(incl - cnt);
    uint32_t m = mine;
    while (m) {
      const int j = __builtin_ctz(m);
      m &= m - 1;
      if (o >= e_lo && o < e_hi) {
        const int p = tid + kSelThreads * j;
        const int lo = max(p * kPage, Pe) - p * kPage, hi = min(p * kPage + kPage, Ws) - p * kPage;
        const int phys = S.sphys[p];
        if (J.slice) J.slice[o - e_lo] = make_int4(p, phys, lo, hi);
        if (J.sel_work) put_item(J.sel_work, o, p, phys, lo, hi);
      }
      ++o;
    }
  }

  // ---- 5. outputs in page order (the selected pages, the stand-alone work
  // list): per-wave ballot words in page order, every wave scanning the
  // words' popcounts itself, so the slot of a taken page is a word prefix
  // plus a popcount within its word
  if (J.sel || J.work) {
    uint32_t wc = 0;
#pragma unroll
    for (int j = 0; j < COLS; ++j) {
      const unsigned long long g = __ballot((mine >> j) & 1u);
      wc = lane == j ? (uint32_t)__popcll(g) : wc;
    }
    if (lane < COLS) S.cnt[1][lane * kSelWaves + wave] = wc;
    __syncthreads();
    const uint32_t P = wave_word_prefix(S.cnt[1], nwords, wave, lane);
    int32_t* selw = J.work ? J.work + 4 * n_pre : nullptr;  // item o of the selection
#pragma unroll
    for (int j = 0; j < COLS; ++j) {
      const bool t = (mine >> j) & 1u;
      const unsigned long long g = __ballot(t);
      // read the word prefix with every lane active: a lane read inside the
      // branch below may be inactive and hold no defined value
      const int base = __builtin_amdgcn_readlane((int)P, 2 * j + (wave >> 3));
      if (t) {
        const int p = tid + kSelThreads * j;
        const int o = base + (int)lanes_below(g);
        if (J.sel) J.sel[o] = p;
        if (selw) {
          const int lo = max(p * kPage, Pe) - p * kPage, hi = min(p * kPage + kPage, Ws) - p * kPage;
          put_item(selw, o, p, S.sphys[p], lo, hi);
        }
      }
    }
  }
  // Stores come last: on this target every load wait also waits for earlier stores.
  if (J.sel)
    for (int i = k + tid; i < J.budget; i += kSelThreads) J.sel[i] = -1;
  if (tid == 0 && J.counts) {
    J.counts[0] = k;
    J.counts[1] = n_items;
  }
  if (J.sel_work)
    for (int i = k + tid; i < J.sel_items; i += kSelThreads) put_item(J.sel_work, i, -1, 0, 0, 0);
  if (J.work) {
    for (int i = n_items + tid; i < J.max_items; i += kSelThreads) put_item(J.work, i, -1, 0, 0, 0);
    for (int i = tid; i < n_pre; i += kSelThreads) put_item(J.work, i, i, S.sphys[i], 0, min(kPage, Pe - i * kPage));
    for (int i = tid; i < n_win; i += kSelThreads) {
      const int p = w_first + i;
      put_item(J.work, n_pre + k + i, p, S.sphys[p], max(p * kPage, w0) - p * kPage,
               min(p * kPage + kPage, L) - p * kPage);
    }
  }
  return SelectResult{k, L, {pf[0], pf[1], pf[2], pf[3]}};
}

}  // namespace fsa
