// Top-k page selection and merge with the pinned prefix and the window.
//
// The paper (Abstract; analysis page "Methodology"; digest "The Move") keeps
// a fixed budget of query-aware top-k pages next to the prefix and the
// window.  Here, per (sequence, KV head), one workgroup:
//   1. finds the k-th largest score exactly by a most-significant-digit radix
//      select over order-preserving 32-bit keys (8-bit digits, LDS histograms,
//      wave-level scan to locate the digit), stopping early once the digit
//      bucket holds exactly the number still needed;
//   2. compacts the selected pages in ascending id order with two block-wide
//      exclusive scans -- one ranks the pages tied with the threshold so that
//      ties go to the lower page id, one gives each thread its output slot;
//   3. writes the attended tokens as work items.  The attended set is split
//      into three disjoint token ranges -- prefix [0, Pe), the middle tokens
//      [Pe, Ws) of selected pages and the window [max(Ws, Pe), L) -- so no
//      token appears twice and no sort or dedup pass is needed.
#include "fsa_internal.h"

namespace fsa {
namespace {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / kWave;

// Exclusive scan of one int per thread over the block; returns the block total in *total.
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) sh[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int s = sh[w];
    base += (w < wave) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

__device__ __forceinline__ void put_item(int32_t* work, int idx, int p, int phys, int lo, int hi) {
  *reinterpret_cast<int4*>(work + 4 * (size_t)idx) = make_int4(p, phys, lo, hi);
}

__global__ __launch_bounds__(kSelThreads) void select_pages_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, int32_t* __restrict__ sel_pages,
    int32_t* __restrict__ work, int32_t* __restrict__ counts, int32_t* __restrict__ attn_counters,
    int hkv, int max_pages, int prefix, int window, int budget, int max_items, int max_seq_len) {
  __shared__ uint32_t hist[256];
  __shared__ int scan_sh[kSelWaves];
  __shared__ uint32_t s_prefix, s_need, s_done;

  const int unit = blockIdx.x, b = unit / hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int L = min(seq_lens[b], max_seq_len);  // lengths beyond the host bound are clamped
  const int Pe = min(prefix, L), Ws = max(0, L - window);
  const int c_lo = Pe / kPage;
  const int C = (Pe < Ws) ? (Ws + kPage - 1) / kPage - c_lo : 0;
  const int k = min(budget, C);
  const bool take_all = (k == C);
  const float* sc = scores + (size_t)unit * max_pages + c_lo;
  const int32_t* pt = page_table + (size_t)b * max_pages;

  // ---- 1. exact k-th largest key: (prefix of the key, its bit shift, count still needed)
  uint32_t kprefix = 0, need = (uint32_t)k;
  int shift = 0;
  if (!take_all && k > 0) {
    for (int pass = 0; pass < 4; ++pass) {
      shift = 24 - 8 * pass;
      for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < C; i += kSelThreads) {
        const uint32_t key = f32_order_key(sc[i]);
        if (pass == 0 || (key >> (shift + 8)) == kprefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < kWave) {
        // lane l owns digits 255 - 4l .. 252 - 4l (largest first)
        uint32_t c[4], s = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) s += (c[j] = hist[255 - 4 * lane - j]);
        uint32_t incl = s;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const uint32_t y = __shfl_up(incl, off);
          if (lane >= off) incl += y;
        }
        const unsigned long long hit = __ballot(incl >= need);
        const int f = __ffsll((long long)hit) - 1;  // first lane reaching `need`
        if (lane == f) {
          uint32_t cum = incl - s;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (cum + c[j] >= need) {
              const uint32_t digit = 255u - 4u * lane - j;
              s_prefix = (kprefix << 8) | digit;
              s_need = need - cum;
              s_done = (c[j] == need - cum);
              break;
            }
            cum += c[j];
          }
        }
      }
      __syncthreads();
      kprefix = s_prefix;
      need = s_need;
      const bool done = s_done;
      __syncthreads();
      if (done) break;
    }
  }

  // ---- 2. ascending compaction of the selected pages
  const int per = (C + kSelThreads - 1) / kSelThreads;
  const int i0 = min(tid * per, C), i1 = min(i0 + per, C);
  int gt = 0, eq = 0;
  if (take_all) {
    gt = i1 - i0;
  } else if (k > 0) {
    for (int i = i0; i < i1; ++i) {
      const uint32_t kt = f32_order_key(sc[i]) >> shift;
      gt += kt > kprefix;
      eq += kt == kprefix;
    }
  }
  int tot;
  const int eq_before = block_excl_scan(eq, scan_sh, &tot);
  const int nsel = gt + max(0, min((int)need - eq_before, eq));
  const int out0 = block_excl_scan(nsel, scan_sh, &tot);

  const int n_pre = (Pe + kPage - 1) / kPage;
  const int w0 = max(Ws, Pe);
  const int n_win = (L > w0) ? (L + kPage - 1) / kPage - w0 / kPage : 0;
  const int n_items = n_pre + k + n_win;
  int32_t* wrk = work ? work + 4 * (size_t)unit * max_items : nullptr;
  int32_t* sel = sel_pages ? sel_pages + (size_t)unit * budget : nullptr;

  if (nsel > 0) {
    int rank = eq_before, o = out0;
    for (int i = i0; i < i1; ++i) {
      bool take = take_all;
      if (!take_all) {
        const uint32_t kt = f32_order_key(sc[i]) >> shift;
        take = kt > kprefix || (kt == kprefix && rank < (int)need);
        rank += kt == kprefix;
      }
      if (take) {
        const int p = c_lo + i;
        if (sel) sel[o] = p;
        if (wrk)
          put_item(wrk, n_pre + o, p, pt[p], max(p * kPage, Pe) - p * kPage,
                   min(p * kPage + kPage, Ws) - p * kPage);
        ++o;
      }
    }
  }

  // ---- 3. prefix and window items, counters
  if (wrk) {
    for (int i = tid; i < n_pre; i += kSelThreads)
      put_item(wrk, i, i, pt[i], 0, min(kPage, Pe - i * kPage));
    for (int i = tid; i < n_win; i += kSelThreads) {
      const int p = w0 / kPage + i;
      put_item(wrk, n_pre + k + i, p, pt[p], max(p * kPage, w0) - p * kPage,
               min(p * kPage + kPage, L) - p * kPage);
    }
  }
  if (sel)
    for (int i = k + tid; i < budget; i += kSelThreads) sel[i] = -1;
  if (tid == 0) {
    if (counts) {
      counts[2 * unit] = k;
      counts[2 * unit + 1] = n_items;
    }
    if (attn_counters) attn_counters[unit] = 0;
  }
  (void)lane;
}

}  // namespace

hipError_t launch_select_pages(const float* scores, const int32_t* page_table,
                               const int32_t* seq_lens, int32_t* sel_pages, int32_t* work,
                               int32_t* counts, int32_t* attn_counters, int batch, int hkv,
                               int max_pages, int prefix, int window, int budget, int max_items,
                               int max_seq_len, hipStream_t stream) {
  hipLaunchKernelGGL(select_pages_kernel, dim3((unsigned)(batch * hkv)), dim3(kSelThreads), 0,
                     stream, scores, page_table, seq_lens, sel_pages, work, counts, attn_counters,
                     hkv, max_pages, prefix, window, budget, max_items, max_seq_len);
  return hipGetLastError();
}

}  // namespace fsa
