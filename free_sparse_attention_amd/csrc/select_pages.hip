// Top-k page selection and merge with the pinned prefix and the window.
//
// The paper (Abstract; analysis page "Methodology"; digest "The Move") keeps
// a fixed budget of query-aware top-k pages next to the prefix and the
// window.  Here, per (sequence, KV head), one workgroup of 1024 threads:
//   1. loads the scores of logical pages [0, n_max) as order-preserving
//      32-bit keys into LDS (128 KiB: up to 32768 pages) and their page-table
//      entries into registers; n_max comes from the host-side length bound,
//      so these loads are issued together with the load of the sequence
//      length instead of after it.  Thread t handles pages t, t + 1024, ...
//      so every load instruction reads 256 contiguous bytes and LDS accesses
//      are bank-conflict free.  Only candidates -- the pages that meet the
//      middle region [Pe, Ws) -- take part in what follows;
//   2. finds the k-th largest key exactly by most-significant-digit radix
//      select.  Digits start right below the bits that the smallest and the
//      largest key share, 11 bits at a time (2048 LDS bins, double-buffered
//      so a pass costs two barriers), so the first histogram already spreads
//      the scores; a wave-level scan locates the digit holding the k-th key,
//      and the search stops as soon as that digit's bin holds exactly the
//      number of keys still needed;
//   3. turns per-wave ballots ("above the threshold", "tied with it") into
//      page-ordered bitmaps; block-wide prefix sums of their popcounts take
//      the tied pages in page order (ties go to the lower page id) and give
//      every selected page its output slot, so pages come out ascending;
//   4. writes the attended tokens as work items.  The attended set is split
//      into three disjoint token ranges -- prefix [0, Pe), the middle tokens
//      [Pe, Ws) of selected pages and the window [max(Ws, Pe), L) -- so no
//      token appears twice and no sort or dedup pass is needed.  The list is
//      padded with empty items up to its fixed length, so a consumer can
//      start on it without first reading how many items it holds.
// Wave-level scans and reductions use DPP row operations.
#include "fsa_internal.h"

namespace fsa {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kCols = 32;  // pages per thread: up to 32768 (512k tokens)
constexpr int kMaxPagesSel = kSelThreads * kCols;
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;

__device__ __forceinline__ int popc64(unsigned long long x) { return __popcll(x); }

// Exclusive prefix sum of one int per thread over the 1024-thread block.
__device__ __forceinline__ int block_excl_sum(int v, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = (int)wave_incl_sum((uint32_t)v);
  if (lane == kWave - 1) sh[wave] = incl;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) base += (w < wave) ? sh[w] : 0;
  __syncthreads();
  return base + incl - v;
}

__device__ __forceinline__ void put_item(int32_t* work, int idx, int p, int phys, int lo, int hi) {
  *reinterpret_cast<int4*>(work + 4 * (size_t)idx) = make_int4(p, phys, lo, hi);
}

__global__ __launch_bounds__(kSelThreads) void select_pages_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, int32_t* __restrict__ sel_pages,
    int32_t* __restrict__ work, int32_t* __restrict__ counts, int hkv, int max_pages, int prefix,
    int window, int budget, int max_items, int max_seq_len) {
  __shared__ uint32_t skey[kMaxPagesSel];
  __shared__ uint32_t hist[2][kBins];
  __shared__ unsigned long long bm_gt[kCols * kSelWaves];  // page-ordered bitmap: key above the threshold
  __shared__ unsigned long long bm_eq[kCols * kSelWaves];  // page-ordered bitmap: key tied with it
  __shared__ int scan_sh[kSelWaves + 1];
  __shared__ uint32_t mm_sh[2 * kSelWaves];
  __shared__ uint32_t s_prefix, s_need, s_done;

  const int unit = blockIdx.x, b = unit / hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_max = (max_seq_len + kPage - 1) / kPage;         // pages any sequence can have
  const int cols = (n_max + kSelThreads - 1) / kSelThreads;  // uniform
  const float* sc = scores + (size_t)unit * max_pages;
  const int32_t* pt = page_table + (size_t)b * max_pages;

  // ---- 1. scores and page-table entries of pages tid + 1024 j, loaded
  // together with the sequence length
  int phys[kCols];
  uint32_t raw[kCols];
#pragma unroll
  for (int j = 0; j < kCols; ++j) {
    if (j < cols) {
      const int p = min(tid + kSelThreads * j, n_max - 1);
      raw[j] = __float_as_uint(sc[p]);
      phys[j] = pt[p];
    }
  }
  const int L = min(seq_lens[b], max_seq_len);  // lengths beyond the host bound are clamped
  const int Pe = min(prefix, L), Ws = max(0, L - window);
  const int c_lo = Pe / kPage;
  const int c_hi = (Pe < Ws) ? (Ws + kPage - 1) / kPage : c_lo;  // candidates: pages [c_lo, c_hi)
  const int C = c_hi - c_lo;
  const int k = min(budget, C);
  const bool radix = k > 0 && k < C;  // otherwise every candidate is taken (k = C) or none is
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < kCols; ++j) {
    if (j < cols) {
      const int p = tid + kSelThreads * j;
      const uint32_t key = f32_order_key(__uint_as_float(raw[j]));  // non-candidates: never used
      skey[p] = key;
      if (p >= c_lo && p < c_hi) {
        kmin = min(kmin, key);
        kmax = max(kmax, key);
      }
    }
  }
  for (int i = tid; i < kBins; i += kSelThreads) hist[0][i] = 0;

  // ---- 2. exact k-th largest key: keys >> shift compared with kprefix, `need` ties to take
  uint32_t kprefix = 0, need = 0;
  int shift = 0;
  if (radix) {
    need = (uint32_t)k;
    kmin = wave_min(kmin);
    kmax = wave_max(kmax);
    if (lane == 0) {
      mm_sh[2 * wave] = kmin;
      mm_sh[2 * wave + 1] = kmax;
    }
    __syncthreads();
    uint32_t gmin = 0xFFFFFFFFu, gmax = 0u;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
      gmin = min(gmin, mm_sh[2 * w]);
      gmax = max(gmax, mm_sh[2 * w + 1]);
    }
    if (gmin == gmax) {
      kprefix = gmin;  // every candidate ties: the lowest ids win
    } else {
      int top = 31 - __clz(gmin ^ gmax);  // highest bit where candidates differ
      kprefix = (uint32_t)((uint64_t)gmax >> (top + 1));  // shared by every key
      for (int pass = 0;; ++pass) {
        uint32_t* h = hist[pass & 1];
        uint32_t* h_next = hist[(pass + 1) & 1];
        const int width = min(kDigitBits, top + 1);
        shift = top + 1 - width;
        for (int j = 0; j < cols; ++j) {
          const int p = tid + kSelThreads * j;
          const uint32_t key = skey[p];
          if (p >= c_lo && p < c_hi && (uint32_t)((uint64_t)key >> (shift + width)) == kprefix)
            atomicAdd(&h[(key >> shift) & ((1u << width) - 1u)], 1u);
        }
        for (int i = tid; i < kBins; i += kSelThreads) h_next[i] = 0;  // for the next pass
        __syncthreads();
        if (wave == 0) {
          // lane l owns digits 2047 - 32 l ... 2016 - 32 l (largest first)
          constexpr int PER_LANE = kBins / kWave;
          uint32_t s = 0;
#pragma unroll
          for (int j = 0; j < PER_LANE; ++j) s += h[kBins - 1 - PER_LANE * lane - j];
          const uint32_t incl = wave_incl_sum(s);
          const int f = __ffsll((long long)__ballot(incl >= need)) - 1;  // first lane reaching `need`
          const uint32_t before = (uint32_t)__builtin_amdgcn_readlane((int)(incl - s), f);
          // the wave scans lane f's 32 digits (lanes 32..63 carry zeros)
          const uint32_t digit = (uint32_t)(kBins - 1 - PER_LANE * f - (lane & (PER_LANE - 1)));
          const uint32_t c = (lane < PER_LANE) ? h[digit] : 0u;
          const uint32_t ic = wave_incl_sum(c);
          const unsigned long long hit = __ballot(lane < PER_LANE && before + ic >= need);
          if (lane == __ffsll((long long)hit) - 1) {
            const uint32_t cum = before + ic - c;
            s_prefix = (kprefix << width) | digit;
            s_need = need - cum;
            s_done = (c == need - cum);
          }
        }
        __syncthreads();
        kprefix = s_prefix;
        need = s_need;
        if (s_done || shift == 0) break;
        top = shift - 1;
      }
    }
  }

  // ---- 3. page-ordered bitmaps: page tid + 1024 j is bit `lane` of word
  // 16 j + wave; page-table entries replace the keys in LDS
  const bool take_all = k == C;
#pragma unroll
  for (int j = 0; j < kCols; ++j) {
    if (j < cols) {
      const int p = tid + kSelThreads * j;
      const bool cand = p >= c_lo && p < c_hi;
      const uint32_t kt = skey[p] >> shift;
      const unsigned long long ga = __ballot(cand && (radix ? kt > kprefix : take_all));
      const unsigned long long ge = __ballot(cand && radix && kt == kprefix);
      if (lane == 0) {
        bm_gt[j * kSelWaves + wave] = ga;
        bm_eq[j * kSelWaves + wave] = ge;
      }
      skey[p] = (uint32_t)phys[j];
    }
  }
  __syncthreads();
  // tied pages are taken in page order up to `need`; then output slots in page order
  const int nwords = cols * kSelWaves;  // <= 512: at most one word per thread
  const unsigned long long eqw = tid < nwords ? bm_eq[tid] : 0ull;
  const int ebase = block_excl_sum(popc64(eqw), scan_sh);
  unsigned long long takew = tid < nwords ? bm_gt[tid] : 0ull;
  int left = (int)need - ebase;  // ties of this word still to take
  for (unsigned long long m = eqw; m && left > 0; m &= m - 1, --left) takew |= m & (~m + 1);
  int o = block_excl_sum(popc64(takew), scan_sh);

  // ---- 4. work items: prefix [0, n_pre), selected [n_pre, n_pre + k), window,
  // then empty items up to max_items
  const int n_pre = (Pe + kPage - 1) / kPage;
  const int w0 = max(Ws, Pe);
  const int n_win = (L > w0) ? (L + kPage - 1) / kPage - w0 / kPage : 0;
  const int n_items = n_pre + k + n_win;
  int32_t* wrk = work ? work + 4 * (size_t)unit * max_items : nullptr;
  int32_t* sel = sel_pages ? sel_pages + (size_t)unit * budget : nullptr;
  const int jw = tid / kSelWaves, ww = tid % kSelWaves;  // word tid covers pages 1024 jw + 64 ww + bit
  for (unsigned long long m = takew; m; m &= m - 1) {
    const int p = kSelThreads * jw + kWave * ww + (__ffsll((long long)m) - 1);
    if (sel) sel[o] = p;
    if (wrk)
      put_item(wrk, n_pre + o, p, (int)skey[p], max(p * kPage, Pe) - p * kPage,
               min(p * kPage + kPage, Ws) - p * kPage);
    ++o;
  }
  if (wrk) {
    for (int i = tid; i < n_pre; i += kSelThreads)
      put_item(wrk, i, i, (int)skey[i], 0, min(kPage, Pe - i * kPage));
    for (int i = tid; i < n_win; i += kSelThreads) {
      const int p = w0 / kPage + i;
      put_item(wrk, n_pre + k + i, p, (int)skey[p], max(p * kPage, w0) - p * kPage,
               min(p * kPage + kPage, L) - p * kPage);
    }
    for (int i = n_items + tid; i < max_items; i += kSelThreads) put_item(wrk, i, -1, 0, 0, 0);
  }
  if (sel)
    for (int i = k + tid; i < budget; i += kSelThreads) sel[i] = -1;
  if (tid == 0 && counts) {
    counts[2 * unit] = k;
    counts[2 * unit + 1] = n_items;
  }
}

}  // namespace

int select_max_candidates() { return kMaxPagesSel; }

hipError_t launch_select_pages(const float* scores, const int32_t* page_table,
                               const int32_t* seq_lens, int32_t* sel_pages, int32_t* work,
                               int32_t* counts, int batch, int hkv, int max_pages, int prefix,
                               int window, int budget, int max_items, int max_seq_len,
                               hipStream_t stream) {
  hipLaunchKernelGGL(select_pages_kernel, dim3((unsigned)(batch * hkv)), dim3(kSelThreads), 0,
                     stream, scores, page_table, seq_lens, sel_pages, work, counts, hkv, max_pages,
                     prefix, window, budget, max_items, max_seq_len);
  return hipGetLastError();
}

}  // namespace fsa
