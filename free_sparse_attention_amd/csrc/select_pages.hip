// Top-k page selection and merge with the pinned prefix and the window.
//
// The paper (Abstract; analysis page "Methodology"; digest "The Move") keeps
// a fixed budget of query-aware top-k pages next to the prefix and the
// window.  Here, per (sequence, KV head), one workgroup of 1024 threads:
//   1. loads the candidates' scores as order-preserving 32-bit keys into LDS
//      (128 KiB: up to 32768 candidates); thread t of the block handles
//      candidates t, t + 1024, ... so every load instruction reads 256
//      contiguous bytes and LDS accesses are bank-conflict free;
//   2. finds the k-th largest key exactly by most-significant-digit radix
//      select.  Digits start right below the bits that the smallest and the
//      largest key share, 11 bits at a time (2048 LDS bins), so the first
//      histogram already spreads the scores; a wave-level scan locates the
//      digit holding the k-th key, and the search stops as soon as that
//      digit's bin holds exactly the number of keys still needed;
//   3. ranks the selected pages in ascending id order from per-wave ballots:
//      a candidate's rank among the keys tied with the threshold (ties go to
//      the lower page id) and its output slot are a popcount within its wave
//      plus a prefix over (column, wave) counts;
//   4. writes the attended tokens as work items.  The attended set is split
//      into three disjoint token ranges -- prefix [0, Pe), the middle tokens
//      [Pe, Ws) of selected pages and the window [max(Ws, Pe), L) -- so no
//      token appears twice and no sort or dedup pass is needed.
#include "fsa_internal.h"

namespace fsa {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kCols = 32;  // keys per thread: up to 32768 candidate pages (512k tokens)
constexpr int kMaxCand = kSelThreads * kCols;
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;

__device__ __forceinline__ int popc64(unsigned long long x) { return __popcll(x); }

__device__ __forceinline__ unsigned long long lanes_below() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__device__ __forceinline__ void put_item(int32_t* work, int idx, int p, int phys, int lo, int hi) {
  *reinterpret_cast<int4*>(work + 4 * (size_t)idx) = make_int4(p, phys, lo, hi);
}

__global__ __launch_bounds__(kSelThreads) void select_pages_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, int32_t* __restrict__ sel_pages,
    int32_t* __restrict__ work, int32_t* __restrict__ counts, int hkv, int max_pages, int prefix,
    int window, int budget, int max_items, int max_seq_len) {
  __shared__ uint32_t skey[kMaxCand];
  __shared__ uint32_t hist[kBins];
  __shared__ int cnt_a[kCols][kSelWaves];  // per (column, wave): keys above the threshold, then output base
  __shared__ int cnt_e[kCols][kSelWaves];  // per (column, wave): keys tied with it, then tie-rank base
  __shared__ uint32_t mm_sh[2 * kSelWaves];
  __shared__ uint32_t s_prefix, s_need, s_done;

  const int unit = blockIdx.x, b = unit / hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = min(seq_lens[b], max_seq_len);  // lengths beyond the host bound are clamped
  const int Pe = min(prefix, L), Ws = max(0, L - window);
  const int c_lo = Pe / kPage;
  const int C = (Pe < Ws) ? (Ws + kPage - 1) / kPage - c_lo : 0;
  const int k = min(budget, C);
  const bool take_all = (k == C);
  const bool radix = !take_all && k > 0;
  const int cols = (C + kSelThreads - 1) / kSelThreads;  // uniform
  const float* sc = scores + (size_t)unit * max_pages + c_lo;
  const int32_t* pt = page_table + (size_t)b * max_pages;

  // ---- 1. keys: candidate i = tid + 1024 j in skey[i]
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  if (radix) {
#pragma unroll 8
    for (int j = 0; j < cols; ++j) {
      const int i = tid + kSelThreads * j;
      const uint32_t key = f32_order_key(sc[min(i, C - 1)]);
      skey[i] = key;
      if (i < C) {
        kmin = min(kmin, key);
        kmax = max(kmax, key);
      }
    }
  }

  // ---- 2. exact k-th largest key: keys >> shift compared with kprefix, `need` ties to take
  uint32_t kprefix = 0, need = (uint32_t)k;
  int shift = 0;
  if (radix) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
    }
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
      while (true) {
        const int width = min(kDigitBits, top + 1);
        shift = top + 1 - width;
        for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0;
        __syncthreads();
#pragma unroll 8
        for (int j = 0; j < cols; ++j) {
          const int i = tid + kSelThreads * j;
          const uint32_t key = skey[i];
          if (i < C && (uint32_t)((uint64_t)key >> (shift + width)) == kprefix)
            atomicAdd(&hist[(key >> shift) & ((1u << width) - 1u)], 1u);
        }
        __syncthreads();
        if (wave == 0) {
          // lane l owns digits 2047 - 32 l ... 2016 - 32 l (largest first)
          constexpr int PER_LANE = kBins / kWave;
          uint32_t s = 0;
#pragma unroll
          for (int j = 0; j < PER_LANE; ++j) s += hist[kBins - 1 - PER_LANE * lane - j];
          uint32_t incl = s;
#pragma unroll
          for (int off = 1; off < kWave; off <<= 1) {
            const uint32_t y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
          }
          const int f = __ffsll((long long)__ballot(incl >= need)) - 1;  // first lane reaching `need`
          const uint32_t before = __shfl(incl - s, f);                   // keys in larger digits
          // the whole wave scans lane f's 32 digits
          const uint32_t digit = (uint32_t)(kBins - 1 - PER_LANE * f - (lane & (PER_LANE - 1)));
          const uint32_t c = (lane < PER_LANE) ? hist[digit] : 0u;
          uint32_t ic = c;
#pragma unroll
          for (int off = 1; off < PER_LANE; off <<= 1) {
            const uint32_t y = __shfl_up(ic, off);
            if (lane >= off) ic += y;
          }
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
        const bool done = s_done;
        __syncthreads();
        if (done || shift == 0) break;
        top = shift - 1;
      }
    }
  }

  // ---- 3. ranks in page-id order: id = tid + 1024 j, i.e. ordered by (j, wave, lane)
  const unsigned long long below = lanes_below();
  if (radix) {
#pragma unroll 8
    for (int j = 0; j < cols; ++j) {
      {
        const bool v = tid + kSelThreads * j < C;
        const uint32_t kt = skey[tid + kSelThreads * j] >> shift;
        const unsigned long long ga = __ballot(v && kt > kprefix);
        const unsigned long long ge = __ballot(v && kt == kprefix);
        if (lane == 0) {
          cnt_a[j][wave] = popc64(ga);
          cnt_e[j][wave] = popc64(ge);
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      // exclusive prefixes over the (column, wave) order, 64 slots per pass:
      // tie-rank base first, then the output slot base
      int e_run = 0, o_run = 0;
      for (int s0 = 0; s0 < cols * kSelWaves; s0 += kWave) {
        const int sidx = s0 + lane;
        const bool in = sidx < cols * kSelWaves;
        const int jj = in ? sidx / kSelWaves : 0, ww = in ? sidx % kSelWaves : 0;
        const int ce = in ? cnt_e[jj][ww] : 0, ca = in ? cnt_a[jj][ww] : 0;
        int ie = ce;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const int y = __shfl_up(ie, off);
          if (lane >= off) ie += y;
        }
        const int ebase = e_run + ie - ce;
        const int taken = ca + max(0, min((int)need - ebase, ce));
        int io = taken;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const int y = __shfl_up(io, off);
          if (lane >= off) io += y;
        }
        if (in) {
          cnt_e[jj][ww] = ebase;
          cnt_a[jj][ww] = o_run + io - taken;
        }
        e_run += __shfl(ie, kWave - 1);
        o_run += __shfl(io, kWave - 1);
      }
    }
    __syncthreads();
  }

  const int n_pre = (Pe + kPage - 1) / kPage;
  const int w0 = max(Ws, Pe);
  const int n_win = (L > w0) ? (L + kPage - 1) / kPage - w0 / kPage : 0;
  const int n_items = n_pre + k + n_win;
  int32_t* wrk = work ? work + 4 * (size_t)unit * max_items : nullptr;
  int32_t* sel = sel_pages ? sel_pages + (size_t)unit * budget : nullptr;

  // ---- 4. selected pages: output slot = base of (column, wave) + taken lanes below
  auto emit = [&](int o, int i, int phys) {
    const int p = c_lo + i;
    if (sel) sel[o] = p;
    if (wrk)
      put_item(wrk, n_pre + o, p, phys, max(p * kPage, Pe) - p * kPage,
               min(p * kPage + kPage, Ws) - p * kPage);
  };
  if (take_all) {
#pragma unroll 4
    for (int j = 0; j < cols; ++j) {
      const int i = tid + kSelThreads * j;
      const int phys = pt[c_lo + min(i, C - 1)];
      if (i < C) emit(i, i, phys);
    }
  } else if (radix) {
    uint32_t mine = 0;  // columns where this lane's page is taken
#pragma unroll 8
    for (int j = 0; j < cols; ++j) {
      {
        const int i = tid + kSelThreads * j;
        const bool v = i < C;
        const uint32_t kt = skey[i] >> shift;
        const bool a = v && kt > kprefix, e = v && kt == kprefix;
        const unsigned long long ge = __ballot(e);
        const int rank = cnt_e[j][wave] + popc64(ge & below);
        const bool take = a || (e && rank < (int)need);
        const unsigned long long gt = __ballot(take);
        if (take) {
          mine |= 1u << j;
          skey[i] = (uint32_t)(cnt_a[j][wave] + popc64(gt & below));  // reuse: output slot
        }
      }
    }
    while (mine) {
      const int j = __ffs(mine) - 1;
      mine &= mine - 1;
      const int i = tid + kSelThreads * j;
      emit((int)skey[i], i, pt[c_lo + i]);
    }
  }

  // ---- 5. prefix and window items, padding, counts
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
  if (tid == 0 && counts) {
    counts[2 * unit] = k;
    counts[2 * unit + 1] = n_items;
  }
}

}  // namespace

int select_max_candidates() { return kMaxCand; }

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
