// Quest page scores on the matrix cores: the scoring launch of the decode
// step (the routine itself is in score_core.h).
#include <algorithm>
#include <atomic>

#include "append_core.h"
#include "score_core.h"

namespace fsa {
namespace {

// wg_per_unit workgroups of W waves score each (sequence, KV head) unit
// (score_wave); the grid is sized to four resident rounds of waves.
//
// In the combined append + decode step the same launch also carries the
// append: its tasks (append_core.h) in the first append_blocks workgroups, one
// per wave; the scoring then takes the lengths after the append (seq_lens +
// len_add).  The host uses this only when no page the append touches can be a
// candidate (window >= n_new + 15), so the two roles write and read disjoint
// data; the scores of the touched pages' tiles that are not candidates are
// computed from metadata being rewritten, but never stored.
template <int D, int W>  // W: waves per workgroup
__global__ __launch_bounds__(W * 64) void quest_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ meta,
    const int32_t* __restrict__ seq_lens, float* __restrict__ scores, int hq, int hkv,
    int max_pages, int prefix, int window, int tiles_per_wave, int wg_per_unit, int max_seq_len,
    const AppendArgs ap, int append_blocks, int append_tasks, int len_add, FastDiv by_wg, FastDiv by_hkv, int G) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if ((int)blockIdx.x < append_blocks) {
    const int w = (int)blockIdx.x * W + wave;
    if (w < append_tasks) append_task<D>(ap, w, lane);
    return;
  }
  const int blk = (int)blockIdx.x - append_blocks;
  const int unit = (int)fdiv((uint32_t)blk, by_wg), wg = blk - unit * wg_per_unit;
  const int b = (int)fdiv((uint32_t)unit, by_hkv), g = unit - b * hkv;
  const ScoreArgs S{q, meta, seq_lens, scores, hq, hkv, max_pages, prefix, window, max_seq_len, len_add, G};
  score_wave<D>(S, unit, b, g, wg * W + wave, W * wg_per_unit, tiles_per_wave);
}

}  // namespace

hipError_t launch_quest_scores(const uint16_t* q, const uint16_t* meta, const int32_t* seq_lens,
                               float* scores, int batch, int hq, int hkv, int d, int max_pages,
                               int prefix, int window, int max_seq_len, hipStream_t stream,
                               const AppendArgs* append) {
  const int units = batch * hkv;
  const int max_cand = (max_seq_len + kPage - 1) / kPage;
  const int tiles_per_unit = (max_cand + kMetaTile - 1) / kMetaTile + 1;  // a range may straddle one more
  // 8-wave workgroups for batches of many units (the 16-sequence serving
  // batch: 128 units, step 171 -> 169 us), 4-wave ones otherwise (64k and
  // 256k: 4 waves 0.1 and 0.9 us faster)
  const int W = units >= 64 ? 8 : 4;
  const void* kern = d == 128 ? (W == 8 ? reinterpret_cast<const void*>(&quest_score_kernel<128, 8>)
                                        : reinterpret_cast<const void*>(&quest_score_kernel<128, 4>))
                              : (W == 8 ? reinterpret_cast<const void*>(&quest_score_kernel<64, 8>)
                                        : reinterpret_cast<const void*>(&quest_score_kernel<64, 4>));
  static std::atomic<int> resident[2][2];  // per head dim and workgroup size, zero until first queried
  int res = resident[d == 128][W == 8].load(std::memory_order_relaxed);
  if (res == 0) {
    res = resident_blocks_per_cu(kern, W * 64);
    resident[d == 128][W == 8].store(res, std::memory_order_relaxed);
  }
  // four resident rounds of workgroups shared out over the units: workgroups
  // whose tiles lie beyond their sequence's length exit at once and the
  // dispatcher gives their slots to the next ones, which evens out batches of
  // unequal lengths (16 sequences of 18k-261k tokens: step 165.9 -> 158.9 us)
  const int round = 4 * res * device_cu_count();
  const int wg_per_unit_max = (tiles_per_unit + W - 1) / W;
  const int wg_per_unit = std::max(1, std::min(wg_per_unit_max, round / std::max(1, units)));
  const int tpw = (tiles_per_unit + W * wg_per_unit - 1) / (W * wg_per_unit);
  AppendArgs ap{};
  int append_tasks = 0, len_add = 0;
  if (append) {
    ap = *append;
    append_tasks = units * ap.touch;
    len_add = ap.n_new;
  }
  const int append_blocks = (append_tasks + W - 1) / W;
  const dim3 grid((unsigned)((long)append_blocks + (long)units * wg_per_unit));
#define FSA_SCORE(DD, WW)                                                                                       \
  hipLaunchKernelGGL((quest_score_kernel<DD, WW>), grid, dim3(WW * 64), 0, stream, q, meta, seq_lens, scores, hq, \
                     hkv, max_pages, prefix, window, tpw, wg_per_unit, max_seq_len, ap, append_blocks, append_tasks,  \
                     len_add, make_fastdiv((uint32_t)wg_per_unit), make_fastdiv((uint32_t)hkv), hq / hkv)
  if (d == 128) {
    if (W == 8) FSA_SCORE(128, 8); else FSA_SCORE(128, 4);
  } else {
    if (W == 8) FSA_SCORE(64, 8); else FSA_SCORE(64, 4);
  }
#undef FSA_SCORE
  return hipGetLastError();
}

}  // namespace fsa
