// Stand-alone top-k page selection and merge with the prefix and the window:
// one 1024-thread workgroup per (sequence, KV head) runs the selection of
// select_core.h on scores in memory.
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
  select_unit<COLS>(S, J);
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

}  // namespace fsa
