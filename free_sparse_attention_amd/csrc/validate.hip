// Debug check of the device-resident inputs of a decode step: lengths, page
// table entries of the pages in use, and finiteness of q.  Reads only; the
// values checked are never used as addresses.
#include <algorithm>

#include "fsa_internal.h"

namespace fsa {
namespace {

// scratch: [0] number of violations, [1] kind of the first one recorded
// (1 length, 2 page-table entry, 3 non-finite q, 4 an append that would run
// past the page table), [2] sequence or element, [3] page or length.
__global__ void validate_init_kernel(int32_t* scratch) {
  if (threadIdx.x == 0) {
    scratch[0] = 0;
    scratch[1] = -1;
    scratch[2] = -1;
    scratch[3] = -1;
  }
}

__device__ __forceinline__ void record(int32_t* scratch, int kind, int a, int b) {
  atomicAdd(scratch, 1);
  if (atomicCAS(scratch + 1, -1, kind) == -1) {
    scratch[2] = a;
    scratch[3] = b;
  }
}

// Blocks [0, batch): sequence blockIdx.x; the rest: a grid-stride scan of q.
__global__ __launch_bounds__(256) void validate_kernel(const uint16_t* __restrict__ q,
                                                       const int32_t* __restrict__ page_table,
                                                       const int32_t* __restrict__ seq_lens,
                                                       int32_t* scratch, int batch, int max_pages,
                                                       int pool, int max_seq_len, int n_new, long q_elems) {
  if ((int)blockIdx.x < batch) {
    const int b = blockIdx.x;
    const int L0 = seq_lens[b];
    // with n_new tokens about to be appended, the pages in use afterwards
    // must be mapped and the new length must fit the page table
    if (n_new > 0 && L0 >= 0 && (long)L0 + n_new > (long)max_pages * kPage) {
      if (threadIdx.x == 0) record(scratch, 4, b, L0);
      return;
    }
    const long Lw = (long)L0 + n_new;
    if (L0 < (n_new > 0 ? 0 : 1) || Lw > max_seq_len) {
      if (threadIdx.x == 0) record(scratch, 1, b, L0);
      return;
    }
    const int L = (int)Lw;
    const int n = min((L + kPage - 1) / kPage, max_pages);
    for (int p = threadIdx.x; p < n; p += blockDim.x) {
      const int phys = page_table[(size_t)b * max_pages + p];
      if (phys < 0 || phys >= pool) record(scratch, 2, b, p);
    }
  } else {
    const long stride = (long)(gridDim.x - batch) * blockDim.x;
    for (long i = (long)(blockIdx.x - batch) * blockDim.x + threadIdx.x; i < q_elems; i += stride)
      if ((q[i] & 0x7F80u) == 0x7F80u) record(scratch, 3, (int)i, 0);  // exponent all ones: inf or NaN
  }
}

}  // namespace

hipError_t launch_validate(const uint16_t* q, const int32_t* page_table, const int32_t* seq_lens,
                           int32_t* scratch, int batch, int hq, int d, int max_pages, int pool,
                           int max_seq_len, int n_new, hipStream_t stream) {
  hipLaunchKernelGGL(validate_init_kernel, dim3(1), dim3(64), 0, stream, scratch);
  const long q_elems = (long)batch * hq * d;
  const int q_blocks = (int)std::min<long>(1024, (q_elems + 255) / 256);
  hipLaunchKernelGGL(validate_kernel, dim3((unsigned)(batch + q_blocks)), dim3(256), 0, stream, q, page_table,
                     seq_lens, scratch, batch, max_pages, pool, max_seq_len, n_new, q_elems);
  return hipGetLastError();
}

}  // namespace fsa
