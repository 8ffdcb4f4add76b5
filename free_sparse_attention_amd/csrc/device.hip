// Device properties used to size grids: compute-unit count and how many
// workgroups of a kernel fit on one compute unit.  Values are cached after
// the first query (one device model per process is assumed); concurrent
// first calls may both query, with the same result.
#include <atomic>

#include "fsa_internal.h"

namespace fsa {

int device_cu_count() {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_relaxed);
  if (n == 0) {
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
      n = c;
    else
      n = 256;  // MI355X
    cached.store(n, std::memory_order_relaxed);
  }
  return n;
}

int resident_blocks_per_cu(const void* kernel, int block_threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, block_threads, 0) != hipSuccess || n < 1)
    n = 1;
  return n;
}

}  // namespace fsa
