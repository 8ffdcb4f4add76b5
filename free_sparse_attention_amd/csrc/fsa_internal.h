// Internal definitions shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsa {

constexpr int kPage = 16;  // tokens per page
constexpr int kWave = 64;  // CDNA wavefront width
constexpr int kXcds = 8;   // MI355X: accelerator dies (XCDs), 32 CUs and one L2 each

// Debug builds (-DFSA_DEBUG_POISON_LDS, libfsa_poison.so) fill a kernel's LDS
// with a NaN pattern when the kernel starts and where a later stage reuses the
// LDS of an earlier one, then wait for the whole workgroup: a read of LDS that
// no stage of the kernel wrote then shows up in the outputs.  Release builds
// compile this to nothing.
#ifdef FSA_DEBUG_POISON_LDS
constexpr int kBuildFlags = 1;
__device__ __forceinline__ void poison_lds(void* p, size_t bytes) {
  uint32_t* w = static_cast<uint32_t*>(p);
  for (size_t i = threadIdx.x; i < bytes / 4; i += blockDim.x) w[i] = 0x7FC07FC0u;  // NaN as fp32 and as bf16
  __syncthreads();
}
#else
constexpr int kBuildFlags = 0;
__device__ __forceinline__ void poison_lds(void*, size_t) {}
#endif

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// nearest-even fp32 -> bf16 bits (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Order-preserving map of bf16 bits to uint16 (numeric order, -0 just below +0).
__device__ __forceinline__ uint32_t bf16_order_key(uint32_t b) {
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}
// Inverse of bf16_order_key, with -0 written as +0.
__device__ __forceinline__ uint32_t bf16_from_order_key(uint32_t k) {
  uint32_t b = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
  return b == 0x8000u ? 0u : b;
}

// Order-preserving map of fp32 scores to uint32 (-0 and +0 map to one key).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- page metadata layout
// Metadata is kept per (sequence b, KV head g, logical page p) -- it is derived
// state of the sequence, so it needs no page-table lookup -- in tiles of 16
// logical pages: tile t of unit (b, g) holds [2D/32 steps][16 pages][32 values],
// where value e of page p is the minimum of key channel e (e < D) or the
// maximum of channel e - D (e >= D).  One 16-page, 32-value slab is 1 KiB of
// contiguous memory: exactly the operand that one MFMA step of the scoring
// kernel loads.
constexpr int kMetaTile = 16;
__host__ __device__ inline int meta_tiles(int max_pages) { return (max_pages + kMetaTile - 1) / kMetaTile; }
__host__ __device__ inline size_t meta_offset(int unit, int p, int e, int tiles, int D) {
  const int ns = 2 * D / 32;
  return (((size_t)unit * tiles + p / kMetaTile) * ns + e / 32) * (kMetaTile * 32) +
         (size_t)(p % kMetaTile) * 32 + e % 32;
}

// ---------------------------------------------------------------- wave-level DPP primitives
// Inclusive prefix sum over the 64 lanes of a wave: row shifts within each
// 16-lane row, then row broadcasts of lanes 15 and 31 across rows.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}
// Wave-wide minimum and maximum (every lane receives the result).
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
  const uint32_t id = 0xFFFFFFFFu;
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x111, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x112, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x114, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x118, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x142, 0xa, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) loads of data read once per step.
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_nt(const uint2* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}

// ---------------------------------------------------------------- device

int device_cu_count();
// plain streaming read of bytes (a multiple of 16) at buf; sink is written at
// most once, with a value of no meaning
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);
int resident_blocks_per_cu(const void* kernel, int block_threads);

// ---------------------------------------------------------------- launchers
// All launchers enqueue on `stream` and return the launch status.

// Launch selection of a decode step (measurement only): `count` numbers the
// step's launches in order, and take() lets through launches [first, last]
// (by default all), so a part of the step can be timed on its own.
struct LaunchFilter {
  int first = 0, last = 1 << 30;
  int count = 0;
  bool take() {
    const int i = count++;
    return i >= first && i <= last;
  }
};

hipError_t launch_import_kv_plain(const uint16_t* k_plain, const uint16_t* v_plain, uint16_t* kc,
                                  uint16_t* vc, int pool, int hkv, int d, hipStream_t stream);

hipError_t launch_append_kv(int n_new, const uint16_t* k_new, const uint16_t* v_new,
                            const int32_t* page_table, const int32_t* seq_lens,
                            int32_t* seq_lens_out, uint16_t* kc, uint16_t* vc, uint16_t* meta,
                            int batch, int hkv, int d, int max_pages, hipStream_t stream);

hipError_t launch_build_page_meta(const uint16_t* kc, const int32_t* page_table,
                                  const int32_t* seq_lens, uint16_t* meta, int batch, int hkv,
                                  int d, int max_pages, int max_seq_len, hipStream_t stream);

struct AppendArgs;
// With `append` (combined append + decode step), the launch also performs the
// append, and seq_lens are the lengths before it.
hipError_t launch_quest_scores(const uint16_t* q, const uint16_t* meta, const int32_t* seq_lens,
                               float* scores, int batch, int hq, int hkv, int d, int max_pages,
                               int prefix, int window, int max_seq_len, hipStream_t stream,
                               const AppendArgs* append = nullptr);

hipError_t launch_select_pages(const float* scores, const int32_t* page_table,
                               const int32_t* seq_lens, int32_t* sel_pages, int32_t* work,
                               int32_t* counts, int batch, int hkv, int max_pages, int prefix,
                               int window, int budget, int max_items, int max_seq_len,
                               hipStream_t stream);

// Largest candidate count one selection workgroup holds.
int select_max_candidates();
int select_columns(int max_seq_len);  // pages per selection thread for this length bound

struct AttnPlan {
  int items_per_wave;  // work items each wave walks through
  int wg_per_unit;     // workgroups launched per (b, KV head)
};

// Debug validation of device inputs into scratch (int32[4]); see fsa_validate_inputs.
hipError_t launch_validate(const uint16_t* q, const int32_t* page_table, const int32_t* seq_lens,
                           int32_t* scratch, int batch, int hq, int d, int max_pages, int pool,
                           int max_seq_len, int n_new, hipStream_t stream);

// One decode step's selection launch: the top-k selection of every (sequence,
// KV head) with the attention over the selected pages, plus the attention over
// the prefix and window pages.
// Division by a launch-invariant divisor without the reciprocal sequence a
// runtime division compiles to: m = min(floor(2^32 / d), 2^32 - 1) makes
// umulhi(n, m) equal n / d or one less for every 32-bit n (d >= 1), and one
// compare settles it (Granlund and Montgomery, "Division by invariant
// integers using multiplication", 1994).  The host fills d and m.
struct FastDiv {
  uint32_t d, m;
};
inline FastDiv make_fastdiv(uint32_t d) {
  const uint64_t m = (uint64_t{1} << 32) / (d ? d : 1);
  return FastDiv{d, (uint32_t)(m > 0xFFFFFFFFull ? 0xFFFFFFFFull : m)};
}
__host__ __device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
  uint32_t q = (uint32_t)(((uint64_t)n * f.m) >> 32);  // a multiply-high on the device
  if (n - q * f.d >= f.d) ++q;
  return q;
}

struct StepArgs {
  const float* scores;        // [B][Hkv][max_pages] Quest scores
  const int32_t* page_table;  // [B][max_pages]
  const int32_t* seq_lens;    // [B]
  int32_t* sel_pages;         // [B][Hkv][budget] or null
  // wide plan (sel_rep > 0): sel_rep workgroups per unit each select and attend
  // selected items [r per, (r + 1) per)
  int sel_rep, per;
  // narrow plan (sel_rep == 0): one selection workgroup per unit writes the
  // selected items to sel_work ([B][Hkv][sel_items][4]) for the split-K kernel
  int32_t* sel_work;
  int sel_items;
  // both plans: pw_wg further workgroups per unit attend the prefix and window pages
  int batch, hq, hkv, d, max_pages, prefix, window, budget, max_seq_len;
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  float* part_o;       // partial slots [B][Hkv][slots_per_unit][G][D]
  float* part_ml;      // [B][Hkv][slots_per_unit][G][2]
  int slots_per_unit;  // prefix/window workgroups first, then the selection replicas (wide)
  int pw_ipw;          // prefix/window items per wave
  int pw_wg;           // prefix/window workgroups per unit
  int sel_blocks;      // selection workgroups at the front of the grid
  int xcd_grouped;     // wide plan: workgroup -> (unit, replica) keeps a unit on one XCD
  int prefetch;        // wide plan: replicas prefetch known-taken pages into their L2
  float scale_log2;
  int G;                          // hq / hkv
  FastDiv by_hkv, by_rep, by_pw;  // divisions by hkv, sel_rep (or 1), pw_wg (or 1)
  uint16_t* out;                  // [B][Hq][D]: written by the one-launch step's merge
};

// Prefix/window attention plan: at most max_items items per unit, ipw per wave,
// wg_per_unit 1024-thread workgroups per unit (0 when there are none).
struct PwPlan {
  int max_items, ipw, wg_per_unit;
};
PwPlan plan_prefix_window(int units, int pw_cus, int prefix, int window, int max_seq_len);

// Plan of the step's selection launch: wide (sel_rep > 0) when selection
// replicas with at most 2 selected pages per wave fit on half the CUs;
// otherwise narrow, followed by the split-K attention over sel_items items.
constexpr int kSliceMax = 256;  // selected items one replica can take
struct StepPlan {
  int sel_rep, per, sel_items;
  PwPlan pw;
  int sel_blocks;   // selection workgroups at the front of the grid
  int xcd_grouped;  // wide plan: a unit's replicas share one XCD (see the kernel)
  int prefetch;     // wide plan: replicas prefetch known-taken pages into their L2
};
StepPlan plan_step(int units, int head_dim, int prefix, int window, int budget, int max_seq_len);
hipError_t launch_select_attend(const StepArgs& a, hipStream_t stream);

// One-launch step (wide plan on a device of kXcds XCDs of 32 CUs): a single
// launch runs the scoring, the selection replicas, the prefix/window
// attention and the merge of the partials as tasks, taken in order from one
// queue per XCD; the units of XCD x (units x, x + 8, ...) have all their tasks
// on that XCD, so what one task leaves for another is in the XCD's L2.
constexpr int kOneMaxUnits = 64;  // units of a one-launch step, at most
constexpr int kSyncSlots = 32;    // one-launch steps in flight on one GPU, at most
struct OneLaunchArgs {
  void* sync;            // this step's synchronisation slot (device memory of the library)
  const uint16_t* meta;  // the page metadata the scoring tasks read
  int units;
  int n_score;        // scoring tasks per unit (16 waves each)
  int score_tpw;      // 16-page tiles per scoring wave, at most
  FastDiv by_score;   // division by n_score
};
// Whether the one-launch step applies (the wide plan, at most kOneMaxUnits
// units, at most 16 query heads per KV head and few partials per unit, a
// device of kXcds XCDs of 32 CUs; mode 1: also a unit count that is a multiple
// of kXcds, mode 2: any; mode 0: never), and its task sizes.
bool plan_one_launch(const StepPlan& p, int units, int head_dim, int G, int prefix, int window, int max_seq_len,
                     int mode, OneLaunchArgs* o);
// Device address of the next synchronisation slot on the current device.
hipError_t one_launch_slot(void** slot);
hipError_t launch_one_step(const StepArgs& a, const OneLaunchArgs& o, hipStream_t stream);
// Waits the one-launch kernel gave up on (bounded waits), summed over the
// slots of the current device; synchronises the device (measurement and tests).
hipError_t one_launch_stalls(long long* n);

// Attention work-item sources: every page of the sequence, or the selection's work list.
enum AttnMode { kDense = 0, kList = 1 };
constexpr int kMaxPartials = 1024;  // partial results per unit, at most

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* work;    // selection work items (kList)
  float* part_o;
  float* part_ml;
  int slots_per_unit;  // partial slots per unit in part_o/part_ml; 0: the plan's workgroups
  int slot_base;       // first slot of this launch's workgroups (with slots_per_unit > 0)
  uint16_t* out;
  int batch, hq, hkv, d, max_pages, max_items;
  float scale_log2;
  int max_seq_len;
};

// Plan for `max_items` items per unit (at most kMaxPartials workgroups per unit).
AttnPlan plan_attention(int units, int max_items);

// Split-K attention over the unit's items, then (when a unit can need more
// than one workgroup) the combine of its partials.
hipError_t launch_attention(AttnMode mode, const AttnPlan& plan, const AttnArgs& a, hipStream_t stream,
                            LaunchFilter* filter = nullptr);

// Merge of all `slots` partials of every unit into the output (decode step).
hipError_t launch_combine(const AttnArgs& a, int slots, hipStream_t stream);

}  // namespace fsa
