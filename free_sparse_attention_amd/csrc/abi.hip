// C-ABI entry points declared in include/fsa.h and include/fsa_measure.h: host-side argument checks,
// workspace layout and launch sequencing on the caller's stream.
#include <dlfcn.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>

#include "fsa.h"
#include "fsa_measure.h"
#include "append_core.h"

namespace {

thread_local std::string g_err;

// Optional tracing: with FSA_TRACE=1 in the environment every entry point that
// launches work opens a roctx range named after itself (rocprofv3
// --marker-trace shows them beside the kernels).  The roctx library is opened
// at run time on first use, so libfsa.so has no link-time dependency on it;
// without FSA_TRACE=1, or without the library, the ranges cost one branch.
struct Roctx {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};

const Roctx& roctx() {
  static const Roctx r = [] {
    Roctx t;
    const char* e = getenv("FSA_TRACE");
    if (e == nullptr || strcmp(e, "1") != 0) return t;
    void* h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
    if (h == nullptr) h = dlopen("libroctx64.so.4", RTLD_NOW | RTLD_LOCAL);
    if (h == nullptr) return t;
    t.push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
    t.pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
    if (t.push == nullptr || t.pop == nullptr) t = Roctx{};
    return t;
  }();
  return r;
}

struct TraceRange {
  explicit TraceRange(const char* name) {
    if (roctx().push) roctx().push(name);
  }
  ~TraceRange() {
    if (roctx().pop) roctx().pop();
  }
  TraceRange(const TraceRange&) = delete;
  TraceRange& operator=(const TraceRange&) = delete;
};

fsa_status fail(fsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

fsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return FSA_OK;
  return fail(FSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define FSA_CHECK(expr)              \
  do {                               \
    const fsa_status _s = (expr);    \
    if (_s != FSA_OK) return _s;     \
  } while (0)

fsa_status check_dims(const fsa_dims* d) {
  if (!d) return fail(FSA_ERR_INVALID_ARG, "dims is NULL");
  if (d->batch < 1 || d->num_kv_heads < 1 || d->num_q_heads < 1 || d->max_pages_per_seq < 1 ||
      d->num_pool_pages < 1)
    return fail(FSA_ERR_INVALID_ARG, "dims: batch, heads, max_pages_per_seq and num_pool_pages must be >= 1");
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(FSA_ERR_INVALID_ARG, "dims: num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                d->num_q_heads, d->num_kv_heads);
  if (d->num_q_heads / d->num_kv_heads > 16)
    return fail(FSA_ERR_UNSUPPORTED, "dims: query group of %d heads; at most 16 are supported",
                d->num_q_heads / d->num_kv_heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(FSA_ERR_UNSUPPORTED, "dims: head_dim %d; supported are 64 and 128", d->head_dim);
  if (d->page_size != fsa::kPage)
    return fail(FSA_ERR_UNSUPPORTED, "dims: page_size %d; supported is 16", d->page_size);
  if ((long long)d->batch * d->max_pages_per_seq > (1LL << 31) ||
      (long long)d->num_pool_pages * d->num_kv_heads > (1LL << 31))
    return fail(FSA_ERR_UNSUPPORTED, "dims: page table or pool too large");
  return FSA_OK;
}

fsa_status check_cfg(fsa_layer_cfg c) {
  if (c.prefix_tokens < 0 || c.window_tokens < 0 || c.budget_pages < 0)
    return fail(FSA_ERR_INVALID_ARG, "cfg: prefix, window and budget must be >= 0");
  if (c.prefix_tokens == 0 && c.window_tokens == 0 && c.budget_pages == 0)
    return fail(FSA_ERR_INVALID_ARG, "cfg: prefix = window = budget = 0 attends to nothing");
  return FSA_OK;
}

fsa_status check_len(const fsa_dims* d, int32_t max_seq_len) {
  if (max_seq_len < 1 || (long long)max_seq_len > (long long)d->max_pages_per_seq * d->page_size)
    return fail(FSA_ERR_INVALID_ARG, "max_seq_len %d outside [1, max_pages_per_seq * page_size]",
                max_seq_len);
  if ((max_seq_len + fsa::kPage - 1) / fsa::kPage > fsa::select_max_candidates())
    return fail(FSA_ERR_UNSUPPORTED, "max_seq_len %d: more than %d pages per sequence", max_seq_len,
                fsa::select_max_candidates());
  return FSA_OK;
}

fsa_status need(const void* p, const char* name) {
  if (!p) return fail(FSA_ERR_INVALID_ARG, "%s is NULL", name);
  return FSA_OK;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int n_pages_max(int32_t max_seq_len) { return (max_seq_len + fsa::kPage - 1) / fsa::kPage; }

int max_items_of(const fsa_dims* d, fsa_layer_cfg c, int32_t max_seq_len) {
  const long n = n_pages_max(max_seq_len);
  const long pre = std::min<long>((c.prefix_tokens + fsa::kPage - 1) / fsa::kPage, n);
  const long sel = std::min<long>(c.budget_pages, n);
  const long win = std::min<long>((c.window_tokens + fsa::kPage - 1) / fsa::kPage + 1, n);
  (void)d;
  return (int)std::max<long>(1, pre + sel + win);
}

// Candidate pages of a sequence of length L: pages meeting [min(P, L), L - W).
// Nondecreasing in L, so its value at the host bound bounds every sequence.
int candidate_pages(fsa_layer_cfg c, int32_t L) {
  const int Pe = std::min(c.prefix_tokens, L), Ws = std::max(0, L - c.window_tokens);
  return Pe < Ws ? (Ws + fsa::kPage - 1) / fsa::kPage - Pe / fsa::kPage : 0;
}

// Workspace of the sparse step: [scores][selected items (narrow plan)]
// [part_ml][part_o].  Partial slots per unit: the prefix/window workgroups
// first, then one per selection replica (wide plan) or the split-K workgroups
// over the selected items (narrow plan).  When no sequence can have more
// candidate pages than the budget, every candidate is taken, the attended set
// is the whole sequence and the step runs the dense kernels (dense plan).
struct SparseWs {
  size_t scores, sel_work, part_ml, part_o, total;
  int slots;
  bool all_taken;
  fsa::StepPlan step;
  fsa::AttnPlan plan;  // dense plan (all candidates taken) or split-K plan (narrow)
  bool one;            // wide plan as one launch; `one_launch` holds its task sizes
  fsa::OneLaunchArgs one_launch;
};

// When the one-launch form of the wide plan is used (fsa_set_one_launch): 0
// never (the default: it measured no faster than the separate launches from
// 4k to 512k tokens, and slower at 64k and 256k), 1 where it applies and the
// units spread evenly over the XCDs, 2 wherever it applies.
std::atomic<int> g_one_launch_mode{0};

SparseWs sparse_ws(const fsa_dims* d, fsa_layer_cfg c, int32_t max_seq_len) {
  SparseWs w;
  const int units = d->batch * d->num_kv_heads;
  const int G = d->num_q_heads / d->num_kv_heads;
  w.all_taken = candidate_pages(c, max_seq_len) <= c.budget_pages;
  w.one = false;
  w.one_launch = fsa::OneLaunchArgs{};
  size_t o = 0;
  w.scores = o;   o = align256(o + (size_t)units * d->max_pages_per_seq * sizeof(float));
  w.sel_work = o;
  if (w.all_taken) {
    w.step = fsa::StepPlan{0, 0, 0, fsa::PwPlan{0, 1, 0}};
    w.plan = fsa::plan_attention(units, n_pages_max(max_seq_len));
    w.slots = w.plan.wg_per_unit;
  } else {
    w.step = fsa::plan_step(units, d->head_dim, c.prefix_tokens, c.window_tokens, c.budget_pages, max_seq_len);
    w.one = fsa::plan_one_launch(w.step, units, d->head_dim, G, c.prefix_tokens, c.window_tokens, max_seq_len,
                                 g_one_launch_mode.load(std::memory_order_relaxed), &w.one_launch);
    if (w.step.sel_rep > 0) {
      w.plan = fsa::AttnPlan{0, 0};
      w.slots = w.step.pw.wg_per_unit + w.step.sel_rep;
    } else {
      w.plan = fsa::plan_attention(units, w.step.sel_items);
      w.slots = w.step.pw.wg_per_unit + w.plan.wg_per_unit;
      o = align256(o + (size_t)units * w.step.sel_items * 4 * sizeof(int32_t));
    }
  }
  w.part_ml = o;  o = align256(o + (size_t)units * w.slots * G * 2 * sizeof(float));
  w.part_o = o;   o = align256(o + (size_t)units * w.slots * G * d->head_dim * sizeof(float));
  w.total = o;
  return w;
}

struct DenseWs {
  size_t part_ml, part_o, total;
  int max_items;
  fsa::AttnPlan plan;
};

DenseWs dense_ws(const fsa_dims* d, int32_t max_seq_len) {
  DenseWs w;
  const size_t units = (size_t)d->batch * d->num_kv_heads;
  const int G = d->num_q_heads / d->num_kv_heads;
  w.max_items = n_pages_max(max_seq_len);
  w.plan = fsa::plan_attention((int)units, w.max_items);
  size_t o = 0;
  w.part_ml = o;  o = align256(o + units * w.plan.wg_per_unit * G * 2 * sizeof(float));
  w.part_o = o;   o = align256(o + units * w.plan.wg_per_unit * G * d->head_dim * sizeof(float));
  w.total = o;
  return w;
}

fsa::AttnArgs attn_args(const fsa_dims* dims, int max_items, float sm_scale, int32_t max_seq_len,
                        const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* page_table, const int32_t* seq_lens, const int32_t* work,
                        float* part_o, float* part_ml, void* out) {
  fsa::AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.kc = static_cast<const uint16_t*>(k_cache);
  a.vc = static_cast<const uint16_t*>(v_cache);
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.work = work;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.slots_per_unit = 0;
  a.slot_base = 0;
  a.out = static_cast<uint16_t*>(out);
  a.batch = dims->batch;
  a.hq = dims->num_q_heads;
  a.hkv = dims->num_kv_heads;
  a.d = dims->head_dim;
  a.max_pages = dims->max_pages_per_seq;
  a.max_items = max_items;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.max_seq_len = max_seq_len;
  return a;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

}  // namespace

extern "C" {

const char* fsa_last_error(void) { return g_err.c_str(); }

fsa_status fsa_import_kv_plain(const fsa_dims* dims, const void* k_plain, const void* v_plain,
                               void* k_cache, void* v_cache, void* stream) {
  TraceRange trace("fsa_import_kv_plain");
  FSA_CHECK(check_dims(dims));
  FSA_CHECK(need(k_plain, "k_plain"));
  FSA_CHECK(need(v_plain, "v_plain"));
  FSA_CHECK(need(k_cache, "k_cache"));
  FSA_CHECK(need(v_cache, "v_cache"));
  return hip_status(fsa::launch_import_kv_plain(
                        static_cast<const uint16_t*>(k_plain), static_cast<const uint16_t*>(v_plain),
                        static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                        dims->num_pool_pages, dims->num_kv_heads, dims->head_dim,
                        static_cast<hipStream_t>(stream)),
                    "import_kv_plain launch");
}

fsa_status fsa_append_kv(const fsa_dims* dims, int32_t n_new, const void* k_new, const void* v_new,
                         const int32_t* page_table, const int32_t* seq_lens, int32_t* seq_lens_out,
                         void* k_cache, void* v_cache, void* meta, void* stream) {
  TraceRange trace("fsa_append_kv");
  FSA_CHECK(check_dims(dims));
  if (n_new < 1) return fail(FSA_ERR_INVALID_ARG, "n_new must be >= 1");
  FSA_CHECK(need(k_new, "k_new"));
  FSA_CHECK(need(v_new, "v_new"));
  FSA_CHECK(need(page_table, "page_table"));
  FSA_CHECK(need(seq_lens, "seq_lens"));
  FSA_CHECK(need(k_cache, "k_cache"));
  FSA_CHECK(need(v_cache, "v_cache"));
  FSA_CHECK(need(meta, "meta"));
  if (seq_lens_out == seq_lens)
    return fail(FSA_ERR_INVALID_ARG, "seq_lens_out must not alias seq_lens");
  return hip_status(
      fsa::launch_append_kv(n_new, static_cast<const uint16_t*>(k_new),
                            static_cast<const uint16_t*>(v_new), page_table, seq_lens, seq_lens_out,
                            static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                            static_cast<uint16_t*>(meta), dims->batch, dims->num_kv_heads,
                            dims->head_dim, dims->max_pages_per_seq, static_cast<hipStream_t>(stream)),
      "append_kv launch");
}

fsa_status fsa_build_page_meta(const fsa_dims* dims, const void* k_cache, const int32_t* page_table,
                               const int32_t* seq_lens, void* meta, void* stream) {
  TraceRange trace("fsa_build_page_meta");
  FSA_CHECK(check_dims(dims));
  FSA_CHECK(need(k_cache, "k_cache"));
  FSA_CHECK(need(page_table, "page_table"));
  FSA_CHECK(need(seq_lens, "seq_lens"));
  FSA_CHECK(need(meta, "meta"));
  return hip_status(
      fsa::launch_build_page_meta(static_cast<const uint16_t*>(k_cache), page_table, seq_lens,
                                  static_cast<uint16_t*>(meta), dims->batch, dims->num_kv_heads,
                                  dims->head_dim, dims->max_pages_per_seq,
                                  dims->max_pages_per_seq * dims->page_size,
                                  static_cast<hipStream_t>(stream)),
      "build_page_meta launch");
}

fsa_status fsa_quest_scores(const fsa_dims* dims, fsa_layer_cfg cfg, int32_t max_seq_len,
                            const void* q, const void* meta, const int32_t* seq_lens, float* scores,
                            void* stream) {
  TraceRange trace("fsa_quest_scores");
  FSA_CHECK(check_dims(dims));
  FSA_CHECK(check_cfg(cfg));
  FSA_CHECK(check_len(dims, max_seq_len));
  FSA_CHECK(need(q, "q"));
  FSA_CHECK(need(meta, "meta"));
  FSA_CHECK(need(seq_lens, "seq_lens"));
  FSA_CHECK(need(scores, "scores"));
  return hip_status(
      fsa::launch_quest_scores(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(meta),
                               seq_lens, scores, dims->batch, dims->num_q_heads, dims->num_kv_heads,
                               dims->head_dim, dims->max_pages_per_seq, cfg.prefix_tokens,
                               cfg.window_tokens, max_seq_len, static_cast<hipStream_t>(stream)),
      "quest_scores launch");
}

size_t fsa_meta_bytes(const fsa_dims* dims) {
  if (check_dims(dims) != FSA_OK) return 0;
  return (size_t)dims->batch * dims->num_kv_heads * fsa::meta_tiles(dims->max_pages_per_seq) *
         fsa::kMetaTile * 2 * dims->head_dim * sizeof(uint16_t);
}

int32_t fsa_max_work_items(const fsa_dims* dims, fsa_layer_cfg cfg, int32_t max_seq_len) {
  if (check_dims(dims) != FSA_OK || check_cfg(cfg) != FSA_OK || check_len(dims, max_seq_len) != FSA_OK)
    return -1;
  return max_items_of(dims, cfg, max_seq_len);
}

fsa_status fsa_select_pages(const fsa_dims* dims, fsa_layer_cfg cfg, int32_t max_seq_len,
                            const float* scores, const int32_t* page_table, const int32_t* seq_lens,
                            int32_t* sel_pages, int32_t* work, int32_t* counts, void* stream) {
  TraceRange trace("fsa_select_pages");
  FSA_CHECK(check_dims(dims));
  FSA_CHECK(check_cfg(cfg));
  FSA_CHECK(check_len(dims, max_seq_len));
  FSA_CHECK(need(scores, "scores"));
  FSA_CHECK(need(page_table, "page_table"));
  FSA_CHECK(need(seq_lens, "seq_lens"));
  return hip_status(fsa::launch_select_pages(scores, page_table, seq_lens, sel_pages, work, counts,
                                             dims->batch, dims->num_kv_heads,
                                             dims->max_pages_per_seq, cfg.prefix_tokens,
                                             cfg.window_tokens, cfg.budget_pages,
                                             max_items_of(dims, cfg, max_seq_len), max_seq_len,
                                             static_cast<hipStream_t>(stream)),
                    "select_pages launch");
}

size_t fsa_sparse_decode_workspace_bytes(const fsa_dims* dims, fsa_layer_cfg cfg, int32_t max_seq_len) {
  if (check_dims(dims) != FSA_OK || check_cfg(cfg) != FSA_OK || check_len(dims, max_seq_len) != FSA_OK)
    return 0;
  return sparse_ws(dims, cfg, max_seq_len).total;
}

}  // extern "C" (reopened below)

namespace {

// Every host check of a decode step but the workspace's.
fsa_status check_step_args(const fsa_dims* dims, fsa_layer_cfg cfg, float sm_scale, int32_t max_seq_len,
                           const void* q, const void* k_cache, const void* v_cache, const void* meta,
                           const int32_t* page_table, const int32_t* seq_lens, void* out) {
  FSA_CHECK(check_dims(dims));
  FSA_CHECK(check_cfg(cfg));
  FSA_CHECK(check_len(dims, max_seq_len));
  FSA_CHECK(need(q, "q"));
  FSA_CHECK(need(k_cache, "k_cache"));
  FSA_CHECK(need(v_cache, "v_cache"));
  FSA_CHECK(need(meta, "meta"));
  FSA_CHECK(need(page_table, "page_table"));
  FSA_CHECK(need(seq_lens, "seq_lens"));
  FSA_CHECK(need(out, "out"));
  if (!(sm_scale > 0.f)) return fail(FSA_ERR_INVALID_ARG, "sm_scale must be > 0");
  return FSA_OK;
}

fsa_status check_step(const fsa_dims* dims, fsa_layer_cfg cfg, float sm_scale, int32_t max_seq_len, const void* q,
                      const void* k_cache, const void* v_cache, const void* meta, const int32_t* page_table,
                      const int32_t* seq_lens, void* out, void* workspace, size_t workspace_bytes) {
  FSA_CHECK(check_step_args(dims, cfg, sm_scale, max_seq_len, q, k_cache, v_cache, meta, page_table, seq_lens, out));
  const size_t total = sparse_ws(dims, cfg, max_seq_len).total;
  if (!workspace || workspace_bytes < total)
    return fail(FSA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, total);
  return FSA_OK;
}

// The decode step over seq_lens.  With `append`, the step first appends its
// tokens (seq_lens are then the lengths after the append, which it writes):
// inside the scoring launch when that is safe, else as a launch of its own.
fsa_status run_sparse_step(const fsa_dims* dims, fsa_layer_cfg cfg, float sm_scale, int32_t max_seq_len,
                           const void* q, const void* k_cache, const void* v_cache, const void* meta,
                           const int32_t* page_table, const int32_t* seq_lens, void* out, int32_t* sel_pages,
                           void* workspace, hipStream_t st, const fsa::AppendArgs* append,
                           fsa::LaunchFilter* filter = nullptr) {
  fsa::LaunchFilter all;
  fsa::LaunchFilter& mk = filter ? *filter : all;
  const SparseWs w = sparse_ws(dims, cfg, max_seq_len);
  // The scoring launch carries the append when no page the append touches can
  // be a candidate: the touched pages start at or after 16 floor(L0 / 16) and
  // candidates end before L0 + n_new - window, so window >= n_new + 15 suffices.
  const bool fused = append && !w.all_taken && cfg.window_tokens >= append->n_new + fsa::kPage - 1;
  if (append && !fused && mk.take())
    FSA_CHECK(hip_status(fsa::launch_append_kv(append->n_new, append->k_new, append->v_new, append->page_table,
                                               append->seq_lens, append->seq_lens_out, append->kc, append->vc,
                                               append->meta, dims->batch, dims->num_kv_heads, dims->head_dim,
                                               dims->max_pages_per_seq, st),
                         "append_kv launch"));
  if (w.all_taken) {
    // every candidate page is selected: the attended set is [0, L), i.e. dense
    // attention; the selection runs only to report the selected pages (it
    // takes all candidates without looking at scores)
    if (sel_pages && mk.take())
      FSA_CHECK(hip_status(fsa::launch_select_pages(at<float>(workspace, w.scores), page_table, seq_lens, sel_pages,
                                                    nullptr, nullptr, dims->batch, dims->num_kv_heads,
                                                    dims->max_pages_per_seq, cfg.prefix_tokens, cfg.window_tokens,
                                                    cfg.budget_pages, 0, max_seq_len, st),
                           "select_pages launch"));
    const fsa::AttnArgs a = attn_args(dims, n_pages_max(max_seq_len), sm_scale, max_seq_len, q, k_cache, v_cache,
                                      page_table, seq_lens, nullptr, at<float>(workspace, w.part_o),
                                      at<float>(workspace, w.part_ml), out);
    return hip_status(fsa::launch_attention(fsa::kDense, w.plan, a, st, &mk), "dense decode attention launch");
  }
  // one launch for the whole step (the plain step only: the combined call's
  // append runs inside the scoring launch)
  const bool one = w.one && !append;
  if (!one && mk.take())
    FSA_CHECK(hip_status(
      fsa::launch_quest_scores(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(meta),
                               fused ? append->seq_lens : seq_lens, at<float>(workspace, w.scores), dims->batch,
                               dims->num_q_heads, dims->num_kv_heads, dims->head_dim,
                               dims->max_pages_per_seq, cfg.prefix_tokens, cfg.window_tokens,
                               max_seq_len, st, fused ? append : nullptr),
      "quest_scores launch"));
  fsa::StepArgs sa;
  sa.scores = at<float>(workspace, w.scores);
  sa.page_table = page_table;
  sa.seq_lens = seq_lens;
  sa.sel_pages = sel_pages;
  sa.sel_rep = w.step.sel_rep;
  sa.per = w.step.per;
  sa.sel_work = at<int32_t>(workspace, w.sel_work);
  sa.sel_items = w.step.sel_items;
  sa.batch = dims->batch;
  sa.hq = dims->num_q_heads;
  sa.hkv = dims->num_kv_heads;
  sa.d = dims->head_dim;
  sa.max_pages = dims->max_pages_per_seq;
  sa.prefix = cfg.prefix_tokens;
  sa.window = cfg.window_tokens;
  sa.budget = cfg.budget_pages;
  sa.max_seq_len = max_seq_len;
  sa.q = static_cast<const uint16_t*>(q);
  sa.kc = static_cast<const uint16_t*>(k_cache);
  sa.vc = static_cast<const uint16_t*>(v_cache);
  sa.part_o = at<float>(workspace, w.part_o);
  sa.part_ml = at<float>(workspace, w.part_ml);
  sa.slots_per_unit = w.slots;
  sa.pw_ipw = w.step.pw.ipw;
  sa.pw_wg = w.step.pw.wg_per_unit;
  sa.sel_blocks = w.step.sel_blocks;
  sa.xcd_grouped = w.step.xcd_grouped;
  sa.prefetch = w.step.prefetch;
  sa.scale_log2 = sm_scale * 1.4426950408889634f;
  sa.G = dims->num_q_heads / dims->num_kv_heads;
  sa.by_hkv = fsa::make_fastdiv((uint32_t)dims->num_kv_heads);
  sa.by_rep = fsa::make_fastdiv((uint32_t)std::max(1, sa.sel_rep));
  sa.by_pw = fsa::make_fastdiv((uint32_t)std::max(1, sa.pw_wg));
  sa.out = static_cast<uint16_t*>(out);
  if (one) {
    if (!mk.take()) return FSA_OK;
    fsa::OneLaunchArgs o = w.one_launch;
    o.meta = static_cast<const uint16_t*>(meta);
    FSA_CHECK(hip_status(fsa::one_launch_slot(&o.sync), "one-launch step: synchronisation slot"));
    return hip_status(fsa::launch_one_step(sa, o, st), "one-launch step launch");
  }
  if (mk.take()) FSA_CHECK(hip_status(fsa::launch_select_attend(sa, st), "selection launch"));
  fsa::AttnArgs a = attn_args(dims, w.step.sel_items, sm_scale, max_seq_len, q, k_cache, v_cache, page_table, seq_lens,
                              at<int32_t>(workspace, w.sel_work), at<float>(workspace, w.part_o),
                              at<float>(workspace, w.part_ml), out);
  if (w.step.sel_rep > 0)
    return mk.take() ? hip_status(fsa::launch_combine(a, w.slots, st), "combine launch") : FSA_OK;
  a.slots_per_unit = w.slots;
  a.slot_base = w.step.pw.wg_per_unit;
  return hip_status(fsa::launch_attention(fsa::kList, w.plan, a, st, &mk), "decode attention launch");
}

// ---------------------------------------------------------------- allocation-free step
// Workspace of fsa_sparse_decode_attn_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  In host code its name is only a
// host-side stand-in, never a device address: the address of each GPU's copy
// is looked up once per device (with that device current) and kept here.
static __device__ __align__(256) uint8_t scratch[FSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

fsa_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  FSA_CHECK(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices) return fail(FSA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    FSA_CHECK(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (!p) return fail(FSA_ERR_HIP, "hipGetSymbolAddress(scratch) gave no address");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return FSA_OK;
}

}  // namespace

extern "C" {

fsa_status fsa_sparse_decode_attn(const fsa_dims* dims, fsa_layer_cfg cfg, float sm_scale,
                                  int32_t max_seq_len, const void* q, const void* k_cache,
                                  const void* v_cache, const void* meta, const int32_t* page_table,
                                  const int32_t* seq_lens, void* out, int32_t* sel_pages,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  TraceRange trace("fsa_sparse_decode_attn");
  FSA_CHECK(check_step(dims, cfg, sm_scale, max_seq_len, q, k_cache, v_cache, meta, page_table, seq_lens, out,
                       workspace, workspace_bytes));
  return run_sparse_step(dims, cfg, sm_scale, max_seq_len, q, k_cache, v_cache, meta, page_table, seq_lens, out,
                         sel_pages, workspace, static_cast<hipStream_t>(stream), nullptr);
}

fsa_status fsa_sparse_decode_attn_noalloc(const fsa_dims* dims, fsa_layer_cfg cfg, float sm_scale,
                                          int32_t max_seq_len, const void* q, const void* k_cache,
                                          const void* v_cache, const void* meta, const int32_t* page_table,
                                          const int32_t* seq_lens, void* out, int32_t* sel_pages, void* stream) {
  TraceRange trace("fsa_sparse_decode_attn_noalloc");
  // every host check, the size limit included, before any HIP call
  FSA_CHECK(check_step_args(dims, cfg, sm_scale, max_seq_len, q, k_cache, v_cache, meta, page_table, seq_lens, out));
  const size_t total = sparse_ws(dims, cfg, max_seq_len).total;
  if (total > (size_t)FSA_NOALLOC_SCRATCH_BYTES)
    return fail(FSA_ERR_WORKSPACE,
                "this step needs %zu bytes of workspace; the allocation-free call holds at most %zu "
                "(use fsa_sparse_decode_attn with a caller-owned workspace)",
                total, (size_t)FSA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  FSA_CHECK(scratch_of_current_device(&ws));
  return run_sparse_step(dims, cfg, sm_scale, max_seq_len, q, k_cache, v_cache, meta, page_table, seq_lens, out,
                         sel_pages, ws, static_cast<hipStream_t>(stream), nullptr);
}

fsa_status fsa_append_decode_attn(const fsa_dims* dims, int32_t n_new, const void* k_new, const void* v_new,
                                  const int32_t* seq_lens, int32_t* seq_lens_out, fsa_layer_cfg cfg,
                                  float sm_scale, int32_t max_seq_len, const void* q, void* k_cache,
                                  void* v_cache, void* meta, const int32_t* page_table, void* out,
                                  int32_t* sel_pages, void* workspace, size_t workspace_bytes, void* stream) {
  TraceRange trace("fsa_append_decode_attn");
  FSA_CHECK(check_step(dims, cfg, sm_scale, max_seq_len, q, k_cache, v_cache, meta, page_table, seq_lens_out, out,
                       workspace, workspace_bytes));
  if (n_new < 1) return fail(FSA_ERR_INVALID_ARG, "n_new must be >= 1");
  FSA_CHECK(need(k_new, "k_new"));
  FSA_CHECK(need(v_new, "v_new"));
  FSA_CHECK(need(seq_lens, "seq_lens"));
  if (seq_lens_out == seq_lens) return fail(FSA_ERR_INVALID_ARG, "seq_lens_out must not alias seq_lens");
  const fsa::AppendArgs a = fsa::append_args(
      n_new, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), page_table, seq_lens,
      seq_lens_out, static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), static_cast<uint16_t*>(meta),
      dims->num_kv_heads, dims->max_pages_per_seq);
  return run_sparse_step(dims, cfg, sm_scale, max_seq_len, q, k_cache, v_cache, meta, page_table, seq_lens_out,
                         out, sel_pages, workspace, static_cast<hipStream_t>(stream), &a);
}

int32_t fsa_sparse_decode_attn_launches(const fsa_dims* dims, fsa_layer_cfg cfg, float sm_scale,
                                        int32_t max_seq_len, const void* q, const void* k_cache, const void* v_cache,
                                        const void* meta, const int32_t* page_table, const int32_t* seq_lens,
                                        void* out, int32_t* sel_pages, void* workspace, size_t workspace_bytes,
                                        int32_t first, int32_t last, void* stream) {
  TraceRange trace("fsa_sparse_decode_attn_launches");
  if (check_step(dims, cfg, sm_scale, max_seq_len, q, k_cache, v_cache, meta, page_table, seq_lens, out, workspace,
                 workspace_bytes) != FSA_OK)
    return -1;
  fsa::LaunchFilter count;  // how many launches the step has (none is enqueued)
  count.first = 1 << 30;
  if (run_sparse_step(dims, cfg, sm_scale, max_seq_len, q, k_cache, v_cache, meta, page_table, seq_lens, out,
                      sel_pages, workspace, static_cast<hipStream_t>(stream), nullptr, &count) != FSA_OK)
    return -1;
  if (first < 0 || last < first || last >= count.count) {
    fail(FSA_ERR_INVALID_ARG, "launches [%d, %d]: this step has %d launches", first, last, count.count);
    return -1;
  }
  fsa::LaunchFilter some;
  some.first = first;
  some.last = last;
  if (run_sparse_step(dims, cfg, sm_scale, max_seq_len, q, k_cache, v_cache, meta, page_table, seq_lens, out,
                      sel_pages, workspace, static_cast<hipStream_t>(stream), nullptr, &some) != FSA_OK)
    return -1;
  return count.count;
}

int32_t fsa_describe_step(const fsa_dims* dims, fsa_layer_cfg cfg, int32_t max_seq_len, int32_t* info,
                          int32_t n_info) {
  if (check_dims(dims) != FSA_OK || check_cfg(cfg) != FSA_OK || check_len(dims, max_seq_len) != FSA_OK) return -1;
  if (!info || n_info < 0) {
    fail(FSA_ERR_INVALID_ARG, "info must be non-null and n_info >= 0");
    return -1;
  }
  const SparseWs w = sparse_ws(dims, cfg, max_seq_len);
  const int32_t v[11] = {w.all_taken ? 0 : (w.step.sel_rep > 0 ? 1 : 2),
                        w.step.sel_rep,
                        w.step.sel_rep > 0 ? w.step.per : 0,
                        w.step.xcd_grouped,
                        w.step.prefetch,
                        w.all_taken ? 0 : w.step.pw.wg_per_unit,
                        w.slots,
                        fsa::select_columns(max_seq_len),
                        w.all_taken ? 0 : w.step.pw.ipw,
                        w.one ? 1 : 0,
                        w.one ? w.one_launch.n_score : 0};
  const int32_t n = std::min<int32_t>(n_info, 11);
  for (int32_t i = 0; i < n; ++i) info[i] = v[i];
  return n;
}

int32_t fsa_build_flags(void) { return fsa::kBuildFlags; }

int32_t fsa_set_one_launch(int32_t mode) { return g_one_launch_mode.exchange(std::min(2, std::max(0, mode))); }

fsa_status fsa_one_launch_stalls(int64_t* n) {
  FSA_CHECK(need(n, "n"));
  long long v = 0;
  FSA_CHECK(hip_status(fsa::one_launch_stalls(&v), "one-launch stall count"));
  *n = v;
  return FSA_OK;
}

int32_t fsa_device_memory(int32_t* info, int32_t n_info) {
  if (!info || n_info < 0) {
    fail(FSA_ERR_INVALID_ARG, "info must be non-null and n_info >= 0");
    return -1;
  }
  int dev = 0;
  hipDeviceProp_t p;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || hipGetDeviceProperties(&p, dev) != hipSuccess) {
    fail(FSA_ERR_HIP, "no device properties: %s", hipGetErrorString(e));
    return -1;
  }
  const int32_t v[4] = {p.memoryClockRate, p.memoryBusWidth, p.multiProcessorCount, p.l2CacheSize};
  const int32_t n = std::min<int32_t>(n_info, 4);
  for (int32_t i = 0; i < n; ++i) info[i] = v[i];
  return n;
}

fsa_status fsa_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  TraceRange trace("fsa_read_probe");
  FSA_CHECK(need(buf, "buf"));
  FSA_CHECK(need(sink, "sink"));
  if (bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return fail(FSA_ERR_INVALID_ARG, "buf must be 16-byte aligned and bytes a positive multiple of 16 (%zu)", bytes);
  return hip_status(fsa::launch_read_probe(buf, bytes, sink, static_cast<hipStream_t>(stream)), "read probe launch");
}

size_t fsa_dense_decode_workspace_bytes(const fsa_dims* dims, int32_t max_seq_len) {
  if (check_dims(dims) != FSA_OK || check_len(dims, max_seq_len) != FSA_OK) return 0;
  return dense_ws(dims, max_seq_len).total;
}

fsa_status fsa_dense_decode_attn(const fsa_dims* dims, float sm_scale, int32_t max_seq_len,
                                 const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* page_table, const int32_t* seq_lens, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  TraceRange trace("fsa_dense_decode_attn");
  FSA_CHECK(check_dims(dims));
  FSA_CHECK(check_len(dims, max_seq_len));
  FSA_CHECK(need(q, "q"));
  FSA_CHECK(need(k_cache, "k_cache"));
  FSA_CHECK(need(v_cache, "v_cache"));
  FSA_CHECK(need(page_table, "page_table"));
  FSA_CHECK(need(seq_lens, "seq_lens"));
  FSA_CHECK(need(out, "out"));
  if (!(sm_scale > 0.f)) return fail(FSA_ERR_INVALID_ARG, "sm_scale must be > 0");
  const DenseWs w = dense_ws(dims, max_seq_len);
  if (!workspace || workspace_bytes < w.total)
    return fail(FSA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, w.total);
  const fsa::AttnArgs a = attn_args(dims, w.max_items, sm_scale, max_seq_len, q, k_cache, v_cache,
                                    page_table, seq_lens, nullptr, at<float>(workspace, w.part_o),
                                    at<float>(workspace, w.part_ml), out);
  return hip_status(fsa::launch_attention(fsa::kDense, w.plan, a, static_cast<hipStream_t>(stream)),
                    "dense decode attention launch");
}

fsa_status fsa_validate_inputs(const fsa_dims* dims, int32_t n_new, int32_t max_seq_len, const void* q,
                               const int32_t* page_table, const int32_t* seq_lens, int32_t* scratch,
                               void* stream) {
  TraceRange trace("fsa_validate_inputs");
  FSA_CHECK(check_dims(dims));
  FSA_CHECK(check_len(dims, max_seq_len));
  if (n_new < 0) return fail(FSA_ERR_INVALID_ARG, "n_new must be >= 0");
  FSA_CHECK(need(page_table, "page_table"));
  FSA_CHECK(need(seq_lens, "seq_lens"));
  FSA_CHECK(need(scratch, "scratch"));
  hipStream_t st = static_cast<hipStream_t>(stream);
  FSA_CHECK(hip_status(fsa::launch_validate(static_cast<const uint16_t*>(q), page_table, seq_lens, scratch,
                                            dims->batch, q ? dims->num_q_heads : 0, dims->head_dim,
                                            dims->max_pages_per_seq, dims->num_pool_pages, max_seq_len, n_new,
                                            st),
                       "validate launch"));
  int32_t h[4];
  FSA_CHECK(hip_status(hipMemcpyAsync(h, scratch, sizeof(h), hipMemcpyDeviceToHost, st), "validate copy"));
  FSA_CHECK(hip_status(hipStreamSynchronize(st), "validate sync"));
  if (h[0] == 0) return FSA_OK;
  switch (h[1]) {
    case 1:
      if (n_new > 0)
        return fail(FSA_ERR_INVALID_ARG, "%d invalid inputs; e.g. seq_lens[%d] = %d: with %d new tokens outside [0, %d]",
                    h[0], h[2], h[3], n_new, max_seq_len - n_new);
      return fail(FSA_ERR_INVALID_ARG, "%d invalid inputs; e.g. seq_lens[%d] = %d outside [1, %d]", h[0], h[2], h[3],
                  max_seq_len);
    case 4:
      return fail(FSA_ERR_INVALID_ARG,
                  "%d invalid inputs; e.g. sequence %d overflows its page table: seq_lens[%d] = %d plus %d new tokens "
                  "exceeds %d pages of 16 tokens",
                  h[0], h[2], h[2], h[3], n_new, dims->max_pages_per_seq);
    case 2:
      return fail(FSA_ERR_INVALID_ARG, "%d invalid inputs; e.g. page_table[%d][%d] outside [0, %d)", h[0], h[2], h[3],
                  dims->num_pool_pages);
    default:
      return fail(FSA_ERR_INVALID_ARG, "%d invalid inputs; e.g. q element %d is not finite", h[0], h[2]);
  }
}

}  // extern "C"
