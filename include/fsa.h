/*
 * fsa.h -- combined sparse decode attention on gfx950 (AMD Instinct MI355X).
 *
 * One decode step of one full-attention layer: every query attends to the
 * union of a pinned prefix, a sliding window of recent tokens and a fixed
 * budget of KV pages picked query-aware from per-page key bounds.
 *   - Paper "Accelerating Long-Context Decoding in Large-Scale Hybrid LLMs
 *     Without Retraining" (Batista, Vatai, Wahib), Abstract: window, prefix and
 *     a fixed budget of the most relevant tokens, configured per layer.
 *   - Same paper, analysis page "Methodology" and digest page "The Move":
 *     the budget is a Quest-style, query-aware paged top-k.
 *   - Digest page "Why It Matters": the KV cache is kept at full size, so any
 *     page can be selected.
 *   - Quest (Tang et al., ICML 2024): per page the elementwise min m and max M
 *     of its keys; sum_i max(q_i m_i, q_i M_i) bounds q.k over the page.
 *
 * Conventions for every entry point
 *   - Pointers marked "device" point to GPU memory; the caller allocates and
 *     owns every buffer.  The library allocates nothing; its only state is a
 *     thread-local error message and device properties (CU count, kernel
 *     occupancy) cached on first use.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *     returns without synchronising: no allocation, no memset, no host
 *     synchronisation, so calls can be captured into a HIP graph.
 *   - Host-detectable argument errors return a non-zero fsa_status before any
 *     launch; fsa_last_error() then describes it.  A failed launch returns
 *     FSA_ERR_HIP.  Device-resident data (page tables, lengths) is trusted.
 *   - bf16 tensors are raw IEEE bfloat16 bit patterns.
 *
 * Why the cache layout is not the common token-major [pool][Hkv][S][D]
 *   The decode step reads each selected page once, straight into the matrix
 *   cores.  With K stored chunk-major ([D/8][S][8]) one 64-lane load of a
 *   page's K is one contiguous 1 KiB row in exactly the operand order of a
 *   16x16x32 bf16 MFMA step, and with V stored channel-major ([D][S]) the P.V
 *   operand of a lane is 8 contiguous bytes.  A cache kept by a model in the
 *   token-major layout is adopted once with fsa_import_kv_plain (and its
 *   metadata built with fsa_build_page_meta); fsa_append_kv then keeps both
 *   current.  Metadata is per (sequence, logical page) rather than per pool
 *   page: it is derived state of the sequence, so the scoring pass streams it
 *   without a page-table lookup.
 *
 * Device layouts (row-major, no padding)
 *   q, out      bf16  [B][Hq][D]            query head h reads KV head h / (Hq/Hkv)
 *   k_cache     bf16  [pool][Hkv][D/8][S][8] K of token slot j, channel c of a page
 *                                           sits at [c/8][j][c%8]
 *   v_cache     bf16  [pool][Hkv][D][S]      V stored channel-major inside a page
 *   meta        bf16  [B][Hkv][T][2D/32][16][32] with T = ceil(max_pages_per_seq / 16):
 *                                           the elementwise min and max of the valid
 *                                           keys of logical page p of sequence b, KV
 *                                           head g, in tiles of 16 logical pages.
 *                                           Value e of page p (e < D: min of channel e;
 *                                           e >= D: max of channel e - D) sits at
 *                                           [b][g][p / 16][e / 32][p % 16][e % 32].
 *                                           A zero is stored as +0.  Size in bytes:
 *                                           fsa_meta_bytes().
 *   page_table  int32 [B][max_pages_per_seq] logical page -> pool page
 *   seq_lens    int32 [B]                    tokens in the cache, including the
 *                                           current token (the query's position
 *                                           is seq_lens[b] - 1)
 * Supported: D in {64, 128}; S = 16; Hq / Hkv in 1..16; seq_lens[b] >= 1;
 * at most 32768 pages (512k tokens) per sequence.  max_seq_len arguments are
 * host-side upper bounds of seq_lens used to size grids and workspaces;
 * device lengths above the bound are clamped to it.
 */
#ifndef FSA_H
#define FSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FSA_OK = 0,
  FSA_ERR_INVALID_ARG = 1, /* a null pointer, a negative size, an inconsistent shape */
  FSA_ERR_UNSUPPORTED = 2, /* a shape outside the supported set above */
  FSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the sizing call says */
  FSA_ERR_HIP = 4          /* a HIP runtime call or launch failed */
} fsa_status;

typedef struct {
  int32_t batch;             /* B */
  int32_t num_q_heads;       /* Hq, a multiple of Hkv */
  int32_t num_kv_heads;      /* Hkv */
  int32_t head_dim;          /* D */
  int32_t page_size;         /* S, tokens per page */
  int32_t max_pages_per_seq; /* columns of page_table; also sizes meta (kept per sequence) */
  int32_t num_pool_pages;    /* pages in k_cache and v_cache */
} fsa_dims;

/* Per-layer configuration (paper, Abstract: window and budget are chosen per
 * layer; the prefix is pinned).  The attended set of a sequence of length L is
 * [0, min(P, L)) U [max(0, L - W), L) U the tokens of the selected pages.
 * Candidates for selection are the pages that intersect [min(P, L), L - W);
 * k = min(budget_pages, candidates) of them are kept. */
typedef struct {
  int32_t prefix_tokens; /* P >= 0 */
  int32_t window_tokens; /* W >= 0 */
  int32_t budget_pages;  /* >= 0; P = W = budget = 0 is rejected */
} fsa_layer_cfg;

/* Text of the last non-OK status returned on the calling thread. */
const char* fsa_last_error(void);

/* Adopt a cache written in the common token-major paged layout: converts
 * k_plain and v_plain, bf16 [pool][Hkv][S][D] (device), into k_cache and
 * v_cache (device, layouts above) for every pool page.  Inputs and outputs
 * must not overlap.  Metadata is not touched (see fsa_build_page_meta). */
fsa_status fsa_import_kv_plain(const fsa_dims* dims, const void* k_plain, const void* v_plain,
                               void* k_cache, void* v_cache, void* stream);

/* Append n_new >= 1 tokens to every sequence and keep the page metadata
 * current: the per-page elementwise key minimum and maximum that Quest's
 * bound needs (analysis page "Methodology" and digest page "The Move" name
 * Quest as the selection rule; the decode step of the paper's Abstract runs
 * after each new token).  Token i of sequence b goes to position
 * seq_lens[b] + i, i.e. page page_table[b][pos / S], slot pos % S; those
 * page-table entries must already be mapped.
 *   k_new, v_new  bf16 [B][n_new][Hkv][D] (device)
 *   seq_lens      int32 [B] (device), lengths before the append
 *   seq_lens_out  int32 [B] (device) or NULL; receives the lengths after the
 *                 append, seq_lens[b] + n_new (must not alias seq_lens)
 * A page whose slot 0 is written by this call gets fresh metadata from the
 * new tokens only; otherwise the new tokens' min/max are merged into the
 * existing entry.  The result equals fsa_build_page_meta bit for bit.
 * Capacity: positions at or past max_pages_per_seq * S have no page and are
 * not written; seq_lens_out then counts only the tokens written
 * (min(seq_lens[b] + n_new, max_pages_per_seq * S)).  Lengths live on the
 * device, so the host cannot see this; fsa_validate_inputs with n_new
 * reports it before the append. */
fsa_status fsa_append_kv(const fsa_dims* dims, int32_t n_new, const void* k_new, const void* v_new,
                         const int32_t* page_table, const int32_t* seq_lens, int32_t* seq_lens_out,
                         void* k_cache, void* v_cache, void* meta, void* stream);

/* Recompute the metadata of every page in use (logical pages
 * [0, ceil(seq_lens[b] / S)) of every sequence) from k_cache, over each
 * page's valid slots only: Quest's per-page elementwise key minimum and
 * maximum (the selection rule of the analysis page's "Methodology" and the
 * digest's "The Move"), for a cache filled by prefill or adopted with
 * fsa_import_kv_plain.  Entries of pages not in use are not written.
 *   k_cache   bf16, layout above (device)
 *   meta      bf16, layout above (device), fsa_meta_bytes() bytes
 * Exact (min and max involve no rounding); asynchronous on stream. */
fsa_status fsa_build_page_meta(const fsa_dims* dims, const void* k_cache, const int32_t* page_table,
                               const int32_t* seq_lens, void* meta, void* stream);

/* Bytes of the page-metadata buffer for these dims (0 on invalid dims). */
size_t fsa_meta_bytes(const fsa_dims* dims);

/* Quest scores of the candidate pages: the query-aware relevance that the
 * paged top-k ranks by (analysis page "Methodology", digest page "The
 * Move"; the bound is Quest's).  For every (b, KV head g) and every
 * candidate logical page p:
 *     scores[b][g][p] = max over query heads h of group g of
 *                       sum_i max(q[b][h][i] * m[p][i], q[b][h][i] * M[p][i])
 * in fp32 (the group shares one selection; the maximum bounds every head).
 * scores: fp32 [B][Hkv][max_pages_per_seq] (device); entries of
 * non-candidate pages are not written.  max_seq_len is a host-side upper
 * bound of seq_lens used to size the grid. */
fsa_status fsa_quest_scores(const fsa_dims* dims, fsa_layer_cfg cfg, int32_t max_seq_len,
                            const void* q, const void* meta, const int32_t* seq_lens, float* scores,
                            void* stream);

/* Number of work items per (b, KV head) that fsa_select_pages can emit. */
int32_t fsa_max_work_items(const fsa_dims* dims, fsa_layer_cfg cfg, int32_t max_seq_len);

/* Top-k selection and merge with the prefix and the window: the fixed
 * budget of most relevant pages next to the pinned prefix and the sliding
 * window (paper, Abstract; a paged top-k per the digest's "The Move").
 * For every (b, g): the k = min(budget, C) candidate pages with the largest
 * scores; equal scores go to the lower logical page id; -0 equals +0.
 *   sel_pages  int32 [B][Hkv][budget_pages] (device) or NULL: selected logical
 *              page ids, ascending, then -1 padding
 *   work       int32 [B][Hkv][max_items][4] (device) or NULL, max_items =
 *              fsa_max_work_items(): the attended tokens as (logical page,
 *              pool page, first slot, end slot) items in ascending token
 *              order; every attended token appears in exactly one item, and
 *              every such item is non-empty.  Entries after the last item
 *              are empty items (-1, 0, 0, 0), so the whole array is defined.
 *   counts     int32 [B][Hkv][2] (device) or NULL: (k, number of items)
 * Scores of non-candidate pages below ceil(max_seq_len / S) are read but not
 * used, so they need not be initialised. */
fsa_status fsa_select_pages(const fsa_dims* dims, fsa_layer_cfg cfg, int32_t max_seq_len,
                            const float* scores, const int32_t* page_table, const int32_t* seq_lens,
                            int32_t* sel_pages, int32_t* work, int32_t* counts, void* stream);

/* Workspace (device bytes) that fsa_sparse_decode_attn needs. */
size_t fsa_sparse_decode_workspace_bytes(const fsa_dims* dims, fsa_layer_cfg cfg, int32_t max_seq_len);

/* The whole decode step of one full-attention layer (paper, Abstract: the
 * query attends to the pinned prefix, the sliding window and a fixed budget
 * of the most relevant tokens; analysis page "Methodology" and digest page
 * "The Move": chosen by a Quest-style paged top-k; digest page "Why It
 * Matters": the cache stays full size, so every page can be chosen):
 * scores, selection and merge, then split-K flash decoding over the
 * attended tokens (fp32 logits, online softmax and fp32 accumulation) and
 * the cross-split combine.
 *   out        bf16 [B][Hq][D] (device): softmax(sm_scale * q.K) V over the
 *              attended set, rounded to nearest-even bf16
 *   sel_pages  as in fsa_select_pages, or NULL
 *   workspace  device, at least fsa_sparse_decode_workspace_bytes(); no
 *              initial contents needed; calls that share one workspace must
 *              be ordered (same stream) */
fsa_status fsa_sparse_decode_attn(const fsa_dims* dims, fsa_layer_cfg cfg, float sm_scale,
                                  int32_t max_seq_len, const void* q, const void* k_cache,
                                  const void* v_cache, const void* meta, const int32_t* page_table,
                                  const int32_t* seq_lens, void* out, int32_t* sel_pages,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes the allocation-free decode step holds per GPU. */
#define FSA_NOALLOC_SCRATCH_BYTES (16u << 20)

/* fsa_sparse_decode_attn without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The caller still passes every
 * input and output; the step's workspace (scores, selected items, split
 * partials) is a device array inside the library of FSA_NOALLOC_SCRATCH_BYTES
 * bytes, one per GPU, held until the process ends.  The call allocates
 * nothing; its first call on a device looks up that device's copy of the
 * array.  Steps whose workspace (fsa_sparse_decode_workspace_bytes) exceeds
 * the array return FSA_ERR_WORKSPACE before any HIP call.  Every call on one
 * GPU shares that GPU's array: calls that may overlap (different streams, or
 * several threads) race and must be ordered by the caller.  The array needs
 * no initial contents.  Arguments and results otherwise as in
 * fsa_sparse_decode_attn, whose kernels it runs: the results are the same
 * bit for bit. */
fsa_status fsa_sparse_decode_attn_noalloc(const fsa_dims* dims, fsa_layer_cfg cfg, float sm_scale,
                                          int32_t max_seq_len, const void* q, const void* k_cache,
                                          const void* v_cache, const void* meta, const int32_t* page_table,
                                          const int32_t* seq_lens, void* out, int32_t* sel_pages, void* stream);

/* How fsa_sparse_decode_attn will run a step of these shapes on the current
 * device (host only: no device memory is touched; queries the device's
 * compute-unit count, 256 when there is no device).  Writes up to n_info of:
 *   info[0]  plan: 0 = every candidate fits the budget (dense kernels),
 *            1 = wide (selection replicas attend the selected pages),
 *            2 = narrow (one selection per unit, split-K launch)
 *   info[1]  selection replicas per (b, KV head) unit (wide plan), else 0
 *   info[2]  selected items each replica attends (wide plan), else 0
 *   info[3]  1 if a unit's replicas are placed on one XCD
 *   info[4]  1 if the replicas prefetch known-taken pages into that L2
 *   info[5]  prefix/window workgroups per unit
 *   info[6]  partial slots per unit (merged by the combine)
 *   info[7]  pages per selection thread (a power of two)
 *   info[8]  prefix/window items each wave of a prefix/window workgroup
 *            attends (16 waves per workgroup)
 *   info[9]  1 if the wide plan runs as one launch (scoring, selection,
 *            prefix/window attention and the merge of the partials as tasks
 *            of one launch, each unit's tasks on one XCD); the call with an
 *            append (fsa_append_decode_attn) keeps the separate launches
 *   info[10] scoring tasks per unit in that launch, else 0
 * Returns the number of entries written, or -1 with fsa_last_error() set. */
int32_t fsa_describe_step(const fsa_dims* dims, fsa_layer_cfg cfg, int32_t max_seq_len, int32_t* info,
                          int32_t n_info);

/* fsa_append_kv followed by fsa_sparse_decode_attn on the same stream, as one
 * call: the decode step of a model that has just produced the new tokens'
 * K/V (the per-layer decode step of the paper's Abstract and the digest
 * page's "The Move", over a cache that grows by n_new tokens first).  Results (caches, metadata, seq_lens_out, out, sel_pages) equal those
 * of the two calls bit for bit.  When no page the append writes can be a
 * candidate of the step (window_tokens >= n_new + 15, and more candidates
 * than the budget) the append runs inside the scoring launch, one launch
 * fewer; otherwise it runs as its own launch first.
 *   seq_lens      int32 [B] (device), lengths before the append
 *   seq_lens_out  int32 [B] (device), receives seq_lens[b] + n_new: the
 *                 lengths the decode step uses; must not alias seq_lens
 *   max_seq_len   host upper bound on the lengths after the append
 *   workspace     fsa_sparse_decode_workspace_bytes(dims, cfg, max_seq_len)
 * Other arguments as in fsa_append_kv and fsa_sparse_decode_attn. */
fsa_status fsa_append_decode_attn(const fsa_dims* dims, int32_t n_new, const void* k_new, const void* v_new,
                                  const int32_t* seq_lens, int32_t* seq_lens_out, fsa_layer_cfg cfg,
                                  float sm_scale, int32_t max_seq_len, const void* q, void* k_cache,
                                  void* v_cache, void* meta, const int32_t* page_table, void* out,
                                  int32_t* sel_pages, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace (device bytes) that fsa_dense_decode_attn needs. */
size_t fsa_dense_decode_workspace_bytes(const fsa_dims* dims, int32_t max_seq_len);

/* Plain decode attention over all tokens [0, seq_lens[b]) with the same
 * split-K kernels: the full attention whose every-step read of all keys the
 * method avoids (digest page, opening and "Why It Matters"), kept as the
 * baseline that the sparse step is measured against, and the result the
 * sparse step must equal when its budget covers every page.
 *   q, out  bf16 [B][Hq][D] (device); caches and page table as above
 * The workspace needs no initial contents; FSA_ERR_WORKSPACE if it is
 * smaller than fsa_dense_decode_workspace_bytes(). */
fsa_status fsa_dense_decode_attn(const fsa_dims* dims, float sm_scale, int32_t max_seq_len,
                                 const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* page_table, const int32_t* seq_lens, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Debug check of the device-resident inputs of a decode step or of an
 * append; unlike every other call it synchronises `stream` and is not
 * graph-capturable.  With n_new = 0 (a decode step) it checks that every
 * seq_lens[b] lies in [1, max_seq_len].  With n_new > 0 (an append of n_new
 * tokens, before it runs) it checks that seq_lens[b] >= 0, that
 * seq_lens[b] + n_new fits the page table (max_pages_per_seq * S tokens;
 * a sequence that does not is named as overflowing it) and that it is at
 * most max_seq_len.  Either way page_table[b][p] must lie in
 * [0, num_pool_pages) for every page p < ceil((seq_lens[b] + n_new) / S),
 * and every value of q (bf16 [B][Hq][D], device; may be NULL to skip) must
 * be finite.  The other entry points trust these values.
 *   scratch  int32[4] (device), caller-owned, no initial contents needed
 * Returns FSA_OK, or FSA_ERR_INVALID_ARG with fsa_last_error() naming the
 * number of violations and one of them. */
fsa_status fsa_validate_inputs(const fsa_dims* dims, int32_t n_new, int32_t max_seq_len, const void* q,
                               const int32_t* page_table, const int32_t* seq_lens, int32_t* scratch,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FSA_H */
