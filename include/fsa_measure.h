/*
 * fsa_measure.h -- measurement helpers exported by the same library as fsa.h.
 *
 * They are not part of the decode step.  Long-context decoding is bound by
 * reading keys from memory (digest page "Accelerating Long-Context Decoding
 * in Large-Scale Hybrid LLMs Without Retraining", opening paragraph and "Why
 * It Matters"), so the step's kernels are compared with what this device's
 * memory can deliver; these calls report that ceiling.
 */
#ifndef FSA_MEASURE_H
#define FSA_MEASURE_H

#include "fsa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Properties of the current device, up to n_info of
 *   info[0] memory clock (kHz), info[1] memory bus width (bits),
 *   info[2] compute units, info[3] L2 cache bytes (one XCD's).
 * Returns the number written, or -1 with fsa_last_error() set (no device, or
 * info NULL / n_info < 0). */
int32_t fsa_device_memory(int32_t* info, int32_t n_info);

/* Reads the `bytes` at buf once with coalesced 16-byte non-temporal loads, on
 * all compute units; its rate is the plain-read ceiling.
 *   buf   device, 16-byte aligned; bytes a positive multiple of 16
 *   sink  one device word, written at most once with a value of no meaning
 * Asynchronous on stream; FSA_ERR_INVALID_ARG before any launch on bad
 * arguments. */
fsa_status fsa_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* How this library was built: bit 0 set in the debug build whose kernels fill
 * their LDS with a NaN pattern at the start and between stages that reuse it
 * (libfsa_poison.so, -DFSA_DEBUG_POISON_LDS); 0 in the release build.  Host
 * only, no device needed. */
int32_t fsa_build_flags(void);

/* When later calls in this process use the one-launch form of the wide plan
 * (fsa_describe_step info[9]), so that both forms can be timed and checked on
 * the same inputs: mode 0 never (the default), 1 where it applies and the
 * (sequence, KV head) units are a multiple of 8 (each unit's tasks run on one
 * of the 8 XCDs), 2 wherever it applies (any unit count up to 64).  Other
 * values are clamped to 0..2.  Returns the previous mode.  Host only. */
int32_t fsa_set_one_launch(int32_t mode);

/* Waits that one-launch steps on the current device gave up on, summed since
 * the library was loaded: each wait of the one-launch kernel for another
 * task is bounded (about a second), and a step whose queues were not all
 * emptied counts one too.  Nonzero means a step's result is wrong.
 * Synchronises the device.  FSA_ERR_HIP on a failed device call. */
fsa_status fsa_one_launch_stalls(int64_t* n);

/* Some of the launches of the fsa_sparse_decode_attn step, so that parts of
 * the step can be timed: runs only launches first..last (0-based, inclusive)
 * of the step these arguments describe.  The launches, in order: dense plan
 * -- [selection, when sel_pages is given], split-K attention, [combine]; wide
 * plan -- scoring, selection launch (selection replicas + prefix/window
 * attention), combine, or in its one-launch form that one launch; narrow
 * plan -- scoring, selection launch, split-K
 * attention, combine (fsa_describe_step names the plan).  A launch reads what
 * the earlier ones left in the workspace, so when first > 0 a whole step with
 * the same arguments and workspace must have run before on the stream.
 * Returns the number of launches of the step, or -1 with fsa_last_error() set
 * (the checks of fsa_sparse_decode_attn, a range outside [0, launches), a
 * failed launch). */
int32_t fsa_sparse_decode_attn_launches(const fsa_dims* dims, fsa_layer_cfg cfg, float sm_scale,
                                        int32_t max_seq_len, const void* q, const void* k_cache, const void* v_cache,
                                        const void* meta, const int32_t* page_table, const int32_t* seq_lens,
                                        void* out, int32_t* sel_pages, void* workspace, size_t workspace_bytes,
                                        int32_t first, int32_t last, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FSA_MEASURE_H */
