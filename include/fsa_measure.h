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

#ifdef __cplusplus
}
#endif

#endif /* FSA_MEASURE_H */
