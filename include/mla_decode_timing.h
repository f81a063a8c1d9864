/*
 * mla_decode_timing.h -- measurement hook of the MI355X (gfx950) MLA decode
 * library.  Not part of the decode interface (include/mla_decode.h): it exists
 * so that a benchmark can time the split-KV decode kernel alone, apart from
 * the split combine that mla_decode_partial enqueues after it, with events
 * recorded on the stream the kernel runs on.
 */
#ifndef MLA_DECODE_TIMING_H
#define MLA_DECODE_TIMING_H

#include "mla_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/* mla_decode_partial (same arguments, results, validation and errors), which
 * additionally records the two hipEvent_t (passed as void*; either may be
 * NULL) on `stream` immediately before and after the split-KV decode kernel.
 * The events add a few microseconds to the call; a caller that does not time
 * the kernel uses mla_decode_partial. */
int mla_decode_partial_timed(const mla_decode_desc* desc, const void* q, const void* kv_cache,
                             const float* kv_scale, const int32_t* block_table,
                             const int32_t* seq_lens, float scale, void* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* event_before_decode, void* event_after_decode);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_TIMING_H */
