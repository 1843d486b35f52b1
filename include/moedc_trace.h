/*
 * moedc_trace.h -- the trace build of libmoedc (libmoedc_trace.so): the
 * same library, entry points and results, except that every wave of the
 * large-batch dispatch kernel records when it passes each phase of the
 * token pipeline of "CloudMatrix384: Co-Designing Supernodes for
 * Trillion-Parameter LLM Inference", section "FusedDispatch and
 * FusedCombine" (load, quantize/address, write), in the manner of the
 * per-core phase probes of "StrataCL 深度技术分析" (its NPU-side profiler
 * section).  Debug and measurement only; libmoedc.so carries none of it.
 *
 * Record (64 bytes, eight uint64 words) per (token t, wave c) of a
 * moedc_dispatch call on a batch above 16 tokens (or with one scale per
 * token), at index t * waves_per_token + c, waves_per_token = ceil(H / 512):
 *   [0] t << 32 | c
 *   [1] XCC_ID << 32 | HW_ID   (the wave's die, shader engine, CU, SIMD)
 *   [2] start   [3] chunk loaded   [4] scales known   [5] quantized
 *   [6] stores issued   [7] stores complete
 * Times are ticks of the GPU's 100 MHz constant clock (10 ns).  Records
 * past the buffer's capacity are not written.
 */
#ifndef MOEDC_TRACE_H
#define MOEDC_TRACE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Sets the trace buffer of the current device for later dispatch calls:
 * buf = device memory of `bytes` bytes (64-byte records), or NULL to stop
 * tracing.  The caller owns the buffer and must not free it while a traced
 * dispatch may run.  Synchronous with respect to the device (a symbol
 * copy); call it while no dispatch is in flight.  Returns the hipError_t of
 * the copies (0 on success).  Exported by libmoedc_trace.so only. */
int32_t moedc_trace_set(void *buf, int64_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* MOEDC_TRACE_H */
