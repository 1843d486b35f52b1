/*
 * moedc_ceiling.h -- measurement kernels (libmoedc_ceiling.so), not part of
 * the MoE path: what one MI355X's memory system delivers for plain streams
 * and for the exact access patterns of dispatch and combine, so that their
 * achieved bandwidth can be read against a measured ceiling as well as the
 * 8 TB/s HBM peak, and the compute floor of the expert layer's instruction
 * mix, read against the 5 POP/s int8 peak likewise.  The pages measure their operators the same way against
 * their fabric ("StrataCL 深度技术分析", section 4.1: bus bandwidth of
 * dispatch and combine).
 *
 * Every call enqueues one kernel on `stream` and returns the launch's
 * hipError_t (0 on success).  Device pointers are 16-byte aligned, byte
 * counts multiples of 16.  No arithmetic of the method runs in them: the
 * memory kernels move data only, the MFMA kernel computes on constants.
 */
#ifndef MOEDC_CEILING_H
#define MOEDC_CEILING_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` at src with 16-byte non-temporal loads, one workgroup per
 * 16 KiB (4 loads per thread); a fold of the values goes to sink[0] only if
 * it equals a value no input produces, so the loads cannot be dropped.
 * sink: device uint32 [1].  The plain streams use short-lived workgroups
 * started in address order, the fastest pattern measured on MI355X. */
int32_t moedc_ceiling_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream);

/* Writes `bytes` at dst with 16-byte ordinary stores, one workgroup per
 * 4 KiB. */
int32_t moedc_ceiling_write(void *dst, int64_t bytes, hipStream_t stream);

/* Copies `bytes` from src to dst with 16-byte non-temporal loads and
 * stores, one workgroup per 4 KiB. */
int32_t moedc_ceiling_copy(void *dst, const void *src, int64_t bytes, hipStream_t stream);

/* Dispatch's store pattern without its loads or arithmetic: for each of T
 * tokens, a workgroup writes bytes [0, row_bytes) of each of the token's K
 * slots (slots: device int32 [T][K], -1 skipped) at slot * slot_stride in
 * dbuf, one wave per 512 bytes, 8 bytes per lane per store, ordinary
 * (cached) stores -- the payload stores of moedc_dispatch.  row_bytes: a multiple of 8, at most
 * 8192. */
int32_t moedc_ceiling_scatter(const int32_t *slots, int32_t T, int32_t K, void *dbuf,
                              int64_t slot_stride, int32_t row_bytes, hipStream_t stream);

/* Combine's load pattern without its arithmetic: for each token and each
 * 1024-byte chunk of a row of row_bytes, one wave reads that chunk of the
 * token's K rows (rows + slot * row_stride; -1 skipped) with 16-byte
 * non-temporal loads and writes their bitwise XOR to out[t] (row_bytes per
 * token), 16-waves workgroups -- the traffic of moedc_combine on BF16
 * expert outputs.  row_bytes: a multiple of 16, at most 16384. */
int32_t moedc_ceiling_gather(const void *rows, const int32_t *slots, int32_t T, int32_t K,
                             int64_t row_stride, int32_t row_bytes, void *out, hipStream_t stream);

/* The expert layer's compute floor: about mfma_total v_mfma_i32_16x16x64_i8
 * (rounded down to whole steps of 32 per wave) issued from registers by 256
 * workgroups of 8 waves (two per SIMD), with no memory traffic; with fold
 * != 0 each wave also folds its 64 int32 sums into fp32 after every 32
 * MFMAs (a convert and an FMA each), the per-group work of 128-input
 * activation scales.  sink: device uint32 [1], written only if a fold of
 * the results hits a value none produces. */
int32_t moedc_ceiling_mfma(int64_t mfma_total, int32_t fold, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEDC_CEILING_H */
