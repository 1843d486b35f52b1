/*
 * moedc_oracle.h -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.
 *
 * Plain, slow, single-threaded CPU oracle for MoE token routing, INT8
 * dispatch and gate-weighted combine.  Only the test suite, the package's
 * smoke entry point and the benchmark's CPU-baseline leg may load or call
 * it.  It shares no header, helper, table or constant with the HIP library
 * (libmoedc); the two are written independently from the same pages.
 *
 * Sources (page title, section):
 *  [CM]  "CloudMatrix384: Co-Designing Supernodes for Trillion-Parameter LLM
 *        Inference" -- sections "Decode Phase" (EP320 expert placement:
 *        256 routed + 32 shared + 32 redundant experts, 96 local tokens,
 *        30,720 global), "FusedDispatch and FusedCombine" (three exchanges
 *        fused into two operators; INT8 with a scale before sending;
 *        separate statically pre-allocated dispatch and combine buffers;
 *        token-granular pipeline) and "INT8 Quantization" (dynamic
 *        per-token activation scales; gating left in BF16).
 *  [SC]  "StrataCL 深度技术分析" -- section 4.1 (MoE dispatch/combine at
 *        hidden 7168, top-8).
 *
 * Where the pages leave a step open, the readings used are listed next to
 * each function below.
 */
#ifndef MOEDC_ORACLE_H
#define MOEDC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_SCORE_SOFTMAX = 0, ORC_SCORE_SIGMOID_NORM = 1 };
enum { ORC_FMT_BF16 = 0, ORC_FMT_Q8 = 1 };

/* Error returns (negative).  0 = success. */
enum {
  ORC_OK = 0,
  ORC_EINVAL = -1,     /* inconsistent configuration */
  ORC_ENONFINITE = -2  /* NaN/Inf in an input that must be finite */
};

typedef struct orc_cfg {
  int32_t hidden;         /* H, a multiple of 128 */
  int32_t group_size;     /* values per fp32 scale: 128, or H (one scale per token) */
  int32_t num_logical;    /* logical routed experts the router scores */
  int32_t num_phys;       /* physical expert instances (replicas + shared included) */
  int32_t top_k;          /* routed picks per token */
  int32_t num_shared;     /* 0 or 1; the shared expert is physical id num_phys-1 */
  int32_t score_fn;       /* ORC_SCORE_* */
  int32_t max_replicas;   /* R >= 1 columns in replica_table */
  const int32_t *replica_table; /* [num_logical][R] physical ids, -1 pads; NULL = identity */
  const int32_t *capacity;      /* [num_phys] slots reserved per physical expert */
} orc_cfg;

/* Validates cfg; returns ORC_OK or ORC_EINVAL. */
int orc_check_cfg(const orc_cfg *c);

/* Top-k of one logit row by repeated arg-max; ties go to the lower id. */
int orc_topk_row(int32_t num_experts, int32_t k, const float *row, int32_t *out_ids);

/* Nearest bfloat16 to f, ties to even significand (IEEE overflow to inf). */
uint16_t orc_f32_to_bf16(float f);
void orc_f32_to_bf16_array(int64_t n, const float *in, uint16_t *out);

/* Full routing for T tokens: top-k, gates, physical mapping, per-expert
 * counts, exclusive offsets, slot indices and the drop count. */
int orc_route(const orc_cfg *c, int32_t T, const float *logits,
              int32_t *topk_ids, float *topk_w, int32_t *counts,
              int32_t *offsets, int32_t *slots, int32_t *dropped);

/* Quantize n BF16 values (one group) to INT8 with one fp32 scale. */
int orc_quantize_group(int32_t n, const uint16_t *x, int8_t *q, float *scale);

/* Quantize one token of H values in groups of gs: q[H], scales[H/gs]. */
int orc_quantize_token(int32_t H, int32_t gs, const uint16_t *x, int8_t *q, float *scales);

/* Dispatch T tokens into a host slot buffer of the given byte stride:
 * payload at byte 0, fp32 scales at byte H.  Bytes past H + 4*(H/gs) of
 * each slot and unoccupied slots are not written. */
int orc_dispatch(const orc_cfg *c, int32_t T, const uint16_t *x,
                 const int32_t *slots, uint8_t *dbuf, int64_t slot_stride);

/* Stand-in expert used to fill combine inputs: occupied slot of physical
 * expert p holds bf16( dequant(slot) * (1 + 0.01*p) ). */
int orc_expert_stub(const orc_cfg *c, const int32_t *counts,
                    const uint8_t *dbuf, int64_t slot_stride,
                    uint16_t *ebuf, int64_t ebuf_stride);

/* Stand-in expert with real arithmetic, one W8A8 linear layer per physical
 * expert (hidden -> hidden): for each occupied slot row of expert p and
 * output channel n, with q the row's INT8 payload and s_x its scales,
 *   isum_g = sum over group g of q[k] * W[p][n][k]   (exact int32)
 *   acc = +0; acc = fmaf(s_x[g], (float)isum_g, acc) for g ascending
 *   y[n] = bf16(acc * w_scale[p][n])
 * W is int8 [num_phys][H][H] (row n = output channel), w_scale fp32
 * [num_phys][H].  Weights per output channel, activations per token or per
 * group ("INT8 Quantization": mixed granularity). */
int orc_expert_w8a8(const orc_cfg *c, const int32_t *counts, const uint8_t *dbuf,
                    int64_t slot_stride, const int8_t *W, const float *w_scale,
                    uint16_t *ebuf, int64_t ebuf_stride);

/* Combine: per token, fp32 multiply-add chain over its slots in route
 * order (dropped slots skipped), rounded once to BF16. */
int orc_combine(const orc_cfg *c, int32_t T, const void *eout, int32_t fmt,
                int64_t eout_stride, const int32_t *slots, const float *topk_w,
                uint16_t *y);

#ifdef __cplusplus
}
#endif

#endif /* MOEDC_ORACLE_H */
