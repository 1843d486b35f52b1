/*
 * moedc_oracle.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.
 *
 * A plain, slow, obviously-correct single-threaded CPU oracle for the MoE
 * route -> INT8 dispatch -> combine path.  Only the tests, the smoke entry
 * point and the benchmark's CPU-baseline leg may use it.  It shares no code
 * with the HIP library.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math (no FMA
 * contraction, IEEE single-precision division, default rounding mode).
 *
 * Pages (title, section) are abbreviated as in moedc_oracle.h:
 *  [CM] CloudMatrix384 article; [SC] StrataCL analysis.
 *
 * Readings of what the pages leave open (each repeated at its function):
 *  R1  experts are picked by the raw fp32 router logit, highest first, ties
 *      to the lower expert id; row order is pick order.
 *  R2  gates: softmax over all logical experts (not renormalised) or the
 *      logistic sigmoid of each pick normalised over the picks; computed in
 *      fp64 and rounded once to fp32.  A shared expert takes weight 1.
 *  R3  INT8 granularity: one fp32 scale per group of consecutive hidden
 *      values, the group being 128 values or the whole token ("INT8
 *      Quantization": activation scales are per token and dynamic);
 *      scale = amax/127 in fp32, q = clamp(round-half-even(x/scale), +-127);
 *      an all-zero group has scale 0 and q = 0.
 *  R4  slot layout: within each physical expert, occupied slots hold tokens
 *      in ascending token order starting at that expert's static base (the
 *      exclusive prefix sum of capacities); a token past capacity is dropped
 *      (slot -1) and counted.
 *  R5  combine: acc = +0; acc = fma(w_k, y_k, acc) for k in route order over
 *      kept slots; output = nearest BF16 (ties to even).
 */
#include "moedc_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- BF16 helpers ------------------------------------------------------ */

static float bf16_to_f32(uint16_t b) {
  /* A bfloat16 is the upper half of an IEEE binary32 with the same value. */
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Magnitude of a bf16 bit pattern taken as if the exponent range were
 * unbounded: the pattern one past the largest finite value stands for 2^128,
 * which is what IEEE round-to-nearest compares against before overflowing. */
static double bf16_mag_unbounded(uint16_t b) {
  if ((b & 0x7FFFu) == 0x7F80u) return ldexp(1.0, 128);
  return fabs((double)bf16_to_f32(b));
}

uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
  if (isinf(f)) return (uint16_t)(u >> 16);
  uint16_t lo = (uint16_t)(u >> 16);           /* same sign, |lo| <= |f| */
  if ((u & 0xFFFFu) == 0) return lo;           /* exactly representable */
  uint16_t hi = (uint16_t)(lo + 1u);           /* next value away from 0 */
  double v = fabs((double)f);
  double a = bf16_mag_unbounded(lo);
  double b = bf16_mag_unbounded(hi);
  double below = v - a, above = b - v;         /* exact in binary64 */
  if (below < above) return lo;
  if (above < below) return hi;
  return (lo & 1u) ? hi : lo;                  /* tie: even significand */
}

void orc_f32_to_bf16_array(int64_t n, const float *in, uint16_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(in[i]);
}

/* ---- configuration ----------------------------------------------------- */

static int replica_count(const orc_cfg *c, int32_t e) {
  if (!c->replica_table) return 1;
  int r = 0;
  while (r < c->max_replicas && c->replica_table[(int64_t)e * c->max_replicas + r] >= 0) ++r;
  return r;
}

static int32_t replica_id(const orc_cfg *c, int32_t e, int32_t copy) {
  if (!c->replica_table) return e;
  return c->replica_table[(int64_t)e * c->max_replicas + copy];
}

int orc_check_cfg(const orc_cfg *c) {
  if (!c || !c->capacity) return ORC_EINVAL;
  if (c->hidden <= 0 || c->hidden % 128 != 0) return ORC_EINVAL;
  if (c->group_size != 128 && c->group_size != c->hidden) return ORC_EINVAL;
  if (c->num_logical <= 0 || c->top_k <= 0 || c->top_k > c->num_logical) return ORC_EINVAL;
  if (c->top_k > 64) return ORC_EINVAL;
  if (c->num_shared != 0 && c->num_shared != 1) return ORC_EINVAL;
  if (c->score_fn != ORC_SCORE_SOFTMAX && c->score_fn != ORC_SCORE_SIGMOID_NORM) return ORC_EINVAL;
  if (c->max_replicas < 1) return ORC_EINVAL;
  int32_t routed_phys = c->num_phys - c->num_shared;
  if (routed_phys < 1) return ORC_EINVAL;
  for (int32_t p = 0; p < c->num_phys; ++p)
    if (c->capacity[p] < 0) return ORC_EINVAL;
  /* Every physical routed id must belong to exactly one logical expert, so a
   * token that picks distinct logical experts never holds one physical id
   * twice. */
  char *owner = calloc((size_t)routed_phys, 1);
  if (!owner) return ORC_EINVAL;
  int bad = 0;
  for (int32_t e = 0; e < c->num_logical && !bad; ++e) {
    int r = replica_count(c, e);
    if (r < 1) { bad = 1; break; }
    for (int k = 0; k < r; ++k) {
      int32_t p = replica_id(c, e, k);
      if (p < 0 || p >= routed_phys || owner[p]) { bad = 1; break; }
      owner[p] = 1;
    }
    if (c->replica_table)
      for (int k = r; k < c->max_replicas; ++k)
        if (c->replica_table[(int64_t)e * c->max_replicas + k] != -1) bad = 1;
  }
  free(owner);
  return bad ? ORC_EINVAL : ORC_OK;
}

/* ---- route ------------------------------------------------------------- */

/* Reading R1: repeated arg-max over the not-yet-picked experts.  Scanning
 * ids upward with a strict ">" keeps the lower id on equal logits; -0.0 and
 * +0.0 compare equal. */
int orc_topk_row(int32_t E, int32_t k, const float *row, int32_t *out) {
  if (k < 1 || k > E) return ORC_EINVAL;
  char *taken = calloc((size_t)E, 1);
  if (!taken) return ORC_EINVAL;
  for (int32_t j = 0; j < k; ++j) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || row[e] > row[best]) best = e;
    }
    taken[best] = 1;
    out[j] = best;
  }
  free(taken);
  return ORC_OK;
}

int orc_route(const orc_cfg *c, int32_t T, const float *logits,
              int32_t *topk_ids, float *topk_w, int32_t *counts,
              int32_t *offsets, int32_t *slots, int32_t *dropped) {
  int rc = orc_check_cfg(c);
  if (rc) return rc;
  if (T < 0) return ORC_EINVAL;
  const int32_t E = c->num_logical, KR = c->top_k;
  const int32_t K = KR + c->num_shared, P = c->num_phys;
  for (int64_t i = 0; i < (int64_t)T * E; ++i)
    if (!isfinite(logits[i])) return ORC_ENONFINITE;

  int32_t *pick = malloc(sizeof(int32_t) * (size_t)KR);
  if (!pick) return ORC_EINVAL;
  for (int32_t t = 0; t < T; ++t) {
    const float *row = logits + (int64_t)t * E;
    int32_t *ids = topk_ids + (int64_t)t * K;
    float *w = topk_w + (int64_t)t * K;
    orc_topk_row(E, KR, row, pick);

    /* Reading R2: gates in binary64, rounded once to binary32. */
    if (c->score_fn == ORC_SCORE_SOFTMAX) {
      double m = row[0];
      for (int32_t e = 1; e < E; ++e) if (row[e] > m) m = row[e];
      double Z = 0.0;
      for (int32_t e = 0; e < E; ++e) Z += exp((double)row[e] - m);
      for (int32_t j = 0; j < KR; ++j) w[j] = (float)(exp((double)row[pick[j]] - m) / Z);
    } else {
      double S = 0.0;
      double s[64];
      for (int32_t j = 0; j < KR; ++j) {
        s[j] = 1.0 / (1.0 + exp(-(double)row[pick[j]]));
        S += s[j];
      }
      for (int32_t j = 0; j < KR; ++j) w[j] = (float)(s[j] / S);
    }

    /* Physical instance: a logical expert with r copies sends token t to
     * copy (t mod r); the shared expert, when present, is last, weight 1. */
    for (int32_t j = 0; j < KR; ++j) {
      int32_t e = pick[j];
      int r = replica_count(c, e);
      ids[j] = replica_id(c, e, t % r);
    }
    if (c->num_shared) {
      ids[K - 1] = P - 1;
      w[K - 1] = 1.0f;
    }
  }
  free(pick);

  /* Per-expert histogram and its exclusive prefix sum. */
  for (int32_t p = 0; p < P; ++p) counts[p] = 0;
  for (int64_t i = 0; i < (int64_t)T * K; ++i) counts[topk_ids[i]]++;
  offsets[0] = 0;
  for (int32_t p = 0; p < P; ++p) offsets[p + 1] = offsets[p] + counts[p];

  /* Reading R4: static per-expert bases, then ranks in token order. */
  int64_t *base = malloc(sizeof(int64_t) * (size_t)P);
  int32_t *next = calloc((size_t)P, sizeof(int32_t));
  if (!base || !next) { free(base); free(next); return ORC_EINVAL; }
  base[0] = 0;
  for (int32_t p = 1; p < P; ++p) base[p] = base[p - 1] + c->capacity[p - 1];
  int32_t drop = 0;
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t j = 0; j < K; ++j) {
      int64_t i = (int64_t)t * K + j;
      int32_t p = topk_ids[i];
      int32_t rank = next[p]++;
      if (rank < c->capacity[p]) {
        slots[i] = (int32_t)(base[p] + rank);
      } else {
        slots[i] = -1;
        ++drop;
      }
    }
  }
  *dropped = drop;
  free(base);
  free(next);
  return ORC_OK;
}

/* ---- dispatch ---------------------------------------------------------- */

/* Reading R3 for one group.  Division is IEEE binary32 (this file is built
 * without fast-math or contraction); rintf rounds half to even. */
int orc_quantize_group(int32_t n, const uint16_t *x, int8_t *q, float *scale) {
  float amax = 0.0f;
  for (int32_t i = 0; i < n; ++i) {
    float v = bf16_to_f32(x[i]);
    if (!isfinite(v)) return ORC_ENONFINITE;
    float a = fabsf(v);
    if (a > amax) amax = a;
  }
  float s = amax / 127.0f;
  for (int32_t i = 0; i < n; ++i) {
    if (s == 0.0f) { q[i] = 0; continue; }
    float r = rintf(bf16_to_f32(x[i]) / s);
    if (r < -127.0f) r = -127.0f;
    if (r > 127.0f) r = 127.0f;
    q[i] = (int8_t)r;
  }
  *scale = s;
  return ORC_OK;
}

int orc_quantize_token(int32_t H, int32_t gs, const uint16_t *x, int8_t *q, float *scales) {
  if (H <= 0 || gs <= 0 || H % gs) return ORC_EINVAL;
  for (int32_t g = 0; g < H / gs; ++g) {
    int rc = orc_quantize_group(gs, x + (int64_t)gs * g, q + (int64_t)gs * g, scales + g);
    if (rc) return rc;
  }
  return ORC_OK;
}

int orc_dispatch(const orc_cfg *c, int32_t T, const uint16_t *x,
                 const int32_t *slots, uint8_t *dbuf, int64_t slot_stride) {
  int rc = orc_check_cfg(c);
  if (rc) return rc;
  const int32_t H = c->hidden, gs = c->group_size, G = H / gs;
  const int32_t K = c->top_k + c->num_shared;
  if (slot_stride < (int64_t)H + 4 * G) return ORC_EINVAL;
  int8_t *q = malloc((size_t)H);
  float *s = malloc(sizeof(float) * (size_t)G);
  if (!q || !s) { free(q); free(s); return ORC_EINVAL; }
  for (int32_t t = 0; t < T && rc == ORC_OK; ++t) {
    rc = orc_quantize_token(H, gs, x + (int64_t)t * H, q, s);
    for (int32_t j = 0; j < K && rc == ORC_OK; ++j) {
      int32_t slot = slots[(int64_t)t * K + j];
      if (slot < 0) continue;
      uint8_t *dst = dbuf + (int64_t)slot * slot_stride;
      memcpy(dst, q, (size_t)H);
      memcpy(dst + H, s, sizeof(float) * (size_t)G);  /* little-endian host */
    }
  }
  free(q);
  free(s);
  return rc;
}

/* ---- expert stand-in --------------------------------------------------- */

int orc_expert_stub(const orc_cfg *c, const int32_t *counts,
                    const uint8_t *dbuf, int64_t slot_stride,
                    uint16_t *ebuf, int64_t ebuf_stride) {
  int rc = orc_check_cfg(c);
  if (rc) return rc;
  const int32_t H = c->hidden, gs = c->group_size;
  int64_t base = 0;
  for (int32_t p = 0; p < c->num_phys; ++p) {
    float m = 1.0f + 0.01f * (float)p;  /* two roundings: product, then sum */
    int32_t used = counts[p] < c->capacity[p] ? counts[p] : c->capacity[p];
    for (int32_t j = 0; j < used; ++j) {
      const uint8_t *src = dbuf + (base + j) * slot_stride;
      uint16_t *dst = (uint16_t *)((uint8_t *)ebuf + (base + j) * ebuf_stride);
      for (int32_t i = 0; i < H; ++i) {
        float s;
        memcpy(&s, src + H + 4 * (i / gs), sizeof s);
        float dq = (float)(int8_t)src[i] * s;
        dst[i] = orc_f32_to_bf16(dq * m);
      }
    }
    base += c->capacity[p];
  }
  return ORC_OK;
}

/* ---- expert: one W8A8 linear layer -------------------------------------- */

int orc_expert_w8a8(const orc_cfg *c, const int32_t *counts, const uint8_t *dbuf,
                    int64_t slot_stride, const int8_t *W, const float *w_scale,
                    uint16_t *ebuf, int64_t ebuf_stride) {
  int rc = orc_check_cfg(c);
  if (rc) return rc;
  const int32_t H = c->hidden, gs = c->group_size, G = H / gs;
  int64_t base = 0;
  for (int32_t p = 0; p < c->num_phys; ++p) {
    int32_t used = counts[p] < c->capacity[p] ? counts[p] : c->capacity[p];
    const int8_t *Wp = W + (int64_t)p * H * H;
    for (int32_t j = 0; j < used; ++j) {
      const uint8_t *row = dbuf + (base + j) * slot_stride;
      const int8_t *q = (const int8_t *)row;
      uint16_t *out = (uint16_t *)((uint8_t *)ebuf + (base + j) * ebuf_stride);
      for (int32_t n = 0; n < H; ++n) {
        const int8_t *w = Wp + (int64_t)n * H;
        float acc = 0.0f;
        for (int32_t g = 0; g < G; ++g) {
          int32_t isum = 0;  /* |isum| <= H * 127 * 127 < 2^31 for H <= 8192 */
          for (int32_t k = g * gs; k < (g + 1) * gs; ++k) isum += (int32_t)q[k] * (int32_t)w[k];
          float sx;
          memcpy(&sx, row + H + 4 * g, sizeof sx);
          acc = fmaf(sx, (float)isum, acc);
        }
        out[n] = orc_f32_to_bf16(acc * w_scale[(int64_t)p * H + n]);
      }
    }
    base += c->capacity[p];
  }
  return ORC_OK;
}

/* ---- combine ----------------------------------------------------------- */

int orc_combine(const orc_cfg *c, int32_t T, const void *eout, int32_t fmt,
                int64_t eout_stride, const int32_t *slots, const float *topk_w,
                uint16_t *y) {
  int rc = orc_check_cfg(c);
  if (rc) return rc;
  if (fmt != ORC_FMT_BF16 && fmt != ORC_FMT_Q8) return ORC_EINVAL;
  const int32_t H = c->hidden, gs = c->group_size, K = c->top_k + c->num_shared;
  const uint8_t *E = (const uint8_t *)eout;
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t i = 0; i < H; ++i) {
      float acc = 0.0f;
      for (int32_t j = 0; j < K; ++j) {
        int32_t slot = slots[(int64_t)t * K + j];
        if (slot < 0) continue;
        const uint8_t *row = E + (int64_t)slot * eout_stride;
        float v;
        if (fmt == ORC_FMT_BF16) {
          uint16_t b;
          memcpy(&b, row + 2 * (int64_t)i, sizeof b);
          v = bf16_to_f32(b);
        } else {
          float s;
          memcpy(&s, row + H + 4 * (i / gs), sizeof s);
          v = (float)(int8_t)row[i] * s;
        }
        acc = fmaf(topk_w[(int64_t)t * K + j], v, acc);
      }
      y[(int64_t)t * H + i] = orc_f32_to_bf16(acc);
    }
  }
  return ORC_OK;
}
