// quant.hpp -- the INT8 group quantizer shared by dispatch.hip and
// fused.hip: BF16 magnitude max and q = clamp(rne(x / s), +-127) with the
// correctly rounded fp32 quotient, and the size of a slot's scale region.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace moedc {

// Dwords of a slot's scale region as stored: the G scales, then zero words
// up to the next 128-byte boundary.  A slot that ended partway through a
// 128-byte line made the HBM write path slower (a partial line per slot,
// 2.7% of dispatch time at H = 7168) than the up to 124 padding bytes cost.
__device__ __forceinline__ int scale_words(int G) { return (G + 31) & ~31; }

// Scale word `lane` of a slot as the wave of 512-value chunk c of nch
// stores it, from its per-group scales sc (DPP row r holds group 4c + r):
// the chunk's own groups, and in the last chunk also the zero words after
// group G - 1, so the padding adds no store instruction.  Returns whether
// this lane stores; *val is the word.  Called by the whole wave.
__device__ __forceinline__ bool chunk_scale_word(int c, int nch, int G, float sc, int lane,
                                                 float *val) {
  const float own = __shfl(sc, ((lane - 4 * c) & 3) * 16);
  *val = lane < G ? own : 0.0f;
  return (lane >= 4 * c && lane < min(4 * c + 4, G)) ||
         (c == nch - 1 && lane >= G && lane < scale_words(G));
}

// Max of |x| over 8 BF16 values as a BF16 magnitude bit pattern.
__device__ __forceinline__ uint32_t absmax8(const uint4 &v) {
  const uint32_t a0 = v.x & 0x7FFF7FFFu, a1 = v.y & 0x7FFF7FFFu;
  const uint32_t a2 = v.z & 0x7FFF7FFFu, a3 = v.w & 0x7FFF7FFFu;
  uint32_t m = max(max(a0 & 0xFFFFu, a0 >> 16), max(a1 & 0xFFFFu, a1 >> 16));
  m = max(m, max(max(a2 & 0xFFFFu, a2 >> 16), max(a3 & 0xFFFFu, a3 >> 16)));
  return m;
}

__device__ __forceinline__ uint32_t clamp_q(float r) {
  return (uint32_t)((int)fminf(fmaxf(r, -127.0f), 127.0f)) & 0xFFu;
}

// q = clamp(rne(x / s)) with the IEEE quotient computed by the compiler's
// correctly rounded division.  Used when 1/s would not be a normal number.
__device__ __forceinline__ uint32_t q8_div(float x, float s) { return clamp_q(rintf(x / s)); }

// Same result with one division per group: y = RN(1/s) (IEEE), q0 = RN(x*y),
// r = x - q0*s (exact in one fma), q1 = RN(q0 + r*y).  By Markstein's
// correction theorem q1 = RN(x/s) whenever y is the correctly rounded
// reciprocal and nothing under- or overflows, which holds for s >= 2^-100
// (the device test checks every BF16 (x, amax) pair).
__device__ __forceinline__ uint32_t q8_rcp(float x, float s, float y) {
  const float q0 = x * y;
  const float r = __builtin_fmaf(-q0, s, x);
  return clamp_q(rintf(__builtin_fmaf(r, y, q0)));
}

__device__ __forceinline__ uint2 quant8(const uint4 &v, float s) {
  uint32_t b[8];
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
  if (s >= 0x1p-100f) {
    const float y = 1.0f / s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      b[2 * i] = q8_rcp(bf16_lo(d[i]), s, y);
      b[2 * i + 1] = q8_rcp(bf16_hi(d[i]), s, y);
    }
  } else if (s > 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      b[2 * i] = q8_div(bf16_lo(d[i]), s);
      b[2 * i + 1] = q8_div(bf16_hi(d[i]), s);
    }
  } else {
    return make_uint2(0, 0);  // all-zero group: scale 0, codes 0
  }
  return make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                    b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
}

}  // namespace moedc
