// dispatch.hip -- early INT8 quantization with per-group fp32 scales and a
// K-way direct store of each token into its static expert slots (gfx950).
//
// Behaviour: "CloudMatrix384: Co-Designing Supernodes for Trillion-Parameter
// LLM Inference", section "FusedDispatch and FusedCombine" -- quantize to
// INT8 with a scale before the data moves, write straight into
// pre-allocated receiver buffers, and run load -> quantize/address -> write
// per token.  Granularity follows section "INT8 Quantization" (dynamic
// activation scales), refined to one scale per 128 values.
//
// Mapping: one wave64 per token.  A token row of H BF16 values is read as
// ceil(H/512) chunks; in chunk c lane l holds values [512c + 8l, +8) from
// one 16-byte load, so a 16-lane DPP row holds exactly one 128-value group.
// amax is a DPP row max over the BF16 magnitudes (bit patterns, no float
// compare needed), the scale is one IEEE fp32 division per group, and each
// value's quotient x/scale is the correctly rounded fp32 quotient, obtained
// from one IEEE reciprocal per group plus an fma correction.  The wave then
// writes the token's payload (8 bytes per lane, 512 contiguous bytes per
// store instruction) and its scales (one dword per lane) into each of the
// K slots, with the non-temporal hint (slots are written once and read by
// a later kernel).  Many waves per CU overlap one token's loads with other
// tokens' quantize and store phases.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"

namespace moedc {

namespace {

constexpr int kWavesPerBlock = 4;

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

template <int NCH>
__global__ __launch_bounds__(256) void dispatch_kernel(DispatchArgs a) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + uniform(threadIdx.x >> 6);
  if (t >= a.T) return;
  const int H = a.H;
  const uint4 *xrow = reinterpret_cast<const uint4 *>(a.x + t * H);

  uint4 v[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int e = c * 512 + lane * 8;
    v[c] = e < H ? xrow[c * 64 + lane] : make_uint4(0, 0, 0, 0);
  }

  uint2 q[NCH];
  float my_scale = 0.0f;  // scale of group `lane`
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const uint32_t m = row16_max_u32(absmax8(v[c]));
    const float s = __uint_as_float(m << 16) / 127.0f;
    q[c] = quant8(v[c], s);
    // Group 4c + r lives in DPP row r; lane 4c + r collects its scale.
    const float sg = __shfl(s, (lane & 3) * 16);
    if ((lane >> 2) == c) my_scale = sg;
  }

  const int32_t *srow = a.slots + t * a.K;
  for (int k = 0; k < a.K; ++k) {
    const int slot = uniform(srow[k]);
    if (slot < 0) continue;
    uint8_t *dst = a.dbuf + (int64_t)slot * a.slot_stride;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e = c * 512 + lane * 8;
      if (e < H) {
        const u32x2 qq = {q[c].x, q[c].y};
        __builtin_nontemporal_store(qq, reinterpret_cast<u32x2 *>(dst + e));
      }
    }
    if (lane < a.G) __builtin_nontemporal_store(my_scale, reinterpret_cast<float *>(dst + H + 4 * lane));
  }
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int nch = (a.H + 511) / 512;
  const unsigned grid = (unsigned)((a.T + kWavesPerBlock - 1) / kWavesPerBlock);
  switch (nch) {
#define MOEDC_CASE(n)                                  \
  case n:                                              \
    dispatch_kernel<n><<<grid, 256, 0, s>>>(a);        \
    break;
    MOEDC_CASE(1) MOEDC_CASE(2) MOEDC_CASE(3) MOEDC_CASE(4) MOEDC_CASE(5) MOEDC_CASE(6)
    MOEDC_CASE(7) MOEDC_CASE(8) MOEDC_CASE(9) MOEDC_CASE(10) MOEDC_CASE(11) MOEDC_CASE(12)
    MOEDC_CASE(13) MOEDC_CASE(14) MOEDC_CASE(15) MOEDC_CASE(16)
#undef MOEDC_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moedc
