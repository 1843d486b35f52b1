// combine.hip -- gather of each token's expert outputs, dequantization and
// gate-weighted fp32 reduction to BF16 (gfx950).
//
// Behaviour: "CloudMatrix384: Co-Designing Supernodes for Trillion-Parameter
// LLM Inference", section "FusedDispatch and FusedCombine" (combine brings
// expert outputs back to the token's owner and weights them).  Arithmetic:
// acc = +0; acc = fma(w_j, y_j, acc) over the token's entries in route
// order, dropped entries skipped; BF16 round-to-nearest-even at the end.
//
// Mapping: one wave64 per token; per 512-value chunk every lane issues the
// K independent 16-byte (BF16) or 8-byte (INT8) gathers before the FMA
// chain, so K * 1 KiB per wave is in flight.  A dropped entry loads nothing
// and contributes fma(0, 0, acc) = acc, which leaves acc bit-identical.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"

namespace moedc {

namespace {

constexpr int kWavesPerBlock = 4;

template <int K>
__global__ __launch_bounds__(256) void combine_bf16_kernel(CombineArgs a) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + uniform(threadIdx.x >> 6);
  if (t >= a.T) return;
  const int H = a.H;
  int slot[K];
  float w[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    slot[k] = uniform(a.slots[t * K + k]);
    w[k] = slot[k] >= 0 ? a.w[t * K + k] : 0.0f;
  }
  uint4 *yrow = reinterpret_cast<uint4 *>(a.y + t * H);
  const int nch = (H + 511) / 512;
#pragma unroll 2
  for (int c = 0; c < nch; ++c) {
    const int e = c * 512 + lane * 8;
    if (e >= H) continue;
    uint4 v[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      v[k] = make_uint4(0, 0, 0, 0);
      if (slot[k] >= 0)
        v[k] = *reinterpret_cast<const uint4 *>(a.eout + (int64_t)slot[k] * a.eout_stride +
                                                 (int64_t)e * 2);
    }
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint32_t d[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __builtin_fmaf(w[k], bf16_lo(d[i]), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(w[k], bf16_hi(d[i]), acc[2 * i + 1]);
      }
    }
    yrow[c * 64 + lane] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                     pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  }
}

template <int K>
__global__ __launch_bounds__(256) void combine_q8_kernel(CombineArgs a) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + uniform(threadIdx.x >> 6);
  if (t >= a.T) return;
  const int H = a.H;
  int slot[K];
  float w[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    slot[k] = uniform(a.slots[t * K + k]);
    w[k] = slot[k] >= 0 ? a.w[t * K + k] : 0.0f;
  }
  uint4 *yrow = reinterpret_cast<uint4 *>(a.y + t * H);
  const int nch = (H + 511) / 512;
#pragma unroll 2
  for (int c = 0; c < nch; ++c) {
    const int e = c * 512 + lane * 8;
    if (e >= H) continue;
    uint2 v[K];
    float sc[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      v[k] = make_uint2(0, 0);
      sc[k] = 0.0f;
      if (slot[k] >= 0) {
        const uint8_t *row = a.eout + (int64_t)slot[k] * a.eout_stride;
        v[k] = *reinterpret_cast<const uint2 *>(row + e);
        sc[k] = *reinterpret_cast<const float *>(row + H + 4 * (e >> 7));
      }
    }
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint32_t d[2] = {v[k].x, v[k].y};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int qi = (int)(int8_t)((d[i >> 2] >> (8 * (i & 3))) & 0xFFu);
        const float dq = (float)qi * sc[k];
        acc[i] = __builtin_fmaf(w[k], dq, acc[i]);
      }
    }
    yrow[c * 64 + lane] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                     pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const unsigned grid = (unsigned)((a.T + kWavesPerBlock - 1) / kWavesPerBlock);
  const bool q8 = a.fmt == MOEDC_FMT_Q8;
  switch (a.K) {
#define MOEDC_CASE(k)                                                  \
  case k:                                                              \
    if (q8)                                                            \
      combine_q8_kernel<k><<<grid, 256, 0, s>>>(a);                    \
    else                                                               \
      combine_bf16_kernel<k><<<grid, 256, 0, s>>>(a);                  \
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
