// combine.hip -- gather of each token's expert outputs, dequantization and
// gate-weighted fp32 reduction to BF16 (gfx950).
//
// Behaviour: "CloudMatrix384: Co-Designing Supernodes for Trillion-Parameter
// LLM Inference", section "FusedDispatch and FusedCombine" (combine brings
// expert outputs back to the token's owner and weights them).  Arithmetic:
// acc = +0; acc = fma(w_j, y_j, acc) over the token's entries in route
// order, dropped entries skipped; BF16 round-to-nearest-even at the end.
//
// Mapping: one wave64 per token (a grid-stride loop when the caller caps
// the number of workgroups).  The token's H values are covered in
// groups of kChunks 512-value chunks (lane l holds values 512c + 8l .. +8
// of chunk c).  Within a group the wave walks the K expert rows in route
// order and, for each row, issues the loads of all kChunks chunks back to
// back: a contiguous 7 KiB (BF16) run of one row instead of 1 KiB pieces of
// K rows in turn, which keeps HBM row-buffer locality on a gather whose rows
// are scattered over the slot buffer.  Expert rows and the output are
// touched once, so loads and stores carry the non-temporal hint.  A dropped
// entry loads nothing and contributes fma(0, 0, acc) = acc exactly.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"

namespace moedc {

namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kChunks = 7;  // 512-value chunks per group: 7168 = 2 groups

__device__ __forceinline__ uint4 load_nt16(const uint8_t *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint2 load_nt8(const uint8_t *p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
  return make_uint2(v.x, v.y);
}

__device__ __forceinline__ void store_nt16(uint16_t *p, const float (&acc)[8]) {
  const u32x4 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                   pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(p));
}

template <int K, bool Q8>
__device__ __forceinline__ void combine_token(const CombineArgs &a, int64_t t, int lane) {
  const int H = a.H;
  int slot[K];
  float w[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    slot[k] = uniform(a.slots[t * K + k]);
    w[k] = slot[k] >= 0 ? a.w[t * K + k] : 0.0f;
  }
  uint16_t *yrow = a.y + t * H;
  const int nch = (H + 511) / 512;
  for (int g0 = 0; g0 < nch; g0 += kChunks) {
    float acc[kChunks][8];
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[c][i] = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint8_t *row = a.eout + (int64_t)(slot[k] < 0 ? 0 : slot[k]) * a.eout_stride;
      if (!Q8) {
        uint4 v[kChunks];
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
          const int e = (g0 + c) * 512 + lane * 8;
          v[c] = make_uint4(0, 0, 0, 0);
          if (slot[k] >= 0 && e < H) v[c] = load_nt16(row + (int64_t)e * 2);
        }
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
          const uint32_t d[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[c][2 * i] = __builtin_fmaf(w[k], bf16_lo(d[i]), acc[c][2 * i]);
            acc[c][2 * i + 1] = __builtin_fmaf(w[k], bf16_hi(d[i]), acc[c][2 * i + 1]);
          }
        }
      } else {
        uint2 v[kChunks];
        float sc[kChunks];
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
          const int e = (g0 + c) * 512 + lane * 8;
          v[c] = make_uint2(0, 0);
          sc[c] = 0.0f;
          if (slot[k] >= 0 && e < H) {
            v[c] = load_nt8(row + e);
            sc[c] = *reinterpret_cast<const float *>(row + H + (a.per_token ? 0 : 4 * (e >> 7)));
          }
        }
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
          const uint32_t d[2] = {v[c].x, v[c].y};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int qi = (int)(int8_t)((d[i >> 2] >> (8 * (i & 3))) & 0xFFu);
            acc[c][i] = __builtin_fmaf(w[k], (float)qi * sc[c], acc[c][i]);
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int e = (g0 + c) * 512 + lane * 8;
      if (e < H) store_nt16(yrow + e, acc[c]);
    }
  }
}

template <int K, bool Q8>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int lane = lane_id();
  const int64_t stride = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + uniform(threadIdx.x >> 6); t < a.T;
       t += stride) {
    combine_token<K, Q8>(a, t, lane);
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int64_t need = (a.T + kWavesPerBlock - 1) / kWavesPerBlock;
  const unsigned grid = (unsigned)(need < a.max_blocks ? need : a.max_blocks);
  const bool q8 = a.fmt == MOEDC_FMT_Q8;
  switch (a.K) {
#define MOEDC_CASE(k)                                                  \
  case k:                                                              \
    if (q8)                                                            \
      combine_kernel<k, true><<<grid, 256, 0, s>>>(a);                 \
    else                                                               \
      combine_kernel<k, false><<<grid, 256, 0, s>>>(a);                \
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
