// combine.hip -- gather of each token's expert outputs, dequantization and
// gate-weighted fp32 reduction to BF16 (gfx950).
//
// Behaviour: "CloudMatrix384: Co-Designing Supernodes for Trillion-Parameter
// LLM Inference", section "FusedDispatch and FusedCombine" (combine brings
// expert outputs back to the token's owner and weights them).  Arithmetic:
// acc = +0; acc = fma(w_j, y_j, acc) over the token's entries in route
// order, dropped entries skipped; BF16 round-to-nearest-even at the end.
//
// Mapping: a wave per work unit, a grid-stride loop when the caller caps
// the number of workgroups.  A unit is one 512-value chunk of a token (lane
// l holds values 512c + 8l .. +8), so a token's K expert rows are read by
// its ceil(H/512) chunk waves at once: on a 30720-token batch, with 16-wave
// workgroups, 7% faster than one wave per token walking each row in 7 KiB
// runs, and a decode batch of ~100 tokens (4-wave workgroups) still spreads
// over every CU.  Under a workgroup cap the workgroups have 16 waves and,
// below 2048 tokens, units of wide_chunks(K) chunks.
// A unit's wave loads the token's slots and gates together, then for each
// expert row in route order issues the loads of its chunks back to back.
// Expert rows and the output are touched once, so loads and stores carry
// the non-temporal hint.  A dropped entry (slot -1), like any slot outside
// the plan's buffer, loads nothing: its weight is 0 and its values are -0,
// so it contributes fma(0, -0, acc) = 0 * -0 + acc = -0 + acc, which is acc
// for every acc including both signed zeros (with +0 values an acc of -0,
// left by a product that underflowed, would turn into +0).
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"

namespace moedc {

namespace {

constexpr int kWavesPerBlock = 4;  // below kWideTokens: spread over every CU
constexpr int kWideTokens = 2048;   // from here on, 16-wave workgroups
constexpr uint32_t kNegZero2 = 0x80008000u;  // two BF16 -0 values
// Chunks per unit under a workgroup cap: 2 (twice the loads in flight per
// wave), 1 from K = 14 on, where two chunks' loads no longer fit in the
// 128 registers of a 16-wave workgroup.
__host__ __device__ constexpr int wide_chunks(int k) { return k >= 14 ? 1 : 2; }

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

// Chunks [c0, c1) of token t, CH chunks at a time.  Each output value sees
// the same K fmas in the same order whatever the unit shape.
template <int K, bool Q8, int CH>
__device__ __forceinline__ void combine_unit(const CombineArgs &a, int64_t t, int c0, int c1,
                                             int lane) {
  const int H = a.H;
  int slot[K];  // -1 for an entry that is skipped
  float w[K];
  // All 2K loads of the token's slots and gates are issued before any is
  // used: one memory latency instead of K dependent ones.
#pragma unroll
  for (int k = 0; k < K; ++k) slot[k] = a.slots[t * K + k];
#pragma unroll
  for (int k = 0; k < K; ++k) w[k] = a.w[t * K + k];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int s = uniform(slot[k]);
    slot[k] = (uint32_t)s < (uint32_t)a.total_slots ? s : -1;
    w[k] = slot[k] >= 0 ? w[k] : 0.0f;
  }
  uint16_t *yrow = a.y + t * H;
  const int hend = min(H, 512 * c1);  // values of this unit end here
  for (int g0 = c0; g0 < c1; g0 += CH) {
    float acc[CH][8];
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[c][i] = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint8_t *row = a.eout + (int64_t)(slot[k] < 0 ? 0 : slot[k]) * a.eout_stride;
      if (!Q8) {
        uint4 v[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const int e = (g0 + c) * 512 + lane * 8;
          v[c] = make_uint4(kNegZero2, kNegZero2, kNegZero2, kNegZero2);
          if (slot[k] >= 0 && e < hend) v[c] = load_nt16(row + (int64_t)e * 2);
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const uint32_t d[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[c][2 * i] = __builtin_fmaf(w[k], bf16_lo(d[i]), acc[c][2 * i]);
            acc[c][2 * i + 1] = __builtin_fmaf(w[k], bf16_hi(d[i]), acc[c][2 * i + 1]);
          }
        }
      } else {
        uint2 v[CH];
        float sc[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const int e = (g0 + c) * 512 + lane * 8;
          v[c] = make_uint2(0, 0);
          sc[c] = -0.0f;  // (float)0 * -0 = -0
          if (slot[k] >= 0 && e < hend) {
            v[c] = load_nt8(row + e);
            sc[c] = *reinterpret_cast<const float *>(row + H + (a.per_token ? 0 : 4 * (e >> 7)));
          }
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
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
    for (int c = 0; c < CH; ++c) {
      const int e = (g0 + c) * 512 + lane * 8;
      if (e < hend) store_nt16(yrow + e, acc[c]);
    }
  }
}

// Units of UC consecutive 512-value chunks of a token; WPB waves per
// workgroup (16 when the caller caps the workgroup count, so the few CUs it
// gets still hold many loads in flight; their units are then
// wide_chunks(K) chunks).
template <int K, bool Q8, int WPB, int UC>
__global__ __launch_bounds__(64 * WPB) void combine_kernel(CombineArgs a) {
  const int lane = lane_id();
  const int nch = (a.H + 511) / 512;
  const int nu = (nch + UC - 1) / UC;  // units per token
  const int64_t units = (int64_t)a.T * nu;
  const int64_t stride = (int64_t)gridDim.x * WPB;
  for (int64_t u = (int64_t)blockIdx.x * WPB + uniform(threadIdx.x >> 6); u < units;
       u += stride) {
    // units <= 2^24 tokens x 16 chunks: 32-bit division
    const int t = (int)u / nu;
    const int c = ((int)u - t * nu) * UC;
    combine_unit<K, Q8, UC>(a, t, c, min(c + UC, nch), lane);
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  // One-chunk units.  Large batches run them on 16-wave workgroups (686-692
  // against 708-712 us with 4, 8, 12 or 14 waves on a 30720-token batch);
  // small ones on 4-wave workgroups so ~100 tokens reach every CU, or, when
  // the caller's cap leaves fewer of those than units, on 16-wave
  // workgroups of wide_chunks(K)-chunk units.
  const int nch = (a.H + 511) / 512;
  const int64_t units = a.T * (int64_t)nch;
  const bool big = a.T >= kWideTokens;
  const bool wide = !big && (int64_t)a.max_blocks * kWavesPerBlock < units;
  const int wpb = big || wide ? 16 : kWavesPerBlock;
  const int uc = wide_chunks(a.K);
  const int64_t wunits = wide ? a.T * (int64_t)((nch + uc - 1) / uc) : units;
  const int64_t need = (wunits + wpb - 1) / wpb;
  const unsigned grid = (unsigned)(need < a.max_blocks ? need : a.max_blocks);
  const bool q8 = a.fmt == MOEDC_FMT_Q8;
  switch (a.K) {
#define MOEDC_LAUNCH(k, q)                                                 \
  if (big)                                                                 \
    combine_kernel<k, q, 16, 1><<<grid, 1024, 0, s>>>(a);                  \
  else if (!wide)                                                          \
    combine_kernel<k, q, kWavesPerBlock, 1><<<grid, 256, 0, s>>>(a);       \
  else                                                                     \
    combine_kernel<k, q, 16, wide_chunks(k)><<<grid, 1024, 0, s>>>(a);
#define MOEDC_CASE(k)          \
  case k:                      \
    if (q8) {                  \
      MOEDC_LAUNCH(k, true)    \
    } else {                   \
      MOEDC_LAUNCH(k, false)   \
    }                          \
    break;
    MOEDC_CASE(1) MOEDC_CASE(2) MOEDC_CASE(3) MOEDC_CASE(4) MOEDC_CASE(5) MOEDC_CASE(6)
    MOEDC_CASE(7) MOEDC_CASE(8) MOEDC_CASE(9) MOEDC_CASE(10) MOEDC_CASE(11) MOEDC_CASE(12)
    MOEDC_CASE(13) MOEDC_CASE(14) MOEDC_CASE(15) MOEDC_CASE(16)
#undef MOEDC_CASE
#undef MOEDC_LAUNCH
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moedc
