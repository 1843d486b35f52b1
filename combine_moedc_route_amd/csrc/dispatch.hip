// dispatch.hip -- early INT8 quantization with per-group fp32 scales and a
// K-way direct store of each token into its static expert slots (gfx950).
//
// Behaviour: "CloudMatrix384: Co-Designing Supernodes for Trillion-Parameter
// LLM Inference", section "FusedDispatch and FusedCombine" -- quantize to
// INT8 with a scale before the data moves, write straight into
// pre-allocated receiver buffers, and run load -> quantize/address -> write
// per token.  Granularity follows section "INT8 Quantization" (dynamic
// activation scales): one scale per 128 values, or one per token.
//
// Mapping: one wave64 per token.  A token row of H BF16 values is read as
// ceil(H/512) chunks; in chunk c lane l holds values [512c + 8l, +8) from
// one 16-byte load, so a 16-lane DPP row holds exactly one 128-value group.
// amax is a DPP row max over the BF16 magnitudes (bit patterns, no float
// compare needed), the scale is one IEEE fp32 division per group, and each
// value's quotient x/scale is the correctly rounded fp32 quotient, obtained
// from one IEEE reciprocal per group plus an fma correction.  The wave then
// writes the token's payload (8 bytes per lane, 512 contiguous bytes per
// store instruction) and its scales (one dword per lane, zero words after
// them up to a 128-byte boundary) into each of the K slots, with the
// non-temporal hint (slots are written once and read by a later kernel).  Entries with slot -1 (dropped), or any slot outside the
// plan's buffer, are skipped.  Many waves per CU overlap one token's loads with other
// tokens' quantize and store phases.
//
// Small batches (below kSplitTokens tokens) use one wave per 512-value chunk
// of a token instead (with one scale per token, a workgroup per token whose
// waves share the token's amax through LDS), so ~100 decode tokens still
// keep every CU busy; the bytes written are the same.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"
#include "quant.hpp"

namespace moedc {

namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kSplitTokens = 2048;

template <int NCH, bool PER_TOKEN>
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
  if (PER_TOKEN) {
    // One group per token: DPP row max over all chunks, then across rows.
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) m = max(m, absmax8(v[c]));
    m = row16_max_u32(m);
    m = max(m, (uint32_t)__shfl_xor((int)m, 16));
    m = max(m, (uint32_t)__shfl_xor((int)m, 32));
    const float s = __uint_as_float(m << 16) / 127.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) q[c] = quant8(v[c], s);
    my_scale = s;
  } else {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint32_t m = row16_max_u32(absmax8(v[c]));
      const float s = __uint_as_float(m << 16) / 127.0f;
      q[c] = quant8(v[c], s);
      // Group 4c + r lives in DPP row r; lane 4c + r collects its scale.
      const float sg = __shfl(s, (lane & 3) * 16);
      if ((lane >> 2) == c) my_scale = sg;
    }
  }

  const int32_t *srow = a.slots + t * a.K;
  const int sw = scale_words(a.G);
  for (int k = 0; k < a.K; ++k) {
    const int slot = uniform(srow[k]);
    if ((uint32_t)slot >= (uint32_t)a.total_slots) continue;  // -1: dropped
    uint8_t *dst = a.dbuf + (int64_t)slot * a.slot_stride;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e = c * 512 + lane * 8;
      if (e < H) {
        const u32x2 qq = {q[c].x, q[c].y};
        __builtin_nontemporal_store(qq, reinterpret_cast<u32x2 *>(dst + e));
      }
    }
    if (lane < sw)
      __builtin_nontemporal_store(lane < a.G ? my_scale : 0.0f,
                                  reinterpret_cast<float *>(dst + H + 4 * lane));
  }
}

// One wave per (token, 512-value chunk); 128-value groups only.
__global__ __launch_bounds__(256) void dispatch_split(DispatchArgs a, int nch) {
  const int lane = lane_id();
  // Below kSplitTokens tokens of at most 16 chunks: 32-bit unit indices.
  const int u = (int)blockIdx.x * kWavesPerBlock + uniform(threadIdx.x >> 6);
  const int t = u / nch;
  if (t >= a.T) return;
  const int c = u - t * nch;
  const int H = a.H;
  const int e = c * 512 + lane * 8;
  // The token's slots (lane k holds entry k) load alongside the values.
  const int my_slot = lane < a.K ? a.slots[t * a.K + lane] : -1;
  const uint4 v = e < H ? reinterpret_cast<const uint4 *>(a.x + t * H)[c * 64 + lane]
                        : make_uint4(0, 0, 0, 0);
  const uint32_t m = row16_max_u32(absmax8(v));
  const float sc = __uint_as_float(m << 16) / 127.0f;
  const uint2 q = quant8(v, sc);
  float word;
  const bool has_word = chunk_scale_word(c, nch, a.G, sc, lane, &word);
  for (int k = 0; k < a.K; ++k) {
    const int slot = __builtin_amdgcn_readlane(my_slot, k);
    if ((uint32_t)slot >= (uint32_t)a.total_slots) continue;  // -1: dropped
    uint8_t *dst = a.dbuf + (int64_t)slot * a.slot_stride;
    if (e < H) {
      const u32x2 qq = {q.x, q.y};
      __builtin_nontemporal_store(qq, reinterpret_cast<u32x2 *>(dst + e));
    }
    if (has_word) __builtin_nontemporal_store(word, reinterpret_cast<float *>(dst + H + 4 * lane));
  }
}

// Small batches with one scale per token: one 16-wave workgroup per token,
// wave c holding chunk c; the token's amax is a workgroup max through LDS.
// (A wave per whole token leaves a decode batch on ~100 waves: 2.2x slower.)
__global__ __launch_bounds__(1024) void dispatch_token_block(DispatchArgs a) {
  __shared__ uint32_t wave_max[16];
  __shared__ int slot_of[kMaxK];
  const int t = blockIdx.x;
  const int wave = uniform(threadIdx.x >> 6), lane = lane_id();
  const int H = a.H;
  const int e = wave * 512 + lane * 8;
  if ((int)threadIdx.x < a.K) {
    const int s = a.slots[(int64_t)t * a.K + threadIdx.x];
    slot_of[threadIdx.x] = (uint32_t)s < (uint32_t)a.total_slots ? s : -1;
  }
  const uint4 v = e < H ? reinterpret_cast<const uint4 *>(a.x + (int64_t)t * H)[wave * 64 + lane]
                        : make_uint4(0, 0, 0, 0);
  uint32_t m = row16_max_u32(absmax8(v));
  m = max(m, (uint32_t)__shfl_xor((int)m, 16));
  m = max(m, (uint32_t)__shfl_xor((int)m, 32));
  if (lane == 0) wave_max[wave] = m;
  __syncthreads();
  m = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) m = max(m, wave_max[w]);
  const float sc = __uint_as_float(m << 16) / 127.0f;
  const uint2 q = quant8(v, sc);
  // Wave 0 stores the scale and the zero words after it (one line).
  const bool has_word = wave == 0 && lane < scale_words(1);
  const float word = lane == 0 ? sc : 0.0f;
  for (int k = 0; k < a.K; ++k) {
    const int slot = slot_of[k];
    if (slot < 0) continue;  // dropped, or outside the buffer
    uint8_t *dst = a.dbuf + (int64_t)slot * a.slot_stride;
    if (e < H) {
      const u32x2 qq = {q.x, q.y};
      __builtin_nontemporal_store(qq, reinterpret_cast<u32x2 *>(dst + e));
    }
    if (has_word) __builtin_nontemporal_store(word, reinterpret_cast<float *>(dst + H + 4 * lane));
  }
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.T < kSplitTokens && a.per_token) {
    dispatch_token_block<<<(unsigned)a.T, 1024, 0, s>>>(a);
    return hipGetLastError();
  }
  if (a.T < kSplitTokens && !a.per_token) {
    const int nch = (a.H + 511) / 512;
    const int64_t units = (int64_t)a.T * nch;
    dispatch_split<<<(unsigned)((units + kWavesPerBlock - 1) / kWavesPerBlock), 256, 0, s>>>(a, nch);
    return hipGetLastError();
  }
  const int nch = (a.H + 511) / 512;
  const unsigned grid = (unsigned)((a.T + kWavesPerBlock - 1) / kWavesPerBlock);
  switch (nch) {
#define MOEDC_CASE(n)                                  \
  case n:                                              \
    if (a.per_token)                                   \
      dispatch_kernel<n, true><<<grid, 256, 0, s>>>(a);  \
    else                                               \
      dispatch_kernel<n, false><<<grid, 256, 0, s>>>(a); \
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
