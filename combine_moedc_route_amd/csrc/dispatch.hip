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
// Mapping: a workgroup per token with one wave per 512-value chunk (at
// most 16).  In chunk c lane l holds values [512c + 8l, +8) from one 16-byte
// load, so a 16-lane DPP row holds exactly one 128-value group.  amax is a
// DPP row max over the BF16 magnitudes (bit patterns, no float compare
// needed); with one scale per token the waves combine their maxima through
// LDS.  The scale is one IEEE fp32 division per group, and each value's
// quotient x/scale is the correctly rounded fp32 quotient, obtained from
// one IEEE reciprocal per group plus an fma correction.  Each wave then
// writes its chunk's payload (8 bytes per lane, 512 contiguous bytes per
// store instruction) into each of the token's K slots, and one wave writes
// the slot's scale region -- the scales, gathered through LDS, then zero
// words up to a 128-byte boundary -- as whole lines with the non-temporal
// hint.  The payload goes through non-temporal stores while the batch's
// BF16 input fits in the memory-side cache (256 MiB) and through ordinary
// (cached) stores above that, each the faster one there in the route ->
// dispatch -> combine sequence at hidden 7168: non-temporal 188 against
// 224 us at 16384 tokens (cached stores evict the input from that cache),
// cached 277 against 286 us at 20480 and 411-413 against 430 us at 30720
// tokens; on decode batches non-temporal 4.1 against 4.3 us at 96 tokens
// and 4.7 against 5.6 us at 256.
// A token's K slots are thus written by all its waves at once: 6% faster on
// a 30720-token batch than one wave walking the token's K x 7 KiB of slots,
// and 2.2x faster on a 96-token decode batch with one scale per token.
// Entries with slot -1 (dropped), or any slot outside the plan's buffer,
// are skipped.
//
// Batches of at most kSplitMaxTokens tokens with 128-value groups use one
// wave per (token, chunk) in 4-wave workgroups instead, with each chunk's
// wave storing its own groups' scales: as fast at 16 tokens, 0.5 us faster
// for one.  The bytes written are the same.
//
// Trace build (compiled with MOEDC_TRACE into libmoedc_trace.so only; see
// include/moedc_trace.h): every wave of dispatch_token_block stamps the
// 100 MHz constant clock at its phase boundaries -- start, chunk loaded,
// scales known, quantized, stores issued, stores complete -- and writes
// them with its hardware placement into a caller buffer, so that the
// token-level load -> quantize -> write pipeline, which this kernel gets
// from many resident waves per CU at different phases, can be seen.  The
// analog of the per-core phase probes of "StrataCL 深度技术分析", section
// on the NPU-side profiler.  The bytes dispatch writes are the same.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"
#include "quant.hpp"

namespace moedc {

#ifdef MOEDC_TRACE
__device__ uint64_t *g_trace = nullptr;  // 8 words per (token, wave) record
__device__ int64_t g_trace_records = 0;
#endif

namespace {

constexpr int kWavesPerBlock = 4;

// A lane's 8 payload bytes: ordinary (cached) or non-temporal store.  A
// compile-time choice: with a run-time branch the compiler merges the two
// stores of the same value into one ordinary store.
template <bool CACHED>
__device__ __forceinline__ void store_payload(const uint2 &q, uint8_t *dst) {
  const u32x2 qq = {q.x, q.y};
  if (CACHED)
    *reinterpret_cast<u32x2 *>(dst) = qq;
  else
    __builtin_nontemporal_store(qq, reinterpret_cast<u32x2 *>(dst));
}
constexpr int kSplitMaxTokens = 16;

// One wave per (token, 512-value chunk); 128-value groups only.
__global__ __launch_bounds__(256) void dispatch_split(DispatchArgs a, int nch) {
  const int lane = lane_id();
  // At most kSplitMaxTokens tokens of at most 16 chunks: 32-bit unit indices.
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
    if (e < H) store_payload<false>(q, dst + e);  // at most 16 tokens: always non-temporal
    if (has_word) __builtin_nontemporal_store(word, reinterpret_cast<float *>(dst + H + 4 * lane));
  }
}

// One workgroup per token, wave c holding chunk c (blockDim = 64 x chunks).
// wave_max: the waves' maxima (one scale per token) or the groups' scales.
template <bool PER_TOKEN, bool CACHED>
__global__ __launch_bounds__(1024) void dispatch_token_block(DispatchArgs a) {
  __shared__ uint32_t wave_max[64];
  __shared__ int slot_of[kMaxK];
  const int t = blockIdx.x;
  const int wave = uniform(threadIdx.x >> 6), lane = lane_id();
  const int H = a.H;
  const int e = wave * 512 + lane * 8;
  if ((int)threadIdx.x < a.K) {
    const int s = a.slots[(int64_t)t * a.K + threadIdx.x];
    slot_of[threadIdx.x] = (uint32_t)s < (uint32_t)a.total_slots ? s : -1;
  }
#ifdef MOEDC_TRACE
  // The empty asm statements pin each stamp after the value it follows.
  uint64_t ts[6];
  ts[0] = wall_clock64();
#endif
  const uint4 v = e < H ? reinterpret_cast<const uint4 *>(a.x + (int64_t)t * H)[wave * 64 + lane]
                        : make_uint4(0, 0, 0, 0);
  uint32_t m = row16_max_u32(absmax8(v));
#ifdef MOEDC_TRACE
  asm volatile("" : : "v"(m) : "memory");
  ts[1] = wall_clock64();
#endif
  float sc, word;
  bool has_word;
  if (PER_TOKEN) {
    m = max(m, (uint32_t)__shfl_xor((int)m, 16));
    m = max(m, (uint32_t)__shfl_xor((int)m, 32));
    if (lane == 0) wave_max[wave] = m;
    __syncthreads();
    m = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) m = max(m, wave_max[w]);
    sc = __uint_as_float(m << 16) / 127.0f;
    // Wave 0 stores the scale and the zero words after it (one line).
    has_word = wave == 0 && lane < scale_words(1);
    word = lane == 0 ? sc : 0.0f;
  } else {
    sc = __uint_as_float(m << 16) / 127.0f;  // this lane's group
    if ((lane & 15) == 0 && e < H) wave_max[e >> 7] = __float_as_uint(sc);
    __syncthreads();
    // The last wave stores every group's scale and the zero padding.
    has_word = wave == (int)(blockDim.x >> 6) - 1 && lane < scale_words(a.G);
    word = lane < a.G ? __uint_as_float(wave_max[lane]) : 0.0f;
  }
#ifdef MOEDC_TRACE
  asm volatile("" : : "v"(sc) : "memory");
  ts[2] = wall_clock64();
#endif
  const uint2 q = quant8(v, sc);
#ifdef MOEDC_TRACE
  asm volatile("" : : "v"(q.x), "v"(q.y) : "memory");
  ts[3] = wall_clock64();
#endif
  for (int k = 0; k < a.K; ++k) {
    const int slot = slot_of[k];
    if (slot < 0) continue;  // dropped, or outside the buffer
    uint8_t *dst = a.dbuf + (int64_t)slot * a.slot_stride;
    if (e < H) store_payload<CACHED>(q, dst + e);
    if (has_word) __builtin_nontemporal_store(word, reinterpret_cast<float *>(dst + H + 4 * lane));
  }
#ifdef MOEDC_TRACE
  ts[4] = wall_clock64();
  __builtin_amdgcn_s_waitcnt(0);  // the stores have completed
  ts[5] = wall_clock64();
  // Record: [token << 32 | wave, XCC_ID << 32 | HW_ID, stamps 0..5].
  const int64_t rec = (int64_t)t * (int64_t)(blockDim.x >> 6) + wave;
  if (g_trace != nullptr && lane < 8 && rec < g_trace_records) {
    const uint64_t hw = ((uint64_t)__builtin_amdgcn_s_getreg((15 << 11) | 20) << 32) |
                        (uint64_t)__builtin_amdgcn_s_getreg((31 << 11) | 4);
    uint64_t w = lane == 0 ? (((uint64_t)(uint32_t)t << 32) | (uint32_t)wave) : hw;
#pragma unroll
    for (int k = 0; k < 6; ++k) w = lane == k + 2 ? ts[k] : w;
    g_trace[8 * rec + lane] = w;
  }
#endif
}

}  // namespace

#ifdef MOEDC_TRACE
extern "C" int32_t moedc_trace_set(void *buf, int64_t bytes) {
  uint64_t *ptr = static_cast<uint64_t *>(buf);
  const int64_t n = (buf != nullptr && bytes > 0) ? bytes / 64 : 0;
  hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(g_trace), &ptr, sizeof(ptr));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(g_trace_records), &n, sizeof(n));
  return (int32_t)e;
}
#endif

hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int nch = (a.H + 511) / 512;
  if (a.T <= kSplitMaxTokens && !a.per_token) {
    const int64_t units = (int64_t)a.T * nch;
    dispatch_split<<<(unsigned)((units + kWavesPerBlock - 1) / kWavesPerBlock), 256, 0, s>>>(a, nch);
  } else if (a.per_token) {
    if (a.cached_payload)
      dispatch_token_block<true, true><<<(unsigned)a.T, 64 * nch, 0, s>>>(a);
    else
      dispatch_token_block<true, false><<<(unsigned)a.T, 64 * nch, 0, s>>>(a);
  } else {
    if (a.cached_payload)
      dispatch_token_block<false, true><<<(unsigned)a.T, 64 * nch, 0, s>>>(a);
    else
      dispatch_token_block<false, false><<<(unsigned)a.T, 64 * nch, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moedc
