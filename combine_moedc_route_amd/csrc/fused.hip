// fused.hip -- the small-batch routing path (T <= 256 tokens) and the
// route + dispatch entry for decode batches, gfx950.
//
// Latency, not bandwidth, bounds a decode batch of one die's share ("Decode
// Phase" of the CloudMatrix384 article: 96 tokens per die), and the pages'
// operators fuse routing metadata with the token exchange ("FusedDispatch
// and FusedCombine").  Two launches, no host synchronisation in between:
//
//  1. topk_wave: one wave per token spread over many CUs.  Each lane holds
//     the logits of experts lane, lane+64, ...; K rounds of a wave-wide
//     argmax over (value desc, id asc) pick the experts in order, then the
//     gates and the physical ids (replica copy t mod r_e, shared expert
//     last) are written.
//  2. rank_dispatch: one block per token.  Every block rebuilds per-expert
//     token bit masks from the T x K ids in LDS (a few KB from L2), so the
//     rank of token t at expert p -- the number of lower tokens that chose
//     p -- is a popcount; its slots follow from the static bases.  Block 0
//     also writes counts, offsets and the drop total.  The block then
//     quantizes its token and stores it into its slots.
//
// moedc_route on a small batch runs step 1 and rank_single, the mask and
// rank work of step 2 in one block for all tokens.  Picks, counts, offsets,
// slots and dispatched bytes equal those of the large-batch kernels bit for
// bit; sigmoid gates too (same per-token arithmetic), while a softmax
// denominator is summed in another order (within the stated gate tolerance).
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"
#include "quant.hpp"

namespace moedc {

namespace {

constexpr int kBlock = 1024;                      // rank / dispatch blocks
constexpr int kMaskWords = kFusedMaxTokens / 64;  // token bits per expert
constexpr int kVals = kMaxExperts / 64;           // logits per lane, at most

// Order-preserving unsigned key of a float with -0 and +0 equal.
__device__ __forceinline__ uint32_t fkey(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);  // -0 + +0 = +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-wide max / min of a 32-bit value, returned wave-uniform: DPP within
// rows of 16 lanes, then the four row results read as scalars.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = row16_max_u32(v);
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return ~wave_max_u32(~v);
}

// Wave-wide sum, lanes added in a fixed tree order; wave-uniform result.
__device__ __forceinline__ float wave_sum(float z) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) z += __shfl_xor(z, d);
  return z;
}

// ---- 1. top-k, gates and physical ids: one wave per token -------------------
template <int KR, bool SHARED>
__global__ __launch_bounds__(256) void topk_wave(RouteArgs a) {
  constexpr int KT = KR + (SHARED ? 1 : 0);
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (t >= a.T) return;
  const int E = a.E, P = a.P;
  const float *row = a.logits + (int64_t)t * E;

  float v[kVals];
  uint32_t live = 0;  // bit i: expert lane + 64 i exists and is not yet picked
#pragma unroll
  for (int i = 0; i < kVals; ++i) {
    const int e = lane + 64 * i;
    v[i] = 0.0f;
    if (64 * i < E && e < E) {
      v[i] = row[e];
      live |= 1u << i;
    }
  }

  float pv[KR];
  int pid[KR];
#pragma unroll
  for (int j = 0; j < KR; ++j) {
    // Best live entry of this lane: ids ascend with i, so the first of equal
    // keys is the lower id.
    uint32_t bk = 0;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kVals; ++i) {
      const uint32_t k = fkey(v[i]);
      if (((live >> i) & 1u) && (bi == 0x7FFFFFFF || k > bk)) {
        bk = k;
        bi = lane + 64 * i;
      }
    }
    const uint32_t m = wave_max_u32(bi == 0x7FFFFFFF ? 0u : bk);
    const uint64_t cand = __ballot(bi != 0x7FFFFFFF && bk == m);
    int id;
    if (__popcll(cand) == 1) {
      id = __builtin_amdgcn_readlane(bi, (int)__ffsll((long long)cand) - 1);
    } else {  // equal keys in several lanes: the lowest id wins
      id = (int)wave_min_u32((cand >> lane) & 1u ? (uint32_t)bi : 0xFFFFFFFFu);
    }
    // Only non-finite rows can leave nothing to pick; keep the id valid.
    if (id >= E) id = 0;
    pid[j] = id;
    // The winning lane retires the entry and broadcasts its value.
    float val = 0.0f;
#pragma unroll
    for (int i = 0; i < kVals; ++i)
      if (lane + 64 * i == id) {
        val = v[i];
        live &= ~(1u << i);
      }
    pv[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(val), id & 63));
  }

  // ---- gates (every lane holds the same picks) ----
  float w[KT];
  if (a.score_fn == MOEDC_SCORE_SOFTMAX) {
    const float mx = pv[0];
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < kVals; ++i)
      if ((lane + 64 * i) < E && 64 * i < E) z += expf(v[i] - mx);
    const float Z = wave_sum(z);
#pragma unroll
    for (int j = 0; j < KR; ++j) w[j] = expf(pv[j] - mx) / Z;
  } else {
    float sg[KR];
    float S = 0.0f;
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      sg[j] = 1.0f / (1.0f + expf(-pv[j]));
      S += sg[j];
    }
#pragma unroll
    for (int j = 0; j < KR; ++j) w[j] = sg[j] / S;
  }
  int pk[KT];
#pragma unroll
  for (int j = 0; j < KR; ++j) pk[j] = a.rep_table[pid[j] * a.R + t % a.rep_count[pid[j]]];
  if (SHARED) {
    pk[KT - 1] = P - 1;
    w[KT - 1] = 1.0f;
  }
#pragma unroll
  for (int j = 0; j < KT; ++j)
    if (lane == j) {
      a.topk_ids[(int64_t)t * KT + j] = pk[j];
      a.topk_w[(int64_t)t * KT + j] = w[j];
    }
}

// ---- shared pieces of the rank kernels ----------------------------------------
struct RankLds {
  unsigned long long mask[kMaxExperts][kMaskWords];
  int wave_sum[kBlock / 64];
  int wave_drop[kBlock / 64];
};

// mask[p] bit t: token t chose physical expert p (from the written ids).
__device__ __forceinline__ void build_masks(const RouteArgs &a, RankLds &L) {
  const int tid = threadIdx.x;
  for (int i = tid; i < a.P * kMaskWords; i += kBlock) L.mask[i / kMaskWords][i % kMaskWords] = 0ull;
  __syncthreads();
  const int n = a.T * a.K;
  for (int i = tid; i < n; i += kBlock) {
    const int t = i / a.K;
    atomicOr(&L.mask[a.topk_ids[i]][t >> 6], 1ull << (t & 63));
  }
  __syncthreads();
}

// Tokens below t that chose p.
__device__ __forceinline__ int rank_of(const RankLds &L, int p, int t) {
  const int word = t >> 6;
  const uint64_t below = (t & 63) ? (~0ull >> (64 - (t & 63))) : 0ull;
  int r = __popcll(L.mask[p][word] & below);
  for (int wd = 0; wd < word; ++wd) r += __popcll(L.mask[p][wd]);
  return r;
}

// counts, offsets (block scan, one expert per thread) and the drop total.
__device__ __forceinline__ void counts_offsets(const RouteArgs &a, RankLds &L) {
  const int tid = threadIdx.x, P = a.P;
  int cnt = 0;
  if (tid < P) {
#pragma unroll
    for (int wd = 0; wd < kMaskWords; ++wd) cnt += __popcll(L.mask[tid][wd]);
    a.counts[tid] = cnt;
  }
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d);
    if ((tid & 63) >= d) incl += u;
  }
  if ((tid & 63) == 63) L.wave_sum[tid >> 6] = incl;
  const int drop = tid < P ? max(0, cnt - a.cap[tid]) : 0;
  int dsum = drop;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) dsum += __shfl_xor(dsum, d);
  if ((tid & 63) == 0) L.wave_drop[tid >> 6] = dsum;
  __syncthreads();
  int base = 0;
  for (int w2 = 0; w2 < (tid >> 6); ++w2) base += L.wave_sum[w2];
  if (tid < P) a.offsets[tid] = base + incl - cnt;
  if (tid == P - 1) a.offsets[P] = base + incl;
  if (tid == 0) {
    int tot = 0;
    for (int w2 = 0; w2 < kBlock / 64; ++w2) tot += L.wave_drop[w2];
    a.dropped[0] = tot;
  }
}

// ---- 2a. ranks and slots of every token in one block (moedc_route) ----------
__global__ __launch_bounds__(kBlock) void rank_single(RouteArgs a) {
  __shared__ RankLds L;
  build_masks(a, L);
  counts_offsets(a, L);
  const int n = a.T * a.K;
  for (int i = threadIdx.x; i < n; i += kBlock) {
    const int t = i / a.K, p = a.topk_ids[i];
    const int r = rank_of(L, p, t);
    a.slots[i] = r < a.cap[p] ? a.capbase[p] + r : -1;
  }
}

// ---- 2b. ranks of token blockIdx.x, then its dispatch ------------------------
template <bool PER_TOKEN>
__global__ __launch_bounds__(kBlock) void rank_dispatch(RouteArgs ra, DispatchArgs da) {
  __shared__ RankLds L;
  __shared__ int slot_of[kMaxK];
  __shared__ uint32_t chunk_max[kBlock / 64];
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  build_masks(ra, L);
  if (blockIdx.x == 0) counts_offsets(ra, L);
  if (tid < ra.K) {
    const int p = ra.topk_ids[(int64_t)t * ra.K + tid];
    const int r = rank_of(L, p, t);
    const int slot = r < ra.cap[p] ? ra.capbase[p] + r : -1;
    slot_of[tid] = slot;
    ra.slots[(int64_t)t * ra.K + tid] = slot;
  }
  __syncthreads();

  // wave c quantizes values 512 c .. 512 c + 511 of the token
  const int wave = uniform(tid >> 6), lane = lane_id();
  const int H = da.H;
  const int e = wave * 512 + lane * 8;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (e < H) v = reinterpret_cast<const uint4 *>(da.x + (int64_t)t * H)[wave * 64 + lane];
  uint32_t m = row16_max_u32(absmax8(v));
  if (PER_TOKEN) {
    m = max(m, (uint32_t)__shfl_xor((int)m, 16));
    m = max(m, (uint32_t)__shfl_xor((int)m, 32));
    if (lane == 0) chunk_max[wave] = m;
    __syncthreads();
    m = 0;
#pragma unroll
    for (int w2 = 0; w2 < kBlock / 64; ++w2) m = max(m, chunk_max[w2]);
  }
  const float s = __uint_as_float(m << 16) / 127.0f;
  const uint2 q = quant8(v, s);
  if (e < H) {
    for (int k = 0; k < da.K; ++k) {
      const int slot = slot_of[k];
      if (slot < 0) continue;
      uint8_t *dst = da.dbuf + (int64_t)slot * da.slot_stride;
      const u32x2 qq = {q.x, q.y};
      __builtin_nontemporal_store(qq, reinterpret_cast<u32x2 *>(dst + e));
      if (PER_TOKEN) {
        if (wave == 0 && lane == 0) __builtin_nontemporal_store(s, reinterpret_cast<float *>(dst + H));
      } else if ((lane & 15) == 0) {
        __builtin_nontemporal_store(s, reinterpret_cast<float *>(dst + H + 4 * (e >> 7)));
      }
    }
  }
}

template <int KR>
hipError_t launch_topk_kr(const RouteArgs &a, hipStream_t s) {
  const unsigned grid = (unsigned)((a.T + 3) / 4);
  if (a.shared)
    topk_wave<KR, true><<<grid, 256, 0, s>>>(a);
  else
    topk_wave<KR, false><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_topk_small(const RouteArgs &a, hipStream_t s) {
  switch (a.KR) {
#define MOEDC_CASE(k) \
  case k:             \
    return launch_topk_kr<k>(a, s);
    MOEDC_CASE(1) MOEDC_CASE(2) MOEDC_CASE(3) MOEDC_CASE(4) MOEDC_CASE(5) MOEDC_CASE(6)
    MOEDC_CASE(7) MOEDC_CASE(8) MOEDC_CASE(9) MOEDC_CASE(10) MOEDC_CASE(11) MOEDC_CASE(12)
    MOEDC_CASE(13) MOEDC_CASE(14) MOEDC_CASE(15) MOEDC_CASE(16)
#undef MOEDC_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_route_small(const RouteArgs &ra, hipStream_t s) {
  if (ra.T <= 0 || ra.T > kFusedMaxTokens || ra.P > kBlock) return hipErrorInvalidValue;
  hipError_t e = launch_topk_small(ra, s);
  if (e != hipSuccess) return e;
  rank_single<<<1, kBlock, 0, s>>>(ra);
  return hipGetLastError();
}

hipError_t launch_route_dispatch_fused(const RouteArgs &ra, const DispatchArgs &da,
                                       hipStream_t s) {
  if (ra.T <= 0 || ra.T > kFusedMaxTokens || ra.P > kBlock || da.H > 512 * (kBlock / 64))
    return hipErrorInvalidValue;
  hipError_t e = launch_topk_small(ra, s);
  if (e != hipSuccess) return e;
  if (da.per_token)
    rank_dispatch<true><<<ra.T, kBlock, 0, s>>>(ra, da);
  else
    rank_dispatch<false><<<ra.T, kBlock, 0, s>>>(ra, da);
  return hipGetLastError();
}

}  // namespace moedc
