// route.hip -- top-k routing, per-expert histogram, scans and slot
// assignment on gfx950.
//
// What is computed follows the routing metadata of "CloudMatrix384:
// Co-Designing Supernodes for Trillion-Parameter LLM Inference", sections
// "Decode Phase" (routed/shared/redundant experts) and "FusedDispatch and
// FusedCombine" (metadata that tells each sender where in the receiver's
// pre-allocated buffer a token goes).  The slot of (token t, pick j) is the
// expert's static base plus the rank of t among that expert's tokens in
// ascending token order, so the layout is deterministic without atomics:
//
//   K1 route_topk_rank  one thread per token: top-k over LDS tiles of the
//                       logits, gates, replica mapping; in-wave ranks from
//                       bit-sliced ballots (a match-any over expert ids),
//                       in-block ranks from an LDS table of per-wave counts;
//                       writes per-block expert counts.
//   K2 route_block_scan one wave per expert: exclusive scan over blocks of
//                       the per-block counts (DPP/shuffle wave scan); the
//                       total is counts[p].
//   K3 route_slots      one thread per entry: slot = base + block base +
//                       in-block rank, or -1 past capacity; the last block
//                       does the LDS-staged scan counts -> offsets and the
//                       drop count.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"

namespace moedc {

namespace {

constexpr int kTileE = 32;                 // experts per LDS tile
constexpr int kWaves = kRouteTokens / 64;  // waves per route block
constexpr int kIdBits = 11;                // ids 0..1024 (1024 = inactive lane)

// Insert (v, e) into a list kept in descending value order; equal values
// keep the earlier (lower-id) entry first because ids arrive ascending.
template <int KR>
__device__ __forceinline__ void topk_insert(float (&val)[KR], int (&id)[KR], float v, int e) {
#pragma unroll
  for (int j = KR - 1; j >= 0; --j) {
    const int jp = j > 0 ? j - 1 : 0;
    const bool shift = j > 0 && v > val[jp];  // the new value lands above slot j
    if (v > val[j]) {
      val[j] = shift ? val[jp] : v;
      id[j] = shift ? id[jp] : e;
    }
  }
}

template <int KR, bool SHARED>
__global__ __launch_bounds__(kRouteTokens) void route_topk_rank(RouteArgs a) {
  constexpr int KT = KR + (SHARED ? 1 : 0);
  __shared__ float tile[kRouteTokens][kTileE + 1];
  __shared__ int32_t hist[kWaves][kMaxExperts];
  __shared__ int32_t ids_lds[KT][kRouteTokens];
  __shared__ int32_t rank_lds[KT][kRouteTokens];

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int64_t row0 = (int64_t)blockIdx.x * kRouteTokens;
  const int64_t t = row0 + tid;
  const bool active = t < a.T;
  const int E = a.E, P = a.P;

  for (int i = tid; i < kWaves * P; i += kRouteTokens) hist[i / P][i % P] = 0;

  // ---- top-k over tiles of kTileE experts ------------------------------
  float val[KR];
  int id[KR];
#pragma unroll
  for (int j = 0; j < KR; ++j) {
    val[j] = -__builtin_inff();
    id[j] = j;  // valid distinct ids even if a row has no finite logit
  }
  for (int e0 = 0; e0 < E; e0 += kTileE) {
    const int ec = min(kTileE, E - e0);
    __syncthreads();
    for (int f = tid; f < kRouteTokens * kTileE; f += kRouteTokens) {
      const int r = f / kTileE, c = f % kTileE;
      float v = -__builtin_inff();
      if (row0 + r < a.T && c < ec) v = a.logits[(row0 + r) * E + e0 + c];
      tile[r][c] = v;
    }
    __syncthreads();
    for (int c = 0; c < ec; ++c) topk_insert<KR>(val, id, tile[tid][c], e0 + c);
  }

  // ---- gates -------------------------------------------------------------
  float w[KT];
  if (a.score_fn == MOEDC_SCORE_SOFTMAX) {
    const float m = val[0];
    float Z = 0.0f;
    for (int e0 = 0; e0 < E; e0 += kTileE) {
      const int ec = min(kTileE, E - e0);
      __syncthreads();
      for (int f = tid; f < kRouteTokens * kTileE; f += kRouteTokens) {
        const int r = f / kTileE, c = f % kTileE;
        float v = -__builtin_inff();
        if (row0 + r < a.T && c < ec) v = a.logits[(row0 + r) * E + e0 + c];
        tile[r][c] = v;
      }
      __syncthreads();
      for (int c = 0; c < ec; ++c) Z += expf(tile[tid][c] - m);
    }
#pragma unroll
    for (int j = 0; j < KR; ++j) w[j] = expf(val[j] - m) / Z;
  } else {
    float s[KR];
    float S = 0.0f;
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      s[j] = 1.0f / (1.0f + expf(-val[j]));
      S += s[j];
    }
#pragma unroll
    for (int j = 0; j < KR; ++j) w[j] = s[j] / S;
  }

  // ---- physical mapping ----------------------------------------------------
  int pk[KT];
#pragma unroll
  for (int j = 0; j < KR; ++j) {
    const int e = id[j];
    const int r = a.rep_count[e];
    pk[j] = a.rep_table[e * a.R + (int)t % r];
  }
  if (SHARED) {
    pk[KT - 1] = P - 1;
    w[KT - 1] = 1.0f;
  }
  if (active) {
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      a.topk_ids[t * KT + j] = pk[j];
      a.topk_w[t * KT + j] = w[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < KT; ++j) pk[j] = kMaxExperts;  // matches no real id
  }

  // ---- in-wave ranks: bit-sliced ballots ------------------------------------
  // For entry (lane, j) with id v, the lanes whose entry j2 also holds v are
  // AND over id bits b of (bit b of v ? ballot(bit b) : ~ballot(bit b)) -- a
  // match-any built from ballots.  A token holds an id at most once, so the
  // rank of the lane for v is the number of lower lanes holding v at any
  // position, and the lane with rank 0 is the wave's leader for v.
#pragma unroll
  for (int j = 0; j < KT; ++j) ids_lds[j][tid] = pk[j];
  __syncthreads();  // ids staged; hist zeroed; tiles consumed
  const uint64_t act = __ballot(active);
  const uint64_t lt = lanemask_lt();
#pragma unroll 1
  for (int j = 0; j < KT; ++j) {
    const int v = ids_lds[j][tid];
    int rank = 0, cnt = 0;
#pragma unroll 1
    for (int j2 = 0; j2 < KT; ++j2) {
      const int other = ids_lds[j2][tid];
      uint64_t m = act;
#pragma unroll
      for (int b = 0; b < kIdBits; ++b) {
        const uint64_t B = __ballot((other >> b) & 1);
        m &= ((v >> b) & 1) ? B : ~B;
      }
      rank += __popcll(m & lt);
      cnt += __popcll(m);
    }
    rank_lds[j][tid] = rank;
    if (active && rank == 0) hist[wave][v] = cnt;
  }
  __syncthreads();

  // ---- in-block ranks via per-wave counts in LDS ----------------------------
  if (active) {
#pragma unroll 1
    for (int j = 0; j < KT; ++j) {
      const int v = ids_lds[j][tid];
      int base = 0;
      for (int w2 = 0; w2 < wave; ++w2) base += hist[w2][v];
      a.slots[t * KT + j] = base + rank_lds[j][tid];  // finished by route_slots
    }
  }
  int32_t *bc = a.block_counts + (int64_t)blockIdx.x * P;
  for (int p = tid; p < P; p += kRouteTokens) {
    int c = 0;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) c += hist[w2][p];
    bc[p] = c;
  }
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d);
    if (l >= d) v += u;
  }
  return v;
}

// One wave per physical expert: block counts -> exclusive block bases.
__global__ __launch_bounds__(256) void route_block_scan(int32_t *bc, int32_t *counts, int nblk,
                                                        int P) {
  const int p = blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (p >= P) return;
  const int l = lane_id();
  int carry = 0;
  for (int b0 = 0; b0 < nblk; b0 += 64) {
    const int b = b0 + l;
    const int v = b < nblk ? bc[(int64_t)b * P + p] : 0;
    const int incl = wave_inclusive_scan(v);
    if (b < nblk) bc[(int64_t)b * P + p] = carry + incl - v;
    carry += __shfl(incl, 63);
  }
  if (l == 0) counts[p] = carry;
}

// Entries -> slots; the last block also scans counts into offsets and
// counts the drops (LDS-staged block scan).
__global__ __launch_bounds__(256) void route_slots(RouteArgs a, int64_t entries) {
  const int tid = threadIdx.x;
  if (blockIdx.x == gridDim.x - 1) {
    __shared__ int wave_tot[4];
    __shared__ int wave_drop[4];
    const int P = a.P;
    constexpr int per = kMaxExperts / 256;  // experts per thread
    int loc[per];
    int sum = 0, drop = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const int p = tid * per + i;
      loc[i] = p < P ? a.counts[p] : 0;
      if (p < P) drop += max(0, loc[i] - a.cap[p]);
      sum += loc[i];
    }
    const int incl = wave_inclusive_scan(sum);
    int dsum = drop;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) dsum += __shfl_xor(dsum, d);
    const int w = tid >> 6;
    if (lane_id() == 63) wave_tot[w] = incl;
    if (lane_id() == 0) wave_drop[w] = dsum;
    __syncthreads();
    int base = 0;
    for (int w2 = 0; w2 < w; ++w2) base += wave_tot[w2];
    int run = base + incl - sum;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const int p = tid * per + i;
      if (p < P) a.offsets[p] = run;
      run += loc[i];
    }
    if (tid == 255) a.offsets[P] = run;
    if (tid == 0) a.dropped[0] = wave_drop[0] + wave_drop[1] + wave_drop[2] + wave_drop[3];
    return;
  }
  const int64_t i = (int64_t)blockIdx.x * 256 + tid;
  if (i >= entries) return;
  const int64_t t = i / a.K;
  const int p = a.topk_ids[i];
  const int j = a.block_counts[(t / kRouteTokens) * a.P + p] + a.slots[i];
  a.slots[i] = j < a.cap[p] ? a.capbase[p] + j : -1;
}

template <int KR>
hipError_t launch_topk(const RouteArgs &a, int nblk, hipStream_t s) {
  if (a.shared)
    route_topk_rank<KR, true><<<nblk, kRouteTokens, 0, s>>>(a);
  else
    route_topk_rank<KR, false><<<nblk, kRouteTokens, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t s) {
  const int nblk = (a.T + kRouteTokens - 1) / kRouteTokens;
  hipError_t e = hipSuccess;
  if (nblk > 0) {
    switch (a.KR) {
#define MOEDC_CASE(k) \
  case k:             \
    e = launch_topk<k>(a, nblk, s); \
    break;
      MOEDC_CASE(1) MOEDC_CASE(2) MOEDC_CASE(3) MOEDC_CASE(4) MOEDC_CASE(5) MOEDC_CASE(6)
      MOEDC_CASE(7) MOEDC_CASE(8) MOEDC_CASE(9) MOEDC_CASE(10) MOEDC_CASE(11) MOEDC_CASE(12)
      MOEDC_CASE(13) MOEDC_CASE(14) MOEDC_CASE(15) MOEDC_CASE(16)
#undef MOEDC_CASE
      default:
        return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  // counts: zero when no block ran.
  route_block_scan<<<(a.P + 3) / 4, 256, 0, s>>>(a.block_counts, a.counts, nblk, a.P);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t entries = (int64_t)a.T * a.K;
  const int64_t grid = (entries + 255) / 256 + 1;
  route_slots<<<(unsigned)grid, 256, 0, s>>>(a, entries);
  return hipGetLastError();
}

}  // namespace moedc
