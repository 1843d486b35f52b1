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
//   K1 route_topk_rank  64 tokens x 4 lanes per block: top-k over LDS tiles
//                       of the logits (next tile prefetched into registers),
//                       4-way merge, gates, replica mapping; block-local
//                       ranks and counts from per-expert 64-bit token masks
//                       in LDS (popcounts); writes per-block expert counts.
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

constexpr int kSub = 4;                    // lanes per token in the top-k scan
constexpr int kTileE = 64;                 // experts per LDS tile (16 per lane)
static_assert(kRouteTokens * kSub == 256, "one token per lane of wave 0");

// Insert (v, e) into a list kept in descending value order; equal values
// keep the earlier (lower-id) entry first because ids arrive ascending.
// Branch-free (selects only): slot j takes the new entry, or slot j-1's old
// one when the new entry lands above it; slots are updated from the bottom
// up, so slot j-1 is still unmodified when slot j reads it.
template <int KR>
__device__ __forceinline__ void topk_insert(float (&val)[KR], int (&id)[KR], float v, int e) {
#pragma unroll
  for (int j = KR - 1; j > 0; --j) {
    const bool take = v > val[j];
    const bool shift = v > val[j - 1];  // the new value lands above slot j
    const float nv = shift ? val[j - 1] : v;
    const int ni = shift ? id[j - 1] : e;
    val[j] = take ? nv : val[j];
    id[j] = take ? ni : id[j];
  }
  const bool take0 = v > val[0];
  val[0] = take0 ? v : val[0];
  id[0] = take0 ? e : id[0];
}

// A thread's share of one 64-expert tile of the block's logits, held in
// registers so the next tile's loads are in flight while this one is scanned.
struct TileRegs {
  float v[kRouteTokens * kTileE / 256];
};

__device__ __forceinline__ void tile_fetch(TileRegs &tr, const RouteArgs &a, int64_t row0,
                                           int e0, int ec, bool vec4) {
  const int tid = threadIdx.x;
  if (vec4) {  // E % 4 == 0: rows are 16-byte aligned and ec is a multiple of 4
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f = tid + 256 * j, r = f / (kTileE / 4), c = (f % (kTileE / 4)) * 4;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (row0 + r < a.T && c < ec)
        x = *reinterpret_cast<const float4 *>(a.logits + (row0 + r) * a.E + e0 + c);
      tr.v[4 * j] = x.x;
      tr.v[4 * j + 1] = x.y;
      tr.v[4 * j + 2] = x.z;
      tr.v[4 * j + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int f = tid + 256 * j, r = f / kTileE, c = f % kTileE;
      tr.v[j] = (row0 + r < a.T && c < ec) ? a.logits[(row0 + r) * a.E + e0 + c] : 0.f;
    }
  }
}

__device__ __forceinline__ void tile_store(float (&tile)[kRouteTokens][kTileE + 1],
                                           const TileRegs &tr, bool vec4) {
  const int tid = threadIdx.x;
  if (vec4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f = tid + 256 * j, r = f / (kTileE / 4), c = (f % (kTileE / 4)) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) tile[r][c + i] = tr.v[4 * j + i];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int f = tid + 256 * j;
      tile[f / kTileE][f % kTileE] = tr.v[j];
    }
  }
}

// One block = kRouteTokens tokens x kSub lanes.  Lane `sub` of token r scans
// columns [16 sub, 16 sub + 16) of every 64-expert tile and keeps a local
// top-KR; wave 0 (lane = token) merges the four lists, computes gates and the
// physical ids.  Ranks come from one 64-bit token mask per expert in LDS:
// bit l of mask[p] is set iff token l of the block routes to p (atomic OR,
// so the result does not depend on arrival order); a token's rank for p is
// the popcount of the mask below its bit, the block's count the full
// popcount.
template <int KR, bool SHARED>
__global__ __launch_bounds__(256) void route_topk_rank(RouteArgs a) {
  constexpr int KT = KR + (SHARED ? 1 : 0);
  __shared__ float tile[kRouteTokens][kTileE + 1];
  // Token-minor, so the merge's reads (lane = token, each at its own list
  // position) hit distinct banks.
  __shared__ float lval[kSub][KR][kRouteTokens];
  __shared__ int lid[kSub][KR][kRouteTokens];
  __shared__ float zpart[kRouteTokens][kSub];
  __shared__ float mrow[kRouteTokens];
  __shared__ unsigned long long tokmask[kMaxExperts];

  const int tid = threadIdx.x;
  const int r = tid >> 2, sub = tid & 3;
  const int64_t row0 = (int64_t)blockIdx.x * kRouteTokens;
  const int E = a.E, P = a.P;
  const bool vec4 = (E & 3) == 0;

  for (int i = tid; i < P; i += 256) tokmask[i] = 0ull;

  // ---- scan: local top-KR over this lane's columns ----------------------
  float val[KR];
  int id[KR];
#pragma unroll
  for (int j = 0; j < KR; ++j) {
    val[j] = -__builtin_inff();
    id[j] = j;  // valid ids even if a row has no finite logit
  }
  TileRegs tr;
  tile_fetch(tr, a, row0, 0, min(kTileE, E), vec4);
  for (int e0 = 0; e0 < E; e0 += kTileE) {
    const int ec = min(kTileE, E - e0);
    __syncthreads();
    tile_store(tile, tr, vec4);
    __syncthreads();
    if (e0 + kTileE < E) tile_fetch(tr, a, row0, e0 + kTileE, min(kTileE, E - e0 - kTileE), vec4);
    if (ec == kTileE) {  // full tile (block-uniform): a fixed, unrolled scan
#pragma unroll
      for (int i = 0; i < kTileE / kSub; ++i)
        topk_insert<KR>(val, id, tile[r][16 * sub + i], e0 + 16 * sub + i);
    } else {
      const int c1 = min(16 * sub + 16, ec);
      for (int c = 16 * sub; c < c1; ++c) topk_insert<KR>(val, id, tile[r][c], e0 + c);
    }
  }
#pragma unroll
  for (int j = 0; j < KR; ++j) {
    lval[sub][j][r] = val[j];
    lid[sub][j][r] = id[j];
  }
  __syncthreads();

  // ---- wave 0: merge the four lists (value desc, id asc) -----------------
  const int64_t t = row0 + tid;
  const bool active = tid < kRouteTokens && t < a.T;
  if (tid < kRouteTokens) {
    int h[kSub] = {0, 0, 0, 0};  // next unread entry of each lane's list
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      float bv = -__builtin_inff();
      int bi = 0, bs = -1;
#pragma unroll
      for (int s2 = 0; s2 < kSub; ++s2) {
        if (h[s2] < KR) {
          const float v = lval[s2][h[s2]][tid];
          const int i = lid[s2][h[s2]][tid];
          if (bs < 0 || v > bv || (v == bv && i < bi)) {
            bv = v;
            bi = i;
            bs = s2;
          }
        }
      }
      val[j] = bv;
      id[j] = bi;
#pragma unroll
      for (int s2 = 0; s2 < kSub; ++s2) h[s2] += bs == s2;
    }
    mrow[tid] = val[0];
  }

  // ---- softmax denominator: second pass over the tiles ---------------------
  float Z = 0.0f;
  if (a.score_fn == MOEDC_SCORE_SOFTMAX) {
    __syncthreads();
    const float m = mrow[r];
    float z = 0.0f;
    tile_fetch(tr, a, row0, 0, min(kTileE, E), vec4);
    for (int e0 = 0; e0 < E; e0 += kTileE) {
      const int ec = min(kTileE, E - e0);
      __syncthreads();
      tile_store(tile, tr, vec4);
      __syncthreads();
      if (e0 + kTileE < E) tile_fetch(tr, a, row0, e0 + kTileE, min(kTileE, E - e0 - kTileE), vec4);
      if (ec == kTileE) {
#pragma unroll
        for (int i = 0; i < kTileE / kSub; ++i) z += expf(tile[r][16 * sub + i] - m);
      } else {
        const int c1 = min(16 * sub + 16, ec);
        for (int c = 16 * sub; c < c1; ++c) z += expf(tile[r][c] - m);
      }
    }
    zpart[r][sub] = z;
    __syncthreads();
    if (tid < kRouteTokens) Z = ((zpart[tid][0] + zpart[tid][1]) + zpart[tid][2]) + zpart[tid][3];
  }

  // ---- wave 0: gates, physical ids, outputs, token masks --------------------
  int pk[KT];
  if (tid < kRouteTokens) {
    float w[KT];
    if (a.score_fn == MOEDC_SCORE_SOFTMAX) {
#pragma unroll
      for (int j = 0; j < KR; ++j) w[j] = expf(val[j] - val[0]) / Z;
    } else {
      float sg[KR];
      float S = 0.0f;
#pragma unroll
      for (int j = 0; j < KR; ++j) {
        sg[j] = 1.0f / (1.0f + expf(-val[j]));
        S += sg[j];
      }
#pragma unroll
      for (int j = 0; j < KR; ++j) w[j] = sg[j] / S;
    }
#pragma unroll
    for (int j = 0; j < KR; ++j) {  // replica copy t mod r_e
      const int e = id[j];
      pk[j] = a.rep_identity ? e : a.rep_table[e * a.R + (int)t % a.rep_count[e]];
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
        atomicOr(&tokmask[pk[j]], 1ull << tid);
      }
    }
  }
  __syncthreads();
  if (active) {
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int j = 0; j < KT; ++j)  // block-local rank, finished by route_slots
      a.slots[t * KT + j] = __popcll(tokmask[pk[j]] & lt);
  }
  int32_t *bc = a.block_counts + (int64_t)blockIdx.x * P;
  for (int p = tid; p < P; p += 256) bc[p] = __popcll(tokmask[p]);
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
  for (int b0 = 0; b0 < nblk; b0 += 256) {
    int v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int b = b0 + 64 * u + l;
      v[u] = b < nblk ? bc[(int64_t)b * P + p] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int b = b0 + 64 * u + l;
      const int incl = wave_inclusive_scan(v[u]);
      if (b < nblk) bc[(int64_t)b * P + p] = carry + incl - v[u];
      carry += __shfl(incl, 63);
    }
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
    route_topk_rank<KR, true><<<nblk, 256, 0, s>>>(a);
  else
    route_topk_rank<KR, false><<<nblk, 256, 0, s>>>(a);
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
