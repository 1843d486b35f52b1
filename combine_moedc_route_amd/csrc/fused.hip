// fused.hip -- single-launch route + dispatch for small decode batches
// (T <= 256 tokens), gfx950.
//
// Latency, not bandwidth, bounds a decode batch of one die's share ("Decode
// Phase" of the CloudMatrix384 article: 96 tokens per die), and the pages'
// operators fuse routing metadata with the token exchange ("FusedDispatch
// and FusedCombine").  Here one kernel does both, with no inter-block
// synchronisation: every block recomputes the routing of all T tokens (a
// few hundred KB of L2-resident logits) and then quantizes and stores the
// one token with index blockIdx.x.  Block 0 also writes the route outputs.
//
// Routing in a block: L lanes per token (L = 4, 8 or 16); lane s of a token
// scans columns s, s+L, s+2L, ... (ascending ids) into a register top-K
// list; the L lists are merged with log2(L) shuffle rounds of a bitonic
// top-K merge over (value desc, id asc).  Ranks and counts come from
// per-expert token bit masks in LDS (atomic OR; order-free), slots from the
// static bases.  Picks, ids, counts, offsets, slots and the dispatched bytes
// equal those of moedc_route + moedc_dispatch bit for bit; sigmoid gates
// too (same per-token arithmetic), while the softmax denominator is summed
// in another order (both within the stated gate tolerance).
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"
#include "quant.hpp"

namespace moedc {

namespace {

constexpr int kThreads = 1024;
constexpr int kMaskWords = kFusedMaxTokens / 64;

struct Cand {
  float v;
  int id;
};

__device__ __forceinline__ bool better(const Cand &a, const Cand &b) {
  return a.v > b.v || (a.v == b.v && a.id < b.id);
}

// Descending bitonic clean-up of n (power of two) candidates.
template <int N>
__device__ __forceinline__ void bitonic_clean(Cand (&c)[N]) {
#pragma unroll
  for (int s = N / 2; s >= 1; s >>= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if ((i & s) == 0) {
        if (better(c[i + s], c[i])) {
          const Cand t = c[i];
          c[i] = c[i + s];
          c[i + s] = t;
        }
      }
    }
  }
}

// Top-N of two descending lists: C[i] = better of A[i], B[N-1-i] is bitonic
// and holds the N best; a clean-up sorts it.
template <int N>
__device__ __forceinline__ void merge_with_lane(Cand (&c)[N], int xor_mask) {
  Cand o[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    o[i].v = __shfl_xor(c[i].v, xor_mask);
    o[i].id = __shfl_xor(c[i].id, xor_mask);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const Cand b = o[N - 1 - i];
    if (better(b, c[i])) c[i] = b;
  }
  bitonic_clean<N>(c);
}

template <int N>
__device__ __forceinline__ void insert(Cand (&c)[N], float v, int e) {
  // Lists stay descending; an equal value never displaces an earlier
  // (lower-id) entry because ids arrive ascending.
#pragma unroll
  for (int j = N - 1; j >= 0; --j) {
    const int jp = j > 0 ? j - 1 : 0;
    const bool shift = j > 0 && v > c[jp].v;
    if (v > c[j].v) {
      c[j].v = shift ? c[jp].v : v;
      c[j].id = shift ? c[jp].id : e;
    }
  }
}

template <int KR, int KRP, bool SHARED, int L, bool PER_TOKEN>
__global__ __launch_bounds__(kThreads) void route_dispatch_fused(RouteArgs ra, DispatchArgs da) {
  constexpr int KT = KR + (SHARED ? 1 : 0);
  __shared__ unsigned long long tokmask[kMaxExperts][kMaskWords];
  __shared__ int slots_lds[kFusedMaxTokens][KT];
  __shared__ int wave_sum[kThreads / 64];
  __shared__ int wave_drop[kThreads / 64];
  __shared__ uint32_t chunk_max[kThreads / 64];

  const int tid = threadIdx.x;
  const int T = ra.T, E = ra.E, P = ra.P;
  const int tok = tid / L, sub = tid % L;
  const bool have_tok = tok < T;

  for (int i = tid; i < P * kMaskWords; i += kThreads) tokmask[i / kMaskWords][i % kMaskWords] = 0ull;

  // ---- top-k of token `tok`: strided columns per lane, then lane merges ----
  Cand c[KRP];
#pragma unroll
  for (int j = 0; j < KRP; ++j) {
    c[j].v = -__builtin_inff();
    c[j].id = kMaxExperts + j;  // padding sorts after every real id
  }
  const float *row = ra.logits + (int64_t)(have_tok ? tok : 0) * E;
  for (int e0 = sub; e0 < E; e0 += 16 * L) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = e0 + i * L;
      v[i] = (have_tok && e < E) ? row[e] : -__builtin_inff();
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (e0 + i * L < E) insert<KRP>(c, v[i], e0 + i * L);
  }
#pragma unroll
  for (int d = 1; d < L; d <<= 1) merge_with_lane<KRP>(c, d);
  // Every lane of the token now holds the same top list; clamp padding ids
  // (only reachable with non-finite logits) to a valid expert.
#pragma unroll
  for (int j = 0; j < KR; ++j)
    if (c[j].id >= E) c[j].id = 0;

  // ---- gates ----------------------------------------------------------------
  float w[KT];
  if (ra.score_fn == MOEDC_SCORE_SOFTMAX) {
    const float m = c[0].v;
    float z = 0.0f;
    for (int e = sub; e < E; e += L) z += have_tok ? expf(row[e] - m) : 0.0f;
#pragma unroll
    for (int d = 1; d < L; d <<= 1) z += __shfl_xor(z, d);
#pragma unroll
    for (int j = 0; j < KR; ++j) w[j] = expf(c[j].v - m) / z;
  } else {
    float sg[KR];
    float S = 0.0f;
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      sg[j] = 1.0f / (1.0f + expf(-c[j].v));
      S += sg[j];
    }
#pragma unroll
    for (int j = 0; j < KR; ++j) w[j] = sg[j] / S;
  }

  // ---- physical ids, token masks ------------------------------------------------
  int pk[KT];
#pragma unroll
  for (int j = 0; j < KR; ++j) {
    const int e = c[j].id;
    pk[j] = ra.rep_table[e * ra.R + tok % ra.rep_count[e]];
  }
  if (SHARED) {
    pk[KT - 1] = P - 1;
    w[KT - 1] = 1.0f;
  }
  const bool owner = have_tok && sub == 0;
  if (owner) {
#pragma unroll
    for (int j = 0; j < KT; ++j) atomicOr(&tokmask[pk[j]][tok >> 6], 1ull << (tok & 63));
  }
  __syncthreads();

  // ---- ranks -> slots; block 0 writes the route outputs ----------------------
  if (owner) {
    const int word = tok >> 6;
    const uint64_t below = (tok & 63) ? (~0ull >> (64 - (tok & 63))) : 0ull;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const int p = pk[j];
      int rank = __popcll(tokmask[p][word] & below);
      for (int wd = 0; wd < word; ++wd) rank += __popcll(tokmask[p][wd]);
      const int slot = rank < ra.cap[p] ? ra.capbase[p] + rank : -1;
      slots_lds[tok][j] = slot;
      if (blockIdx.x == 0) {
        ra.topk_ids[tok * KT + j] = p;
        ra.topk_w[tok * KT + j] = w[j];
        ra.slots[tok * KT + j] = slot;
      }
    }
  }
  if (blockIdx.x == 0) {
    // counts, offsets (LDS-staged block scan, one expert per thread), drops
    int cnt = 0;
    if (tid < P) {
#pragma unroll
      for (int wd = 0; wd < kMaskWords; ++wd) cnt += __popcll(tokmask[tid][wd]);
      ra.counts[tid] = cnt;
    }
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(incl, d);
      if ((tid & 63) >= d) incl += u;
    }
    if ((tid & 63) == 63) wave_sum[tid >> 6] = incl;
    const int drop = tid < P ? max(0, cnt - ra.cap[tid]) : 0;
    __syncthreads();
    int base = 0;
    for (int w2 = 0; w2 < (tid >> 6); ++w2) base += wave_sum[w2];
    if (tid < P) ra.offsets[tid] = base + incl - cnt;
    if (tid == P - 1) ra.offsets[P] = base + incl;
    int dsum = drop;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) dsum += __shfl_xor(dsum, d);
    if ((tid & 63) == 0) wave_drop[tid >> 6] = dsum;
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int w2 = 0; w2 < kThreads / 64; ++w2) tot += wave_drop[w2];
      ra.dropped[0] = tot;
    }
  }
  __syncthreads();

  // ---- dispatch token blockIdx.x: wave c quantizes chunk c ---------------------
  const int t = blockIdx.x;
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
    for (int w2 = 0; w2 < kThreads / 64; ++w2) m = max(m, chunk_max[w2]);
  }
  const float s = __uint_as_float(m << 16) / 127.0f;
  const uint2 q = quant8(v, s);
  if (e < H) {
    for (int k = 0; k < KT; ++k) {
      const int slot = slots_lds[t][k];
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

template <int KR, bool SHARED, int L, bool PT>
hipError_t launch4(const RouteArgs &ra, const DispatchArgs &da, hipStream_t s) {
  constexpr int KRP = KR <= 1 ? 1 : KR <= 2 ? 2 : KR <= 4 ? 4 : KR <= 8 ? 8 : 16;
  route_dispatch_fused<KR, KRP, SHARED, L, PT><<<ra.T, kThreads, 0, s>>>(ra, da);
  return hipGetLastError();
}

template <int KR>
hipError_t launch_kr(const RouteArgs &ra, const DispatchArgs &da, hipStream_t s) {
  const int L = ra.T <= 64 ? 16 : ra.T <= 128 ? 8 : 4;
  const bool pt = da.per_token != 0;
#define MOEDC_L(LL)                                                          \
  if (L == LL) {                                                             \
    if (ra.shared)                                                           \
      return pt ? launch4<KR, true, LL, true>(ra, da, s)                      \
                : launch4<KR, true, LL, false>(ra, da, s);                    \
    return pt ? launch4<KR, false, LL, true>(ra, da, s)                       \
              : launch4<KR, false, LL, false>(ra, da, s);                     \
  }
  MOEDC_L(16) MOEDC_L(8) MOEDC_L(4)
#undef MOEDC_L
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_route_dispatch_fused(const RouteArgs &ra, const DispatchArgs &da,
                                       hipStream_t s) {
  if (ra.T <= 0 || ra.T > kFusedMaxTokens) return hipErrorInvalidValue;
  switch (ra.KR) {
#define MOEDC_CASE(k) \
  case k:             \
    return launch_kr<k>(ra, da, s);
    MOEDC_CASE(1) MOEDC_CASE(2) MOEDC_CASE(3) MOEDC_CASE(4) MOEDC_CASE(5) MOEDC_CASE(6)
    MOEDC_CASE(7) MOEDC_CASE(8) MOEDC_CASE(9) MOEDC_CASE(10) MOEDC_CASE(11) MOEDC_CASE(12)
    MOEDC_CASE(13) MOEDC_CASE(14) MOEDC_CASE(15) MOEDC_CASE(16)
#undef MOEDC_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace moedc
