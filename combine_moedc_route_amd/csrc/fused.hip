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
//     argmax over (value desc, id asc) pick the experts in order, lane j
//     keeping pick j; lane j then evaluates pick j's gate and physical id
//     (replica copy t mod r_e, shared expert last) and writes them.
//  2. rank_dispatch: one block per token.  Every block rebuilds per-expert
//     token bit masks from the T x K ids in LDS (a few KB from L2), so the
//     rank of token t at expert p -- the number of lower tokens that chose
//     p -- is a popcount; its slots follow from the static bases.  The
//     block then quantizes its token and stores it into its slots; one
//     extra block writes counts, offsets and the drop total.
//
// moedc_route on a small batch runs step 1 and rank_single, the mask and
// rank work of step 2 for all tokens in one block (a second one writes the
// counts, offsets and drops).
//
// Up to kOneLaunchTokens tokens (one per wave of a block) both entries are a
// single launch instead: every block runs the whole batch's top-k itself
// and goes straight on to its ranks, which saves a launch and a round trip
// through memory.  A wave's top-k of one token is ~1.7 us of dependent
// cross-lane steps (K rounds of ~460 cycles), so beyond one token per wave
// the two-launch path is faster (at 96 tokens the one-launch form measured
// 22 us against 9.7).  Picks, counts, offsets, slots and dispatched bytes
// equal those of the large-batch kernels bit for bit; sigmoid gates too
// (same per-token arithmetic), while a softmax denominator is summed in
// another order (within the stated gate tolerance).
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"
#include "quant.hpp"

namespace moedc {

namespace {

constexpr int kBlock = 1024;                      // rank / dispatch blocks
constexpr int kMaskWords = kFusedMaxTokens / 64;  // token bits per expert
constexpr int kOneLaunchTokens = 16;  // one launch up to one token per wave

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

// Float back from a key (the -0 of a tie pair comes back as +0, which no
// gate can tell apart).
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ---- 1. top-k, gates and physical ids: one wave per token -------------------
// The pieces below are shared by every small-batch kernel, so all of them
// pick, weight and map a token's experts with the same instructions.

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// K_R rounds of a wave-wide argmax over (value desc, id asc); lane j < K_R
// receives pick j's value (pv) and logical id (pe); v[] keeps the token's
// logits.  NV = logits per lane (a power of two >= E / 64).  A key of 0
// marks an empty or already picked entry: every finite logit's key is
// above it.  The rounds are bound by the dependent cross-lane steps (DPP
// row max, readlanes, ballot); sorting each lane's candidates once instead
// of scanning them every round measured no faster.
template <int NV>
__device__ __forceinline__ void topk_picks(const RouteArgs &a, int t, int lane, float (&v)[NV],
                                           float &pv, int &pe) {
  const int E = a.E, KR = a.KR;
  const float *row = a.logits + (int64_t)t * E;
  uint32_t key[NV];
  // Unconditional loads (lanes past E read entry E-1 and drop it) so that
  // all NV loads are in flight together behind one wait.
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = row[min(lane + 64 * i, E - 1)];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? fkey(v[i]) : 0u;
    v[i] = e < E ? v[i] : 0.0f;
  }

  pv = 0.0f;
  pe = 0;
  for (int j = 0; j < KR; ++j) {
    // This lane's best candidate (ids ascend with i, so the first of equal
    // keys is the lower id).
    uint32_t bk = key[0];
    int bi = lane;
#pragma unroll
    for (int i = 1; i < NV; ++i)
      if (key[i] > bk) {
        bk = key[i];
        bi = lane + 64 * i;
      }
    const uint32_t m = wave_max_u32(bk);
    const uint64_t cand = __ballot(bk == m);
    int id;
    if (__popcll(cand) == 1)
      id = __builtin_amdgcn_readlane(bi, (int)__ffsll((long long)cand) - 1);
    else  // equal keys in several lanes: the lowest id wins
      id = (int)wave_min_u32(bk == m ? (uint32_t)bi : 0xFFFFFFFFu);
    if (m == 0u || id >= E) id = 0;  // nothing left: only non-finite rows
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + 64 * i == id) key[i] = 0u;
    if (lane == j) {
      pv = key_float(m);
      pe = id;
    }
  }
}

// Gate of pick `lane` (lanes < K_R; sums in pick order, as the large-batch
// kernel does).  pv: this lane's pick value from topk_picks.
template <int NV>
__device__ __forceinline__ float topk_gate(const RouteArgs &a, int lane, const float (&v)[NV],
                                           float pv) {
  const int E = a.E, KR = a.KR;
  float wj = 0.0f;
  if (a.score_fn == MOEDC_SCORE_SOFTMAX) {
    const float mx = readlane_f(pv, 0);
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + 64 * i < E) z += expf(v[i] - mx);
    const float Z = wave_sum(z);
    if (lane < KR) wj = expf(pv - mx) / Z;
  } else {
    // Lane j evaluates pick j's sigmoid; the sum still runs in pick order.
    const float sg = 1.0f / (1.0f + expf(-pv));
    float S = 0.0f;
    for (int j = 0; j < KR; ++j) S += readlane_f(sg, j);
    wj = sg / S;
  }
  return wj;
}

// Physical id of entry `lane` of token t: pick `lane` (pe) mapped to its
// replica copy t mod r_e, the shared expert after the routed picks, -1
// past K.
template <bool SHARED>
__device__ __forceinline__ int entry_id(const RouteArgs &a, int t, int lane, int pe) {
  if (lane < a.KR) return a.rep_identity ? pe : a.rep_table[pe * a.R + t % a.rep_count[pe]];
  return SHARED && lane == a.KR ? a.P - 1 : -1;
}

template <int NV, bool SHARED>
__global__ __launch_bounds__(256) void topk_wave(RouteArgs a) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (t >= a.T) return;
  float v[NV], pv;
  int pe;
  topk_picks<NV>(a, t, lane, v, pv, pe);
  const float wj = topk_gate<NV>(a, lane, v, pv);
  const int id = entry_id<SHARED>(a, t, lane, pe);
  if (lane < a.K) {
    a.topk_ids[(int64_t)t * a.K + lane] = id;
    a.topk_w[(int64_t)t * a.K + lane] = lane < a.KR ? wj : 1.0f;
  }
}

// ---- shared pieces of the rank kernels ----------------------------------------
struct RankLds {
  unsigned long long mask[kMaxExperts][kMaskWords];
  int cap[kMaxExperts];
  int capbase[kMaxExperts];
  int wave_sum[kBlock / 64];
  int wave_drop[kBlock / 64];
};

// mask[p] bit t: token t chose physical expert p.  clear_masks zeroes the
// masks and stages the static capacities and bases (P <= kBlock); the
// caller synchronises before the masks are filled.
__device__ __forceinline__ void clear_masks(const RouteArgs &a, RankLds &L) {
  const int tid = threadIdx.x;
  for (int i = tid; i < a.P * kMaskWords; i += kBlock) L.mask[i / kMaskWords][i % kMaskWords] = 0ull;
  if (tid < a.P) {
    L.cap[tid] = a.cap[tid];
    L.capbase[tid] = a.capbase[tid];
  }
}

// Masks from the ids written by topk_wave.  The ids (at most kIdsPerThread
// per thread) are loaded before the masks are cleared, so their latency
// overlaps that of the capacities instead of following it.
// Entry i = threadIdx.x + r * kBlock of the batch goes to id[r].
constexpr int kIdsPerThread = kFusedMaxTokens * kMaxK / kBlock;
__device__ __forceinline__ void build_masks(const RouteArgs &a, RankLds &L,
                                            int (&id)[kIdsPerThread]) {
  const int n = a.T * a.K;  // >= 1
#pragma unroll
  for (int r = 0; r < kIdsPerThread; ++r) id[r] = a.topk_ids[min((int)threadIdx.x + r * kBlock, n - 1)];
  clear_masks(a, L);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kIdsPerThread; ++r) {
    const int i = threadIdx.x + r * kBlock;
    if (i < n) {
      const int t = i / a.K;
      atomicOr(&L.mask[id[r]][t >> 6], 1ull << (t & 63));
    }
  }
  __syncthreads();
}

// Masks from ids[t][j] in LDS (the one-launch kernels).
__device__ __forceinline__ void fill_masks(const RouteArgs &a, RankLds &L,
                                           const int (*ids)[kMaxK]) {
  const int n = a.T * a.K;
  for (int i = threadIdx.x; i < n; i += kBlock) {
    const int t = i / a.K;
    atomicOr(&L.mask[ids[t][i - t * a.K]][t >> 6], 1ull << (t & 63));
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
  const int drop = tid < P ? max(0, cnt - L.cap[tid]) : 0;
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

// ---- 2a. ranks and slots of every token (moedc_route): block 0 writes the
// slots, block 1 counts, offsets and drops, side by side -------------------
__global__ __launch_bounds__(kBlock) void rank_single(RouteArgs a) {
  __shared__ RankLds L;
  int id[kIdsPerThread];
  build_masks(a, L, id);
  if (blockIdx.x == 1) {
    counts_offsets(a, L);
    return;
  }
  const int n = a.T * a.K;
#pragma unroll
  for (int r = 0; r < kIdsPerThread; ++r) {
    const int i = threadIdx.x + r * kBlock;
    if (i < n) {
      const int t = i / a.K, p = id[r];
      const int rk = rank_of(L, p, t);
      a.slots[i] = rk < L.cap[p] ? L.capbase[p] + rk : -1;
    }
  }
}

// Quantize and store one token after its slots are in slot_of[]: wave c
// holds values 512 c .. 512 c + 511 in v (called by the whole block).
// chunk_lds: 64 words of LDS for the chunks' maxima (one scale per token)
// or the groups' scales.
template <bool PER_TOKEN>
__device__ __forceinline__ void store_token(const DispatchArgs &da, const uint4 &v,
                                            const int *slot_of, uint32_t *chunk_lds) {
  const int wave = uniform(threadIdx.x >> 6), lane = lane_id();
  const int H = da.H;
  const int e = wave * 512 + lane * 8;
  uint32_t m = row16_max_u32(absmax8(v));
  if (PER_TOKEN) {
    m = max(m, (uint32_t)__shfl_xor((int)m, 16));
    m = max(m, (uint32_t)__shfl_xor((int)m, 32));
    if (lane == 0) chunk_lds[wave] = m;
    __syncthreads();
    m = 0;
#pragma unroll
    for (int w2 = 0; w2 < kBlock / 64; ++w2) m = max(m, chunk_lds[w2]);
  }
  const float s = __uint_as_float(m << 16) / 127.0f;
  const uint2 q = quant8(v, s);
  // Scale words with their zero padding, as one store of whole 128-byte
  // lines per slot: wave 0 stores the token's one scale and the zeros after
  // it; with 128-value groups the chunks' scales are gathered in LDS and
  // the last wave stores them all (instead of 16 bytes from each chunk's
  // wave: 3-7% faster from 64 tokens up).
  float word = lane == 0 ? s : 0.0f;
  bool has_word = PER_TOKEN && wave == 0 && lane < scale_words(1);
  if (!PER_TOKEN) {
    if ((lane & 15) == 0 && e < H) chunk_lds[e >> 7] = __float_as_uint(s);
    __syncthreads();
    word = lane < da.G ? __uint_as_float(chunk_lds[lane]) : 0.0f;
    has_word = wave == kBlock / 64 - 1 && lane < scale_words(da.G);
  }
  for (int k = 0; k < da.K; ++k) {
    const int slot = slot_of[k];
    if (slot < 0) continue;
    uint8_t *dst = da.dbuf + (int64_t)slot * da.slot_stride;
    if (e < H) {
      const u32x2 qq = {q.x, q.y};
      __builtin_nontemporal_store(qq, reinterpret_cast<u32x2 *>(dst + e));
    }
    if (has_word) __builtin_nontemporal_store(word, reinterpret_cast<float *>(dst + H + 4 * lane));
  }
}

// ---- 2b. ranks of token blockIdx.x, then its dispatch ------------------------
template <bool PER_TOKEN>
__global__ __launch_bounds__(kBlock) void rank_dispatch(RouteArgs ra, DispatchArgs da) {
  __shared__ RankLds L;
  __shared__ int slot_of[kMaxK];
  __shared__ uint32_t chunk_lds[64];  // store_token's exchange
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  int id[kIdsPerThread];
  if (t == ra.T) {  // the extra last block: counts, offsets, drops only
    build_masks(ra, L, id);
    counts_offsets(ra, L);
    return;
  }
  // wave c quantizes values 512 c .. 512 c + 511 of the token; its load is
  // issued first so that it overlaps the rank work.
  const int wave = uniform(tid >> 6), lane = lane_id();
  const int H = da.H;
  const int e = wave * 512 + lane * 8;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (e < H) v = reinterpret_cast<const uint4 *>(da.x + (int64_t)t * H)[wave * 64 + lane];
  const int own = ra.topk_ids[(int64_t)t * ra.K + min(tid, ra.K - 1)];  // entry tid, tid < K

  build_masks(ra, L, id);
  if (tid < ra.K) {
    const int p = own;
    const int r = rank_of(L, p, t);
    const int slot = r < L.cap[p] ? L.capbase[p] + r : -1;
    slot_of[tid] = slot;
    ra.slots[(int64_t)t * ra.K + tid] = slot;
  }
  __syncthreads();
  store_token<PER_TOKEN>(da, v, slot_of, chunk_lds);
}

// ---- 3. one launch for batches of at most kOneLaunchTokens tokens ----------
// Every block runs the top-k of the whole batch itself (16 waves, tokens w,
// w + 16, ...; after the first block the logits come from L2) instead of
// waiting for another kernel's ids: one launch and one global round trip
// fewer.  Same device code as topk_wave, so the same picks and gates; only
// the block that owns a token writes its route outputs.

// Physical ids of every token into ids[t][*]; gates and route outputs of
// token `own`, or of every token when own < 0.
template <int NV, bool SHARED>
__device__ __forceinline__ void topk_all(const RouteArgs &a, int own, int (*ids)[kMaxK]) {
  const int wave = uniform(threadIdx.x >> 6), lane = lane_id();
  for (int t = wave; t < a.T; t += kBlock / 64) {
    float v[NV], pv;
    int pe;
    topk_picks<NV>(a, t, lane, v, pv, pe);
    const int id = entry_id<SHARED>(a, t, lane, pe);
    if (lane < a.K) ids[t][lane] = id;
    if (own < 0 || t == own) {
      const float wj = topk_gate<NV>(a, lane, v, pv);
      if (lane < a.K) {
        a.topk_ids[(int64_t)t * a.K + lane] = id;
        a.topk_w[(int64_t)t * a.K + lane] = lane < a.KR ? wj : 1.0f;
      }
    }
  }
}

struct OneLds {
  RankLds L;
  int ids[kOneLaunchTokens][kMaxK];
  int slot_of[kMaxK];
  uint32_t chunk_lds[64];  // store_token's exchange
};

// moedc_route: block 0 writes every token's outputs and slots, block 1
// counts, offsets and drops.
template <int NV, bool SHARED>
__global__ __launch_bounds__(kBlock) void route_one(RouteArgs a) {
  __shared__ OneLds S;
  clear_masks(a, S.L);
  topk_all<NV, SHARED>(a, blockIdx.x == 0 ? -1 : a.T, S.ids);
  __syncthreads();
  fill_masks(a, S.L, S.ids);
  if (blockIdx.x == 1) {
    counts_offsets(a, S.L);
    return;
  }
  const int n = a.T * a.K;
  for (int i = threadIdx.x; i < n; i += kBlock) {
    const int t = i / a.K, p = S.ids[t][i - t * a.K];
    const int r = rank_of(S.L, p, t);
    a.slots[i] = r < S.L.cap[p] ? S.L.capbase[p] + r : -1;
  }
}

// moedc_route_dispatch: block t < T routes the batch, then ranks, quantizes
// and stores token t; block T writes counts, offsets and drops.
template <int NV, bool SHARED, bool PER_TOKEN>
__global__ __launch_bounds__(kBlock) void route_dispatch_one(RouteArgs ra, DispatchArgs da) {
  __shared__ OneLds S;
  const int tid = threadIdx.x, t = blockIdx.x;
  const int wave = uniform(tid >> 6), lane = lane_id();
  const int H = da.H;
  const int e = wave * 512 + lane * 8;
  uint4 v = make_uint4(0, 0, 0, 0);  // the token's load overlaps the routing
  if (t < ra.T && e < H) v = reinterpret_cast<const uint4 *>(da.x + (int64_t)t * H)[wave * 64 + lane];
  clear_masks(ra, S.L);
  topk_all<NV, SHARED>(ra, t, S.ids);
  __syncthreads();
  fill_masks(ra, S.L, S.ids);
  if (t == ra.T) {
    counts_offsets(ra, S.L);
    return;
  }
  if (tid < ra.K) {
    const int p = S.ids[t][tid];
    const int r = rank_of(S.L, p, t);
    const int slot = r < S.L.cap[p] ? S.L.capbase[p] + r : -1;
    S.slot_of[tid] = slot;
    ra.slots[(int64_t)t * ra.K + tid] = slot;
  }
  __syncthreads();
  store_token<PER_TOKEN>(da, v, S.slot_of, S.chunk_lds);
}

template <int NV>
hipError_t launch_one_nv(const RouteArgs &ra, const DispatchArgs *da, hipStream_t s) {
  if (!da) {
    if (ra.shared)
      route_one<NV, true><<<2, kBlock, 0, s>>>(ra);
    else
      route_one<NV, false><<<2, kBlock, 0, s>>>(ra);
  } else if (da->per_token) {
    if (ra.shared)
      route_dispatch_one<NV, true, true><<<ra.T + 1, kBlock, 0, s>>>(ra, *da);
    else
      route_dispatch_one<NV, false, true><<<ra.T + 1, kBlock, 0, s>>>(ra, *da);
  } else {
    if (ra.shared)
      route_dispatch_one<NV, true, false><<<ra.T + 1, kBlock, 0, s>>>(ra, *da);
    else
      route_dispatch_one<NV, false, false><<<ra.T + 1, kBlock, 0, s>>>(ra, *da);
  }
  return hipGetLastError();
}

hipError_t launch_one(const RouteArgs &a, const DispatchArgs *da, hipStream_t s) {
  if (a.KR < 1 || a.KR > kMaxK || a.E > kMaxExperts) return hipErrorInvalidValue;
  if (a.E <= 64) return launch_one_nv<1>(a, da, s);
  if (a.E <= 128) return launch_one_nv<2>(a, da, s);
  if (a.E <= 256) return launch_one_nv<4>(a, da, s);
  if (a.E <= 512) return launch_one_nv<8>(a, da, s);
  return launch_one_nv<16>(a, da, s);
}

template <int NV>
hipError_t launch_topk_nv(const RouteArgs &a, hipStream_t s) {
  const unsigned grid = (unsigned)((a.T + 3) / 4);
  if (a.shared)
    topk_wave<NV, true><<<grid, 256, 0, s>>>(a);
  else
    topk_wave<NV, false><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_topk_small(const RouteArgs &a, hipStream_t s) {
  if (a.KR < 1 || a.KR > kMaxK || a.E > kMaxExperts) return hipErrorInvalidValue;
  if (a.E <= 64) return launch_topk_nv<1>(a, s);
  if (a.E <= 128) return launch_topk_nv<2>(a, s);
  if (a.E <= 256) return launch_topk_nv<4>(a, s);
  if (a.E <= 512) return launch_topk_nv<8>(a, s);
  return launch_topk_nv<16>(a, s);
}

}  // namespace

hipError_t launch_route_small(const RouteArgs &ra, hipStream_t s) {
  if (ra.T <= 0 || ra.T > kFusedMaxTokens || ra.P > kBlock) return hipErrorInvalidValue;
  if (ra.T <= kOneLaunchTokens) return launch_one(ra, nullptr, s);
  hipError_t e = launch_topk_small(ra, s);
  if (e != hipSuccess) return e;
  rank_single<<<2, kBlock, 0, s>>>(ra);
  return hipGetLastError();
}

hipError_t launch_route_dispatch_fused(const RouteArgs &ra, const DispatchArgs &da,
                                       hipStream_t s) {
  if (ra.T <= 0 || ra.T > kFusedMaxTokens || ra.P > kBlock || da.H > 512 * (kBlock / 64))
    return hipErrorInvalidValue;
  if (ra.T <= kOneLaunchTokens) return launch_one(ra, &da, s);
  hipError_t e = launch_topk_small(ra, s);
  if (e != hipSuccess) return e;
  // One block per token plus one for counts, offsets and drops.
  if (da.per_token)
    rank_dispatch<true><<<ra.T + 1, kBlock, 0, s>>>(ra, da);
  else
    rank_dispatch<false><<<ra.T + 1, kBlock, 0, s>>>(ra, da);
  return hipGetLastError();
}

}  // namespace moedc
