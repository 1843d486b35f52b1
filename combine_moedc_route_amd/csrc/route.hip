// route.hip -- top-k routing, per-expert histogram, scans and slot
// assignment for batches of more than 256 tokens (gfx950).
//
// What is computed follows the routing metadata of "CloudMatrix384:
// Co-Designing Supernodes for Trillion-Parameter LLM Inference", sections
// "Decode Phase" (routed/shared/redundant experts) and "FusedDispatch and
// FusedCombine" (metadata that tells each sender where in the receiver's
// pre-allocated buffer a token goes).  The slot of (token t, pick j) is the
// expert's static base plus the rank of t among that expert's tokens in
// ascending token order, so the layout is deterministic without atomics.
//
// K1 route_topk (a workgroup per 64 tokens, 4 lanes per token; lane `sub`
//    holds columns 4 sub + 16 i + c, i < 16, c < 4, of each 256-column
//    chunk of the logits, loaded as 16-byte vectors):
//    - Top-k on packed keys.  A logit v of expert e becomes the 32-bit key
//      (ok(v) with its low b bits replaced by 2^b - 1 - e), ok being the
//      order-preserving integer image of the float and 2^b >= E: larger key
//      = larger value, or the same high part and a lower id.  Each lane
//      keeps its top KR + 1 keys sorted, one v_med3_u32 per list entry per
//      logit (insertion is L[j] = med3(L[j-1], L[j], c), L[0] = max(L[0],
//      c)), and the token's four lists merge through quad DPP.  Rows of
//      exactly 256 logits (one chunk) take a path with unguarded loads
//      (compute starts on the first while the rest are in flight) and 5
//      instructions of key building per logit besides the 9 of the
//      insertion; with it the scan overlaps the arrival of the logits.
//    - Exactness.  Where the high parts (the key without the id bits) of
//      the merged top KR + 1 strictly decrease, the first KR keys are the
//      top KR logits by (value desc, id asc) in that order: every other
//      logit has a smaller high part than the KR-th, hence a smaller value.
//      Two cases need more.  If the KR-th and the (KR+1)-th key share their
//      high part h, the logits with high part h (the boundary class) are
//      ranked again on their own, by a second med3 pass keyed on the low b
//      bits of ok (the part the packed key dropped) and the id -- exact,
//      since the class shares h -- and fill the positions below the picks
//      with higher high parts (one max per logit when only the last
//      position is open).  If picks share a high part, their set is right
//      and only their order needs the exact values, which are re-read for
//      the gates anyway: each lane ranks its picks by (ok desc, id asc)
//      against the token's others and writes them at that rank.
//    - Gates, replica mapping, outputs; the token's bit in a per-expert
//      64-bit mask in LDS (atomic OR, order free).  The block-local rank of
//      an entry, the popcount of the lower bits of its expert's mask, goes
//      into slots; the block's count of each expert into block_counts[p][b]
//      (expert-major, so K2 reads one contiguous row per expert).
// K2 route_scan: a wave per expert: exclusive scan of its row of block
//    counts (in place) and the expert's total, counts[p].
// K3 route_slots: a thread per entry: slot = base + block prefix +
//    block-local rank, or -1 past capacity; workgroup 0 scans counts into
//    offsets through LDS and sums the drops.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"

namespace moedc {

namespace {

constexpr int kSub = 4;           // lanes per token
constexpr int kLaneCols = 64;     // columns per lane per chunk (256 per token)
constexpr int kChunkCols = kSub * kLaneCols;
static_assert(kRouteTokens * kSub == 256, "64 tokens x 4 lanes per workgroup");

// Order-preserving integer image of a float; -0 and +0 map to one key
// (adding +0 turns -0 into +0).  Negative floats get every bit flipped, the
// others only the sign bit: an arithmetic shift makes the mask, no branch.
__device__ __forceinline__ uint32_t okey(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float okey_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// v_med3_u32, written as an instruction: the same median spelled as nested
// min/max makes LLVM's n-ary reassociation pass run for minutes on the long
// insertion chains below.
__device__ __forceinline__ uint32_t med3u(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Insert c into a descending list (the smallest entry falls off).
template <int N>
__device__ __forceinline__ void list_insert(uint32_t (&L)[N], uint32_t c) {
#pragma unroll
  for (int j = N - 1; j > 0; --j) L[j] = med3u(L[j - 1], L[j], c);
  L[0] = max(L[0], c);
}

// L := the top N of L and the list of the quad lane selected by CTRL.  The
// partner's entries arrive in descending order, so entry j can only land
// at position j or below: its insertion skips the positions above.
template <int N, int CTRL>
__device__ __forceinline__ void list_merge(uint32_t (&L)[N]) {
  uint32_t o[N];
#pragma unroll
  for (int j = 0; j < N; ++j) o[j] = dpp<CTRL>(L[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) {
#pragma unroll
    for (int i = N - 1; i > j; --i) L[i] = med3u(L[i - 1], L[i], o[j]);
    L[j] = max(L[j], o[j]);
  }
}

// quad_perm control that broadcasts quad lane q to all four lanes.
__host__ __device__ constexpr int quad_bcast(int q) { return q | (q << 2) | (q << 4) | (q << 6); }

__device__ __forceinline__ uint32_t quad_get(uint32_t v, int q) {
  switch (q) {
    case 0: return dpp<quad_bcast(0)>(v);
    case 1: return dpp<quad_bcast(1)>(v);
    case 2: return dpp<quad_bcast(2)>(v);
    default: return dpp<quad_bcast(3)>(v);
  }
}

// Lane `sub` of token t loads its 64 columns of chunk c0 (columns past E and
// tokens past T read as -inf).
__device__ __forceinline__ void load_chunk(float (&v)[kLaneCols], const RouteArgs &a, int64_t t,
                                           bool active, int c0, int sub, bool vec4) {
  const float *row = a.logits + t * a.E + c0;
  const int left = a.E - c0;
  if (vec4) {  // E % 4 == 0: 16-byte aligned rows, and left is a multiple of 4
#pragma unroll
    for (int i = 0; i < kLaneCols / 4; ++i) {
      const int c = 4 * sub + 16 * i;
      float4 x = make_float4(-__builtin_inff(), -__builtin_inff(), -__builtin_inff(),
                             -__builtin_inff());
      if (active && c < left) x = *reinterpret_cast<const float4 *>(row + c);
      v[4 * i] = x.x;
      v[4 * i + 1] = x.y;
      v[4 * i + 2] = x.z;
      v[4 * i + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kLaneCols; ++i) {
      const int c = 4 * sub + 16 * (i >> 2) + (i & 3);
      v[i] = (active && c < left) ? row[c] : -__builtin_inff();
    }
  }
}

__device__ __forceinline__ int lane_col(int c0, int sub, int i) {
  return c0 + 4 * sub + 16 * (i >> 2) + (i & 3);
}

// Group g (of 4) of a lane's chunk, columns lane_col(c0, sub, 16 g + u),
// u < 16, for the rare passes over rows of more than 256 logits (read again
// from memory, L2-resident by then).  Reading group by group in a loop that
// is not unrolled keeps those passes short without indexing a register
// array by a loop counter.
__device__ __forceinline__ void load_group(float (&w)[16], const RouteArgs &a, int64_t t, int c0,
                                           int g, int sub, bool vec4) {
  const float *row = a.logits + t * a.E + c0;
  const int left = a.E - c0;
  if (vec4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = 4 * sub + 16 * (4 * g + u);
      float4 x = make_float4(-__builtin_inff(), -__builtin_inff(), -__builtin_inff(),
                             -__builtin_inff());
      if (c < left) x = *reinterpret_cast<const float4 *>(row + c);
      w[4 * u] = x.x;
      w[4 * u + 1] = x.y;
      w[4 * u + 2] = x.z;
      w[4 * u + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int c = 4 * sub + 16 * (4 * g + (u >> 2)) + (u & 3);
      w[u] = c < left ? row[c] : -__builtin_inff();
    }
  }
}

// Boundary-class key: logits whose high part is h, ranked by the low bits
// of ok and then the id; everything else 0.
__device__ __forceinline__ uint32_t class_key(float x, int e, int E, uint32_t h, int idbits,
                                              uint32_t idmask) {
  const uint32_t k = okey(x);
  return (e < E && (k >> idbits) == h) ? (((k & idmask) << idbits) | (idmask - (uint32_t)e)) : 0u;
}

// The boundary class ranked over a lane's columns into the top NC class keys,
// merged over the token's quad.  REG: the row (E <= 256) is still in v;
// otherwise its chunks are read again from memory.
template <int NC, bool REG>
__device__ __forceinline__ void class_pass(uint32_t (&C)[NC], const float (&v)[kLaneCols],
                                           const RouteArgs &a, int64_t t, int sub, bool vec4,
                                           uint32_t h, int idbits, uint32_t idmask) {
#pragma unroll
  for (int j = 0; j < NC; ++j) C[j] = 0u;
  if (REG) {
#pragma unroll
    for (int i = 0; i < kLaneCols; ++i)
      list_insert<NC>(C, class_key(v[i], lane_col(0, sub, i), a.E, h, idbits, idmask));
  } else {
    for (int c0 = 0; c0 < a.E; c0 += kChunkCols) {
#pragma unroll 1
      for (int g = 0; g < kLaneCols / 16; ++g) {
        float w[16];
        load_group(w, a, t, c0, g, sub, vec4);
#pragma unroll
        for (int u = 0; u < 16; ++u)
          list_insert<NC>(C, class_key(w[u], lane_col(c0, sub, 16 * g + u), a.E, h, idbits,
                                       idmask));
      }
    }
  }
  list_merge<NC, kDppQuadXor1>(C);
  list_merge<NC, kDppQuadXor2>(C);
}

template <int KR, bool SHARED>
__global__ __launch_bounds__(256) void route_topk(RouteArgs a, int idbits, int nblk) {
  constexpr int KT = KR + (SHARED ? 1 : 0);
  constexpr int N = KR + 1;                   // one key past the picks, for the exactness test
  constexpr int NP = (KT + kSub - 1) / kSub;  // picks per lane
  __shared__ unsigned long long tokmask[kMaxExperts];
  __shared__ float sorted_s[kRouteTokens][KR];  // sigmoid numerators in pick order (ties only)

  const int tid = threadIdx.x;
  const int r = tid >> 2, sub = tid & 3;
  const int E = a.E, P = a.P;
  const int blk = blockIdx.x;
  for (int i = tid; i < P; i += 256) tokmask[i] = 0ull;

  const int64_t t = (int64_t)blk * kRouteTokens + r;
  const bool active = t < a.T;
  const bool vec4 = (E & 3) == 0;
  const uint32_t idmask = (1u << idbits) - 1u;

  // ---- packed-key top-(KR+1) per lane, merged over the token's quad -------
  uint32_t L[N];
#pragma unroll
  for (int j = 0; j < N; ++j) L[j] = 0u;  // below every real key
  float v[kLaneCols];
  const bool full = E == kChunkCols;  // one chunk, every column in range
  if (full) {
    // Unguarded 16-byte loads (a padding token past T reads row T - 1 and is
    // never written out), so the keys can start on the first loads while the
    // rest are in flight.  A key is built as (ok | idmask) - (column within
    // the lane's stripe); the lane's own offset 4 sub comes off the merged-in
    // entries at the end, all of them real keys by then (N <= 64 inserted),
    // which leaves each entry's low bits at idmask - e.
    const int64_t tl = active ? t : (int64_t)a.T - 1;
    const float4 *row = reinterpret_cast<const float4 *>(a.logits + tl * kChunkCols) + sub;
#pragma unroll
    for (int i = 0; i < kLaneCols / 4; ++i) {
      const float4 x = row[4 * i];
      v[4 * i] = x.x;
      v[4 * i + 1] = x.y;
      v[4 * i + 2] = x.z;
      v[4 * i + 3] = x.w;
    }
#pragma unroll
    for (int i = 0; i < kLaneCols; ++i)
      list_insert<N>(L, (okey(v[i]) | idmask) - (uint32_t)lane_col(0, 0, i));
    const uint32_t off = 4u * (uint32_t)sub;
#pragma unroll
    for (int j = 0; j < N; ++j) L[j] -= off;
  } else {
    for (int c0 = 0; c0 < E; c0 += kChunkCols) {
      load_chunk(v, a, t, active, c0, sub, vec4);
#pragma unroll
      for (int i = 0; i < kLaneCols; ++i) {
        const int e = lane_col(c0, sub, i);
        const uint32_t key = (okey(v[i]) & ~idmask) | (idmask - (uint32_t)e);
        list_insert<N>(L, e < E ? key : 0u);
      }
    }
  }
  list_merge<N, kDppQuadXor1>(L);
  list_merge<N, kDppQuadXor2>(L);

  int id[KR];
#pragma unroll
  for (int j = 0; j < KR; ++j) id[j] = (int)(idmask - (L[j] & idmask));
  bool inner = false;
#pragma unroll
  for (int j = 0; j + 1 < KR; ++j) inner |= (L[j] >> idbits) == (L[j + 1] >> idbits);
  const uint32_t hmin = L[KR - 1] >> idbits;
  const bool bnd = active && hmin == (L[KR] >> idbits);
  inner = inner && active;

  // ---- boundary class: rank the logits of high part hmin by their low bits
  // (whole quads take this together: the merged list is the quad's).  The
  // picks with a higher high part keep their places; the class fills the
  // KR - above positions below them, most often just the last one, for
  // which one max per logit does.
  int above = 0;
#pragma unroll
  for (int j = 0; j < KR; ++j) above += (L[j] >> idbits) > hmin;
  if (__builtin_amdgcn_ballot_w64(bnd)) {
    const bool one = !__builtin_amdgcn_ballot_w64(bnd && above + 1 < KR);
    if (bnd && one) {
      uint32_t C[1];
      if (E <= kChunkCols)
        class_pass<1, true>(C, v, a, t, sub, vec4, hmin, idbits, idmask);
      else
        class_pass<1, false>(C, v, a, t, sub, vec4, hmin, idbits, idmask);
      if (C[0] != 0u) id[KR - 1] = (int)(idmask - (C[0] & idmask));
    } else if (bnd) {
      uint32_t C[KR];
      if (E <= kChunkCols)
        class_pass<KR, true>(C, v, a, t, sub, vec4, hmin, idbits, idmask);
      else
        class_pass<KR, false>(C, v, a, t, sub, vec4, hmin, idbits, idmask);
#pragma unroll
      for (int j = 0; j < KR; ++j) {
        // position j takes class entry j - above (compile-time j, runtime above)
        uint32_t c = 0u;
#pragma unroll
        for (int q = 0; q <= j; ++q) c = (j - q == above) ? C[q] : c;
        // The class holds at least KR - above + 1 logits (positions above..KR
        // of the merged list), so c is a real key; the test keeps ids in range
        // regardless.
        if (j >= above && c != 0u) id[j] = (int)(idmask - (c & idmask));
      }
    }
  }

  // ---- exact logits of this lane's picks (j = sub + 4 i) ---------------------
  int pid[NP];
  float pv[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int j = sub + kSub * i;
    int e = 0;
#pragma unroll
    for (int q = 0; q < kSub; ++q)
      if (kSub * i + q < KR) e = (sub == q) ? id[kSub * i + q] : e;
    pid[i] = e;
    pv[i] = (active && j < KR) ? a.logits[t * E + e] : 0.0f;
  }
  // Picks that share a high part (or came from the boundary class): their set
  // is right, their order is by (value desc, id asc) on the exact values.
  // Each lane ranks its own picks against the quad's KR picks and writes them
  // at that rank; without such ties the rank of pick j is j.
  int prank[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) prank[i] = sub + kSub * i;
  const bool ties = __builtin_amdgcn_ballot_w64(inner || bnd) != 0;  // wave-uniform
  float m = __uint_as_float(dpp<quad_bcast(0)>(__float_as_uint(pv[0])));  // pick 0: the max
  if (ties) {
    uint32_t xk[KR];
    int xe[KR];
#pragma unroll
    for (int q = 0; q < KR; ++q) {
      xk[q] = quad_get(okey(pv[q / kSub]), q % kSub);
      xe[q] = (int)quad_get((uint32_t)pid[q / kSub], q % kSub);
    }
    uint32_t top = xk[0];
#pragma unroll
    for (int q = 1; q < KR; ++q) top = max(top, xk[q]);
    m = okey_float(top);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const uint32_t k = okey(pv[i]);
      int r = 0;
#pragma unroll
      for (int q = 0; q < KR; ++q) r += (xk[q] > k || (xk[q] == k && xe[q] < pid[i])) ? 1 : 0;
      if (sub + kSub * i < KR) prank[i] = r;
    }
  }

  // ---- gates, physical ids, outputs, token masks ------------------------------
  float w[NP];
  if (a.score_fn == MOEDC_SCORE_SOFTMAX) {
    // Z = sum over all logits of exp(l - max), per lane in column order,
    // then lanes 0..3 in order.
    float z = 0.0f;
    if (active) {
      if (E <= kChunkCols) {
#pragma unroll
        for (int i = 0; i < kLaneCols; ++i)
          if (lane_col(0, sub, i) < E) z += expf(v[i] - m);
      } else {
        for (int c0 = 0; c0 < E; c0 += kChunkCols) {
#pragma unroll 1
          for (int g = 0; g < kLaneCols / 16; ++g) {
            float x[16];
            load_group(x, a, t, c0, g, sub, vec4);
#pragma unroll
            for (int u = 0; u < 16; ++u)
              if (lane_col(c0, sub, 16 * g + u) < E) z += expf(x[u] - m);
          }
        }
      }
    }
    const float Z = ((__uint_as_float(quad_get(__float_as_uint(z), 0)) +
                      __uint_as_float(quad_get(__float_as_uint(z), 1))) +
                     __uint_as_float(quad_get(__float_as_uint(z), 2))) +
                    __uint_as_float(quad_get(__float_as_uint(z), 3));
#pragma unroll
    for (int i = 0; i < NP; ++i) w[i] = expf(pv[i] - m) / Z;
  } else {
    // Sigmoid of each pick, normalised by their sum taken in pick order.
    float s[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) s[i] = 1.0f / (1.0f + expf(-pv[i]));
    float S = 0.0f;
    if (ties) {
      // in rank order: through the token's row of sorted_s (one wave's own
      // lanes write and then read it)
#pragma unroll
      for (int i = 0; i < NP; ++i)
        if (sub + kSub * i < KR) sorted_s[r][prank[i]] = s[i];
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = 0; q < KR; ++q) S += sorted_s[r][q];
    } else {
#pragma unroll
      for (int j = 0; j < KR; ++j)
        S += __uint_as_float(quad_get(__float_as_uint(s[j / kSub]), j % kSub));
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) w[i] = s[i] / S;
  }
  int pk[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int j = sub + kSub * i;
    const int e = pid[i];
    pk[i] = -1;
    // (tokens past T hold padding ids: no table lookup for them)
    if (active && j < KR)
      pk[i] = a.rep_identity ? e : a.rep_table[e * a.R + (int)(t % a.rep_count[e])];
    if (SHARED && j == KT - 1) {
      pk[i] = P - 1;
      w[i] = 1.0f;
    }
    if (active && j < KT) {
      a.topk_ids[t * KT + prank[i]] = pk[i];
      a.topk_w[t * KT + prank[i]] = w[i];
      atomicOr(&tokmask[pk[i]], 1ull << r);
    }
  }
  __syncthreads();

  // ---- block-local ranks (finished by route_slots) and block counts ----------
  const uint64_t below = r == 0 ? 0ull : (~0ull >> (64 - r));
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int j = sub + kSub * i;
    if (active && j < KT) a.slots[t * KT + prank[i]] = __popcll(tokmask[pk[i]] & below);
  }
  for (int p = tid; p < P; p += 256)
    a.block_counts[(int64_t)p * nblk + blk] = __popcll(tokmask[p]);
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

// One wave per physical expert: its row of block counts -> exclusive block
// prefixes (in place) and the expert's total.  Lane l takes 8 consecutive
// blocks (two 16-byte loads when the row allows), sums them serially, and
// one wave scan of the lane totals gives every block's prefix.
__global__ __launch_bounds__(256) void route_scan(int32_t *bc, int32_t *counts, int nblk, int P) {
  const int p = blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (p >= P) return;
  const int l = lane_id();
  int32_t *row = bc + (int64_t)p * nblk;
  const bool vec = (nblk & 3) == 0;  // rows 16-byte aligned (the workspace base is)
  int carry = 0;
  for (int b0 = 0; b0 < nblk; b0 += 512) {
    const int b = b0 + 8 * l;
    int v[8];
    if (vec && b + 8 <= nblk) {
      const int4 x = *reinterpret_cast<const int4 *>(row + b);
      const int4 y = *reinterpret_cast<const int4 *>(row + b + 4);
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
      v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = b + u < nblk ? row[b + u] : 0;
    }
    int sum = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += v[u];
    const int incl = wave_inclusive_scan(sum);
    int run = carry + incl - sum;  // blocks before b
    int e[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      e[u] = run;
      run += v[u];
    }
    if (vec && b + 8 <= nblk) {
      *reinterpret_cast<int4 *>(row + b) = make_int4(e[0], e[1], e[2], e[3]);
      *reinterpret_cast<int4 *>(row + b + 4) = make_int4(e[4], e[5], e[6], e[7]);
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (b + u < nblk) row[b + u] = e[u];
    }
    carry += __shfl(incl, 63);
  }
  if (l == 0) counts[p] = carry;
}

// Entries -> slots; workgroup 0 also scans counts into offsets and counts
// the drops (LDS-staged block scan).  It is dispatched first, so that
// small serial job runs beside the entries instead of after them.
__global__ __launch_bounds__(256) void route_slots(RouteArgs a, int64_t entries, int nblk) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {
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
  const int64_t i = (int64_t)(blockIdx.x - 1) * 256 + tid;
  if (i >= entries) return;
  const int64_t t = i / a.K;
  const int p = a.topk_ids[i];
  const int j = a.block_counts[(int64_t)p * nblk + t / kRouteTokens] + a.slots[i];
  a.slots[i] = j < a.cap[p] ? a.capbase[p] + j : -1;
}

template <int KR>
hipError_t launch_topk(const RouteArgs &a, int nblk, int idbits, hipStream_t s) {
  if (a.shared)
    route_topk<KR, true><<<nblk, 256, 0, s>>>(a, idbits, nblk);
  else
    route_topk<KR, false><<<nblk, 256, 0, s>>>(a, idbits, nblk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t s) {
  const int nblk = (a.T + kRouteTokens - 1) / kRouteTokens;
  hipError_t e = hipSuccess;
  if (nblk > 0) {
    int idbits = 0;
    while ((1 << idbits) < a.E) ++idbits;
    switch (a.KR) {
#define MOEDC_CASE(k)                       \
  case k:                                   \
    e = launch_topk<k>(a, nblk, idbits, s); \
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
  // counts: zero when no workgroup ran.
  route_scan<<<(a.P + 3) / 4, 256, 0, s>>>(a.block_counts, a.counts, nblk, a.P);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t entries = (int64_t)a.T * a.K;
  const int64_t grid = (entries + 255) / 256 + 1;
  route_slots<<<(unsigned)grid, 256, 0, s>>>(a, entries, nblk);
  return hipGetLastError();
}

}  // namespace moedc
