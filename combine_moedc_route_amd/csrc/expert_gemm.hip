// expert_gemm.hip -- one W8A8 linear layer per physical expert (hidden ->
// hidden) over the occupied dispatch slots, on int8 MFMA (gfx950).
//
// This is the expert compute that sits between dispatch and combine: the
// CloudMatrix384 article, section "INT8 Quantization", runs the large
// matmuls in INT8 with per-token dynamic activation scales and per-channel
// static weight scales.  The kernel reads the dispatch buffer in place
// (INT8 payload + fp32 scales per slot) and writes BF16 rows of the combine
// buffer, so route -> dispatch -> expert -> combine runs end to end.
//
// For slot row t of expert p and output channel n:
//   isum_g = sum_{k in group g} q[t][k] * W[p][n][k]     exact in int32
//   acc = +0;  acc = fmaf(s_x[t][g], (float)isum_g, acc) for g ascending
//   y[t][n] = bf16(acc * w_scale[p][n])
// (a group is 128 inputs, or the whole row with one scale per token).
//
// Work list: the route's counts give each expert ceil(rows / tile rows) row
// tiles and ceil(H/256) channel tiles.  A band is kBandTiles channel tiles x all
// row tiles of one expert (32 tiles for 8 row tiles), ordered row-major so
// that neighbouring entries share a weight slice or a slot tile.  Bands are
// dealt to the 8 XCDs by an LPT list schedule on their tile counts (or
// round-robin, for comparison) on the device, from the route's counts;
// workgroup b runs on XCD b mod 8 (the hardware's round-robin placement),
// and the 32 workgroups resident on one XCD walk that XCD's band stream
// together.  The tiles of a band then run
// concurrently on one die, so each 256-channel weight slice and each slot
// tile crosses from memory into that die's L2 about once per band instead
// of once per tile.  The placement is only a performance assumption: any
// placement computes the same result.
//
// Per tile, 8 waves (2 token halves x 4 channel quarters); MFMA
// v_mfma_i32_16x16x64_i8 with A = 16 weight rows (channels) and B = 16 slot
// rows (tokens), so each lane ends up with 4 consecutive channels of one
// token (8-byte BF16 stores).  K advances 128 inputs per step; slot rows and
// weight rows are shared by 4 and 2 waves respectively and pass through a
// double-buffered LDS tile, loaded one step ahead into registers.  With
// 128-input groups a tile is 128 slot rows x 256 channels (waves of 64 x
// 64), moves 48 KiB per step for 8.4 MOP (175 op/B), and all eight waves
// meet at one barrier per step.  With one scale per token the int32 sums
// span the whole row and are scaled once in the epilogue, so the registers
// that would hold fp32 partial sums hold a second 64 tokens instead: 256 x
// 256 tiles (waves of 128 tokens x 64 channels), 64 KiB per step for 16.8
// MOP (262 op/B), a quarter fewer LDS reads per MFMA and half the tiles;
// there the two halves of the workgroup take turns between MFMAs and
// staging (see expert_gemm_pt).
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"

namespace moedc {

namespace {

constexpr int BM = 128;   // slot rows (tokens) per tile with 128-input groups
constexpr int BM_PT = 256;  // with one scale per token
constexpr int BN = kGemmChannels;  // output channels per tile
constexpr int BK = 128;   // inputs per K step

// LDS tiles are unpadded rows of BK bytes; the 16-byte chunk c of row r is
// stored at chunk c ^ (r & 7).  The 16-byte fragment reads (16 rows, one
// chunk) and the staging writes (8 chunks of one row) then hit distinct
// banks, and the tiles need no padding.
__device__ __forceinline__ int swz(int r, int chunk) { return 16 * (chunk ^ (r & 7)); }
constexpr int kThreads = 512;   // 8 waves: 2 token halves x 4 channel quarters
constexpr int kDppRowHalfMirror = 0x141;  // row_half_mirror: lane i <-> 7 - i within 8

typedef int v4i __attribute__((ext_vector_type(4)));

// counts -> each XCD's band list and tile prefix.  A band k (expert k / nbe,
// channel tiles kBandTiles (k mod nbe) on) costs its tile count.
//  - LPT (the longest-processing-time list schedule of "StrataCL 深度技术分析",
//    section 3.5, with the 8 XCDs as the workers): bands with tiles, in
//    order of cost descending (equal costs by index), each to the XCD with
//    the fewest tiles so far (ties to the lower XCD).  Its largest XCD load
//    is within 4/3 - 1/24 of the best possible.
//  - Round-robin: band k to XCD k mod 8, in index order.
// band_list[x][j] is XCD x's j-th band, band_pre[x][j] the tiles of its
// bands before j, band_pre[x][band_cnt[x]] its total.  One workgroup; the
// LPT pass sorts 32-bit keys (cost << 13 | 8191 - k, cost saturated at
// 2^19 - 1) in LDS, then one wave places the bands in order.
__device__ __forceinline__ int band_cost(const GemmArgs &a, int k) {
  const int p = k / a.nbe, b = k - p * a.nbe;
  const int rows = min(a.counts[p], a.cap[p]);
  return (rows + a.bm - 1) / a.bm * min(kBandTiles, a.ntiles - b * kBandTiles);
}

__global__ __launch_bounds__(1024) void gemm_tiles(GemmArgs a) {
  __shared__ uint32_t keys[kMaxBands];
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  const int nb = a.P * a.nbe;
  const int Jm = a.Jmax;
  if (a.dealing == MOEDC_DEAL_ROUND_ROBIN) {
    for (int x = 0; x < kXcds; ++x) {
      const int J = nb > x ? (nb - x + kXcds - 1) / kXcds : 0;
      int32_t *pre = a.band_pre + x * (Jm + 1);
      int carry = 0;
      for (int j0 = 0; j0 < J; j0 += 1024) {
        const int j = j0 + tid;
        const int k = x + kXcds * j;
        const int tiles = j < J ? band_cost(a, k) : 0;
        if (j < J) a.band_list[x * Jm + j] = k;
        int incl = tiles;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int u = __shfl_up(incl, d);
          if ((tid & 63) >= d) incl += u;
        }
        if ((tid & 63) == 63) wsum[tid >> 6] = incl;
        __syncthreads();
        int base = carry;
        for (int w = 0; w < (tid >> 6); ++w) base += wsum[w];
        if (j < J) pre[j] = base + incl - tiles;
        int tot = 0;
        for (int w = 0; w < 16; ++w) tot += wsum[w];
        carry += tot;
        __syncthreads();  // wsum is reused
      }
      if (tid == 0) {
        pre[J] = carry;
        a.band_cnt[x] = J;
        if (a.xcd_tiles) a.xcd_tiles[x] = carry;
      }
    }
    return;
  }
  // ---- LPT ----
  int n2 = 1;
  while (n2 < nb) n2 <<= 1;
  for (int i = tid; i < n2; i += 1024) {
    uint32_t key = 0u;
    if (i < nb) key = ((uint32_t)min(band_cost(a, i), (1 << 19) - 1) << 13) | (uint32_t)(8191 - i);
    keys[i] = key;
  }
  __syncthreads();
  // bitonic sort, descending
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (n2 >> 1); i += 1024) {
        const int lo = 2 * stride * (i / stride) + (i % stride), hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint32_t x = keys[lo], y = keys[hi];
        if ((x < y) == desc) {
          keys[lo] = y;
          keys[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  if (tid >= 64) return;
  // One wave places the bands in that order.  Lane x < 8 holds XCD x's
  // tiles and bands so far; the least-loaded XCD (ties to the lower one) is
  // the minimum of (tiles << 3 | x) over lanes 0-7, three DPP steps.  Lane i
  // remembers where band i of the current 64 went, and the 64 placements
  // are stored together after the chunk.
  const int lane = tid;
  int load_l = 0, cnt_l = 0;
  bool more = true;
  for (int base = 0; base < nb && more; base += 64) {
    // 64 bands at a time: each lane fetches one band's exact cost (the key
    // holds a saturated one), then the wave places them one by one.
    const uint32_t mine = base + lane < nb ? keys[base + lane] : 0u;
    const int mine_k = 8191 - (int)(mine & 8191u);
    const int mine_cost = (mine >> 13) ? band_cost(a, mine_k) : 0;
    const int n = min(64, nb - base);
    int my_x = -1, my_j = 0, my_pre = 0;
    for (int i = 0; i < n; ++i) {
      const int cost = __builtin_amdgcn_readlane(mine_cost, i);
      if (cost == 0) {  // the rest have no tiles
        more = false;
        break;
      }
      uint32_t key = lane < kXcds ? ((uint32_t)load_l << 3) | (uint32_t)lane : 0xFFFFFFFFu;
      key = min(key, dpp<kDppQuadXor1>(key));
      key = min(key, dpp<kDppQuadXor2>(key));
      key = min(key, dpp<kDppRowHalfMirror>(key));  // lanes 0-3 with 4-7
      const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)key);
      const int bx = (int)(m & 7u);
      const int j = __builtin_amdgcn_readlane(cnt_l, bx);
      if (lane == i) {
        my_x = bx;
        my_j = j;
        my_pre = (int)(m >> 3);
      }
      if (lane == bx) {
        load_l += cost;
        cnt_l += 1;
      }
    }
    if (my_x >= 0) {
      a.band_list[my_x * Jm + my_j] = mine_k;
      a.band_pre[my_x * (Jm + 1) + my_j] = my_pre;
    }
  }
  if (lane < kXcds) {
    a.band_pre[lane * (Jm + 1) + cnt_l] = load_l;
    a.band_cnt[lane] = cnt_l;
    if (a.xcd_tiles) a.xcd_tiles[lane] = load_l;
  }
}

__device__ __forceinline__ v4i ld16(const void *p) { return *reinterpret_cast<const v4i *>(p); }

// ======== 128-input scale groups: 128 x 256 tiles, one barrier per step ========

// One K step of the tile, as loaded by one thread: 2 x 16 B of slot rows
// (rows r, r+64), 4 x 16 B of weight rows (r, r+64, r+128, r+192) and the
// step's activation scale of slot row `tid` (threads below 128).  Rows past
// the expert's tokens or past H channels read as zero.
struct StepRegs {
  v4i x[2], w[4];
  float s;
};

__device__ __forceinline__ StepRegs fetch_step(const GemmArgs &a, const int8_t *wtile,
                                               int64_t slot0, int rows, int chans, int g,
                                               int tid) {
  const int r = tid >> 3, c = 16 * (tid & 7);
  StepRegs st;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = r + 64 * i;
    st.x[i] = t < rows ? ld16(a.dbuf + (slot0 + t) * a.slot_stride + g * BK + c)
                       : v4i{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = r + 64 * i;
    st.w[i] = n < chans ? ld16(wtile + (int64_t)n * a.H + g * BK + c) : v4i{0, 0, 0, 0};
  }
  st.s = 0.0f;
  if (tid < BM && tid < rows)
    st.s = *reinterpret_cast<const float *>(a.dbuf + (slot0 + tid) * a.slot_stride + a.H + 4 * g);
  return st;
}

// Scales are double-buffered by step parity: step g's scales are written
// with its slot rows and read after its MFMAs (or, by the lagging waves,
// after the next barrier), while step g+1's go to the other buffer.
__device__ __forceinline__ void stage(int8_t (&Xs)[BM][BK], int8_t (&Ws)[BN][BK],
                                      float (&sx)[2][BM], const StepRegs &st, int g, int tid) {
  const int r = tid >> 3, c = tid & 7;  // rows r + 64 i keep r's low 3 bits
#pragma unroll
  for (int i = 0; i < 2; ++i) *reinterpret_cast<v4i *>(&Xs[r + 64 * i][swz(r, c)]) = st.x[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<v4i *>(&Ws[r + 64 * i][swz(r, c)]) = st.w[i];
  if (tid < BM) sx[g & 1][tid] = st.s;
}

// Every K step is one 128-input scale group: the first MFMA of a step
// starts from a zero accumulator and the group's int32 sums are folded into
// fp32 at the end of the step.
__global__ __launch_bounds__(kThreads) void expert_gemm_groups(GemmArgs a) {
  constexpr int TF = BM / 32;  // 16-token blocks per wave (4)
  __shared__ __attribute__((aligned(16))) int8_t Xs[2][BM][BK];
  __shared__ __attribute__((aligned(16))) int8_t Ws[2][BN][BK];
  __shared__ float sx[2][BM];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = uniform(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // token half, channel quarter
  const int H = a.H;
  const int ksteps = H / BK;
  const int xcd = blockIdx.x % kXcds;
  const int nblk = gridDim.x / kXcds;  // workgroups sharing this XCD's stream
  const int32_t *row = a.band_pre + xcd * (a.Jmax + 1);
  const int J = uniform(a.band_cnt[xcd]);
  const int total = uniform(row[J]);

  for (int q = blockIdx.x / kXcds; q < total; q += nblk) {
    // ---- locate the tile: band j of this XCD holds row[j] .. row[j+1) ----
    int lo = 0, hi = J;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (row[mid] <= q) lo = mid; else hi = mid;
    }
    const int k = uniform(a.band_list[xcd * a.Jmax + lo]);
    const int p = k / a.nbe, band = k % a.nbe;
    const int off = q - row[lo];
    const int w = min(kBandTiles, a.ntiles - band * kBandTiles);
    const int mt = off / w, nt = band * kBandTiles + off % w;
    const int used = min(a.counts[p], a.cap[p]);
    const int rows = min(BM, used - mt * BM);
    const int chans = min(BN, H - nt * BN);
    const int64_t slot0 = (int64_t)a.capbase[p] + (int64_t)mt * BM;
    const int8_t *wtile = a.W + ((int64_t)p * H + (int64_t)nt * BN) * H;

    v4i acc[4][TF];
    float accf[4][TF][4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf)
#pragma unroll
      for (int tf = 0; tf < TF; ++tf) {
        acc[nf][tf] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) accf[nf][tf][q2] = 0.0f;
      }

    __syncthreads();  // the previous tile's last reads of the LDS tiles are done
    stage(Xs[0], Ws[0], sx, fetch_step(a, wtile, slot0, rows, chans, 0, tid), 0, tid);
    StepRegs nxt = fetch_step(a, wtile, slot0, rows, chans, min(1, ksteps - 1), tid);

    // Waves 4-7 (the second wave on each SIMD) fold a step's group sums
    // after the next barrier, while waves 0-3 run that step's MFMAs, and run
    // their own MFMAs while waves 0-3 fold: the matrix and vector units of a
    // SIMD stay busy together instead of taking turns.
    const bool lag = wave >= 4;
    for (int g = 0; g < ksteps; ++g) {
      const int buf = g & 1;
      float sv[4];
      if (lag && g > 0) {
#pragma unroll
        for (int tf = 0; tf < 4; ++tf) sv[tf] = sx[(g - 1) & 1][64 * wm + 16 * tf + (lane & 15)];
      }
      __syncthreads();  // step g staged by all; step g-1's reads of buf^1 done
      if (lag && g > 0) {
#pragma unroll
        for (int tf = 0; tf < 4; ++tf)
#pragma unroll
          for (int nf = 0; nf < 4; ++nf)
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2)
              accf[nf][tf][q2] = __builtin_fmaf(sv[tf], (float)acc[nf][tf][q2], accf[nf][tf][q2]);
      }
      // Stage step g+1 into the other buffer (free since this barrier) and
      // issue step g+2's loads before this step's MFMAs, which gives the
      // loads a whole step of lead (1.5% faster than after them).
      if (g + 1 < ksteps) stage(Xs[buf ^ 1], Ws[buf ^ 1], sx, nxt, g + 1, tid);
      if (g + 2 < ksteps) nxt = fetch_step(a, wtile, slot0, rows, chans, g + 2, tid);
      // Raised wave priority while a wave issues its MFMAs, so the SIMD's
      // other wave (staging, loads, folds) does not delay them.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        v4i av[4], bv[4];
#pragma unroll
        for (int nf = 0; nf < 4; ++nf)
          av[nf] = *reinterpret_cast<const v4i *>(
              &Ws[buf][64 * wn + 16 * nf + (lane & 15)][swz(lane, 4 * kk + (lane >> 4))]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          bv[i] = *reinterpret_cast<const v4i *>(
              &Xs[buf][16 * TF * wm + 16 * i + (lane & 15)][swz(lane, 4 * kk + (lane >> 4))]);
#pragma unroll
        for (int nf = 0; nf < 4; ++nf)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[nf][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                av[nf], bv[i], kk == 0 ? v4i{0, 0, 0, 0} : acc[nf][i], 0, 0, 0);
      }
      __builtin_amdgcn_s_setprio(0);
      if (!lag) {  // end of the step's scale group
#pragma unroll
        for (int tf = 0; tf < 4; ++tf) {
          const float sc = sx[g & 1][64 * wm + 16 * tf + (lane & 15)];
#pragma unroll
          for (int nf = 0; nf < 4; ++nf)
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2)
              accf[nf][tf][q2] = __builtin_fmaf(sc, (float)acc[nf][tf][q2], accf[nf][tf][q2]);
        }
      }
    }
    if (lag) {  // the last step's fold (its scales are not restaged before the next tile)
#pragma unroll
      for (int tf = 0; tf < 4; ++tf) {
        const float sc = sx[(ksteps - 1) & 1][64 * wm + 16 * tf + (lane & 15)];
#pragma unroll
        for (int nf = 0; nf < 4; ++nf)
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2)
            accf[nf][tf][q2] = __builtin_fmaf(sc, (float)acc[nf][tf][q2], accf[nf][tf][q2]);
      }
    }

    // ---- epilogue: lane holds channels n0..n0+3 of token 64 wm + 16 tf + lane%16 ----
    // Token rows one after another: the four 32-byte stores that make up a
    // row's 128-byte line issue back to back and the line reaches memory
    // whole (channel-major order left lines partly written in L2: up to
    // 1.85x the output bytes written).  Weight scales load at each store
    // (loaded once per tile they cost two more spilled registers, +3.5%).
#pragma unroll
    for (int tf = 0; tf < TF; ++tf) {
      const int t = 16 * TF * wm + 16 * tf + (lane & 15);
      if (t >= rows) continue;
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        const int nl = 64 * wn + 16 * nf + 4 * (lane >> 4);
        if (nl >= chans) continue;
        const int64_t n0 = (int64_t)nt * BN + nl;
        const float4 w4 = *reinterpret_cast<const float4 *>(a.w_scale + (int64_t)p * H + n0);
        const uint2 o = make_uint2(pack_bf16x2(accf[nf][tf][0] * w4.x, accf[nf][tf][1] * w4.y),
                                   pack_bf16x2(accf[nf][tf][2] * w4.z, accf[nf][tf][3] * w4.w));
        *reinterpret_cast<uint2 *>(a.ebuf + (slot0 + t) * (int64_t)H + n0) = o;
      }
    }
  }
}

// ======== one scale per token: 256 x 256 tiles, two wave groups in turn ========
//
// Waves 0-3 (group A: output channels 0-127) and 4-7 (group B: channels
// 128-255) alternate between a compute phase (a step's 64 MFMAs per wave,
// from LDS fragments) and a memory phase (staging the group's half of a
// later step into LDS and issuing the global loads of the one after), with
// a workgroup barrier between phases; group B starts one phase late, so on
// every SIMD one wave issues MFMAs while the other stages.  Group A stages
// slot rows 0-127 and weight rows 0-127, group B rows 128-255 of both.  A
// computes on step g, then stages step g + 1; B computes on step g, then
// stages step g + 2: every step is complete one phase before either group
// computes on it, and two LDS buffers suffice (a buffer is rewritten only
// after both groups have computed on the step it held).  Against one
// barrier per step with all eight waves in the same phase (the 128-input
// kernel's scheme): 12.1-12.4 ms against 13.3-13.6 ms on the 30720-token
// batch, bit-identical.

// Slot rows 128 grp + r + 32 i and weight rows likewise (r = gt / 8, the
// thread's index in its group over 8), 16-byte column gt % 8 of the step's
// 128 inputs; the loads address a uniform base plus a 32-bit lane offset.
struct PartRegs {
  v4i x[4], w[4];
  float s;
};

__device__ __forceinline__ PartRegs fetch_part(const int8_t *xb, const int8_t *wb, uint32_t xo,
                                               uint32_t wo, uint32_t xstep, uint32_t wstep,
                                               int rows, int chans, int g, int grp, int gt,
                                               const int8_t *sb) {
  const int r = gt >> 3;
  PartRegs st;
  const int8_t *xg = xb + g * BK;
  const int8_t *wg = wb + g * BK;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 128 * grp + r + 32 * i;
    st.x[i] = t < rows ? ld16(xg + (xo + i * xstep)) : v4i{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = 128 * grp + r + 32 * i;
    st.w[i] = n < chans ? ld16(wg + (wo + i * wstep)) : v4i{0, 0, 0, 0};
  }
  // The token's scale, with the first step (slot rows 128 grp + gt, gt < 128).
  st.s = 0.0f;
  if (g == 0 && gt < 128 && 128 * grp + gt < rows) st.s = *reinterpret_cast<const float *>(sb);
  return st;
}

__device__ __forceinline__ void stage_part(int8_t (&Xs)[BM_PT][BK], int8_t (&Ws)[BN][BK],
                                           float (&sx)[BM_PT], const PartRegs &st, int g,
                                           int grp, int gt) {
  const int r = gt >> 3, c = gt & 7;  // rows 128 grp + r + 32 i keep r's low 3 bits
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<v4i *>(&Xs[128 * grp + r + 32 * i][swz(r, c)]) = st.x[i];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<v4i *>(&Ws[128 * grp + r + 32 * i][swz(r, c)]) = st.w[i];
  if (g == 0 && gt < 128) sx[128 * grp + gt] = st.s;
}

__global__ __launch_bounds__(kThreads) void expert_gemm_pt(GemmArgs a) {
  constexpr int TF = BM_PT / 32;  // 16-token blocks per wave (8)
  __shared__ __attribute__((aligned(16))) int8_t Xs[2][BM_PT][BK];
  __shared__ __attribute__((aligned(16))) int8_t Ws[2][BN][BK];
  __shared__ float sx[BM_PT];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = uniform(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // token half, channel quarter
  const int grp = wave >> 2;                // 0: channels 0-127, 1: channels 128-255
  const int gt = tid & 255;                 // thread index within the group
  const int H = a.H;
  const int ksteps = H / BK;
  const int xcd = blockIdx.x % kXcds;
  const int nblk = gridDim.x / kXcds;
  const int32_t *row = a.band_pre + xcd * (a.Jmax + 1);
  const int J = uniform(a.band_cnt[xcd]);
  const int total = uniform(row[J]);

  for (int q = blockIdx.x / kXcds; q < total; q += nblk) {
    int lo = 0, hi = J;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (row[mid] <= q) lo = mid; else hi = mid;
    }
    const int k = uniform(a.band_list[xcd * a.Jmax + lo]);
    const int p = k / a.nbe, band = k % a.nbe;
    const int off = q - row[lo];
    const int w = min(kBandTiles, a.ntiles - band * kBandTiles);
    const int mt = off / w, nt = band * kBandTiles + off % w;
    const int used = min(a.counts[p], a.cap[p]);
    const int rows = min(BM_PT, used - mt * BM_PT);
    const int chans = min(BN, H - nt * BN);
    const int64_t slot0 = (int64_t)a.capbase[p] + (int64_t)mt * BM_PT;
    const int8_t *wtile = a.W + ((int64_t)p * H + (int64_t)nt * BN) * H;
    const int8_t *xb = reinterpret_cast<const int8_t *>(a.dbuf) + slot0 * a.slot_stride;
    const uint32_t xstep = 32u * (uint32_t)a.slot_stride, wstep = 32u * (uint32_t)H;
    const uint32_t xo = (uint32_t)(128 * grp + (gt >> 3)) * (uint32_t)a.slot_stride + 16u * (gt & 7);
    const uint32_t wo = (uint32_t)(128 * grp + (gt >> 3)) * (uint32_t)H + 16u * (gt & 7);
    const int8_t *sb = xb + (int64_t)(128 * grp + gt) * a.slot_stride + H;
    auto fetch = [&](int g) {
      return fetch_part(xb, wtile, xo, wo, xstep, wstep, rows, chans, g, grp, gt, sb);
    };

    v4i acc[4][TF];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf)
#pragma unroll
      for (int tf = 0; tf < TF; ++tf) acc[nf][tf] = v4i{0, 0, 0, 0};

    __syncthreads();  // the previous tile's reads of the LDS tiles and scales are done
    stage_part(Xs[0], Ws[0], sx, fetch(0), 0, grp, gt);
    if (grp == 1 && ksteps > 1) stage_part(Xs[1], Ws[1], sx, fetch(1), 1, grp, gt);
    // The step this group stages next (A: 1, B: 2) is loaded ahead.
    PartRegs nxt;
    const int first = 1 + grp;
    if (first < ksteps) nxt = fetch(first);
    __syncthreads();                // step 0 (and B's half of step 1) staged
    if (grp == 1) __syncthreads();  // group B runs one phase behind group A

    for (int g = 0; g < ksteps; ++g) {
      const int buf = g & 1;
      // ---- compute phase, at raised wave priority ----
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        v4i av[4];
#pragma unroll
        for (int nf = 0; nf < 4; ++nf)
          av[nf] = *reinterpret_cast<const v4i *>(
              &Ws[buf][64 * wn + 16 * nf + (lane & 15)][swz(lane, 4 * kk + (lane >> 4))]);
        // Token fragments four at a time (16 registers live, not 4 TF).
#pragma unroll
        for (int t0 = 0; t0 < TF; t0 += 4) {
          v4i bv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            bv[i] = *reinterpret_cast<const v4i *>(
                &Xs[buf][16 * TF * wm + 16 * (t0 + i) + (lane & 15)][swz(lane, 4 * kk + (lane >> 4))]);
#pragma unroll
          for (int nf = 0; nf < 4; ++nf)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[nf][t0 + i] =
                  __builtin_amdgcn_mfma_i32_16x16x64_i8(av[nf], bv[i], acc[nf][t0 + i], 0, 0, 0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
      // ---- memory phase: stage step st_g, load step st_g + 1 ----
      const int st_g = g + 1 + grp;
      if (st_g < ksteps) {
        stage_part(Xs[st_g & 1], Ws[st_g & 1], sx, nxt, st_g, grp, gt);
        if (st_g + 1 < ksteps) nxt = fetch(st_g + 1);
      }
      // Group B's last memory phase has nothing to do and no partner phase.
      if (grp == 0 || g + 1 < ksteps) __syncthreads();
    }

    // ---- epilogue: lane holds channels n0..n0+3 of token 128 wm + 16 tf + lane%16 ----
    // The one group's fold, fma(s, isum, +0), then the weight scale; token
    // rows one after another, as above.
    float4 ws[4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      const int nl = 64 * wn + 16 * nf + 4 * (lane >> 4);
      ws[nf] = nl < chans ? *reinterpret_cast<const float4 *>(a.w_scale + (int64_t)p * H +
                                                               nt * BN + nl)
                          : float4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int tf = 0; tf < TF; ++tf) {
      const int t = 16 * TF * wm + 16 * tf + (lane & 15);
      if (t >= rows) continue;
      const float sc = sx[t];
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        const int nl = 64 * wn + 16 * nf + 4 * (lane >> 4);
        if (nl >= chans) continue;
        const int64_t n0 = (int64_t)nt * BN + nl;
        float v[4];
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) v[q2] = __builtin_fmaf(sc, (float)acc[nf][tf][q2], 0.0f);
        const uint2 o = make_uint2(pack_bf16x2(v[0] * ws[nf].x, v[1] * ws[nf].y),
                                   pack_bf16x2(v[2] * ws[nf].z, v[3] * ws[nf].w));
        *reinterpret_cast<uint2 *>(a.ebuf + (slot0 + t) * (int64_t)H + n0) = o;
      }
    }
  }
}

}  // namespace

hipError_t launch_expert_gemm(const GemmArgs &args, int grid, hipStream_t s) {
  if (args.Jmax > kMaxBands || grid % kXcds) return hipErrorInvalidValue;
  GemmArgs a = args;
  a.bm = a.steps_per_group == 1 ? BM : BM_PT;  // the tile rows of the kernel below
  gemm_tiles<<<1, 1024, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.steps_per_group == 1)
    expert_gemm_groups<<<grid, kThreads, 0, s>>>(a);
  else
    expert_gemm_pt<<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moedc
