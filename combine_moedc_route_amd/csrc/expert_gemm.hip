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
// Work list: gemm_tiles turns the route's counts into tiles of 64 slot rows
// x 128 channels, expert-major; a persistent grid walks the list.  Per tile,
// 4 waves; MFMA v_mfma_i32_16x16x64_i8 with A = 16 weight rows (channels)
// and B = 16 slot rows (tokens), so each lane ends up with 4 consecutive
// channels of one token (8-byte BF16 stores).  K advances 128 inputs at a
// time through LDS, the next step's loads prefetched into registers.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"

namespace moedc {

namespace {

constexpr int BM = 64;    // slot rows (tokens) per tile
constexpr int BN = 128;   // output channels per tile
constexpr int BK = 128;   // inputs per K step
constexpr int PITCH = BK + 16;  // LDS row pitch: conflict-free 16-byte reads

typedef int v4i __attribute__((ext_vector_type(4)));

// counts -> tile_base[p] = tiles of experts < p; tile_base[P] = total.
__global__ __launch_bounds__(1024) void gemm_tiles(GemmArgs a) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  int tiles = 0;
  if (tid < a.P) {
    const int used = min(a.counts[tid], a.cap[tid]);
    tiles = (used + BM - 1) / BM * a.ntiles;
  }
  int incl = tiles;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d);
    if ((tid & 63) >= d) incl += u;
  }
  if ((tid & 63) == 63) wsum[tid >> 6] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < (tid >> 6); ++w) base += wsum[w];
  if (tid < a.P) a.tile_base[tid] = base + incl - tiles;
  if (tid == a.P - 1) a.tile_base[a.P] = base + incl;
}

// Loads of K step g: 16 KiB of weights (4 x 16 B per thread, rows n, n+32,
// n+64, n+96), 8 KiB of slot payload (2 x 16 B; rows past the expert's
// tokens read as zero) and, at the first step of a scale group, one
// activation scale per slot row.
struct StepRegs {
  uint4 w0, w1, w2, w3, x0, x1;
  float s;
};

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

__device__ __forceinline__ StepRegs fetch_step(const GemmArgs &a, const int8_t *wbase,
                                               int64_t slot0, int rows, int g, int spg, int tid,
                                               float s_prev) {
  const int H = a.H;
  const int n = tid >> 3, c = tid & 7;  // + 32 rows per further 256 chunks
  const int8_t *wp = wbase + (int64_t)n * H + g * BK + 16 * c;
  StepRegs r;
  r.w0 = ld16(wp);
  r.w1 = ld16(wp + 32 * (int64_t)H);
  r.w2 = ld16(wp + 64 * (int64_t)H);
  r.w3 = ld16(wp + 96 * (int64_t)H);
  const uint8_t *xp = a.dbuf + (slot0 + n) * a.slot_stride + g * BK + 16 * c;
  r.x0 = n < rows ? ld16(xp) : make_uint4(0, 0, 0, 0);
  r.x1 = n + 32 < rows ? ld16(xp + 32 * a.slot_stride) : make_uint4(0, 0, 0, 0);
  r.s = s_prev;
  if (tid < BM && g % spg == 0)
    r.s = tid < rows ? *reinterpret_cast<const float *>(a.dbuf + (slot0 + tid) * a.slot_stride +
                                                        H + 4 * (g / spg))
                     : 0.0f;
  return r;
}

__global__ __launch_bounds__(256) void expert_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) int8_t Ws[BN][PITCH];
  __shared__ __attribute__((aligned(16))) int8_t Xs[BM][PITCH];
  __shared__ float sx[BM];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = uniform(tid >> 6);
  const int H = a.H;
  const int ksteps = H / BK;
  const int spg = a.steps_per_group;  // K steps per activation scale
  const int total = uniform(a.tile_base[a.P]);

  for (int lin = blockIdx.x; lin < total; lin += gridDim.x) {
    // ---- locate the tile: expert p owns tile_base[p] .. tile_base[p+1) ----
    int lo = 0, hi = a.P;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.tile_base[mid] <= lin) lo = mid; else hi = mid;
    }
    const int p = uniform(lo);
    const int r = lin - a.tile_base[p];
    const int mt = r / a.ntiles, nt = r % a.ntiles;
    const int used = min(a.counts[p], a.cap[p]);
    const int rows = min(BM, used - mt * BM);
    const int64_t slot0 = (int64_t)a.capbase[p] + (int64_t)mt * BM;
    const int8_t *wbase = a.W + ((int64_t)p * H + (int64_t)nt * BN) * H;

    v4i acc[2][4];
    float accf[2][4][4];
#pragma unroll
    for (int nf = 0; nf < 2; ++nf)
#pragma unroll
      for (int tf = 0; tf < 4; ++tf) {
        acc[nf][tf] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 4; ++q) accf[nf][tf][q] = 0.0f;
      }

    StepRegs st = fetch_step(a, wbase, slot0, rows, 0, spg, tid, 0.0f);
    for (int g = 0; g < ksteps; ++g) {
      __syncthreads();  // LDS free: previous step's reads are done
      {
        const int n = tid >> 3, c = 16 * (tid & 7);
        *reinterpret_cast<uint4 *>(&Ws[n][c]) = st.w0;
        *reinterpret_cast<uint4 *>(&Ws[n + 32][c]) = st.w1;
        *reinterpret_cast<uint4 *>(&Ws[n + 64][c]) = st.w2;
        *reinterpret_cast<uint4 *>(&Ws[n + 96][c]) = st.w3;
        *reinterpret_cast<uint4 *>(&Xs[n][c]) = st.x0;
        *reinterpret_cast<uint4 *>(&Xs[n + 32][c]) = st.x1;
      }
      if (tid < BM && g % spg == 0) sx[tid] = st.s;
      __syncthreads();
      if (g + 1 < ksteps)  // in flight during the MFMAs below
        st = fetch_step(a, wbase, slot0, rows, g + 1, spg, tid, st.s);

#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        v4i av[2], bv[4];
#pragma unroll
        for (int nf = 0; nf < 2; ++nf)
          av[nf] = *reinterpret_cast<const v4i *>(
              &Ws[32 * wave + 16 * nf + (lane & 15)][64 * kk + 16 * (lane >> 4)]);
#pragma unroll
        for (int tf = 0; tf < 4; ++tf)
          bv[tf] = *reinterpret_cast<const v4i *>(
              &Xs[16 * tf + (lane & 15)][64 * kk + 16 * (lane >> 4)]);
#pragma unroll
        for (int nf = 0; nf < 2; ++nf)
#pragma unroll
          for (int tf = 0; tf < 4; ++tf)
            acc[nf][tf] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[nf], bv[tf], acc[nf][tf], 0, 0, 0);
      }

      if (g % spg == spg - 1) {  // end of an activation-scale group
#pragma unroll
        for (int tf = 0; tf < 4; ++tf) {
          const float s = sx[16 * tf + (lane & 15)];
#pragma unroll
          for (int nf = 0; nf < 2; ++nf) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              accf[nf][tf][q] = __builtin_fmaf(s, (float)acc[nf][tf][q], accf[nf][tf][q]);
            acc[nf][tf] = v4i{0, 0, 0, 0};
          }
        }
      }
    }

    // ---- epilogue: lane holds channels n0..n0+3 of token 16 tf + lane%16 ----
#pragma unroll
    for (int nf = 0; nf < 2; ++nf) {
      const int n0 = nt * BN + 32 * wave + 16 * nf + 4 * (lane >> 4);
      const float4 ws = *reinterpret_cast<const float4 *>(a.w_scale + (int64_t)p * H + n0);
#pragma unroll
      for (int tf = 0; tf < 4; ++tf) {
        const int t = 16 * tf + (lane & 15);
        if (t < rows) {
          const uint2 o = make_uint2(pack_bf16x2(accf[nf][tf][0] * ws.x, accf[nf][tf][1] * ws.y),
                                     pack_bf16x2(accf[nf][tf][2] * ws.z, accf[nf][tf][3] * ws.w));
          *reinterpret_cast<uint2 *>(a.ebuf + (slot0 + t) * (int64_t)H + n0) = o;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_expert_gemm(const GemmArgs &a, int grid, hipStream_t s) {
  gemm_tiles<<<1, 1024, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  expert_gemm<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moedc
