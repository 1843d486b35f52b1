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
// Work list: gemm_tiles turns the route's counts into tiles of 128 slot rows
// x 256 channels, expert-major; a persistent grid walks the list.  Per tile,
// 8 waves (2 token halves x 4 channel quarters, 64 x 64 each); MFMA
// v_mfma_i32_16x16x64_i8 with A = 16 weight rows (channels) and B = 16 slot
// rows (tokens), so each lane ends up with 4 consecutive channels of one
// token (8-byte BF16 stores).  K advances 128 inputs per step; slot rows and
// weight rows are shared by 4 and 2 waves respectively and pass through a
// double-buffered LDS tile, loaded one step ahead into registers, with one
// barrier per step.  A tile moves 48 KiB per step for 8.4 MOP (175 op/B),
// twice the reuse of a 64 x 128 tile: the kernel is bound by cache
// bandwidth before MFMA throughput.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"

namespace moedc {

namespace {

constexpr int BM = 128;   // slot rows (tokens) per tile
constexpr int BN = 256;   // output channels per tile
constexpr int BK = 128;   // inputs per K step
constexpr int PITCH = BK + 16;  // LDS row pitch: conflict-free 16-byte reads
constexpr int kThreads = 512;   // 8 waves: 2 token halves x 4 channel quarters

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
__device__ __forceinline__ v4i ld16(const void *p) { return *reinterpret_cast<const v4i *>(p); }

// One K step of the tile, as loaded by one thread: 2 x 16 B of slot rows
// (rows r and r+64), 4 x 16 B of weight rows (r, r+64, r+128, r+192) and, at
// the first step of a scale group, one activation scale (threads < BM).
// Rows past the expert's tokens or past H channels read as zero.
struct StepRegs {
  v4i x[2], w[4];
  float s;
};

__device__ __forceinline__ StepRegs fetch_step(const GemmArgs &a, const int8_t *wtile,
                                               int64_t slot0, int rows, int chans, int g,
                                               int spg, int tid) {
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
  if (tid < BM && g % spg == 0 && tid < rows)
    st.s = *reinterpret_cast<const float *>(a.dbuf + (slot0 + tid) * a.slot_stride + a.H +
                                            4 * (g / spg));
  return st;
}

// Scales are double-buffered by group parity: group j's scale is written
// with its first step and read after its last, while group j+1's goes to
// the other buffer.
__device__ __forceinline__ void stage(int8_t (&Xs)[BM][PITCH], int8_t (&Ws)[BN][PITCH],
                                      float (&sx)[2][BM], const StepRegs &st, int g, int spg,
                                      int tid) {
  const int r = tid >> 3, c = 16 * (tid & 7);
#pragma unroll
  for (int i = 0; i < 2; ++i) *reinterpret_cast<v4i *>(&Xs[r + 64 * i][c]) = st.x[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<v4i *>(&Ws[r + 64 * i][c]) = st.w[i];
  if (tid < BM && g % spg == 0) sx[(g / spg) & 1][tid] = st.s;
}

__global__ __launch_bounds__(kThreads) void expert_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) int8_t Xs[2][BM][PITCH];
  __shared__ __attribute__((aligned(16))) int8_t Ws[2][BN][PITCH];
  __shared__ float sx[2][BM];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = uniform(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // token half, channel quarter
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
    const int chans = min(BN, H - nt * BN);
    const int64_t slot0 = (int64_t)a.capbase[p] + (int64_t)mt * BM;
    const int8_t *wtile = a.W + ((int64_t)p * H + (int64_t)nt * BN) * H;

    v4i acc[4][4];
    float accf[4][4][4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf)
#pragma unroll
      for (int tf = 0; tf < 4; ++tf) {
        acc[nf][tf] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 4; ++q) accf[nf][tf][q] = 0.0f;
      }

    __syncthreads();  // the previous tile's last reads of the LDS tiles are done
    stage(Xs[0], Ws[0], sx, fetch_step(a, wtile, slot0, rows, chans, 0, spg, tid), 0, spg, tid);
    StepRegs nxt = fetch_step(a, wtile, slot0, rows, chans, min(1, ksteps - 1), spg, tid);

    for (int g = 0; g < ksteps; ++g) {
      const int buf = g & 1;
      __syncthreads();  // step g staged by all; step g-1's reads of buf^1 done
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        v4i av[4], bv[4];
#pragma unroll
        for (int nf = 0; nf < 4; ++nf)
          av[nf] = *reinterpret_cast<const v4i *>(
              &Ws[buf][64 * wn + 16 * nf + (lane & 15)][64 * kk + 16 * (lane >> 4)]);
#pragma unroll
        for (int tf = 0; tf < 4; ++tf)
          bv[tf] = *reinterpret_cast<const v4i *>(
              &Xs[buf][64 * wm + 16 * tf + (lane & 15)][64 * kk + 16 * (lane >> 4)]);
#pragma unroll
        for (int nf = 0; nf < 4; ++nf)
#pragma unroll
          for (int tf = 0; tf < 4; ++tf)
            acc[nf][tf] =
                __builtin_amdgcn_mfma_i32_16x16x64_i8(av[nf], bv[tf], acc[nf][tf], 0, 0, 0);
      }
      if (g + 1 < ksteps) stage(Xs[buf ^ 1], Ws[buf ^ 1], sx, nxt, g + 1, spg, tid);
      if (g + 2 < ksteps) nxt = fetch_step(a, wtile, slot0, rows, chans, g + 2, spg, tid);

      if (g % spg == spg - 1) {  // end of an activation-scale group
#pragma unroll
        for (int tf = 0; tf < 4; ++tf) {
          const float s = sx[(g / spg) & 1][64 * wm + 16 * tf + (lane & 15)];
#pragma unroll
          for (int nf = 0; nf < 4; ++nf) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              accf[nf][tf][q] = __builtin_fmaf(s, (float)acc[nf][tf][q], accf[nf][tf][q]);
            acc[nf][tf] = v4i{0, 0, 0, 0};
          }
        }
      }
    }

    // ---- epilogue: lane holds channels n0..n0+3 of token 64 wm + 16 tf + lane%16 ----
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      const int nl = 64 * wn + 16 * nf + 4 * (lane >> 4);
      if (nl >= chans) continue;
      const int n0 = nt * BN + nl;
      const float4 ws = *reinterpret_cast<const float4 *>(a.w_scale + (int64_t)p * H + n0);
#pragma unroll
      for (int tf = 0; tf < 4; ++tf) {
        const int t = 64 * wm + 16 * tf + (lane & 15);
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
  expert_gemm<<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moedc
