// ceiling.hip -- measurement kernels (libmoedc_ceiling.so): the memory
// system's attainable bandwidth for plain streams and for dispatch's store
// and combine's load patterns with their arithmetic taken out, and the
// compute floor of the expert layer's instruction mix with its memory
// traffic taken out.  Not part of the MoE path; the benchmark reads
// dispatch, combine and the expert layer against these.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moedc_ceiling.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kReadUnroll = 4;  // 16-byte loads per thread in the read stream

__device__ __forceinline__ u32x4 ld_nt(const u32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(u32x4 v, u32x4 *p) { __builtin_nontemporal_store(v, p); }

// The plain streams run one short-lived workgroup per 4 KiB (16 KiB for the
// read), one 16-byte access per thread and step: workgroups start in index
// order, so the accesses in flight cover a narrow address window.  On a
// 4 GiB buffer that reads at 7.2, writes at 6.7 and copies at 6.5 TB/s,
// against 6.5 / 5.0 / 4.9 TB/s for 8192 persistent workgroups striding
// through the buffer.  Non-temporal loads read faster than ordinary ones
// (7.2 against 6.7 TB/s); ordinary stores write faster than non-temporal
// ones (6.7 against 6.5); the copy is fastest with both non-temporal.
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4 *src, int64_t n,
                                                        uint32_t *sink) {
  const int64_t i0 = (int64_t)blockIdx.x * (kReadUnroll * kThreads) + threadIdx.x;
  u32x4 v[kReadUnroll];
#pragma unroll
  for (int u = 0; u < kReadUnroll; ++u) {
    const int64_t i = i0 + u * kThreads;
    v[u] = i < n ? ld_nt(src + i) : u32x4{0u, 0u, 0u, 0u};
  }
  u32x4 acc = v[0];
#pragma unroll
  for (int u = 1; u < kReadUnroll; ++u) acc ^= v[u];
  const uint32_t f = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (f == 0x9E3779B9u && acc.x == 0x7F4A7C15u) sink[0] = f;
}

__global__ __launch_bounds__(kThreads) void write_kernel(u32x4 *dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) dst[i] = u32x4{threadIdx.x, blockIdx.x, 0x5A5A5A5Au, 0u};
}

__global__ __launch_bounds__(kThreads) void copy_kernel(u32x4 *dst, const u32x4 *src, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) st_nt(ld_nt(src + i), dst + i);
}

// A workgroup per token, wave c writing bytes [512 c, 512 c + 512) of each
// of the token's slots, 8 bytes per lane, with ordinary stores (as
// dispatch's payload).
__global__ __launch_bounds__(1024) void scatter_kernel(const int32_t *slots, int K,
                                                       uint8_t *dbuf, int64_t slot_stride,
                                                       int row_bytes) {
  const int t = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int off = wave * 512 + lane * 8;
  const u32x2 v = {(uint32_t)t, (uint32_t)threadIdx.x};
  for (int k = 0; k < K; ++k) {
    const int s = slots[(int64_t)t * K + k];
    if (s < 0 || off >= row_bytes) continue;
    *reinterpret_cast<u32x2 *>(dbuf + (int64_t)s * slot_stride + off) = v;
  }
}

// One wave per (token, 1 KiB chunk), 16 waves per workgroup.
__global__ __launch_bounds__(1024) void gather_kernel(const uint8_t *rows, const int32_t *slots,
                                                      int T, int K, int64_t row_stride,
                                                      int row_bytes, uint8_t *out) {
  const int nch = (row_bytes + 1023) / 1024;
  const int64_t u = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 6);
  if (u >= (int64_t)T * nch) return;
  const int t = (int)(u / nch), c = (int)(u - (int64_t)t * nch);
  const int off = c * 1024 + (threadIdx.x & 63) * 16;
  int s[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) s[k] = k < K ? slots[(int64_t)t * K + k] : -1;
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (s[k] >= 0 && off < row_bytes)
      acc ^= ld_nt(reinterpret_cast<const u32x4 *>(rows + (int64_t)s[k] * row_stride + off));
  if (off < row_bytes) st_nt(acc, reinterpret_cast<u32x4 *>(out + (int64_t)t * row_bytes + off));
}

// The expert layer's per-wave instruction mix without memory: per K step,
// 2 x 16 v_mfma_i32_16x16x64_i8 on 16 accumulators from register operands
// and, with FOLD, the fold of the 64 int32 sums into fp32 (a convert and an
// FMA each, the first MFMA of the step on a zero accumulator) -- the
// 128-input-group kernel's step; without FOLD the sums carry on (the
// one-scale-per-token kernel).  512-thread workgroups: two waves per SIMD.
typedef int v4i __attribute__((ext_vector_type(4)));
template <bool FOLD>
__global__ __launch_bounds__(512) void mfma_kernel(int steps, float s, int *sink) {
  // 4 A and 4 B fragments, 16 accumulators (the layer's 4 x 4 blocking).
  v4i av[4], bv[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    av[f] = v4i{(int)threadIdx.x + f, 0x01020304 * (f + 1), 0x7F7F7F7F ^ f, (int)blockIdx.x};
    bv[f] = v4i{0x05060708 + f, (int)threadIdx.x * (3 + f), 0x11223344, 0x7F00FF01 - f};
  }
  v4i acc[16];
  float accf[16][4];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    acc[i] = v4i{i, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < 4; ++q) accf[i][q] = 0.0f;
  }
  for (int g = 0; g < steps; ++g) {
    av[0].x += g;  // operands that change every step: nothing is loop-invariant
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
            av[i >> 2], bv[i & 3], (FOLD && kk == 0) ? v4i{0, 0, 0, 0} : acc[i], 0, 0, 0);
    if (FOLD) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) accf[i][q] = __builtin_fmaf(s, (float)acc[i][q], accf[i][q]);
    }
  }
  int r = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) r += FOLD ? (int)accf[i][q] : acc[i][q];
  if (r == 0x5A5A5A5A) sink[0] = r;
}

// Workgroups for n 16-byte elements at `per` elements each; 0 when the grid
// would not fit a launch.
unsigned stream_grid(int64_t n, int64_t per) {
  const int64_t g = (n + per - 1) / per;
  return g <= 0x7fffffff ? (unsigned)g : 0u;
}

}  // namespace

extern "C" {

int32_t moedc_ceiling_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t s) {
  const int64_t n = bytes / 16;
  if (n <= 0) return 0;
  const unsigned g = stream_grid(n, kReadUnroll * kThreads);
  if (g == 0) return (int32_t)hipErrorInvalidValue;
  read_kernel<<<g, kThreads, 0, s>>>(static_cast<const u32x4 *>(src), n, sink);
  return (int32_t)hipGetLastError();
}

int32_t moedc_ceiling_write(void *dst, int64_t bytes, hipStream_t s) {
  const int64_t n = bytes / 16;
  if (n <= 0) return 0;
  const unsigned g = stream_grid(n, kThreads);
  if (g == 0) return (int32_t)hipErrorInvalidValue;
  write_kernel<<<g, kThreads, 0, s>>>(static_cast<u32x4 *>(dst), n);
  return (int32_t)hipGetLastError();
}

int32_t moedc_ceiling_copy(void *dst, const void *src, int64_t bytes, hipStream_t s) {
  const int64_t n = bytes / 16;
  if (n <= 0) return 0;
  const unsigned g = stream_grid(n, kThreads);
  if (g == 0) return (int32_t)hipErrorInvalidValue;
  copy_kernel<<<g, kThreads, 0, s>>>(static_cast<u32x4 *>(dst), static_cast<const u32x4 *>(src), n);
  return (int32_t)hipGetLastError();
}

int32_t moedc_ceiling_scatter(const int32_t *slots, int32_t T, int32_t K, void *dbuf,
                              int64_t slot_stride, int32_t row_bytes, hipStream_t s) {
  if (T <= 0) return 0;
  if (K < 1 || K > 16 || row_bytes <= 0 || row_bytes > 8192 || row_bytes % 8)
    return (int32_t)hipErrorInvalidValue;
  const int waves = (row_bytes + 511) / 512;
  scatter_kernel<<<(unsigned)T, 64 * waves, 0, s>>>(slots, K, static_cast<uint8_t *>(dbuf),
                                                    slot_stride, row_bytes);
  return (int32_t)hipGetLastError();
}

int32_t moedc_ceiling_gather(const void *rows, const int32_t *slots, int32_t T, int32_t K,
                             int64_t row_stride, int32_t row_bytes, void *out, hipStream_t s) {
  if (T <= 0) return 0;
  if (K < 1 || K > 16 || row_bytes <= 0 || row_bytes > 16384 || row_bytes % 16)
    return (int32_t)hipErrorInvalidValue;
  const int64_t units = (int64_t)T * ((row_bytes + 1023) / 1024);
  gather_kernel<<<(unsigned)((units + 15) / 16), 1024, 0, s>>>(
      static_cast<const uint8_t *>(rows), slots, T, K, row_stride, row_bytes,
      static_cast<uint8_t *>(out));
  return (int32_t)hipGetLastError();
}

int32_t moedc_ceiling_mfma(int64_t mfma_total, int32_t fold, uint32_t *sink, hipStream_t s) {
  // 256 workgroups x 8 waves, 32 MFMAs per wave and step.
  const int64_t steps = mfma_total / (256 * 8 * 32);
  if (steps <= 0 || steps > (1 << 30)) return (int32_t)hipErrorInvalidValue;
  if (fold)
    mfma_kernel<true><<<256, 512, 0, s>>>((int)steps, 1.0e-3f, reinterpret_cast<int *>(sink));
  else
    mfma_kernel<false><<<256, 512, 0, s>>>((int)steps, 1.0e-3f, reinterpret_cast<int *>(sink));
  return (int32_t)hipGetLastError();
}

}  // extern "C"
