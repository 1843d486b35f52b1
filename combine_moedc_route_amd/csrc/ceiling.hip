// ceiling.hip -- measurement kernels for the memory system's attainable
// bandwidth (libmoedc_ceiling.so): plain streams, and dispatch's store and
// combine's load patterns with their arithmetic taken out.  Not part of the
// MoE path; the benchmark reads dispatch and combine against these.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moedc_ceiling.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr unsigned kGrid = 8192;  // 32 workgroups per CU: enough loads in flight
constexpr int kUnroll = 4;        // 16-byte accesses per thread per step

__device__ __forceinline__ u32x4 ld_nt(const u32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(u32x4 v, u32x4 *p) { __builtin_nontemporal_store(v, p); }

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4 *src, int64_t n,
                                                        uint32_t *sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = ld_nt(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= ld_nt(src + i);
  const uint32_t f = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (f == 0x9E3779B9u && acc.x == 0x7F4A7C15u) sink[0] = f;
}

__global__ __launch_bounds__(kThreads) void write_kernel(u32x4 *dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const u32x4 v = {threadIdx.x, blockIdx.x, 0x5A5A5A5Au, 0u};
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) st_nt(v, dst + i);
}

__global__ __launch_bounds__(kThreads) void copy_kernel(u32x4 *dst, const u32x4 *src, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = ld_nt(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) st_nt(v[u], dst + i + u * stride);
  }
  for (; i < n; i += stride) st_nt(ld_nt(src + i), dst + i);
}

// A workgroup per token, wave c writing bytes [512 c, 512 c + 512) of each
// of the token's slots, 8 bytes per lane.
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
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(dbuf + (int64_t)s * slot_stride + off));
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

}  // namespace

extern "C" {

int32_t moedc_ceiling_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t s) {
  read_kernel<<<kGrid, kThreads, 0, s>>>(static_cast<const u32x4 *>(src), bytes / 16, sink);
  return (int32_t)hipGetLastError();
}

int32_t moedc_ceiling_write(void *dst, int64_t bytes, hipStream_t s) {
  write_kernel<<<kGrid, kThreads, 0, s>>>(static_cast<u32x4 *>(dst), bytes / 16);
  return (int32_t)hipGetLastError();
}

int32_t moedc_ceiling_copy(void *dst, const void *src, int64_t bytes, hipStream_t s) {
  copy_kernel<<<kGrid, kThreads, 0, s>>>(static_cast<u32x4 *>(dst),
                                          static_cast<const u32x4 *>(src), bytes / 16);
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

}  // extern "C"
