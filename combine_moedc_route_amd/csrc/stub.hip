// stub.hip -- stand-in expert so the path can run end to end without
// weights: occupied slot of physical expert p gets
//   bf16( ((float)q * scale) * (1 + 0.01f * p) )
// (two rounded fp32 products, one rounded sum; no contraction).  Not a step
// of the method; the real expert is a grouped INT8 GEMM over the slots.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "internal.hpp"

namespace moedc {

namespace {

__global__ __launch_bounds__(256) void stub_kernel(StubArgs a) {
  const int lane = lane_id();
  const int64_t s = (int64_t)blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (s >= a.total_slots) return;
  // Owner: the last expert whose first slot is <= s (experts with zero
  // capacity share their base with the next one and are skipped).
  int lo = 0, hi = a.P;  // number of experts with capbase <= s lies in [1, P]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.capbase[mid] <= s) lo = mid; else hi = mid;
  }
  const int p = uniform(lo);
  const int64_t j = s - a.capbase[p];
  if (j >= min(a.counts[p], a.cap[p])) return;
  const float m = 1.0f + 0.01f * (float)p;
  const uint8_t *src = a.dbuf + s * a.slot_stride;
  uint4 *dst = reinterpret_cast<uint4 *>(reinterpret_cast<uint8_t *>(a.ebuf) + s * a.ebuf_stride);
  const int H = a.H;
  for (int c = 0; c * 512 < H; ++c) {
    const int e = c * 512 + lane * 8;
    if (e >= H) continue;
    const uint2 q = *reinterpret_cast<const uint2 *>(src + e);
    const float sc = *reinterpret_cast<const float *>(src + H + (a.per_token ? 0 : 4 * (e >> 7)));
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t d = i < 4 ? q.x : q.y;
      const int qi = (int)(int8_t)((d >> (8 * (i & 3))) & 0xFFu);
      o[i] = ((float)qi * sc) * m;
    }
    dst[c * 64 + lane] = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                    pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
  }
}

}  // namespace

hipError_t launch_stub(const StubArgs &a, hipStream_t s) {
  if (a.total_slots == 0) return hipSuccess;
  const unsigned grid = (unsigned)((a.total_slots + 3) / 4);
  stub_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moedc
