// noalloc.hip -- moedc_route for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation): the workspace of moedc_route is replaced by a library-owned
// static device array.
//
// Layout of the array (fixed, independent of the plan):
//   [0, kTableBytes)          the plan's table image (capacities, slot bases,
//                             replica copy counts and table), copied in by
//                             every call;
//   [kTableBytes, kScratchBytes)  the route kernels' per-block expert counts.
// Every GPU the library runs on holds its own copy of the array until the
// process ends.  In host code the array's name is only a stand-in for the
// symbol; the device address comes from hipGetSymbolAddress, looked up once
// per device and kept, and only that address reaches kernels and copies.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.hpp"

namespace {

constexpr int64_t kScratchBytes = 16ll << 20;
constexpr int64_t kTableBytes = 64ll << 10;
static_assert(moedc::kMaxTableBytes <= kTableBytes, "table image fits its region");
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, or null

// Device address of the array on the current device (looked up once).
hipError_t scratch_on_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" moedc_status moedc_route_noalloc(const moedc_plan *p, int32_t T, const float *logits,
                                            int32_t *topk_ids, float *topk_w, int32_t *counts,
                                            int32_t *offsets, int32_t *slots, int32_t *dropped,
                                            hipStream_t stream) {
  const moedc_status st =
      moedc::check_route_args(p, T, logits, topk_ids, topk_w, counts, offsets, slots, dropped);
  if (st != MOEDC_OK) return st;
  // Per-block counts of this call: one int32 per (64-token block, physical
  // expert).  Batches of at most kFusedMaxTokens tokens need none.
  const int64_t nblk = ((int64_t)T + moedc::kRouteTokens - 1) / moedc::kRouteTokens;
  const int64_t need = 4 * nblk * p->cfg.num_phys_experts;
  if ((int64_t)p->table_image.size() > kTableBytes || need > kScratchBytes - kTableBytes)
    return MOEDC_ERR_UNSUPPORTED;
  void *base = nullptr;
  hipError_t e = scratch_on_current_device(&base);
  if (e != hipSuccess) return moedc::hip_status(e);
  unsigned char *sp = static_cast<unsigned char *>(base);
  e = hipMemcpyAsync(sp, p->table_image.data(), p->table_image.size(), hipMemcpyHostToDevice,
                     stream);
  if (e != hipSuccess) return moedc::hip_status(e);
  const moedc::RouteArgs ra =
      moedc::route_args_at(p, T, logits, topk_ids, topk_w, counts, offsets, slots, dropped, sp,
                           reinterpret_cast<int32_t *>(sp + kTableBytes));
  return moedc::hip_status(moedc::launch_route_any(ra, stream));
}
