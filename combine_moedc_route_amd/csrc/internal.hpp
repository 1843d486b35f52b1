// internal.hpp -- plan layout and kernel launchers shared by the host code
// (host.cpp) and the HIP kernels (route.hip, dispatch.hip, combine.hip,
// stub.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <vector>

#include "../../include/moedc.h"

namespace moedc {

constexpr int kGroup = 128;          // quantization group (values)
constexpr int kMaxHidden = 8192;     // 16 chunks of 512 values per wave
constexpr int kMaxExperts = 1024;    // logical and physical
constexpr int kMaxK = 16;            // entries per token
constexpr int kMaxReplicas = 8;
constexpr int kRouteTokens = 64;     // tokens per route block (4 lanes per token)
constexpr int kFusedMaxTokens = 256; // largest batch of the small-batch route (+ dispatch) path
constexpr int64_t kSlotAlign = 512;  // dispatch slot stride granularity
constexpr int64_t kWsAlign = 256;
// Expert GEMM work list: bands of kBandTiles channel tiles x all row tiles
// of one expert, dealt round-robin to the kXcds accelerator dies.
constexpr int kXcds = 8;
constexpr int kBandTiles = 4;
constexpr int kGemmChannels = 256;  // output channels per tile
constexpr int kMaxBands = 8192;     // kMaxExperts x ceil(ceil(kMaxHidden / 256) / kBandTiles)

// Workspace byte offsets (all kWsAlign-aligned).  The static tables come
// first and form one contiguous image [0, tables_end) that the host keeps in
// the plan and uploads with a single copy.
struct WsLayout {
  int64_t cap = 0;          // int32 [P]
  int64_t capbase = 0;      // int32 [P]
  int64_t rep_count = 0;    // int32 [E]
  int64_t rep_table = 0;    // int32 [E][R]
  int64_t tables_end = 0;   // end of the table image (<= kMaxTableBytes)
  int64_t block_counts = 0; // int32 [P][nblk_max]: the route's per-block expert counts
  int64_t band_pre = 0;     // int32 [8][Jmax+1]: tile prefix of each XCD's bands (expert GEMM)
  int64_t band_list = 0;    // int32 [8][Jmax]: each XCD's bands in order
  int64_t band_cnt = 0;     // int32 [8]: bands per XCD
  int64_t bytes = 0;
};
// Largest table image: capacities and bases of 1024 physical experts, copy
// counts and an 8-column replica table of 1024 logical experts.
constexpr int64_t kMaxTableBytes = 4 * kMaxExperts * (3 + kMaxReplicas);

struct RouteArgs {
  const float *logits;
  int32_t *topk_ids;
  float *topk_w;
  int32_t *counts;
  int32_t *offsets;
  int32_t *slots;
  int32_t *dropped;
  const int32_t *cap;
  const int32_t *capbase;
  const int32_t *rep_count;
  const int32_t *rep_table;
  int32_t *block_counts;  // [P][ceil(T/64)]: per-block counts, then block prefixes
  int32_t T, E, P, R, K, KR, shared, score_fn;
  int32_t rep_identity;  // every logical expert e is physical expert e (one copy)
};

struct DispatchArgs {
  const uint16_t *x;
  const int32_t *slots;
  uint8_t *dbuf;
  int64_t slot_stride;
  int32_t T, H, G, K;
  int32_t per_token;    // one scale per token (G == 1) instead of per 128 values
  int32_t total_slots;  // entries outside [0, total_slots) are skipped
  int32_t cached_payload;  // payload through ordinary stores (inputs larger than kStreamInputBytes)
};

// Dispatch batches whose BF16 input is at most this many bytes (the MI355X
// memory-side cache's capacity) write their payload with non-temporal
// stores, larger ones with ordinary ones.
constexpr int64_t kStreamInputBytes = int64_t(256) << 20;

struct CombineArgs {
  const uint8_t *eout;
  const int32_t *slots;
  const float *w;
  uint16_t *y;
  int64_t eout_stride;  // bytes per slot row
  int32_t total_slots;  // entries outside [0, total_slots) are skipped
  int32_t T, H, K, fmt;
  int32_t per_token;    // Q8 input: one scale per token
  int32_t max_blocks;   // grid cap in workgroups (4 waves, or 16 from 2048 tokens on and
                        // whenever the cap binds); >= 1
};

struct StubArgs {
  const uint8_t *dbuf;
  uint16_t *ebuf;
  const int32_t *counts;
  const int32_t *cap;
  const int32_t *capbase;
  int64_t slot_stride;
  int64_t ebuf_stride;
  int64_t total_slots;
  int32_t H, P;
  int32_t per_token;
};

struct GemmArgs {
  const uint8_t *dbuf;
  const int8_t *W;
  const float *w_scale;
  uint16_t *ebuf;
  const int32_t *counts;
  const int32_t *cap;
  const int32_t *capbase;
  int32_t *band_pre;        // [kXcds][Jmax+1] exclusive tile prefix of each XCD's bands
  int32_t *band_list;       // [kXcds][Jmax] bands of each XCD, in the order walked
  int32_t *band_cnt;        // [kXcds] bands per XCD
  int32_t *xcd_tiles;       // device [kXcds] tiles per XCD, or null
  int64_t slot_stride;
  int32_t H, P, ntiles, steps_per_group;
  int32_t nbe;              // bands per expert: ceil(ntiles / kBandTiles)
  int32_t Jmax;             // bands in all: P * nbe (an XCD may get any number of them)
  int32_t dealing;          // moedc_xcd_dealing
  int32_t bm;               // slot rows per tile (set by the launcher)
};

hipError_t launch_route(const RouteArgs &a, hipStream_t s);
// Batches of 1..kFusedMaxTokens tokens: wave-per-token top-k + one-block ranks.
hipError_t launch_route_small(const RouteArgs &a, hipStream_t s);
hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t s);
hipError_t launch_combine(const CombineArgs &a, hipStream_t s);
hipError_t launch_stub(const StubArgs &a, hipStream_t s);
hipError_t launch_route_dispatch_fused(const RouteArgs &ra, const DispatchArgs &da,
                                       hipStream_t s);
hipError_t launch_expert_gemm(const GemmArgs &a, int grid, hipStream_t s);

}  // namespace moedc

struct moedc_plan;

namespace moedc {

// Host helpers shared by the entry points (host.cpp).
// Records e as the thread's last HIP error and returns MOEDC_ERR_HIP, or
// MOEDC_OK for hipSuccess.
moedc_status hip_status(hipError_t e);
// Host-side argument checks of a route call, without the workspace.
moedc_status check_route_args(const moedc_plan *p, int32_t T, const float *logits,
                              const int32_t *topk_ids, const float *topk_w,
                              const int32_t *counts, const int32_t *offsets,
                              const int32_t *slots, const int32_t *dropped);
// Route kernel arguments with the plan's table image at `tables` (laid out as
// in the workspace) and the per-block counts at `block_counts`.
RouteArgs route_args_at(const moedc_plan *p, int32_t T, const float *logits, int32_t *topk_ids,
                        float *topk_w, int32_t *counts, int32_t *offsets, int32_t *slots,
                        int32_t *dropped, const void *tables, int32_t *block_counts);
// Runs the route kernels for a small or large batch.
hipError_t launch_route_any(const RouteArgs &a, hipStream_t s);

}  // namespace moedc

struct moedc_plan {
  moedc_config cfg;                 // pointer fields point into the vectors below
  std::vector<int32_t> cap, capbase, rep_count, rep_table;
  std::vector<uint8_t> table_image;  // workspace bytes [0, ws.tables_end)
  int32_t K, G, nblk_max;
  int32_t rep_identity;             // no replicas and logical e == physical e
  int32_t gemm_nbe, gemm_Jmax;      // expert GEMM bands per expert / in all
  int64_t slot_stride, combine_stride, total_slots;
  moedc::WsLayout ws;
};
