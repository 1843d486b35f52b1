// host.cpp -- C ABI of libmoedc: plan validation and sizing, workspace
// binding, argument checks and kernel launches on the caller's stream.
#include <hip/hip_runtime_api.h>

#include <climits>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/moedc.h"
#include "internal.hpp"

namespace {

thread_local int32_t g_last_hip_error = 0;

moedc_status hip_fail(hipError_t e) {
  g_last_hip_error = (int32_t)e;
  return MOEDC_ERR_HIP;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

moedc_status validate_config(const moedc_config *c) {
  using namespace moedc;
  if (!c || !c->capacity) return MOEDC_ERR_INVALID_ARG;
  if (c->hidden <= 0 || c->hidden % kGroup) return MOEDC_ERR_INVALID_ARG;
  if (c->group_size != kGroup && c->group_size != c->hidden) return MOEDC_ERR_UNSUPPORTED;
  if (c->hidden > kMaxHidden) return MOEDC_ERR_UNSUPPORTED;
  if (c->max_tokens < 0) return MOEDC_ERR_INVALID_ARG;
  if (c->max_tokens > (1 << 24)) return MOEDC_ERR_UNSUPPORTED;
  if (c->num_logical_experts < 1 || c->num_phys_experts < 1) return MOEDC_ERR_INVALID_ARG;
  if (c->num_logical_experts > kMaxExperts || c->num_phys_experts > kMaxExperts)
    return MOEDC_ERR_UNSUPPORTED;
  if (c->num_shared != 0 && c->num_shared != 1) return MOEDC_ERR_INVALID_ARG;
  if (c->top_k < 1 || c->top_k > c->num_logical_experts) return MOEDC_ERR_INVALID_ARG;
  if (c->top_k + c->num_shared > kMaxK) return MOEDC_ERR_UNSUPPORTED;
  if (c->score_fn != MOEDC_SCORE_SOFTMAX && c->score_fn != MOEDC_SCORE_SIGMOID_NORM)
    return MOEDC_ERR_INVALID_ARG;
  if (c->max_replicas < 1) return MOEDC_ERR_INVALID_ARG;
  if (c->max_replicas > kMaxReplicas) return MOEDC_ERR_UNSUPPORTED;
  const int32_t routed = c->num_phys_experts - c->num_shared;
  if (routed < 1) return MOEDC_ERR_INVALID_ARG;
  int64_t total = 0;
  for (int32_t p = 0; p < c->num_phys_experts; ++p) {
    if (c->capacity[p] < 0) return MOEDC_ERR_INVALID_ARG;
    total += c->capacity[p];
  }
  if (total > INT32_MAX) return MOEDC_ERR_UNSUPPORTED;
  const int32_t E = c->num_logical_experts, R = c->max_replicas;
  if (!c->replica_table) {
    if (R != 1 || routed < E) return MOEDC_ERR_INVALID_ARG;
    return MOEDC_OK;
  }
  std::vector<char> owned((size_t)routed, 0);
  for (int32_t e = 0; e < E; ++e) {
    const int32_t *row = c->replica_table + (int64_t)e * R;
    int32_t r = 0;
    while (r < R && row[r] >= 0) ++r;
    if (r == 0) return MOEDC_ERR_INVALID_ARG;
    for (int32_t k = 0; k < r; ++k) {
      if (row[k] >= routed || owned[(size_t)row[k]]) return MOEDC_ERR_INVALID_ARG;
      owned[(size_t)row[k]] = 1;
    }
    for (int32_t k = r; k < R; ++k)
      if (row[k] != -1) return MOEDC_ERR_INVALID_ARG;
  }
  return MOEDC_OK;
}

template <typename T>
T *ws_ptr(void *ws, int64_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

}  // namespace

extern "C" {

moedc_status moedc_plan_create(const moedc_config *config, moedc_plan **out) {
  using namespace moedc;
  if (!out) return MOEDC_ERR_INVALID_ARG;
  *out = nullptr;
  const moedc_status st = validate_config(config);
  if (st != MOEDC_OK) return st;
  moedc_plan *p = new (std::nothrow) moedc_plan();
  if (!p) return MOEDC_ERR_NO_MEMORY;
  try {
    const moedc_config &c = *config;
    const int32_t P = c.num_phys_experts, E = c.num_logical_experts, R = c.max_replicas;
    p->cfg = c;
    p->cap.assign(c.capacity, c.capacity + P);
    p->capbase.resize((size_t)P);
    int64_t run = 0;
    for (int32_t i = 0; i < P; ++i) {
      p->capbase[(size_t)i] = (int32_t)run;
      run += p->cap[(size_t)i];
    }
    p->total_slots = run;
    p->rep_count.resize((size_t)E);
    p->rep_table.assign((size_t)E * R, -1);
    for (int32_t e = 0; e < E; ++e) {
      if (!c.replica_table) {
        p->rep_count[(size_t)e] = 1;
        p->rep_table[(size_t)e * R] = e;
        continue;
      }
      int32_t r = 0;
      while (r < R && c.replica_table[(int64_t)e * R + r] >= 0) {
        p->rep_table[(size_t)e * R + r] = c.replica_table[(int64_t)e * R + r];
        ++r;
      }
      p->rep_count[(size_t)e] = r;
    }
    p->rep_identity = 1;
    for (int32_t e = 0; e < E; ++e)
      if (p->rep_count[(size_t)e] != 1 || p->rep_table[(size_t)e * R] != e) p->rep_identity = 0;
    p->cfg.capacity = p->cap.data();
    p->cfg.replica_table = c.replica_table ? p->rep_table.data() : nullptr;
    p->K = c.top_k + c.num_shared;
    p->G = c.hidden / c.group_size;
    p->slot_stride = round_up((int64_t)c.hidden + 4 * (int64_t)p->G, kSlotAlign);
    p->combine_stride = 2 * (int64_t)c.hidden;
    p->nblk_max = c.max_tokens > 0 ? (c.max_tokens + kRouteTokens - 1) / kRouteTokens : 1;
    WsLayout &w = p->ws;
    int64_t o = 0;
    w.cap = o;           o = round_up(o + 4 * (int64_t)P, kWsAlign);
    w.capbase = o;       o = round_up(o + 4 * (int64_t)P, kWsAlign);
    w.rep_count = o;     o = round_up(o + 4 * (int64_t)E, kWsAlign);
    w.rep_table = o;     o = round_up(o + 4 * (int64_t)E * R, kWsAlign);
    w.tables_end = o;
    w.block_counts = o;  o = round_up(o + 4 * (int64_t)p->nblk_max * P, kWsAlign);
    const int32_t ntiles = (c.hidden + kGemmChannels - 1) / kGemmChannels;
    p->gemm_nbe = (ntiles + kBandTiles - 1) / kBandTiles;
    p->gemm_Jmax = P * p->gemm_nbe;
    w.band_pre = o;      o = round_up(o + 4 * (int64_t)kXcds * (p->gemm_Jmax + 1), kWsAlign);
    w.band_list = o;     o = round_up(o + 4 * (int64_t)kXcds * p->gemm_Jmax, kWsAlign);
    w.band_cnt = o;      o = round_up(o + 4 * (int64_t)kXcds, kWsAlign);
    w.bytes = o;
    p->table_image.assign((size_t)w.tables_end, 0);
    const struct { int64_t off; const std::vector<int32_t> &v; } parts[] = {
        {w.cap, p->cap}, {w.capbase, p->capbase}, {w.rep_count, p->rep_count},
        {w.rep_table, p->rep_table}};
    for (const auto &pt : parts)
      std::memcpy(p->table_image.data() + pt.off, pt.v.data(), 4 * pt.v.size());
  } catch (...) {
    delete p;
    return MOEDC_ERR_NO_MEMORY;
  }
  *out = p;
  return MOEDC_OK;
}

void moedc_plan_destroy(moedc_plan *plan) { delete plan; }

moedc_status moedc_plan_sizes(const moedc_plan *p, moedc_sizes *out) {
  if (!p || !out) return MOEDC_ERR_INVALID_ARG;
  out->workspace_bytes = p->ws.bytes;
  out->dispatch_buf_bytes = p->total_slots * p->slot_stride;
  out->combine_buf_bytes = p->total_slots * p->combine_stride;
  out->slot_stride = p->slot_stride;
  out->combine_slot_stride = p->combine_stride;
  out->total_slots = p->total_slots;
  out->k = p->K;
  out->num_groups = p->G;
  return MOEDC_OK;
}

moedc_status moedc_plan_bind_workspace(const moedc_plan *p, void *ws, hipStream_t stream) {
  if (!p || !ws) return MOEDC_ERR_INVALID_ARG;
  if (!aligned16(ws)) return MOEDC_ERR_ALIGN;
  const hipError_t e = hipMemcpyAsync(ws, p->table_image.data(), p->table_image.size(),
                                      hipMemcpyHostToDevice, stream);
  return e == hipSuccess ? MOEDC_OK : hip_fail(e);
}

}  // extern "C"

namespace {

moedc_status check_route(const moedc_plan *p, int32_t T, const float *logits,
                         const int32_t *topk_ids, const float *topk_w, const int32_t *counts,
                         const int32_t *offsets, const int32_t *slots, const int32_t *dropped,
                         const void *ws) {
  const moedc_status st = moedc::check_route_args(p, T, logits, topk_ids, topk_w, counts,
                                                  offsets, slots, dropped);
  if (st != MOEDC_OK) return st;
  if (!ws) return MOEDC_ERR_INVALID_ARG;
  if (!aligned16(ws)) return MOEDC_ERR_ALIGN;
  return MOEDC_OK;
}

moedc_status check_dispatch(const moedc_plan *p, int32_t T, const uint16_t *x,
                            const int32_t *slots, const void *dbuf) {
  if (!p) return MOEDC_ERR_INVALID_ARG;
  if (T < 0 || T > p->cfg.max_tokens) return MOEDC_ERR_SHAPE;
  if (T == 0) return MOEDC_OK;
  if (!x || !slots || !dbuf) return MOEDC_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(dbuf) || !aligned4(slots)) return MOEDC_ERR_ALIGN;
  return MOEDC_OK;
}

moedc::RouteArgs route_args(const moedc_plan *p, int32_t T, const float *logits,
                            int32_t *topk_ids, float *topk_w, int32_t *counts, int32_t *offsets,
                            int32_t *slots, int32_t *dropped, void *ws) {
  return moedc::route_args_at(p, T, logits, topk_ids, topk_w, counts, offsets, slots, dropped,
                              ws, ws_ptr<int32_t>(ws, p->ws.block_counts));
}

}  // namespace

namespace moedc {

moedc_status hip_status(hipError_t e) { return e == hipSuccess ? MOEDC_OK : hip_fail(e); }

moedc_status check_route_args(const moedc_plan *p, int32_t T, const float *logits,
                              const int32_t *topk_ids, const float *topk_w,
                              const int32_t *counts, const int32_t *offsets,
                              const int32_t *slots, const int32_t *dropped) {
  if (!p || !counts || !offsets || !dropped) return MOEDC_ERR_INVALID_ARG;
  if (T < 0 || T > p->cfg.max_tokens) return MOEDC_ERR_SHAPE;
  if (T > 0 && (!logits || !topk_ids || !topk_w || !slots)) return MOEDC_ERR_INVALID_ARG;
  if (!aligned4(counts) || !aligned4(offsets) || !aligned4(dropped)) return MOEDC_ERR_ALIGN;
  if (T > 0 && (!aligned16(logits) || !aligned4(topk_ids) || !aligned4(topk_w) ||
                !aligned4(slots)))
    return MOEDC_ERR_ALIGN;
  return MOEDC_OK;
}

hipError_t launch_route_any(const RouteArgs &a, hipStream_t s) {
  return (a.T > 0 && a.T <= kFusedMaxTokens) ? launch_route_small(a, s) : launch_route(a, s);
}

RouteArgs route_args_at(const moedc_plan *p, int32_t T, const float *logits, int32_t *topk_ids,
                        float *topk_w, int32_t *counts, int32_t *offsets, int32_t *slots,
                        int32_t *dropped, const void *tables, int32_t *block_counts) {
  void *ws = const_cast<void *>(tables);
  moedc::RouteArgs a{};
  a.logits = logits;
  a.topk_ids = topk_ids;
  a.topk_w = topk_w;
  a.counts = counts;
  a.offsets = offsets;
  a.slots = slots;
  a.dropped = dropped;
  a.cap = ws_ptr<const int32_t>(ws, p->ws.cap);
  a.capbase = ws_ptr<const int32_t>(ws, p->ws.capbase);
  a.rep_count = ws_ptr<const int32_t>(ws, p->ws.rep_count);
  a.rep_table = ws_ptr<const int32_t>(ws, p->ws.rep_table);
  a.block_counts = block_counts;
  a.T = T;
  a.E = p->cfg.num_logical_experts;
  a.P = p->cfg.num_phys_experts;
  a.R = p->cfg.max_replicas;
  a.K = p->K;
  a.KR = p->cfg.top_k;
  a.shared = p->cfg.num_shared;
  a.score_fn = p->cfg.score_fn;
  a.rep_identity = p->rep_identity;
  return a;
}

}  // namespace moedc

namespace {

moedc::DispatchArgs dispatch_args(const moedc_plan *p, int32_t T, const uint16_t *x,
                                  const int32_t *slots, void *dbuf) {
  moedc::DispatchArgs a{};
  a.x = x;
  a.slots = slots;
  a.dbuf = static_cast<uint8_t *>(dbuf);
  a.slot_stride = p->slot_stride;
  a.T = T;
  a.H = p->cfg.hidden;
  a.G = p->G;
  a.K = p->K;
  a.per_token = p->G == 1;
  a.total_slots = (int32_t)p->total_slots;
  a.cached_payload = (int64_t)T * 2 * a.H > moedc::kStreamInputBytes;
  return a;
}

moedc_status combine_impl(const moedc_plan *p, int32_t T, const void *eout, int32_t fmt,
                          const int32_t *slots, const float *topk_w, uint16_t *y,
                          int32_t max_blocks, hipStream_t stream) {
  if (!p) return MOEDC_ERR_INVALID_ARG;
  if (fmt != MOEDC_FMT_BF16 && fmt != MOEDC_FMT_Q8) return MOEDC_ERR_INVALID_ARG;
  if (max_blocks < 1) return MOEDC_ERR_INVALID_ARG;
  if (T < 0 || T > p->cfg.max_tokens) return MOEDC_ERR_SHAPE;
  if (T == 0) return MOEDC_OK;
  if (!eout || !slots || !topk_w || !y) return MOEDC_ERR_INVALID_ARG;
  if (!aligned16(eout) || !aligned16(y) || !aligned4(slots) || !aligned4(topk_w))
    return MOEDC_ERR_ALIGN;
  moedc::CombineArgs a{};
  a.eout = static_cast<const uint8_t *>(eout);
  a.slots = slots;
  a.w = topk_w;
  a.y = y;
  a.eout_stride = fmt == MOEDC_FMT_Q8 ? p->slot_stride : p->combine_stride;
  a.total_slots = (int32_t)p->total_slots;
  a.T = T;
  a.H = p->cfg.hidden;
  a.K = p->K;
  a.fmt = fmt;
  a.per_token = p->G == 1;
  a.max_blocks = max_blocks;
  const hipError_t e = moedc::launch_combine(a, stream);
  return e == hipSuccess ? MOEDC_OK : hip_fail(e);
}

}  // namespace

extern "C" {

moedc_status moedc_route(const moedc_plan *p, int32_t T, const float *logits, int32_t *topk_ids,
                         float *topk_w, int32_t *counts, int32_t *offsets, int32_t *slots,
                         int32_t *dropped, void *ws, hipStream_t stream) {
  const moedc_status st =
      check_route(p, T, logits, topk_ids, topk_w, counts, offsets, slots, dropped, ws);
  if (st != MOEDC_OK) return st;
  const moedc::RouteArgs ra =
      route_args(p, T, logits, topk_ids, topk_w, counts, offsets, slots, dropped, ws);
  return moedc::hip_status(moedc::launch_route_any(ra, stream));
}

moedc_status moedc_dispatch(const moedc_plan *p, int32_t T, const uint16_t *x,
                            const int32_t *slots, void *dbuf, hipStream_t stream) {
  const moedc_status st = check_dispatch(p, T, x, slots, dbuf);
  if (st != MOEDC_OK || T == 0) return st;
  const hipError_t e = moedc::launch_dispatch(dispatch_args(p, T, x, slots, dbuf), stream);
  return e == hipSuccess ? MOEDC_OK : hip_fail(e);
}

moedc_status moedc_route_dispatch(const moedc_plan *p, int32_t T, const float *logits,
                                  const uint16_t *x, int32_t *topk_ids, float *topk_w,
                                  int32_t *counts, int32_t *offsets, int32_t *slots,
                                  int32_t *dropped, void *dbuf, void *ws, hipStream_t stream) {
  moedc_status st =
      check_route(p, T, logits, topk_ids, topk_w, counts, offsets, slots, dropped, ws);
  if (st == MOEDC_OK) st = check_dispatch(p, T, x, slots, dbuf);
  if (st != MOEDC_OK) return st;
  const moedc::RouteArgs ra =
      route_args(p, T, logits, topk_ids, topk_w, counts, offsets, slots, dropped, ws);
  const moedc::DispatchArgs da = dispatch_args(p, T, x, slots, dbuf);
  hipError_t e;
  if (T > 0 && T <= moedc::kFusedMaxTokens) {
    e = moedc::launch_route_dispatch_fused(ra, da, stream);
  } else {
    e = moedc::launch_route(ra, stream);
    if (e == hipSuccess && T > 0) e = moedc::launch_dispatch(da, stream);
  }
  return e == hipSuccess ? MOEDC_OK : hip_fail(e);
}

moedc_status moedc_combine(const moedc_plan *p, int32_t T, const void *eout, int32_t fmt,
                           const int32_t *slots, const float *topk_w, uint16_t *y,
                           hipStream_t stream) {
  return combine_impl(p, T, eout, fmt, slots, topk_w, y, INT32_MAX, stream);
}

moedc_status moedc_combine_limited(const moedc_plan *p, int32_t T, const void *eout, int32_t fmt,
                                   const int32_t *slots, const float *topk_w, uint16_t *y,
                                   int32_t max_workgroups, hipStream_t stream) {
  return combine_impl(p, T, eout, fmt, slots, topk_w, y, max_workgroups, stream);
}

moedc_status moedc_expert_w8a8(const moedc_plan *p, const int32_t *counts, const void *dbuf,
                               const int8_t *weights, const float *w_scale,
                               uint16_t *ebuf, void *ws, hipStream_t stream) {
  return moedc_expert_w8a8_dealt(p, counts, dbuf, weights, w_scale, ebuf, ws, MOEDC_DEAL_LPT,
                                 nullptr, stream);
}

moedc_status moedc_expert_w8a8_dealt(const moedc_plan *p, const int32_t *counts, const void *dbuf,
                                     const int8_t *weights, const float *w_scale, uint16_t *ebuf,
                                     void *ws, int32_t dealing, int32_t *xcd_tiles,
                                     hipStream_t stream) {
  if (!p || !counts || !dbuf || !weights || !w_scale || !ebuf || !ws) return MOEDC_ERR_INVALID_ARG;
  if (dealing != MOEDC_DEAL_LPT && dealing != MOEDC_DEAL_ROUND_ROBIN) return MOEDC_ERR_INVALID_ARG;
  if (!aligned16(dbuf) || !aligned16(weights) || !aligned16(w_scale) || !aligned16(ebuf) ||
      !aligned16(ws) || !aligned4(counts) || !aligned4(xcd_tiles))
    return MOEDC_ERR_ALIGN;
  moedc::GemmArgs a{};
  a.dbuf = static_cast<const uint8_t *>(dbuf);
  a.W = weights;
  a.w_scale = w_scale;
  a.ebuf = ebuf;
  a.counts = counts;
  a.cap = ws_ptr<const int32_t>(ws, p->ws.cap);
  a.capbase = ws_ptr<const int32_t>(ws, p->ws.capbase);
  a.band_pre = ws_ptr<int32_t>(ws, p->ws.band_pre);
  a.band_list = ws_ptr<int32_t>(ws, p->ws.band_list);
  a.band_cnt = ws_ptr<int32_t>(ws, p->ws.band_cnt);
  a.xcd_tiles = xcd_tiles;
  a.dealing = dealing;
  a.slot_stride = p->slot_stride;
  a.H = p->cfg.hidden;
  a.P = p->cfg.num_phys_experts;
  a.ntiles = (p->cfg.hidden + moedc::kGemmChannels - 1) / moedc::kGemmChannels;
  a.steps_per_group = p->cfg.group_size / 128;
  a.nbe = p->gemm_nbe;
  a.Jmax = p->gemm_Jmax;
  // One persistent workgroup per CU: 32 on each of the 8 XCDs.
  const hipError_t e = moedc::launch_expert_gemm(a, 32 * moedc::kXcds, stream);
  return e == hipSuccess ? MOEDC_OK : hip_fail(e);
}

moedc_status moedc_expert_stub(const moedc_plan *p, const int32_t *counts, const void *dbuf,
                               uint16_t *ebuf, void *ws, hipStream_t stream) {
  if (!p || !counts || !dbuf || !ebuf || !ws) return MOEDC_ERR_INVALID_ARG;
  if (!aligned16(dbuf) || !aligned16(ebuf) || !aligned16(ws) || !aligned4(counts))
    return MOEDC_ERR_ALIGN;
  moedc::StubArgs a{};
  a.dbuf = static_cast<const uint8_t *>(dbuf);
  a.ebuf = ebuf;
  a.counts = counts;
  a.cap = ws_ptr<const int32_t>(ws, p->ws.cap);
  a.capbase = ws_ptr<const int32_t>(ws, p->ws.capbase);
  a.slot_stride = p->slot_stride;
  a.ebuf_stride = p->combine_stride;
  a.total_slots = p->total_slots;
  a.H = p->cfg.hidden;
  a.P = p->cfg.num_phys_experts;
  a.per_token = p->G == 1;
  const hipError_t e = moedc::launch_stub(a, stream);
  return e == hipSuccess ? MOEDC_OK : hip_fail(e);
}

const char *moedc_status_string(moedc_status s) {
  switch (s) {
    case MOEDC_OK: return "ok";
    case MOEDC_ERR_INVALID_ARG: return "invalid argument";
    case MOEDC_ERR_SHAPE: return "shape outside the plan";
    case MOEDC_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case MOEDC_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOEDC_ERR_HIP: return "HIP runtime error";
    case MOEDC_ERR_NO_MEMORY: return "host allocation failed";
  }
  return "unknown status";
}

int32_t moedc_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
