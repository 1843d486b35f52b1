// sanitize_host.cpp -- the library's host code and the CPU oracle under
// AddressSanitizer and UndefinedBehaviorSanitizer (built with g++ by
// tests/test_host_sanitizers.py; no GPU, no HIP runtime).
//
// host.cpp (plan creation, validation, sizing, workspace layout and kernel
// argument set-up of every C entry point) and planning.cpp (replica
// placement, LPT partitioning) are linked against the stand-ins below:
//  - hipMemcpyAsync copies host to "device" for real, into host memory that
//    plays the workspace, so a wrong size or offset is an ASan report;
//  - each kernel launcher checks the arguments it would launch with: the
//    workspace pointers and the extents the kernels read or write lie
//    inside the workspace, shapes match the plan.
// Random layer descriptions (valid and invalid), random calls with aligned,
// misaligned and null pointers, random planner inputs, and random small
// layers through every oracle function on exactly sized host buffers.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "../../combine_moedc_route_amd/csrc/internal.hpp"
#include "../../include/moedc.h"
#include "../../oracle/moedc_oracle.h"

namespace {

// The workspace of the call in flight (host memory standing in for it).
const char *g_ws = nullptr;
int64_t g_ws_bytes = 0;
const moedc_plan *g_plan = nullptr;
long g_launches = 0;

void fail(const char *what) {
  std::fprintf(stderr, "sanitize_host: %s\n", what);
  std::abort();
}

void in_ws(const void *p, int64_t bytes, const char *what) {
  const char *c = static_cast<const char *>(p);
  if (!g_ws || c < g_ws || bytes < 0 || c + bytes > g_ws + g_ws_bytes) fail(what);
}

}  // namespace

extern "C" hipError_t hipMemcpyAsync(void *dst, const void *src, size_t n, hipMemcpyKind kind,
                                     hipStream_t) {
  if (kind != hipMemcpyHostToDevice) fail("unexpected copy kind");
  in_ws(dst, (int64_t)n, "table upload outside the workspace");
  std::memcpy(dst, src, n);
  return hipSuccess;
}

namespace moedc {

static void check_route(const RouteArgs &a) {
  const moedc_config &c = g_plan->cfg;
  if (a.T < 1 || a.T > c.max_tokens) fail("route: token count");
  if (a.E != c.num_logical_experts || a.P != c.num_phys_experts || a.K != g_plan->K)
    fail("route: shape");
  in_ws(a.cap, 4 * (int64_t)a.P, "route: capacities");
  in_ws(a.capbase, 4 * (int64_t)a.P, "route: bases");
  in_ws(a.rep_count, 4 * (int64_t)a.E, "route: copy counts");
  in_ws(a.rep_table, 4 * (int64_t)a.E * a.R, "route: replica table");
  // the table image uploaded at bind: the capacities must read back
  for (int p = 0; p < a.P; ++p)
    if (a.cap[p] != c.capacity[p]) fail("route: capacity image");
  const int64_t nblk = (a.T + kRouteTokens - 1) / kRouteTokens;
  if (a.T > kFusedMaxTokens) in_ws(a.block_counts, 4 * nblk * a.P, "route: block counts");
}

hipError_t launch_route(const RouteArgs &a, hipStream_t) {
  ++g_launches;
  if (a.T == 0) return hipSuccess;
  check_route(a);
  return hipSuccess;
}
hipError_t launch_route_small(const RouteArgs &a, hipStream_t) {
  ++g_launches;
  check_route(a);
  if (a.T > kFusedMaxTokens) fail("small route: batch too large");
  return hipSuccess;
}
hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t) {
  ++g_launches;
  if (a.T < 1 || a.H != g_plan->cfg.hidden || a.K != g_plan->K || a.G != g_plan->G)
    fail("dispatch: shape");
  if (a.slot_stride < a.H + 4 * ((a.G + 31) / 32 * 32)) fail("dispatch: slot too short");
  if (a.total_slots != g_plan->total_slots) fail("dispatch: total slots");
  return hipSuccess;
}
hipError_t launch_combine(const CombineArgs &a, hipStream_t) {
  ++g_launches;
  if (a.T < 1 || a.max_blocks < 1 || a.H != g_plan->cfg.hidden || a.K != g_plan->K)
    fail("combine: shape");
  if (a.eout_stride != (a.fmt == MOEDC_FMT_Q8 ? g_plan->slot_stride : 2 * (int64_t)a.H))
    fail("combine: row stride");
  return hipSuccess;
}
hipError_t launch_stub(const StubArgs &a, hipStream_t) {
  ++g_launches;
  in_ws(a.cap, 4 * (int64_t)a.P, "stub: capacities");
  in_ws(a.capbase, 4 * (int64_t)a.P, "stub: bases");
  return hipSuccess;
}
hipError_t launch_route_dispatch_fused(const RouteArgs &ra, const DispatchArgs &da,
                                       hipStream_t s) {
  if (ra.T > kFusedMaxTokens) fail("fused route: batch too large");
  const hipError_t e = launch_route_small(ra, s);
  return e == hipSuccess ? launch_dispatch(da, s) : e;
}
hipError_t launch_expert_gemm(const GemmArgs &a, int grid, hipStream_t) {
  ++g_launches;
  if (grid % kXcds) fail("gemm: grid");
  if (a.Jmax != a.P * a.nbe || a.Jmax > kMaxBands) fail("gemm: band count");
  in_ws(a.cap, 4 * (int64_t)a.P, "gemm: capacities");
  in_ws(a.capbase, 4 * (int64_t)a.P, "gemm: bases");
  in_ws(a.band_pre, 4 * (int64_t)kXcds * (a.Jmax + 1), "gemm: band prefixes");
  in_ws(a.band_list, 4 * (int64_t)kXcds * a.Jmax, "gemm: band lists");
  in_ws(a.band_cnt, 4 * (int64_t)kXcds, "gemm: band counts");
  if (a.dealing != MOEDC_DEAL_LPT && a.dealing != MOEDC_DEAL_ROUND_ROBIN) fail("gemm: dealing");
  return hipSuccess;
}

}  // namespace moedc

namespace {

std::mt19937_64 rng(12345);
int ri(int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); }  // inclusive

// A fake device address: 16-aligned, misaligned or null.
void *fake(int mode) {
  static char arena[64];
  char *base = reinterpret_cast<char *>((reinterpret_cast<uintptr_t>(arena) + 15) & ~15ull);
  return mode == 0 ? nullptr : mode == 1 ? static_cast<void *>(base + 1) : static_cast<void *>(base);
}

bool valid_status(moedc_status s) { return s >= MOEDC_OK && s <= MOEDC_ERR_NO_MEMORY; }

void one_layer() {
  moedc_config c{};
  c.max_tokens = ri(-2, 3000);
  c.hidden = 128 * ri(ri(0, 9) == 0 ? 0 : 1, 9) + (ri(0, 15) == 0 ? 64 : 0);
  c.group_size = ri(0, 5) == 0 ? 64 : (ri(0, 1) ? 128 : c.hidden);
  c.num_logical_experts = ri(ri(0, 9) == 0 ? 0 : 1, 70);
  const int extra = ri(0, 12);
  c.num_shared = ri(0, 4) == 0 ? ri(0, 2) : 0;
  c.num_phys_experts = c.num_logical_experts + extra + c.num_shared + (ri(0, 9) == 0 ? -1 : 0);
  c.top_k = ri(0, 9) == 0 ? ri(0, 17) : ri(1, std::max(1, std::min(16 - c.num_shared, c.num_logical_experts)));
  c.score_fn = ri(0, 8) == 0 ? 7 : ri(0, 1);
  c.max_replicas = ri(0, 9) == 0 ? ri(0, 9) : ri(1, 4);
  std::vector<int32_t> cap(std::max(c.num_phys_experts, 1));
  for (auto &x : cap) x = ri(0, 9) == 0 ? -1 : ri(0, 400);
  c.capacity = ri(0, 30) == 0 ? nullptr : cap.data();
  std::vector<int32_t> table;
  if (c.max_replicas > 1 && c.num_logical_experts > 0 && ri(0, 3)) {
    const int E = c.num_logical_experts, R = c.max_replicas;
    table.assign((size_t)E * R, -1);
    int next = E;
    const int routed = c.num_phys_experts - c.num_shared;
    for (int e = 0; e < E; ++e) {
      table[(size_t)e * R] = e;
      for (int r = 1; r < R && next < routed && ri(0, 3) == 0; ++r) table[(size_t)e * R + r] = next++;
    }
    if (ri(0, 15) == 0) table[(size_t)ri(0, E - 1) * R] = routed + 3;  // invalid id
    c.replica_table = table.data();
  }
  moedc_plan *plan = nullptr;
  const moedc_status st = moedc_plan_create(&c, &plan);
  if (!valid_status(st)) fail("plan_create: status");
  if (st != MOEDC_OK) {
    if (plan) fail("plan_create: plan on error");
    return;
  }
  moedc_sizes sz{};
  if (moedc_plan_sizes(plan, &sz) != MOEDC_OK) fail("plan_sizes");
  std::vector<char> wsmem((size_t)sz.workspace_bytes + 32);
  char *ws = reinterpret_cast<char *>((reinterpret_cast<uintptr_t>(wsmem.data()) + 15) & ~15ull);
  g_ws = ws;
  g_ws_bytes = sz.workspace_bytes;
  g_plan = plan;
  if (moedc_plan_bind_workspace(plan, ws, nullptr) != MOEDC_OK) fail("bind");
  for (int call = 0; call < 8; ++call) {
    const int T = ri(-1, c.max_tokens + 1);
    const int m = ri(0, 9) == 0 ? ri(0, 1) : 2;  // mostly good pointers
    void *p = fake(m), *q = fake(2);
    moedc_status s;
    s = moedc_route(plan, T, (float *)p, (int32_t *)q, (float *)q, (int32_t *)q, (int32_t *)q,
                    (int32_t *)q, (int32_t *)q, ws, nullptr);
    if (!valid_status(s)) fail("route status");
    s = moedc_route_dispatch(plan, T, (float *)q, (uint16_t *)p, (int32_t *)q, (float *)q,
                             (int32_t *)q, (int32_t *)q, (int32_t *)q, (int32_t *)q, q, ws,
                             nullptr);
    if (!valid_status(s)) fail("route_dispatch status");
    s = moedc_dispatch(plan, T, (uint16_t *)p, (int32_t *)q, q, nullptr);
    if (!valid_status(s)) fail("dispatch status");
    s = moedc_combine_limited(plan, T, p, ri(0, 2), (int32_t *)q, (float *)q, (uint16_t *)q,
                              ri(-1, 40), nullptr);
    if (!valid_status(s)) fail("combine status");
    s = moedc_expert_w8a8_dealt(plan, (int32_t *)q, q, (int8_t *)p, (float *)q, (uint16_t *)q,
                                ws, ri(0, 2), ri(0, 1) ? (int32_t *)q : nullptr, nullptr);
    if (!valid_status(s)) fail("expert status");
    s = moedc_expert_stub(plan, (int32_t *)q, p, (uint16_t *)q, ws, nullptr);
    if (!valid_status(s)) fail("stub status");
  }
  g_ws = nullptr;
  moedc_plan_destroy(plan);
}

void one_planning() {
  const int E = ri(1, 40), R = ri(1, 8);
  std::vector<double> load(E);
  for (auto &x : load) x = ri(0, 5) == 0 ? 0.0 : ri(0, 100000) / 7.0;
  if (ri(0, 20) == 0) load[ri(0, E - 1)] = -1.0;
  const int N = ri(0, E * (R - 1) + 2);
  std::vector<int32_t> table((size_t)E * R);
  const moedc_status s = moedc_place_replicas(E, load.data(), N, R, table.data());
  if (s == MOEDC_OK)
    for (int32_t v : table)
      if (v < -1 || v >= E + N) fail("place_replicas: id out of range");
  const int U = ri(0, 200), G = ri(1, 12), W = ri(1, 16);
  std::vector<double> cost(U);
  std::vector<int32_t> grp(U), assign(U);
  for (int u = 0; u < U; ++u) {
    cost[u] = ri(0, 1000) / 3.0;
    grp[u] = ri(0, G - 1);
  }
  double ms = 0.0;
  const moedc_status s2 = moedc_lpt_partition(U, cost.data(), grp.data(), G, W, ri(0, 3),
                                              assign.data(), &ms);
  if (s2 == MOEDC_OK)
    for (int u = 0; u < U; ++u)
      if (assign[u] < 0 || assign[u] >= W) fail("lpt: worker out of range");
}

void one_oracle_layer() {
  const int E = ri(1, 24), KR = ri(1, std::min(E, 6)), shared = ri(0, 1);
  const int R = ri(1, 3), H = 128 * ri(1, 3), gs = ri(0, 1) ? 128 : H;
  const int T = ri(0, 150);
  std::vector<int32_t> table((size_t)E * R, -1);
  int next = E;
  for (int e = 0; e < E; ++e) {
    table[(size_t)e * R] = e;
    for (int r = 1; r < R && ri(0, 2) == 0; ++r) table[(size_t)e * R + r] = next++;
  }
  const int P = next + shared;
  std::vector<int32_t> cap(P);
  for (auto &x : cap) x = ri(0, 2 * T / std::max(1, E) + 4);
  if (shared) cap[P - 1] = T;
  orc_cfg c{H, gs, E, P, KR, shared, ri(0, 1), R, table.data(), cap.data()};
  if (orc_check_cfg(&c) != 0) fail("oracle config");
  const int K = KR + shared;
  std::vector<float> logits((size_t)T * E);
  for (auto &x : logits) x = (float)ri(-1000, 1000) / (float)ri(1, 300);
  std::vector<int32_t> ids((size_t)T * K), counts(P), offsets(P + 1), slots((size_t)T * K), dr(1);
  std::vector<float> w((size_t)T * K);
  if (orc_route(&c, T, logits.data(), ids.data(), w.data(), counts.data(), offsets.data(),
                slots.data(), dr.data()) != 0)
    fail("orc_route");
  int64_t S = 0;
  for (int x : cap) S += x;
  const int G = H / gs;
  const int64_t sd = (H + 4 * G + 511) / 512 * 512;
  std::vector<uint16_t> x((size_t)T * H);
  for (auto &v : x) v = (uint16_t)(ri(0, 0xFFFF) & 0xBFFF);  // finite BF16 values
  std::vector<uint8_t> dbuf((size_t)S * sd);
  if (orc_dispatch(&c, T, x.data(), slots.data(), dbuf.data(), sd) != 0) fail("orc_dispatch");
  std::vector<uint16_t> ebuf((size_t)S * H), y((size_t)T * H);
  if (orc_expert_stub(&c, counts.data(), dbuf.data(), sd, ebuf.data(), 2 * H) != 0)
    fail("orc_expert_stub");
  if (orc_combine(&c, T, ebuf.data(), ORC_FMT_BF16, 2 * H, slots.data(), w.data(), y.data()) != 0)
    fail("orc_combine bf16");
  if (orc_combine(&c, T, dbuf.data(), ORC_FMT_Q8, sd, slots.data(), w.data(), y.data()) != 0)
    fail("orc_combine q8");
  if (ri(0, 4) == 0 && H <= 256) {
    std::vector<int8_t> Wt((size_t)P * H * H);
    for (auto &v : Wt) v = (int8_t)ri(-127, 127);
    std::vector<float> wsc((size_t)P * H, 0.01f);
    if (orc_expert_w8a8(&c, counts.data(), dbuf.data(), sd, Wt.data(), wsc.data(), ebuf.data(),
                        2 * H) != 0)
      fail("orc_expert_w8a8");
  }
}

}  // namespace

int main(int argc, char **argv) {
  const int n = argc > 1 ? std::atoi(argv[1]) : 2000;
  for (int i = 0; i < n; ++i) one_layer();
  for (int i = 0; i < n; ++i) one_planning();
  for (int i = 0; i < n / 4; ++i) one_oracle_layer();
  std::printf("sanitize_host ok: %d layer descriptions, %ld launches checked, %d planner "
              "calls, %d oracle layers\n", n, g_launches, 2 * n, n / 4);
  return 0;
}
