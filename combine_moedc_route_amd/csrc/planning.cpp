// planning.cpp -- host-side load balancing for expert-major work:
// load-proportional redundant-expert placement and a longest-processing-
// time-first (LPT) list scheduler with a per-group fan-out cap.
//
// "StrataCL 深度技术分析", section 3.5 (workload-balanced core partitioning):
// traffic per peer is cut into units whose cost depends on size and path,
// and units are assigned to cores to minimise the predicted straggler
// (min-max load) under a cap on how many cores may target one peer, with an
// LPT-style list scheduler as the approximation of this NP-hard problem.
// "CloudMatrix384 ...", section "Decode Phase": redundant copies of experts
// balance load.  Here units are any expert-major work items (an expert's
// token block, a GEMM tile row) and workers are workgroups or devices.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <numeric>
#include <vector>

#include "../../include/moedc.h"

namespace {

bool finite_nonneg(const double *v, int32_t n) {
  for (int32_t i = 0; i < n; ++i)
    if (!(v[i] >= 0.0) || !std::isfinite(v[i])) return false;
  return true;
}

}  // namespace

extern "C" {

moedc_status moedc_place_replicas(int32_t num_logical, const double *load,
                                  int32_t num_redundant, int32_t max_replicas,
                                  int32_t *replica_table) {
  if (num_logical < 1 || num_redundant < 0 || max_replicas < 1 || !load || !replica_table)
    return MOEDC_ERR_INVALID_ARG;
  if ((int64_t)num_logical * (max_replicas - 1) < num_redundant) return MOEDC_ERR_INVALID_ARG;
  if (!finite_nonneg(load, num_logical)) return MOEDC_ERR_INVALID_ARG;
  const int32_t E = num_logical, R = max_replicas;
  std::vector<int32_t> r((size_t)E, 1);
  for (int64_t i = 0; i < (int64_t)E * R; ++i) replica_table[i] = -1;
  for (int32_t e = 0; e < E; ++e) replica_table[(int64_t)e * R] = e;
  // Each extra copy goes to the expert with the largest load per copy
  // (ties to the lower id) among those below the cap.  Repeatedly lowering
  // the current maximum of load/copies is optimal for the min-max objective.
  for (int32_t i = 0; i < num_redundant; ++i) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e) {
      if (r[(size_t)e] >= R) continue;
      if (best < 0 || load[e] * r[(size_t)best] > load[best] * r[(size_t)e]) best = e;
    }
    replica_table[(int64_t)best * R + r[(size_t)best]] = E + i;
    ++r[(size_t)best];
  }
  return MOEDC_OK;
}

moedc_status moedc_lpt_partition(int32_t num_units, const double *cost, const int32_t *group,
                                 int32_t num_groups, int32_t num_workers, int32_t fanout_cap,
                                 int32_t *assign, double *makespan) {
  if (num_units < 0 || num_workers < 1 || !assign || !makespan) return MOEDC_ERR_INVALID_ARG;
  if (num_units > 0 && !cost) return MOEDC_ERR_INVALID_ARG;
  if (!finite_nonneg(cost, num_units)) return MOEDC_ERR_INVALID_ARG;
  const bool capped = fanout_cap > 0;
  if (capped && (!group || num_groups < 1)) return MOEDC_ERR_INVALID_ARG;
  if (capped)
    for (int32_t u = 0; u < num_units; ++u)
      if (group[u] < 0 || group[u] >= num_groups) return MOEDC_ERR_INVALID_ARG;
  // Longest first; equal costs keep unit order.
  std::vector<int32_t> order((size_t)num_units);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t x, int32_t y) { return cost[x] > cost[y]; });
  std::vector<double> load((size_t)num_workers, 0.0);
  // holds[g * W + w]: worker w already serves group g; users[g]: how many.
  std::vector<char> holds(capped ? (size_t)num_groups * num_workers : 0, 0);
  std::vector<int32_t> users(capped ? (size_t)num_groups : 0, 0);
  for (int32_t u : order) {
    const int32_t g = capped ? group[u] : 0;
    const bool open = !capped || users[(size_t)g] < fanout_cap;
    int32_t best = -1;
    for (int32_t w = 0; w < num_workers; ++w) {
      if (!open && !holds[(size_t)g * num_workers + w]) continue;
      if (best < 0 || load[(size_t)w] < load[(size_t)best]) best = w;
    }
    assign[u] = best;
    load[(size_t)best] += cost[u];
    if (capped && !holds[(size_t)g * num_workers + best]) {
      holds[(size_t)g * num_workers + best] = 1;
      ++users[(size_t)g];
    }
  }
  double m = 0.0;
  for (double l : load) m = l > m ? l : m;
  *makespan = m;
  return MOEDC_OK;
}

}  // extern "C"
