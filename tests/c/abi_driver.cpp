// abi_driver.cpp -- drives libmoedc through its C ABI alone (hipMalloc'd
// buffers, no Python, no torch, no oracle): route -> dispatch -> stand-in
// expert -> combine on a small seeded layer, then checks the invariants the
// header promises: counts sum to T*K, offsets are their exclusive scan,
// every kept slot lies in its expert's window in ascending token order and
// none repeats, drops match the capacities, gates are normalised, dispatched
// payload bytes are within +-127 with finite scales, every combine output is
// finite, and invalid arguments are refused before any launch.  Prints
// "abi driver ok" and exits 0 on success.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "moedc.h"

#define CHECK(cond, ...)                         \
  do {                                           \
    if (!(cond)) {                               \
      std::fprintf(stderr, "FAIL: " __VA_ARGS__); \
      std::fprintf(stderr, "\n");                \
      return 1;                                  \
    }                                            \
  } while (0)
#define HIPCK(x) CHECK((x) == hipSuccess, "%s", #x)
#define OK(x) CHECK((x) == MOEDC_OK, "%s -> %s", #x, moedc_status_string(x))

namespace {

uint32_t lcg(uint32_t &s) {
  s = s * 1664525u + 1013904223u;
  return s >> 8;
}

float bf16_to_float(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

}  // namespace

int main() {
  const int T = 300, H = 640, E = 16, KR = 4, K = KR;
  std::vector<int32_t> cap(E, 90);  // mean T*K/E = 75: a few experts overflow
  moedc_config c{};
  c.max_tokens = T;
  c.hidden = H;
  c.group_size = 128;
  c.num_logical_experts = E;
  c.num_phys_experts = E;
  c.top_k = KR;
  c.num_shared = 0;
  c.score_fn = MOEDC_SCORE_SIGMOID_NORM;
  c.max_replicas = 1;
  c.capacity = cap.data();
  c.replica_table = nullptr;

  moedc_plan *plan = nullptr;
  OK(moedc_plan_create(&c, &plan));
  moedc_sizes sz{};
  OK(moedc_plan_sizes(plan, &sz));
  CHECK(sz.k == K && sz.num_groups == H / 128, "sizes");
  CHECK(sz.slot_stride == 1024, "slot stride %lld", (long long)sz.slot_stride);

  // Seeded inputs: skewed logits (expert e favoured by e % 5), BF16 rows.
  uint32_t seed = 12345;
  std::vector<float> logits((size_t)T * E);
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e)
      logits[(size_t)t * E + e] = (float)(lcg(seed) % 1000) / 1000.0f + 0.3f * (float)(e % 5);
  std::vector<uint16_t> x((size_t)T * H);
  for (auto &v : x) {
    const float f = ((float)(lcg(seed) % 2001) - 1000.0f) / 250.0f;
    uint32_t u;
    std::memcpy(&u, &f, 4);
    v = (uint16_t)(u >> 16);
  }

  float *d_logits, *d_w;
  uint16_t *d_x, *d_cbuf, *d_y;
  int32_t *d_ids, *d_counts, *d_offsets, *d_slots, *d_dropped;
  void *d_ws, *d_dbuf;
  HIPCK(hipMalloc(&d_logits, sizeof(float) * T * E));
  HIPCK(hipMalloc(&d_x, sizeof(uint16_t) * T * H));
  HIPCK(hipMalloc(&d_ids, sizeof(int32_t) * T * K));
  HIPCK(hipMalloc(&d_w, sizeof(float) * T * K));
  HIPCK(hipMalloc(&d_counts, sizeof(int32_t) * E));
  HIPCK(hipMalloc(&d_offsets, sizeof(int32_t) * (E + 1)));
  HIPCK(hipMalloc(&d_slots, sizeof(int32_t) * T * K));
  HIPCK(hipMalloc(&d_dropped, sizeof(int32_t)));
  HIPCK(hipMalloc(&d_ws, (size_t)sz.workspace_bytes));
  HIPCK(hipMalloc(&d_dbuf, (size_t)sz.dispatch_buf_bytes));
  HIPCK(hipMalloc(&d_cbuf, (size_t)sz.combine_buf_bytes));
  HIPCK(hipMalloc(&d_y, sizeof(uint16_t) * T * H));
  HIPCK(hipMemcpy(d_logits, logits.data(), sizeof(float) * T * E, hipMemcpyHostToDevice));
  HIPCK(hipMemcpy(d_x, x.data(), sizeof(uint16_t) * T * H, hipMemcpyHostToDevice));

  hipStream_t st;
  HIPCK(hipStreamCreate(&st));
  OK(moedc_plan_bind_workspace(plan, d_ws, st));
  OK(moedc_route(plan, T, d_logits, d_ids, d_w, d_counts, d_offsets, d_slots, d_dropped, d_ws, st));
  OK(moedc_dispatch(plan, T, d_x, d_slots, d_dbuf, st));
  OK(moedc_expert_stub(plan, d_counts, d_dbuf, d_cbuf, d_ws, st));
  OK(moedc_combine(plan, T, d_cbuf, MOEDC_FMT_BF16, d_slots, d_w, d_y, st));
  HIPCK(hipStreamSynchronize(st));

  std::vector<int32_t> ids((size_t)T * K), counts(E), offsets(E + 1), slots((size_t)T * K);
  std::vector<float> w((size_t)T * K);
  int32_t dropped = -1;
  HIPCK(hipMemcpy(ids.data(), d_ids, sizeof(int32_t) * T * K, hipMemcpyDeviceToHost));
  HIPCK(hipMemcpy(w.data(), d_w, sizeof(float) * T * K, hipMemcpyDeviceToHost));
  HIPCK(hipMemcpy(counts.data(), d_counts, sizeof(int32_t) * E, hipMemcpyDeviceToHost));
  HIPCK(hipMemcpy(offsets.data(), d_offsets, sizeof(int32_t) * (E + 1), hipMemcpyDeviceToHost));
  HIPCK(hipMemcpy(slots.data(), d_slots, sizeof(int32_t) * T * K, hipMemcpyDeviceToHost));
  HIPCK(hipMemcpy(&dropped, d_dropped, sizeof(int32_t), hipMemcpyDeviceToHost));

  // Routing invariants.
  std::vector<int> hist(E, 0);
  for (int t = 0; t < T; ++t) {
    float wsum = 0.0f;
    for (int j = 0; j < K; ++j) {
      const int e = ids[(size_t)t * K + j];
      CHECK(e >= 0 && e < E, "id %d", e);
      for (int i = 0; i < j; ++i) CHECK(ids[(size_t)t * K + i] != e, "repeated pick, token %d", t);
      const float g = w[(size_t)t * K + j];
      CHECK(g > 0.0f && g <= 1.0f, "gate %g", g);
      wsum += g;
      ++hist[e];
    }
    CHECK(std::fabs(wsum - 1.0f) < 1e-5f, "gates of token %d sum to %g", t, wsum);
  }
  int total = 0, drops = 0;
  for (int e = 0; e < E; ++e) {
    CHECK(counts[e] == hist[e], "counts[%d]", e);
    CHECK(offsets[e] == total, "offsets[%d]", e);
    total += counts[e];
    drops += counts[e] > cap[e] ? counts[e] - cap[e] : 0;
  }
  CHECK(offsets[E] == total && total == T * K, "sum of counts %d", total);
  CHECK(dropped == drops, "dropped %d != %d", dropped, drops);

  // Slots: expert e's kept entries fill [base_e, base_e + min(count, cap))
  // in ascending token order; the rest are -1.
  std::vector<int> next(E, 0), base(E, 0);
  for (int e = 1; e < E; ++e) base[e] = base[e - 1] + cap[e - 1];
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < K; ++j) {
      const int e = ids[(size_t)t * K + j], s = slots[(size_t)t * K + j];
      const int r = next[e]++;
      CHECK(s == (r < cap[e] ? base[e] + r : -1), "slot of token %d entry %d", t, j);
    }

  // Dispatched bytes: payload within +-127, finite non-negative scales.
  std::vector<uint8_t> dbuf((size_t)sz.dispatch_buf_bytes);
  HIPCK(hipMemcpy(dbuf.data(), d_dbuf, dbuf.size(), hipMemcpyDeviceToHost));
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < K; ++j) {
      const int s = slots[(size_t)t * K + j];
      if (s < 0) continue;
      const uint8_t *row = dbuf.data() + (size_t)s * sz.slot_stride;
      for (int i = 0; i < H; ++i) CHECK((int8_t)row[i] != -128, "INT8 -128 in slot %d", s);
      for (int g = 0; g < H / 128; ++g) {
        float sc;
        std::memcpy(&sc, row + H + 4 * g, 4);
        CHECK(std::isfinite(sc) && sc >= 0.0f, "scale %g", sc);
      }
    }

  // Combine output: finite everywhere.
  std::vector<uint16_t> y((size_t)T * H);
  HIPCK(hipMemcpy(y.data(), d_y, sizeof(uint16_t) * T * H, hipMemcpyDeviceToHost));
  for (uint16_t v : y) CHECK(std::isfinite(bf16_to_float(v)), "non-finite output");

  // Invalid arguments are refused on the host, before any launch.
  CHECK(moedc_route(plan, T, nullptr, d_ids, d_w, d_counts, d_offsets, d_slots, d_dropped, d_ws,
                    st) == MOEDC_ERR_INVALID_ARG, "NULL logits accepted");
  CHECK(moedc_dispatch(plan, T + 1, d_x, d_slots, d_dbuf, st) == MOEDC_ERR_SHAPE,
        "token count above the plan accepted");
  CHECK(moedc_combine(plan, T, (const char *)d_cbuf + 4, MOEDC_FMT_BF16, d_slots, d_w, d_y,
                      st) == MOEDC_ERR_ALIGN, "misaligned expert outputs accepted");
  CHECK(moedc_combine(plan, T, d_cbuf, 7, d_slots, d_w, d_y, st) == MOEDC_ERR_INVALID_ARG,
        "bad format accepted");
  HIPCK(hipStreamSynchronize(st));

  HIPCK(hipStreamDestroy(st));
  for (void *ptr : {(void *)d_logits, (void *)d_x, (void *)d_ids, (void *)d_w, (void *)d_counts,
                    (void *)d_offsets, (void *)d_slots, (void *)d_dropped, d_ws, d_dbuf,
                    (void *)d_cbuf, (void *)d_y})
    HIPCK(hipFree(ptr));
  moedc_plan_destroy(plan);
  std::printf("abi driver ok: %d tokens, %d dropped\n", T, dropped);
  return 0;
}
