// abi_driver.cpp -- drives libmoedc through its C ABI alone (hipMalloc'd
// buffers, no Python, no torch, no oracle).  For each of a few seeded
// layers -- 128-value scales without a shared expert, one scale per token
// with a shared expert and a replica table, a one-launch decode batch with
// softmax gates -- it runs route -> dispatch -> stand-in expert -> combine,
// and moedc_route_dispatch on the same inputs, then checks the invariants
// the header promises: counts sum to T*K, offsets are their exclusive scan,
// every kept slot lies in its expert's window in ascending token order and
// none repeats, replicated experts use copy t mod r, the shared expert is
// the last entry with gate 1, drops match the capacities, routed gates are
// normalised, dispatched payload bytes are within +-127 with finite scales
// and zero padding after them, the fused call writes the same outputs and
// bytes, every combine output is finite, and invalid arguments are refused
// before any launch.  Prints "abi driver ok" and exits 0 on success.
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

struct Layer {
  const char *name;
  int T, H, group, E, KR, shared, score_fn;
  int R;                       // replica table columns (1: no table)
  std::vector<int32_t> table;  // [E][R], -1 padded; empty: identity
  std::vector<int32_t> cap;    // [P]
  uint32_t seed;
};

// Device buffers of one route + dispatch + combine pass.
struct Bufs {
  float *logits = nullptr, *w = nullptr;
  uint16_t *x = nullptr, *cbuf = nullptr, *y = nullptr;
  int32_t *ids = nullptr, *counts = nullptr, *offsets = nullptr, *slots = nullptr,
          *dropped = nullptr;
  void *ws = nullptr, *dbuf = nullptr;
};

int run_layer(const Layer &L) {
  const int T = L.T, H = L.H, E = L.E, P = (int)L.cap.size(), K = L.KR + L.shared;
  const int G = H / L.group;
  moedc_config c{};
  c.max_tokens = T;
  c.hidden = H;
  c.group_size = L.group;
  c.num_logical_experts = E;
  c.num_phys_experts = P;
  c.top_k = L.KR;
  c.num_shared = L.shared;
  c.score_fn = L.score_fn;
  c.max_replicas = L.R;
  c.capacity = L.cap.data();
  c.replica_table = L.table.empty() ? nullptr : L.table.data();

  moedc_plan *plan = nullptr;
  OK(moedc_plan_create(&c, &plan));
  moedc_sizes sz{};
  OK(moedc_plan_sizes(plan, &sz));
  CHECK(sz.k == K && sz.num_groups == G, "%s: sizes", L.name);
  const int scale_end = H + 4 * ((G + 31) / 32 * 32);  // scales + zero padding
  CHECK(scale_end % 128 == 0 && scale_end <= sz.slot_stride, "%s: slot layout", L.name);

  // Seeded inputs: skewed logits (expert e favoured by e % 5), BF16 rows.
  uint32_t seed = L.seed;
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

  Bufs b, f;  // two-step path, fused path
  for (Bufs *q : {&b, &f}) {
    HIPCK(hipMalloc(&q->ids, sizeof(int32_t) * T * K));
    HIPCK(hipMalloc(&q->w, sizeof(float) * T * K));
    HIPCK(hipMalloc(&q->counts, sizeof(int32_t) * P));
    HIPCK(hipMalloc(&q->offsets, sizeof(int32_t) * (P + 1)));
    HIPCK(hipMalloc(&q->slots, sizeof(int32_t) * T * K));
    HIPCK(hipMalloc(&q->dropped, sizeof(int32_t)));
    HIPCK(hipMalloc(&q->ws, (size_t)sz.workspace_bytes));
    HIPCK(hipMalloc(&q->dbuf, (size_t)sz.dispatch_buf_bytes));
    HIPCK(hipMemset(q->dbuf, 0xA5, (size_t)sz.dispatch_buf_bytes));
  }
  HIPCK(hipMalloc(&b.logits, sizeof(float) * T * E));
  HIPCK(hipMalloc(&b.x, sizeof(uint16_t) * T * H));
  HIPCK(hipMalloc(&b.cbuf, (size_t)sz.combine_buf_bytes));
  HIPCK(hipMalloc(&b.y, sizeof(uint16_t) * T * H));
  HIPCK(hipMemcpy(b.logits, logits.data(), sizeof(float) * T * E, hipMemcpyHostToDevice));
  HIPCK(hipMemcpy(b.x, x.data(), sizeof(uint16_t) * T * H, hipMemcpyHostToDevice));

  hipStream_t st;
  HIPCK(hipStreamCreate(&st));
  OK(moedc_plan_bind_workspace(plan, b.ws, st));
  OK(moedc_plan_bind_workspace(plan, f.ws, st));
  OK(moedc_route(plan, T, b.logits, b.ids, b.w, b.counts, b.offsets, b.slots, b.dropped, b.ws, st));
  OK(moedc_dispatch(plan, T, b.x, b.slots, b.dbuf, st));
  OK(moedc_expert_stub(plan, b.counts, b.dbuf, b.cbuf, b.ws, st));
  OK(moedc_combine(plan, T, b.cbuf, MOEDC_FMT_BF16, b.slots, b.w, b.y, st));
  OK(moedc_route_dispatch(plan, T, b.logits, b.x, f.ids, f.w, f.counts, f.offsets, f.slots,
                          f.dropped, f.dbuf, f.ws, st));
  HIPCK(hipStreamSynchronize(st));

  std::vector<int32_t> ids((size_t)T * K), counts(P), offsets(P + 1), slots((size_t)T * K);
  std::vector<float> w((size_t)T * K);
  int32_t dropped = -1;
  HIPCK(hipMemcpy(ids.data(), b.ids, sizeof(int32_t) * T * K, hipMemcpyDeviceToHost));
  HIPCK(hipMemcpy(w.data(), b.w, sizeof(float) * T * K, hipMemcpyDeviceToHost));
  HIPCK(hipMemcpy(counts.data(), b.counts, sizeof(int32_t) * P, hipMemcpyDeviceToHost));
  HIPCK(hipMemcpy(offsets.data(), b.offsets, sizeof(int32_t) * (P + 1), hipMemcpyDeviceToHost));
  HIPCK(hipMemcpy(slots.data(), b.slots, sizeof(int32_t) * T * K, hipMemcpyDeviceToHost));
  HIPCK(hipMemcpy(&dropped, b.dropped, sizeof(int32_t), hipMemcpyDeviceToHost));

  // Which logical expert and copy each physical id is (routed ids only).
  std::vector<int> owner(P, -1), copy(P, -1), ncopies(E, 1);
  for (int e = 0; e < E; ++e) {
    if (L.table.empty()) {
      owner[e] = e;
      copy[e] = 0;
      continue;
    }
    int r = 0;
    while (r < L.R && L.table[(size_t)e * L.R + r] >= 0) {
      owner[L.table[(size_t)e * L.R + r]] = e;
      copy[L.table[(size_t)e * L.R + r]] = r;
      ++r;
    }
    ncopies[e] = r;
  }

  // Routing invariants.
  std::vector<int> hist(P, 0);
  for (int t = 0; t < T; ++t) {
    float wsum = 0.0f;
    for (int j = 0; j < K; ++j) {
      const int p = ids[(size_t)t * K + j];
      CHECK(p >= 0 && p < P, "%s: id %d", L.name, p);
      for (int i = 0; i < j; ++i)
        CHECK(ids[(size_t)t * K + i] != p, "%s: repeated pick, token %d", L.name, t);
      const float g = w[(size_t)t * K + j];
      ++hist[p];
      if (L.shared && j == K - 1) {
        CHECK(p == P - 1 && g == 1.0f, "%s: shared entry of token %d", L.name, t);
        continue;
      }
      CHECK(owner[p] >= 0, "%s: routed pick %d is no logical expert's copy", L.name, p);
      CHECK(copy[p] == t % ncopies[owner[p]], "%s: token %d uses copy %d of expert %d", L.name, t,
            copy[p], owner[p]);
      CHECK(g > 0.0f && g <= 1.0f, "%s: gate %g", L.name, g);
      wsum += g;
    }
    if (L.score_fn == MOEDC_SCORE_SIGMOID_NORM)
      CHECK(std::fabs(wsum - 1.0f) < 1e-5f, "%s: gates of token %d sum to %g", L.name, t, wsum);
    else
      CHECK(wsum > 0.0f && wsum <= 1.0f + 1e-6f, "%s: softmax gates of token %d sum to %g", L.name,
            t, wsum);
  }
  int total = 0, drops = 0;
  for (int p = 0; p < P; ++p) {
    CHECK(counts[p] == hist[p], "%s: counts[%d]", L.name, p);
    CHECK(offsets[p] == total, "%s: offsets[%d]", L.name, p);
    total += counts[p];
    drops += counts[p] > L.cap[p] ? counts[p] - L.cap[p] : 0;
  }
  CHECK(offsets[P] == total && total == T * K, "%s: sum of counts %d", L.name, total);
  CHECK(dropped == drops, "%s: dropped %d != %d", L.name, dropped, drops);

  // Slots: expert p's kept entries fill [base_p, base_p + min(count, cap))
  // in ascending token order; the rest are -1.
  std::vector<int> next(P, 0), base(P, 0);
  for (int p = 1; p < P; ++p) base[p] = base[p - 1] + L.cap[p - 1];
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < K; ++j) {
      const int p = ids[(size_t)t * K + j], s = slots[(size_t)t * K + j];
      const int r = next[p]++;
      CHECK(s == (r < L.cap[p] ? base[p] + r : -1), "%s: slot of token %d entry %d", L.name, t, j);
    }

  // Dispatched bytes: payload within +-127, finite non-negative scales,
  // zero words after them up to the 128-byte boundary, the rest untouched.
  std::vector<uint8_t> dbuf((size_t)sz.dispatch_buf_bytes), fbuf(dbuf.size());
  HIPCK(hipMemcpy(dbuf.data(), b.dbuf, dbuf.size(), hipMemcpyDeviceToHost));
  HIPCK(hipMemcpy(fbuf.data(), f.dbuf, fbuf.size(), hipMemcpyDeviceToHost));
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < K; ++j) {
      const int s = slots[(size_t)t * K + j];
      if (s < 0) continue;
      const uint8_t *row = dbuf.data() + (size_t)s * sz.slot_stride;
      for (int i = 0; i < H; ++i) CHECK((int8_t)row[i] != -128, "%s: INT8 -128 in slot %d", L.name, s);
      for (int g = 0; g < G; ++g) {
        float sc;
        std::memcpy(&sc, row + H + 4 * g, 4);
        CHECK(std::isfinite(sc) && sc >= 0.0f, "%s: scale %g", L.name, sc);
      }
      for (int i = H + 4 * G; i < scale_end; ++i) CHECK(row[i] == 0, "%s: padding byte %d", L.name, i);
      for (int i = scale_end; i < sz.slot_stride; ++i)
        CHECK(row[i] == 0xA5, "%s: tail byte %d of slot %d written", L.name, i, s);
    }

  // The fused call: same route outputs and the same dispatch buffer bytes.
  {
    std::vector<int32_t> i2((size_t)T * K), s2((size_t)T * K), c2(P), o2(P + 1);
    std::vector<float> w2((size_t)T * K);
    int32_t d2 = -1;
    HIPCK(hipMemcpy(i2.data(), f.ids, sizeof(int32_t) * T * K, hipMemcpyDeviceToHost));
    HIPCK(hipMemcpy(w2.data(), f.w, sizeof(float) * T * K, hipMemcpyDeviceToHost));
    HIPCK(hipMemcpy(s2.data(), f.slots, sizeof(int32_t) * T * K, hipMemcpyDeviceToHost));
    HIPCK(hipMemcpy(c2.data(), f.counts, sizeof(int32_t) * P, hipMemcpyDeviceToHost));
    HIPCK(hipMemcpy(o2.data(), f.offsets, sizeof(int32_t) * (P + 1), hipMemcpyDeviceToHost));
    HIPCK(hipMemcpy(&d2, f.dropped, sizeof(int32_t), hipMemcpyDeviceToHost));
    CHECK(i2 == ids && s2 == slots && c2 == counts && o2 == offsets && d2 == dropped,
          "%s: fused route outputs differ", L.name);
    CHECK(std::memcmp(w2.data(), w.data(), sizeof(float) * w.size()) == 0, "%s: fused gates differ",
          L.name);
    CHECK(fbuf == dbuf, "%s: fused dispatch bytes differ", L.name);
  }

  // Combine output: finite everywhere.
  std::vector<uint16_t> y((size_t)T * H);
  HIPCK(hipMemcpy(y.data(), b.y, sizeof(uint16_t) * T * H, hipMemcpyDeviceToHost));
  for (uint16_t v : y) CHECK(std::isfinite(bf16_to_float(v)), "%s: non-finite output", L.name);

  // Invalid arguments are refused on the host, before any launch.
  CHECK(moedc_route(plan, T, nullptr, b.ids, b.w, b.counts, b.offsets, b.slots, b.dropped, b.ws,
                    st) == MOEDC_ERR_INVALID_ARG, "%s: NULL logits accepted", L.name);
  CHECK(moedc_dispatch(plan, T + 1, b.x, b.slots, b.dbuf, st) == MOEDC_ERR_SHAPE,
        "%s: token count above the plan accepted", L.name);
  CHECK(moedc_combine(plan, T, (const char *)b.cbuf + 4, MOEDC_FMT_BF16, b.slots, b.w, b.y,
                      st) == MOEDC_ERR_ALIGN, "%s: misaligned expert outputs accepted", L.name);
  CHECK(moedc_combine(plan, T, b.cbuf, 7, b.slots, b.w, b.y, st) == MOEDC_ERR_INVALID_ARG,
        "%s: bad format accepted", L.name);
  HIPCK(hipStreamSynchronize(st));

  HIPCK(hipStreamDestroy(st));
  for (Bufs *q : {&b, &f})
    for (void *ptr : {(void *)q->logits, (void *)q->x, (void *)q->ids, (void *)q->w,
                      (void *)q->counts, (void *)q->offsets, (void *)q->slots, (void *)q->dropped,
                      q->ws, q->dbuf, (void *)q->cbuf, (void *)q->y})
      if (ptr) HIPCK(hipFree(ptr));
  moedc_plan_destroy(plan);
  std::printf("%s: %d tokens, %d dropped\n", L.name, T, dropped);
  return 0;
}

}  // namespace

int main() {
  // The logits favour experts by e % 5, so picks crowd onto a few experts
  // and every layer drops a large share of its entries (the drop path).
  // 300 tokens, 16 experts, top-4, 128-value scales, capacity 90.
  Layer a{"groups128", 300, 640, 128, 16, 4, 0, MOEDC_SCORE_SIGMOID_NORM, 1, {},
          std::vector<int32_t>(16, 90), 12345u};
  // 200 tokens, 30 logical experts of which 0-3 have a second copy
  // (physical 30-33), a shared expert (physical 34, capacity T), one scale
  // per token, capacity 40.
  Layer b{"per_token_shared_replicas", 200, 1024, 1024, 30, 4, 1, MOEDC_SCORE_SIGMOID_NORM, 2, {},
          {}, 777u};
  b.table.assign(30 * 2, -1);
  for (int e = 0; e < 30; ++e) b.table[e * 2] = e;
  for (int e = 0; e < 4; ++e) b.table[e * 2 + 1] = 30 + e;
  b.cap.assign(35, 40);
  b.cap[34] = 200;
  // 12 tokens (the one-launch decode path), softmax gates, ragged hidden,
  // capacity 3.
  Layer d{"decode_softmax", 12, 1152, 128, 40, 6, 0, MOEDC_SCORE_SOFTMAX, 1, {},
          std::vector<int32_t>(40, 3), 99u};
  for (const Layer *L : {&a, &b, &d})
    if (run_layer(*L) != 0) return 1;
  std::printf("abi driver ok\n");
  return 0;
}
