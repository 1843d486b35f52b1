/*
 * moedc.h -- C ABI of libmoedc: MoE token routing, INT8 dispatch into static
 * per-expert slot buffers, and gate-weighted combine, for AMD MI355X
 * (gfx950).  Simulated expert-parallel ranks are partitions of one GPU's
 * HBM.
 *
 * The three calls follow the problem statement of "CloudMatrix384:
 * Co-Designing Supernodes for Trillion-Parameter LLM Inference", section
 * "FusedDispatch and FusedCombine": a naive all-to-all MoE layer exchanges
 * routing metadata, token data and expert outputs; here routing metadata
 * becomes slot indices (moedc_route), token data is quantized to INT8 with
 * scales and written straight into pre-allocated per-expert slots
 * (moedc_dispatch), and expert outputs are gathered back and weighted
 * (moedc_combine).
 *
 * Conventions for every call:
 *  - Device pointers are HIP device addresses owned by the caller; the
 *    library never allocates or frees device memory and keeps no state
 *    between calls.  Host pointers are read during the call only.
 *  - Work is enqueued on the caller's stream and is asynchronous; no call
 *    synchronises the stream.  A NULL stream means the default stream.
 *  - Arguments are validated on the host before any launch; a failed
 *    validation launches nothing.  Launch failures return MOEDC_ERR_HIP and
 *    the HIP error code is available from moedc_last_hip_error().
 *  - Conditions found on the device (capacity overflow) are reported only
 *    through the `dropped` output, never through the status.
 *  - A plan is immutable after creation; calls on one plan may run
 *    concurrently on different streams if their buffers are disjoint.
 *  - BF16 values are passed as uint16_t bit patterns.
 */
#ifndef MOEDC_H
#define MOEDC_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moedc_status {
  MOEDC_OK = 0,
  MOEDC_ERR_INVALID_ARG = 1,  /* NULL pointer, bad enum, inconsistent config */
  MOEDC_ERR_SHAPE = 2,        /* token count / sizes outside the plan */
  MOEDC_ERR_ALIGN = 3,        /* a device pointer is not 16-byte aligned */
  MOEDC_ERR_UNSUPPORTED = 4,  /* valid but not supported (group size, hidden > 8192, ...) */
  MOEDC_ERR_HIP = 5,          /* a HIP launch or copy failed */
  MOEDC_ERR_NO_MEMORY = 6     /* host allocation for the plan failed */
} moedc_status;

typedef enum moedc_score_fn {
  /* softmax over all logical experts (gates of the picks, not renormalised) */
  MOEDC_SCORE_SOFTMAX = 0,
  /* logistic sigmoid of each pick, divided by the sum over the routed picks */
  MOEDC_SCORE_SIGMOID_NORM = 1
} moedc_score_fn;

typedef enum moedc_xcd_dealing {
  /* the expert layer's bands go to the accelerator dies (XCDs) by an LPT
   * list schedule on their tile counts */
  MOEDC_DEAL_LPT = 0,
  /* band k to die k mod 8 (for comparison) */
  MOEDC_DEAL_ROUND_ROBIN = 1
} moedc_xcd_dealing;

typedef enum moedc_elem_fmt {
  MOEDC_FMT_BF16 = 0,  /* expert outputs: [total_slots][hidden] BF16 rows */
  MOEDC_FMT_Q8 = 1     /* expert outputs in the dispatch slot layout (INT8 + scales) */
} moedc_elem_fmt;

/*
 * Static description of one MoE layer.  Expert placement follows "Decode
 * Phase" of the CloudMatrix384 article (routed experts, shared experts and
 * redundant copies of popular experts, one expert per simulated rank).
 */
typedef struct moedc_config {
  int32_t max_tokens;          /* largest token count any call will pass, 0..2^24 */
  int32_t hidden;              /* H: multiple of 128, 128..8192 */
  int32_t group_size;          /* values per fp32 scale: 128, or hidden (one scale per token) */
  int32_t num_logical_experts; /* E_log: logits per token, 1..1024 */
  int32_t num_phys_experts;    /* E_phys: physical experts incl. replicas and shared, 1..1024 */
  int32_t top_k;               /* routed picks per token, 1..E_log; top_k + num_shared <= 16 */
  int32_t num_shared;          /* 0 or 1; the shared expert is physical id E_phys-1 */
  int32_t score_fn;            /* moedc_score_fn */
  int32_t max_replicas;        /* R: columns of replica_table, 1..8 */
  /* Host [E_phys]: slots reserved for each physical expert (>= 0).  Their
   * exclusive prefix sum is each expert's first slot; the sum is
   * total_slots (< 2^31). */
  const int32_t *capacity;
  /* Host [E_log][R] or NULL.  Row e lists the physical ids of logical
   * expert e's copies, then -1 padding; token t goes to copy (t mod r_e).
   * Every routed physical id (< E_phys - num_shared) may appear once.  NULL
   * means physical id = logical id (needs E_phys - num_shared >= E_log). */
  const int32_t *replica_table;
} moedc_config;

typedef struct moedc_sizes {
  int64_t workspace_bytes;      /* device workspace for route, the expert layer and stand-in (bind once) */
  int64_t dispatch_buf_bytes;   /* total_slots * slot_stride */
  int64_t combine_buf_bytes;    /* total_slots * combine_slot_stride */
  int64_t slot_stride;          /* dispatch slot: round_up(H + 4*G, 512) bytes */
  int64_t combine_slot_stride;  /* BF16 combine slot: 2*H bytes */
  int64_t total_slots;          /* sum of capacities */
  int32_t k;                    /* entries per token: top_k + num_shared */
  int32_t num_groups;           /* G = H / group_size */
} moedc_sizes;

typedef struct moedc_plan moedc_plan;

/* Validates *config and builds a host-only plan (copies the tables; no
 * device memory is touched).  *out receives the plan, or NULL on error.
 * Errors: INVALID_ARG, UNSUPPORTED, NO_MEMORY. */
moedc_status moedc_plan_create(const moedc_config *config, moedc_plan **out);

/* Frees a plan (NULL is ignored). */
void moedc_plan_destroy(moedc_plan *plan);

/* Byte sizes of the buffers the caller must allocate for this plan. */
moedc_status moedc_plan_sizes(const moedc_plan *plan, moedc_sizes *out);

/* Uploads the plan's static tables (capacities, slot bases, replica table)
 * into the caller's device workspace of workspace_bytes (16-byte aligned),
 * asynchronously on `stream`.  Needed once per workspace before route,
 * route_dispatch, the expert layer or the expert stand-in use it.  The
 * copies read the plan's own host memory: keep the plan alive until they
 * have run on `stream`.  Calls that share a workspace must not overlap
 * (route and the expert layer keep per-call work lists in it). */
moedc_status moedc_plan_bind_workspace(const moedc_plan *plan, void *workspace,
                                       hipStream_t stream);

/*
 * Routing: the routing metadata of "FusedDispatch and FusedCombine" in the
 * CloudMatrix384 article (each token's experts, and where in each expert's
 * pre-allocated receive buffer the token lands), over the expert placement
 * of its "Decode Phase" (routed experts, redundant copies of popular
 * experts, a shared expert every token visits).  For each of num_tokens
 * tokens:
 *  - picks top_k logical experts by fp32 logit, highest first, ties to the
 *    lower id (-0 == +0), maps each to a physical copy, and computes its
 *    gate (score_fn); a shared expert, if configured, is appended last with
 *    weight 1.0;
 *  - counts[p]: number of (token, entry) pairs routed to physical expert p
 *    (before capacity); offsets[]: exclusive scan of counts, E_phys+1
 *    entries, offsets[E_phys] = num_tokens * k;
 *  - slots[t][j]: base(p) + rank of token t among the tokens routed to p in
 *    ascending token order, or -1 when that rank reaches capacity[p];
 *    *dropped: number of -1 entries.
 * Device arrays: logits float32 [num_tokens][E_log] (16-byte aligned);
 * topk_ids int32 [num_tokens][k] (physical ids); topk_w float32
 * [num_tokens][k]; counts int32 [E_phys]; offsets int32 [E_phys+1]; slots
 * int32 [num_tokens][k]; dropped int32 [1]; workspace as bound.  counts,
 * offsets and dropped are fully rewritten on every call, also for
 * num_tokens == 0.  Logits must be finite; otherwise picks are unspecified
 * but always valid expert ids.
 * Errors: INVALID_ARG, SHAPE (num_tokens outside [0, max_tokens]), ALIGN, HIP.
 */
moedc_status moedc_route(const moedc_plan *plan, int32_t num_tokens,
                         const float *logits, int32_t *topk_ids, float *topk_w,
                         int32_t *counts, int32_t *offsets, int32_t *slots,
                         int32_t *dropped, void *workspace, hipStream_t stream);

/*
 * moedc_route without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments (minus the workspace), outputs and
 * errors as moedc_route, bit for bit the same results.  The per-block
 * expert counts and the plan's tables live in a static device array of
 * 16 MiB that the library holds on each GPU it runs on until the process
 * ends; each call first copies the plan's tables (at most 44 KiB) into it
 * with a host-to-device copy on `stream` -- the plan must stay alive until
 * that copy has run -- and then runs the route kernels on it.  No device
 * memory is allocated or freed.  Every call on a GPU shares that GPU's
 * array, which keeps the last call's contents: calls that overlap on one
 * GPU (other streams, other threads) race, and the caller must serialise
 * them.  The stream must belong to the current device.
 * Errors: as moedc_route; UNSUPPORTED when a batch needs more than the
 * array holds, i.e. 4 * ceil(num_tokens / 64) * E_phys > 16 MiB - 64 KiB
 * (e.g. more than 1,048,320 tokens at 256 physical experts); HIP when the
 * array's address cannot be obtained or a copy or launch fails.
 */
moedc_status moedc_route_noalloc(const moedc_plan *plan, int32_t num_tokens,
                                 const float *logits, int32_t *topk_ids, float *topk_w,
                                 int32_t *counts, int32_t *offsets, int32_t *slots,
                                 int32_t *dropped, hipStream_t stream);

/*
 * Dispatch: early INT8 quantization with scales, then a direct
 * store of each token into each of its slots ("FusedDispatch and
 * FusedCombine": quantize before sending, write into pre-allocated
 * receiver buffers, token-granular load / quantize / write pipeline).
 * Per token and group (128 values, or the whole token when group_size ==
 * hidden, following "INT8 Quantization": per-token dynamic activation
 * scales): amax = max |x|; scale = amax / 127 in IEEE fp32; q =
 * clamp(round-half-even(x / scale), -127, 127) with a correctly rounded
 * fp32 quotient (scale 0 gives q 0).  Slot s occupies bytes
 * [s*slot_stride, (s+1)*slot_stride) of dispatch_buf: INT8 payload at
 * [0, H), G fp32 scales (little-endian) at [H, H + 4*G), then zero bytes
 * up to the next multiple of 128, H + 4*round_up(G, 32) (so no slot ends
 * inside a 128-byte line); the rest of the slot and slots no token maps to
 * are not written.  Entries with slot -1
 * (dropped) are skipped, and so is any slot outside [0, total_slots), so a
 * corrupt slot table cannot make the kernel write outside dispatch_buf.
 * x: BF16 [num_tokens][H] (16-byte aligned); slots: from moedc_route;
 * dispatch_buf: dispatch_buf_bytes (16-byte aligned).  x must be finite.
 * Errors: INVALID_ARG, SHAPE, ALIGN, HIP.
 */
moedc_status moedc_dispatch(const moedc_plan *plan, int32_t num_tokens,
                            const uint16_t *x, const int32_t *slots,
                            void *dispatch_buf, hipStream_t stream);

/*
 * Combine: for each token t and hidden index i,
 *   acc = +0.0f;  acc = fmaf(topk_w[t][j], y_j[i], acc)  for j = 0..k-1
 * skipping entries with slot -1 (and any slot outside [0, total_slots),
 * which is never read), then y[t][i] = BF16 round-to-nearest-even of acc.
 * slots and topk_w are [num_tokens][k] as written by moedc_route.
 * y_j is the expert output in slot slots[t][j]:
 *  fmt BF16: expert_out is [total_slots][H] BF16 (combine_buf_bytes);
 *  fmt Q8:   expert_out is a dispatch buffer, y_j[i] = (float)q * scale.
 * expert_out and y (BF16 [num_tokens][H]) are 16-byte aligned.
 * Errors: INVALID_ARG, SHAPE, ALIGN, HIP.
 */
moedc_status moedc_combine(const moedc_plan *plan, int32_t num_tokens,
                           const void *expert_out, int32_t fmt,
                           const int32_t *slots, const float *topk_w,
                           uint16_t *y, hipStream_t stream);

/*
 * Routing and dispatch in one call, for small decode batches.  Same outputs
 * and the same dispatch buffer bytes as moedc_route followed by
 * moedc_dispatch, bit for bit.  For 17 <= num_tokens <= 256 it is two
 * launches with no host step between them: a wave-per-token top-k, then
 * one workgroup per token that derives its slots from every token's picks
 * and immediately quantizes and stores that token ("Decode Phase": 96
 * tokens per die; "FusedDispatch and FusedCombine": routing metadata fused
 * with the token exchange).  Up to 16 tokens it is one launch: every
 * workgroup runs the batch's top-k itself.  Larger batches run the
 * two-step path.
 * Arguments, layouts, alignment and errors are those of moedc_route and
 * moedc_dispatch.
 */
moedc_status moedc_route_dispatch(const moedc_plan *plan, int32_t num_tokens,
                                  const float *logits, const uint16_t *x,
                                  int32_t *topk_ids, float *topk_w, int32_t *counts,
                                  int32_t *offsets, int32_t *slots, int32_t *dropped,
                                  void *dispatch_buf, void *workspace, hipStream_t stream);

/*
 * moedc_combine on at most max_workgroups workgroups (each loops over the
 * batch with 16 waves when the cap binds), leaving the other compute units
 * to concurrent work on other streams -- the pages' decode pipeline gives the
 * MoE path a fixed share of the cores ("Micro-batch Decode Pipeline" of the
 * CloudMatrix384 article).  Output identical to moedc_combine.
 * Errors: as moedc_combine; INVALID_ARG if max_workgroups < 1.
 */
moedc_status moedc_combine_limited(const moedc_plan *plan, int32_t num_tokens,
                                   const void *expert_out, int32_t fmt,
                                   const int32_t *slots, const float *topk_w,
                                   uint16_t *y, int32_t max_workgroups,
                                   hipStream_t stream);

/*
 * Stand-in expert (not a step of the method; it fills combine inputs so the
 * path can run end to end without weights).  For every occupied slot of
 * physical expert p (the first min(counts[p], capacity[p]) slots of its
 * window): combine_buf row = BF16( ((float)q * scale) * (1 + 0.01f*p) ),
 * computed as two fp32 products and one fp32 sum.  Other rows are not
 * written.  counts: from moedc_route; workspace as bound.
 * Errors: INVALID_ARG, ALIGN, HIP.
 */
moedc_status moedc_expert_stub(const moedc_plan *plan, const int32_t *counts,
                               const void *dispatch_buf, uint16_t *combine_buf,
                               void *workspace, hipStream_t stream);

/*
 * Expert compute between dispatch and combine: one W8A8 linear layer per
 * physical expert (hidden -> hidden), the INT8 matmul of "INT8
 * Quantization" (CloudMatrix384 article: per-token dynamic activation
 * scales, per-channel static weight scales).  For every occupied slot row t
 * of expert p (the first min(counts[p], capacity[p]) slots of its window)
 * and output channel n:
 *   isum_g = sum over scale group g of q[t][k] * weights[p][n][k]  (int32)
 *   acc = +0; acc = fmaf(s_x[t][g], (float)isum_g, acc), g ascending
 *   combine_buf[t][n] = BF16 round-to-nearest-even of acc * w_scale[p][n]
 * reading q and s_x in place from dispatch_buf.  weights: int8
 * [E_phys][H][H] (row n = output channel); w_scale: fp32 [E_phys][H];
 * combine_buf: BF16 [total_slots][H]; all 16-byte aligned.  Other rows of
 * combine_buf are not written.  Runs on int8 MFMA.  The work is cut into
 * bands (4 x 256 output channels x all slot rows of one expert), which are
 * dealt to the GPU's 8 dies by an LPT schedule built on the device from
 * counts, as moedc_expert_w8a8_dealt with MOEDC_DEAL_LPT.
 * Errors: INVALID_ARG, ALIGN, HIP.
 */
moedc_status moedc_expert_w8a8(const moedc_plan *plan, const int32_t *counts,
                               const void *dispatch_buf, const int8_t *weights,
                               const float *w_scale, uint16_t *combine_buf,
                               void *workspace, hipStream_t stream);

/*
 * moedc_expert_w8a8 with a choice of how the bands reach the dies
 * ("StrataCL 深度技术分析", section 3.5: workload-balanced partitioning of
 * expert-major work by an LPT list scheduler; here the workers are the 8
 * XCDs of one GPU, each walking its band list with 32 workgroups).
 * dealing: MOEDC_DEAL_LPT -- bands with tiles, longest first (equal tile
 * counts in band order), each to the die with the fewest tiles so far
 * (ties to the lower die); the largest die load is at most (4/3 - 1/24)
 * times the best possible.  MOEDC_DEAL_ROUND_ROBIN -- band k to die k mod 8.
 * The schedule is built on the device from counts, so the call can be
 * captured in a graph.  xcd_tiles: device int32 [8] receiving the tiles
 * dealt to each die, or NULL.  Results are identical for either dealing.
 * Errors: INVALID_ARG (also for an unknown dealing), ALIGN, HIP.
 */
moedc_status moedc_expert_w8a8_dealt(const moedc_plan *plan, const int32_t *counts,
                                     const void *dispatch_buf, const int8_t *weights,
                                     const float *w_scale, uint16_t *combine_buf,
                                     void *workspace, int32_t dealing, int32_t *xcd_tiles,
                                     hipStream_t stream);

/*
 * Load-proportional placement of redundant experts ("Decode Phase" of the
 * CloudMatrix384 article: redundant copies of experts balance load).  Given
 * the expected load of each logical expert (>= 0, e.g. the previous batch's
 * counts), assigns num_redundant extra copies, each to the expert with the
 * largest load per copy (ties to the lower id) below max_replicas copies,
 * which minimises the largest load per physical expert.  Writes
 * replica_table [num_logical][max_replicas] in the layout moedc_config
 * takes: row e = e, then the physical ids num_logical, num_logical+1, ...
 * of its extra copies in the order they were assigned, then -1.
 * Host memory only; no device work.
 * Errors: INVALID_ARG (negative or non-finite load, more copies than
 * num_logical * (max_replicas - 1), NULL pointers).
 */
moedc_status moedc_place_replicas(int32_t num_logical, const double *load,
                                  int32_t num_redundant, int32_t max_replicas,
                                  int32_t *replica_table);

/*
 * Workload-balanced partitioning of expert-major work units over workers
 * ("StrataCL 深度技术分析", section 3.5: minimise the largest per-core
 * load under a per-peer fan-out cap, by an LPT list scheduler).  Units are
 * taken longest first (equal costs in index order); each goes to the least
 * loaded worker (ties to the lower index) among those allowed: when
 * fanout_cap > 0, a group already served by fanout_cap workers may only be
 * given to one of those.  assign[u] receives the worker of unit u,
 * *makespan the largest worker load.  Without a cap the makespan is at most
 * (4/3 - 1/(3 * num_workers)) times the optimum.  O(U log U + U * W) on the
 * host; no device work.
 * Errors: INVALID_ARG (negative or non-finite cost, group outside
 * [0, num_groups) when capped, NULL pointers).
 */
moedc_status moedc_lpt_partition(int32_t num_units, const double *cost, const int32_t *group,
                                 int32_t num_groups, int32_t num_workers, int32_t fanout_cap,
                                 int32_t *assign, double *makespan);

/* Static English text for a status code. */
const char *moedc_status_string(moedc_status status);

/* hipError_t of the last MOEDC_ERR_HIP returned on this thread (0 if none). */
int32_t moedc_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOEDC_H */
