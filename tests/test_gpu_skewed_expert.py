"""The expert layer under skew, with planned replicas and the device-built
LPT schedule of its bands over the 8 dies ("StrataCL 深度技术分析", section
3.5; redundant experts: "Decode Phase" of the CloudMatrix384 article).

The replica table comes from moedc_place_replicas on the batch's per-expert
loads (32 redundant copies, at most 8 per expert); capacities are the
planned route's counts plus a margin, so nothing drops.  The path runs
route -> dispatch -> expert layer (LPT and round-robin dealing) -> combine:

- route bit for bit against the oracle on the planned table;
- the two dealings give byte-identical expert outputs;
- the tiles the device dealt to each die equal, for LPT, the per-worker
  loads of the library's host LPT planner (moedc_lpt_partition, pinned
  against brute force in test_planning.py) on the same band costs, and for
  round-robin the sums of every 8th band;
- expert rows and combine output against the oracle: every row and token
  on a reduced batch (hidden 512, 2048 tokens), the hottest and coldest
  copies' rows and a sample of tokens at full size."""
import numpy as np
import pytest
import torch

import oracle
from combine_moedc_route_amd import moedc as M
from combine_moedc_route_amd import workloads as W

from gpu_common import compare_route, dev, dev_i16, gpu_route, host_u16, log

pytestmark = pytest.mark.gpu

REDUNDANT, MAX_REPLICAS = 32, 8
BAND_TILES, CHANNELS, XCDS = 4, 256, 8


def planned_workload(T, H):
    """The skewed recipe (Zipf(1.1) popularity, 8 of every 96 rows x50) at T
    tokens and hidden H, with replicas placed for this batch's loads."""
    base = W.get("skewed")
    E = base.num_logical
    wl = W.Workload("skewed-planned", "", T, H, E, E, base.top_k, 0, base.score_fn,
                    np.full(E, T, np.int32), None, base.seed, "zipf", base.outliers)
    x, logits = W.make_inputs(wl)
    load = oracle.route(oracle.Cfg.from_workload(wl), logits)["counts"].astype(np.float64)
    table = M.place_replicas(load, REDUNDANT, MAX_REPLICAS)
    P = E + REDUNDANT
    wl = W.Workload("skewed-planned", "", T, H, E, P, base.top_k, 0, base.score_fn,
                    np.full(P, T, np.int32), table, base.seed, "zipf", base.outliers)
    counts = oracle.route(oracle.Cfg.from_workload(wl), logits)["counts"]
    cap = ((counts + 64 + 63) // 64 * 64).astype(np.int32)      # room for every token
    wl.capacity = cap
    return wl, x, logits, table


def band_costs(counts, cap, H, bm):
    ntiles = -(-H // CHANNELS)
    nbe = -(-ntiles // BAND_TILES)
    rows = np.minimum(counts, cap).astype(np.int64)
    rt = -(-rows // bm)
    width = np.array([min(BAND_TILES, ntiles - b * BAND_TILES) for b in range(nbe)])
    return (rt[:, None] * width[None, :]).ravel()               # band k = p * nbe + b


def run_case(wl, x, logits, weights, wscale):
    """Device path with both dealings; returns the route, both expert
    buffers, the combine output and the per-die tile totals."""
    plan = M.Plan.from_workload(wl)
    cfg = oracle.Cfg.from_workload(wl)
    r = oracle.route(cfg, logits)
    assert r["dropped"] == 0
    got_r, ws = gpu_route(plan, wl, logits)
    compare_route(wl, got_r, r)
    s = plan.sizes
    dbuf = torch.empty(s.dispatch_buf_bytes, dtype=torch.uint8, device="cuda")
    counts_d, slots_d, w_d = dev(r["counts"]), dev(r["slots"]), dev(r["topk_w"])
    plan.dispatch(dev_i16(x), slots_d, dbuf)
    out, tiles = {}, {}
    for name, deal in (("lpt", M.DEAL_LPT), ("rr", M.DEAL_ROUND_ROBIN)):
        cbuf = torch.full((s.total_slots, wl.hidden), 0x7FC1, dtype=torch.int16, device="cuda")
        xt = torch.full((XCDS,), -1, dtype=torch.int32, device="cuda")
        plan.expert_w8a8_dealt(counts_d, dbuf, weights, wscale, cbuf, ws, deal, xt)
        torch.cuda.synchronize()
        out[name], tiles[name] = cbuf, xt.cpu().numpy()
    assert torch.equal(out["lpt"], out["rr"]), "dealings give different expert outputs"
    y = torch.empty((wl.tokens, wl.hidden), dtype=torch.int16, device="cuda")
    plan.combine(out["lpt"], M.FMT_BF16, slots_d, w_d, y)
    torch.cuda.synchronize()
    del out["rr"], dbuf
    return plan, cfg, r, out["lpt"], y, tiles


def check_schedule(wl, r, tiles, bm):
    cost = band_costs(r["counts"], wl.capacity, wl.hidden, bm)
    assign, makespan = M.lpt_partition(cost.astype(np.float64), XCDS)
    host_lpt = np.bincount(assign, weights=cost, minlength=XCDS).astype(np.int64)
    assert np.array_equal(tiles["lpt"], host_lpt), (tiles["lpt"], host_lpt)
    rr = np.bincount(np.arange(cost.size) % XCDS, weights=cost, minlength=XCDS).astype(np.int64)
    assert np.array_equal(tiles["rr"], rr), (tiles["rr"], rr)
    assert tiles["lpt"].max() == makespan and tiles["lpt"].sum() == cost.sum()
    return cost


def test_skewed_planned_reduced_every_row_and_token():
    wl, x, logits, table = planned_workload(2048, 512)
    log(f"[case] skewed planned T={wl.tokens} H={wl.hidden} P={wl.num_phys} "
        f"copies<= {(table >= 0).sum(1).max()}")
    Wt, wsc = W.make_expert_weights(51, wl.num_phys, wl.hidden)
    plan, cfg, r, ebuf, y, tiles = run_case(wl, x, logits, torch.from_numpy(Wt).cuda(),
                                            dev(wsc))
    check_schedule(wl, r, tiles, 128)
    s = plan.sizes
    dref = oracle.dispatch(cfg, x, r["slots"], s.total_slots, s.slot_stride)
    eref = oracle.expert_w8a8(cfg, r["counts"], dref, s.slot_stride, Wt, wsc,
                              ebuf=np.full((s.total_slots, wl.hidden), 0x7FC1, np.uint16))
    assert np.array_equal(host_u16(ebuf), eref), "expert rows differ"
    want = oracle.combine(cfg, eref, M.FMT_BF16, r["slots"], r["topk_w"])
    assert np.array_equal(host_u16(y), want), "combine differs"
    log(f"  every row and token bit-exact; tiles per die LPT {tiles['lpt'].tolist()} "
        f"round-robin {tiles['rr'].tolist()}")


@pytest.mark.slow
def test_skewed_planned_full_size_hottest_and_coldest_copies():
    wl, x, logits, table = planned_workload(30720, 7168)
    H, P = wl.hidden, wl.num_phys
    log(f"[case] skewed planned full size T={wl.tokens} H={H} P={P}")
    gen = torch.Generator(device="cuda").manual_seed(52)
    Wd = torch.randint(-127, 128, (P, H, H), dtype=torch.int8, device="cuda", generator=gen)
    wsd = (torch.rand((P, H), device="cuda", generator=gen) + 0.5) / (127.0 * H ** 0.5)
    plan, cfg, r, ebuf, y, tiles = run_case(wl, x, logits, Wd, wsd)
    cost = check_schedule(wl, r, tiles, 128)
    s = plan.sizes
    base = np.concatenate([[0], np.cumsum(wl.capacity)[:-1]])
    owner = np.full(s.total_slots, -1, np.int64)                 # slot -> token
    kept = r["slots"] >= 0
    owner[r["slots"][kept]] = np.nonzero(kept)[0]
    used = np.minimum(r["counts"], wl.capacity)
    hot, cold = int(np.argmax(used)), int(np.argmin(np.where(used > 0, used, 1 << 30)))

    def oracle_rows(p, rows):
        one = oracle.Cfg(H, 1, 1, 1, 0, 1, [len(rows)], group_size=wl.group_size)
        d = oracle.dispatch(one, x[owner[base[p] + rows]],
                            np.arange(len(rows), dtype=np.int32)[:, None], len(rows),
                            s.slot_stride)
        return oracle.expert_w8a8(one, np.array([len(rows)], np.int32), d, s.slot_stride,
                                  Wd[p:p + 1].cpu().numpy(), wsd[p:p + 1].cpu().numpy())

    for p in (hot, cold):
        n = int(used[p])
        rows = np.unique(np.concatenate([[0, n - 1], np.arange(0, n, max(1, n // 24))]))
        got = host_u16(ebuf[torch.from_numpy(base[p] + rows).cuda()])
        assert np.array_equal(got, oracle_rows(p, rows)), f"expert {p} rows differ"
    # Combine on sampled tokens: the oracle computes their K expert rows.
    toks = np.random.default_rng(53).choice(wl.tokens, 12, replace=False)
    sl = r["slots"][toks]
    compact = np.zeros((sl.size, H), np.uint16)
    for i, t in enumerate(toks):
        for k in range(wl.K):
            p = int(np.searchsorted(base, sl[i, k], side="right") - 1)
            compact[i * wl.K + k] = oracle_rows(p, np.array([sl[i, k] - base[p]]))[0]
    remap = np.arange(sl.size, dtype=np.int32).reshape(sl.shape)
    want = oracle.combine(cfg, compact, M.FMT_BF16, remap, r["topk_w"][toks])
    assert np.array_equal(host_u16(y[torch.from_numpy(toks).cuda()]), want)
    mean = cost.sum() / XCDS
    log(f"  hottest copy {hot} ({used[hot]} rows), coldest {cold} ({used[cold]}) and 12 tokens "
        f"bit-exact; die load max/mean LPT {tiles['lpt'].max() / mean:.4f} "
        f"round-robin {tiles['rr'].max() / mean:.4f}")
