"""Seeded random layer configurations through the whole C-ABI path.

Each case draws a configuration (hidden size 128..8192, 128-value or
per-token scales, 1..300 logical experts (256 in a quarter of the cases), 1..16 picks, an optional shared
expert, multi-copy replicas, capacities that may overflow, normal, uniform
or tie-heavy logits, token counts on both sides of the small-batch switch)
and checks against the oracle: route (integers exact, gates within the
derived tolerance), dispatch (bytes exact, untouched bytes kept), the fused
route+dispatch entry (equal to the two calls), combine in both formats
(exact), and, where the weights are small, the expert W8A8 layer (exact)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from combine_moedc_route_amd import moedc as M
from combine_moedc_route_amd import workloads as W

from gpu_common import (check_dispatch_tokens, check_dispatch_untouched, compare_route, dev,
                        dev_i16, gpu_dispatch, gpu_route, host_u16, log)

pytestmark = pytest.mark.gpu

SENT = 0x7FC1


def random_case(seed):
    rng = np.random.default_rng(5000 + seed)
    H = int(rng.choice([128, 256, 640, 1152, 4096, 8192]))
    gs = H if rng.random() < 0.3 else 128
    shared = int(rng.random() < 0.3)
    # a quarter of the cases use rows of exactly 256 logits (the large-batch
    # route's one-chunk path)
    E = 256 if rng.random() < 0.25 else int(rng.integers(1, 301))
    KR = int(rng.integers(1, min(E, 16 - shared) + 1))
    R = int(rng.choice([1, 1, 2, 3]))
    rep, extra = None, 0
    if R > 1 and E > 1:
        rep = np.full((E, R), -1, np.int32)
        rep[:, 0] = np.arange(E)
        nxt = E
        for e in rng.choice(E, size=int(rng.integers(1, min(E, 8) + 1)), replace=False):
            c = int(rng.integers(2, R + 1))
            rep[e, 1:c] = np.arange(nxt, nxt + c - 1)
            nxt += c - 1
        extra = nxt - E
    P = E + extra + shared
    T = int(rng.choice([1, 2, 63, 64, 65, 256, 257, int(rng.integers(3, 700))]))
    mean = max(1, T * KR // (E + extra))
    cap = rng.integers(max(1, mean // 2), 2 * mean + 3, size=P).astype(np.int32)
    if shared:
        cap[-1] = T if rng.random() < 0.7 else max(1, T // 2)
    kind = str(rng.choice(["normal", "uniform", "ties"]))
    wl = W.Workload(f"rand{seed}", "", T, H, E, P, KR, shared, int(rng.integers(0, 2)),
                    cap, rep, 7000 + seed, "normal" if kind == "ties" else kind,
                    group_size=gs)
    x, logits = W.make_inputs(wl)
    if kind == "ties":
        menu = np.array([-1.0, -0.0, 0.0, 0.5, 1.0], np.float32)
        logits = menu[rng.integers(0, len(menu), logits.shape)]
    return wl, x, np.ascontiguousarray(logits, np.float32), kind


@pytest.mark.parametrize("seed", range(256))
def test_random_config_full_path(seed):
    wl, x, logits, kind = random_case(seed)
    T, H, K = wl.tokens, wl.hidden, wl.K
    log(f"[case] seed {seed}: T={T} H={H} group={wl.group_size} E={wl.num_logical}/"
        f"{wl.num_phys} K={wl.top_k}+{wl.num_shared} R={0 if wl.replica_table is None else wl.replica_table.shape[1]} "
        f"score={wl.score_fn} logits={kind}")
    plan = M.Plan.from_workload(wl)
    cfg = oracle.Cfg.from_workload(wl)
    s = plan.sizes

    # route
    want = oracle.route(cfg, logits)
    got, ws = gpu_route(plan, wl, logits)
    compare_route(wl, got, want)

    # dispatch (from the oracle's slots, so the bytes are checked on their own)
    dbuf = gpu_dispatch(plan, x, want["slots"])
    check_dispatch_tokens(dbuf, x, want["slots"], np.arange(T), H, wl.group_size)
    check_dispatch_untouched(dbuf, want["slots"], H, group_size=wl.group_size)

    # fused entry == route + dispatch
    i32 = dict(dtype=torch.int32, device="cuda")
    outs = dict(ids=torch.full((T, K), -7, **i32), w=torch.zeros((T, K), device="cuda"),
                counts=torch.full((wl.num_phys,), -7, **i32),
                offsets=torch.full((wl.num_phys + 1,), -7, **i32),
                slots=torch.full((T, K), -7, **i32), dropped=torch.full((1,), -7, **i32))
    fbuf = torch.full((s.total_slots, s.slot_stride), 0xA5, dtype=torch.uint8, device="cuda")
    plan.route_dispatch(dev(logits), dev_i16(x), outs["ids"], outs["w"], outs["counts"],
                        outs["offsets"], outs["slots"], outs["dropped"], fbuf, ws)
    torch.cuda.synchronize()
    assert np.array_equal(outs["ids"].cpu().numpy(), got["topk_ids"])
    assert np.array_equal(outs["slots"].cpu().numpy(), got["slots"])
    assert np.array_equal(outs["counts"].cpu().numpy(), got["counts"])
    assert np.array_equal(outs["offsets"].cpu().numpy(), got["offsets"])
    assert int(outs["dropped"].item()) == got["dropped"]
    assert np.array_equal(outs["w"].cpu().numpy(), got["topk_w"])
    assert torch.equal(fbuf, dbuf), "fused dispatch bytes differ from moedc_dispatch"

    # combine, both formats, on the oracle's dispatch and stand-in expert
    dref = oracle.dispatch(cfg, x, want["slots"], s.total_slots, s.slot_stride)
    ebuf = oracle.expert_stub(cfg, want["counts"], dref, s.slot_stride)
    for fmt, src_host, src in ((M.FMT_BF16, ebuf, dev_i16(ebuf)), (M.FMT_Q8, dref, dev(dref))):
        ref = oracle.combine(cfg, src_host, fmt, want["slots"], want["topk_w"])
        y = torch.full((T, H), -1, dtype=torch.int16, device="cuda")
        plan.combine(src, fmt, dev(want["slots"]), dev(want["topk_w"]), y)
        assert np.array_equal(host_u16(y), ref), f"combine fmt {fmt} differs"

    # expert W8A8 layer where the weights stay small
    if wl.num_phys * H * H <= 64 * 2 ** 20 and T * K <= 2500:
        Wt, wsc = W.make_expert_weights(seed, wl.num_phys, H)
        wref = oracle.expert_w8a8(cfg, want["counts"], dref, s.slot_stride, Wt, wsc,
                                  ebuf=np.full((s.total_slots, H), SENT, np.uint16))
        out = torch.full((s.total_slots, H), SENT, dtype=torch.int16, device="cuda")
        plan.expert_w8a8(dev(want["counts"]), dev(dref), torch.from_numpy(Wt).cuda(),
                         dev(wsc), out, ws)
        torch.cuda.synchronize()
        assert np.array_equal(host_u16(out), wref), "expert layer differs"
        log("  expert layer bit-exact")
    log(f"  route/dispatch/fused/combine bit-exact; dropped {got['dropped']}")
