"""Every size limit of the library at once: 1024 physical experts (1002
logical, 8-copy replicas of three of them, a shared expert), 16 entries per
token (15 routed + shared), hidden 8192 (64 scale groups, 8704-byte slots),
with 128-value and per-token scales, on both sides of the small-batch and
chunked-combine switches.  The expert W8A8 layer then has 1024 x 8 bands:
exactly the largest work list its launch accepts.  Checked against the
oracle: route and dispatch bytes exact, combine exact in both formats, the
expert layer exact on sampled rows of the first, a replica, the last
routed and the shared expert."""
import numpy as np
import pytest
import torch

import oracle
from combine_moedc_route_amd import moedc as M
from combine_moedc_route_amd import workloads as W

from gpu_common import (check_dispatch_tokens, check_dispatch_untouched, compare_route, dev,
                        dev_i16, gpu_dispatch, gpu_route, host_u16, log)

pytestmark = pytest.mark.gpu

H = 8192
E_LOG, R = 1002, 8


def max_workload(T, group_size):
    table = np.full((E_LOG, R), -1, np.int32)
    table[:, 0] = np.arange(E_LOG)
    nxt = E_LOG
    for e in (0, 1, 2):                       # three experts with 8 copies each
        table[e, 1:] = np.arange(nxt, nxt + R - 1)
        nxt += R - 1
    P = nxt + 1                               # + shared expert
    assert P == 1024
    K = 16
    cap = np.full(P, max(2, 2 * T * K // P), np.int32)   # ~2x the mean: few drops
    cap[:3] = max(2, T // 8)                 # the replicated ones overflow on purpose
    cap[-1] = T
    return W.Workload(f"max{T}", "", T, H, E_LOG, P, K - 1, 1, W.SCORE_SIGMOID_NORM, cap,
                      table, 900 + T, "zipf", ("fraction", 0.02, 50.0), group_size=group_size)


@pytest.fixture(scope="module")
def weights():
    gen = torch.Generator(device="cuda").manual_seed(77)
    Wd = torch.randint(-127, 128, (1024, H, H), dtype=torch.int8, device="cuda", generator=gen)
    wsd = (torch.rand((1024, H), device="cuda", generator=gen) + 0.5) / (127.0 * H ** 0.5)
    yield Wd, wsd
    del Wd, wsd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,group", [(1, 128), (256, H), (2048, 128), (3000, 128), (3000, H)])
def test_largest_configuration_full_path(T, group, weights):
    wl = max_workload(T, group)
    log(f"[case] max config T={T} group={group} P={wl.num_phys} K={wl.K} H={H}")
    plan = M.Plan.from_workload(wl)
    cfg = oracle.Cfg.from_workload(wl)
    s = plan.sizes
    assert s.slot_stride == 8704
    x, logits = W.make_inputs(wl)

    want = oracle.route(cfg, logits)
    got, ws = gpu_route(plan, wl, logits)
    compare_route(wl, got, want)
    assert want["dropped"] > 0 or T == 1

    dbuf = gpu_dispatch(plan, x, want["slots"])
    check_dispatch_tokens(dbuf, x, want["slots"], np.arange(T), H, group)
    check_dispatch_untouched(dbuf, want["slots"], H, group_size=group)

    if T <= 256:  # the fused entry equals route + dispatch
        K, P = wl.K, wl.num_phys
        i32 = dict(dtype=torch.int32, device="cuda")
        o = dict(ids=torch.empty((T, K), **i32), w=torch.empty((T, K), device="cuda"),
                 counts=torch.empty(P, **i32), offsets=torch.empty(P + 1, **i32),
                 slots=torch.empty((T, K), **i32), dropped=torch.empty(1, **i32))
        fbuf = torch.full_like(dbuf, 0xA5)
        plan.route_dispatch(dev(logits), dev_i16(x), o["ids"], o["w"], o["counts"], o["offsets"],
                            o["slots"], o["dropped"], fbuf, ws)
        torch.cuda.synchronize()
        assert np.array_equal(o["slots"].cpu().numpy(), want["slots"])
        assert torch.equal(fbuf, dbuf)
        del fbuf

    dref = oracle.dispatch(cfg, x, want["slots"], s.total_slots, s.slot_stride)
    ebuf = oracle.expert_stub(cfg, want["counts"], dref, s.slot_stride)
    for fmt, src_host in ((M.FMT_BF16, ebuf), (M.FMT_Q8, dref)):
        ref = oracle.combine(cfg, src_host, fmt, want["slots"], want["topk_w"])
        y = torch.full((T, H), -1, dtype=torch.int16, device="cuda")
        src = dev_i16(src_host) if fmt == M.FMT_BF16 else dev(src_host)
        plan.combine(src, fmt, dev(want["slots"]), dev(want["topk_w"]), y)
        torch.cuda.synchronize()
        assert np.array_equal(host_u16(y), ref), f"combine fmt {fmt} differs"
        del src
    del ebuf
    log("  route, dispatch, combine bit-exact")

    if T < 3000:
        return
    Wd, wsd = weights
    out = torch.full((s.total_slots, H), 0x7FC1, dtype=torch.int16, device="cuda")
    plan.expert_w8a8(dev(want["counts"]), dbuf, Wd, wsd, out, ws)
    torch.cuda.synchronize()
    base = np.concatenate([[0], np.cumsum(wl.capacity)[:-1]])
    for p in (0, 1002, 1001, 1023):
        n_p = min(int(want["counts"][p]), int(wl.capacity[p]))
        assert n_p > 0, p
        rows = np.unique(np.array([0, n_p // 2, n_p - 1]))
        sl = torch.from_numpy(base[p] + rows).cuda()
        one = oracle.Cfg(H, 1, 1, 1, 0, 1, [len(rows)], group_size=group)
        w_exp = oracle.expert_w8a8(one, np.array([len(rows)], np.int32),
                                   dbuf[sl].cpu().numpy(), s.slot_stride,
                                   Wd[p:p + 1].cpu().numpy(), wsd[p:p + 1].cpu().numpy())
        assert np.array_equal(host_u16(out[sl]), w_exp), f"expert {p} differs"
    log("  expert layer bit-exact on sampled rows")
