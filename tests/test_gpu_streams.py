"""Double-buffered operation on two streams: while batch A's combine reads
buffer set 0 on one stream, batch B is routed and dispatched into buffer set
1 on another (its own workspace and route outputs).  The plan is shared and
the library keeps no state, so both results must equal the oracle's."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from combine_moedc_route_amd import moedc as M
from combine_moedc_route_amd import workloads as W

from gpu_common import check_dispatch_tokens, dev, dev_i16, host_u16, log

pytestmark = pytest.mark.gpu


def _route_bufs(plan, T):
    i32 = dict(dtype=torch.int32, device="cuda")
    ws = torch.empty(plan.sizes.workspace_bytes, dtype=torch.uint8, device="cuda")
    plan.bind_workspace(ws)
    return dict(ids=torch.empty((T, plan.K), **i32), w=torch.empty((T, plan.K), device="cuda"),
                counts=torch.empty(plan.num_phys, **i32), offsets=torch.empty(plan.num_phys + 1, **i32),
                slots=torch.empty((T, plan.K), **i32), dropped=torch.empty(1, **i32), ws=ws)


@pytest.mark.parametrize("T", [96, 3000])
def test_dispatch_of_next_batch_overlaps_combine_of_this_one(T):
    base = W.get("mid")
    wl_a = W.with_tokens(base, T)
    wl_b = dataclasses.replace(wl_a, name="mid-b", seed=base.seed + 100)
    log(f"[case] two streams T={T}")
    plan = M.Plan.from_workload(wl_a)
    cfg = oracle.Cfg.from_workload(wl_a)
    s = plan.sizes
    xa, la = W.make_inputs(wl_a)
    xb, lb = W.make_inputs(wl_b)
    ra = oracle.route(cfg, la)
    dref = oracle.dispatch(cfg, xa, ra["slots"], s.total_slots, s.slot_stride)
    ebuf = oracle.expert_stub(cfg, ra["counts"], dref, s.slot_stride)
    want_y = oracle.combine(cfg, ebuf, M.FMT_BF16, ra["slots"], ra["topk_w"])
    want_b = oracle.route(cfg, lb)

    cbuf0 = dev_i16(ebuf)                                   # set 0: batch A's expert outputs
    dbuf1 = torch.full((s.total_slots, s.slot_stride), 0xA5, dtype=torch.uint8, device="cuda")
    y = torch.full((T, base.hidden), -1, dtype=torch.int16, device="cuda")
    slots_a, w_a = dev(ra["slots"]), dev(ra["topk_w"])
    rb = _route_bufs(plan, T)
    lb_d, xb_d = dev(lb), dev_i16(xb)
    torch.cuda.synchronize()

    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):  # repeat so the two streams really interleave
        with torch.cuda.stream(sa):
            plan.combine(cbuf0, M.FMT_BF16, slots_a, w_a, y, stream=sa)
        with torch.cuda.stream(sb):
            plan.route(lb_d, rb["ids"], rb["w"], rb["counts"], rb["offsets"], rb["slots"],
                       rb["dropped"], rb["ws"], stream=sb)
            plan.dispatch(xb_d, rb["slots"], dbuf1, stream=sb)
    torch.cuda.synchronize()

    assert np.array_equal(host_u16(y), want_y)
    assert np.array_equal(rb["ids"].cpu().numpy(), want_b["topk_ids"])
    assert np.array_equal(rb["slots"].cpu().numpy(), want_b["slots"])
    check_dispatch_tokens(dbuf1, xb, want_b["slots"], np.arange(T), base.hidden)
    log("  combine (set 0) and route+dispatch (set 1) on two streams: both bit-exact")
