"""HIP-graph capture of the decode step, and of a large-batch step with
the expert layer, through the C ABI.

The benchmark times the 96-token decode path as graph replays, so this test
captures moedc_route_dispatch + the stand-in expert + moedc_combine (and,
separately, the two-step moedc_route + moedc_dispatch + moedc_combine) in a
graph, replays it several times with eager work and synchronisations in
between, and checks every replay bit for bit against an eager run, which
itself is checked against the oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from combine_moedc_route_amd import moedc as M
from combine_moedc_route_amd import workloads as W

from gpu_common import assert_within_gate_bound, bf16_to_f32, log

pytestmark = pytest.mark.gpu


def _state(wl):
    plan = M.Plan.from_workload(wl)
    b = plan.alloc("cuda:0")
    x, logits = W.make_inputs(wl)
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    lg = torch.from_numpy(logits).cuda()
    y = torch.full((wl.tokens, wl.hidden), -1, dtype=torch.int16, device="cuda")
    return plan, b, x, logits, xd, lg, y


@pytest.mark.parametrize("fused", [True, False])
def test_decode_step_graph_replays_match_eager(fused):
    wl = W.get("decode")
    log(f"[case] decode graph fused={fused}")
    plan, b, x, logits, xd, lg, y = _state(wl)
    rargs = (b["topk_ids"], b["topk_w"], b["counts"], b["offsets"], b["slots"], b["dropped"])

    def step():
        if fused:
            plan.route_dispatch(lg, xd, *rargs, b["dispatch_buf"], b["workspace"])
        else:
            plan.route(lg, *rargs, b["workspace"])
            plan.dispatch(xd, b["slots"], b["dispatch_buf"])
        plan.expert_stub(b["counts"], b["dispatch_buf"], b["combine_buf"], b["workspace"])
        plan.combine(b["combine_buf"], M.FMT_BF16, b["slots"], b["topk_w"], y)

    def snapshot():
        torch.cuda.synchronize()
        return {"ids": b["topk_ids"].clone(), "w": b["topk_w"].clone(),
                "slots": b["slots"].clone(), "counts": b["counts"].clone(),
                "offsets": b["offsets"].clone(), "y": y.clone()}

    step()
    ref = snapshot()
    # The eager result itself against the oracle (integer outputs exact).
    cfg = oracle.Cfg.from_workload(wl)
    want = oracle.route(cfg, logits)
    assert np.array_equal(ref["ids"].cpu().numpy(), want["topk_ids"])
    assert np.array_equal(ref["slots"].cpu().numpy(), want["slots"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        # Eager work between replays: clobber every output, then replay.
        for k in ("topk_ids", "slots", "counts", "offsets"):
            b[k].fill_(-3)
        b["topk_w"].fill_(-3.0)
        y.fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"replay {rep}: {k} differs from the eager run"
    log("  4 replays bit-identical to the eager step")


def test_large_batch_step_with_expert_layer_graph_replays_match_eager():
    """The large-batch path in a graph: 3000 tokens (the large-batch route,
    a workgroup per token in dispatch, one wave per 512-value chunk on
    16-wave workgroups in combine) and the W8A8 expert layer between
    dispatch and combine, whose tile list is rebuilt on the device from
    the route's counts on every replay.  The eager output is checked against
    the oracle's expert layer and combine on every token."""
    # capacity 470 per expert against a mean of 450 entries: a few drops
    wl = dataclasses.replace(W.with_tokens(W.get("ragged"), 3000),
                             capacity=np.full(40, 470, np.int32))
    log(f"[case] large-batch graph T={wl.tokens} H={wl.hidden} P={wl.num_phys}")
    plan, b, x, logits, xd, lg, y = _state(wl)
    Wt, wsc = W.make_expert_weights(7, wl.num_phys, wl.hidden)
    Wd, wsd = torch.from_numpy(Wt).cuda(), torch.from_numpy(wsc).cuda()
    rargs = (b["topk_ids"], b["topk_w"], b["counts"], b["offsets"], b["slots"], b["dropped"])

    def step():
        plan.route(lg, *rargs, b["workspace"])
        plan.dispatch(xd, b["slots"], b["dispatch_buf"])
        plan.expert_w8a8(b["counts"], b["dispatch_buf"], Wd, wsd, b["combine_buf"], b["workspace"])
        plan.combine(b["combine_buf"], M.FMT_BF16, b["slots"], b["topk_w"], y)

    def snapshot():
        torch.cuda.synchronize()
        return {"ids": b["topk_ids"].clone(), "w": b["topk_w"].clone(),
                "slots": b["slots"].clone(), "counts": b["counts"].clone(),
                "offsets": b["offsets"].clone(), "dropped": b["dropped"].clone(),
                "y": y.clone()}

    step()
    ref = snapshot()
    cfg = oracle.Cfg.from_workload(wl)
    want = oracle.route(cfg, logits)
    assert np.array_equal(ref["ids"].cpu().numpy(), want["topk_ids"])
    assert np.array_equal(ref["slots"].cpu().numpy(), want["slots"])
    assert int(ref["dropped"].item()) == want["dropped"] > 0
    s = plan.sizes
    dref = oracle.dispatch(cfg, x, want["slots"], s.total_slots, s.slot_stride)
    eref = oracle.expert_w8a8(cfg, want["counts"], dref, s.slot_stride, Wt, wsc)
    ywant = oracle.combine(cfg, eref, M.FMT_BF16, want["slots"], want["topk_w"])
    assert_within_gate_bound(ref["y"].cpu().numpy().view(np.uint16), ywant, want["slots"],
                             ref["w"].cpu().numpy(), want["topk_w"],
                             lambda idx: bf16_to_f32(eref[idx]).astype(np.float64))
    log("  eager step within the end-to-end bound of the oracle on every token")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for k in ("topk_ids", "slots", "counts", "offsets", "dropped"):
            b[k].fill_(-3)
        b["topk_w"].fill_(-3.0)
        b["combine_buf"].fill_(-3)
        y.fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"replay {rep}: {k} differs from the eager run"
    log("  4 replays bit-identical to the eager step")
