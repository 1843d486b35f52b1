"""HIP-graph capture of the decode step through the C ABI.

The benchmark times the 96-token decode path as graph replays, so this test
captures moedc_route_dispatch + the stand-in expert + moedc_combine (and,
separately, the two-step moedc_route + moedc_dispatch + moedc_combine) in a
graph, replays it several times with eager work and synchronisations in
between, and checks every replay bit for bit against an eager run, which
itself is checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from combine_moedc_route_amd import moedc as M
from combine_moedc_route_amd import workloads as W

from gpu_common import log

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
