"""The expert W8A8 layer on seeded shapes with many rows per expert: hidden
128..1152 (partial 256-channel tiles), 1..12 experts, 200..3000 tokens, so
experts span several 128-row (128-input groups) or 256-row (one scale per
token) tiles with ragged tails, and capacities that may cut an expert's
rows.  The whole output buffer is compared with the oracle: occupied rows
bit for bit, every other row untouched."""
import numpy as np
import pytest
import torch

import oracle
from combine_moedc_route_amd import moedc as M
from combine_moedc_route_amd import workloads as W

from gpu_common import dev, log

pytestmark = pytest.mark.gpu

SENT = 0x7FC1


def shape_case(seed):
    rng = np.random.default_rng(9000 + seed)
    H = 128 * int(rng.integers(1, 10))
    gs = H if rng.random() < 0.5 else 128
    E = int(rng.integers(1, 13))
    KR = int(rng.integers(1, min(E, 4) + 1))
    T = int(rng.integers(200, 3001))
    cap = rng.integers(T * KR // E // 2 + 1, T * KR // E + 300, size=E).astype(np.int32)
    return W.Workload(f"shape{seed}", "", T, H, E, E, KR, 0, W.SCORE_SIGMOID_NORM, cap, None,
                      300 + seed, "normal", group_size=gs)


@pytest.mark.parametrize("seed", range(16))
def test_expert_layer_many_rows_per_expert(seed):
    wl = shape_case(seed)
    H, E = wl.hidden, wl.num_phys
    plan, cfg = M.Plan.from_workload(wl), oracle.Cfg.from_workload(wl)
    s = plan.sizes
    x, logits = W.make_inputs(wl)
    r = oracle.route(cfg, logits)
    rows = np.minimum(r["counts"], wl.capacity)
    log(f"[case] seed {seed}: H={H} group={wl.group_size} E={E} K={wl.top_k} T={wl.tokens} "
        f"rows/expert max {rows.max()}")
    dref = oracle.dispatch(cfg, x, r["slots"], s.total_slots, s.slot_stride)
    Wt, wsc = W.make_expert_weights(seed, E, H)
    want = oracle.expert_w8a8(cfg, r["counts"], dref, s.slot_stride, Wt, wsc,
                              ebuf=np.full((s.total_slots, H), SENT, np.uint16))
    ws = torch.empty(s.workspace_bytes, dtype=torch.uint8, device="cuda")
    plan.bind_workspace(ws)
    out = torch.full((s.total_slots, H), SENT, dtype=torch.int16, device="cuda")
    plan.expert_w8a8(dev(r["counts"]), dev(dref), torch.from_numpy(Wt).cuda(), dev(wsc), out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want), f"{(got != want).any(axis=1).sum()} rows differ"
