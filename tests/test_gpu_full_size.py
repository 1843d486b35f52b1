"""GPU parity at full size, every token: the 30720-token global batch, the
skewed batch (288 physical experts with replicas) and the 65536-token
prefill batch (top-8 + shared), in the launch shapes the benchmark times.

- route: every id, count, offset and slot bit for bit, gates within the
  derived tolerance;
- dispatch: the bytes of every occupied slot (payload, scales and the zero
  padding that ends the slot's last 128-byte line) against the oracle's
  dispatch of the same tokens; every other byte keeps its sentinel;
- combine, Q8 (reading the GPU's own dispatch buffer) and BF16 (expert
  outputs from a seeded pool of rows, slot s holding row s mod POOL_ROWS):
  every output value of every token against the oracle's combine.

The oracle runs 4096 tokens at a time over a compact slot buffer: the
chunk's kept slots renumbered 0..n-1 in (token, entry) order.  Dispatch and
combine are defined slot by slot, so this is the same definition on a
smaller buffer; the combine inputs of both sides are the oracle's gates and
slots."""
import numpy as np
import pytest
import torch

import oracle
from combine_moedc_route_amd import moedc as M
from combine_moedc_route_amd import workloads as W

from gpu_common import (SENTINEL, check_dispatch_untouched, compare_route, dev, dev_i16,
                        gpu_route, host_u16, log, scale_region_end)

pytestmark = pytest.mark.gpu

CHUNK = 4096
POOL_ROWS = 8191  # prime, so neighbouring and nearby slots hold different rows


def compact(rows):
    """(kept slot ids in (token, entry) order, the rows renumbered to 0..n-1)."""
    keep = rows >= 0
    remap = np.full(rows.shape, -1, np.int32)
    remap[keep] = np.arange(int(keep.sum()), dtype=np.int32)
    return rows[keep].astype(np.int64), remap


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.slow
@pytest.mark.parametrize("name", ["global", "skewed", "prefill"])
def test_every_token_at_full_size(name):
    wl = W.get(name)
    T, H, K = wl.tokens, wl.hidden, wl.K
    G = H // wl.group_size
    log(f"[case] full size {name} T={T} H={H} E={wl.num_logical}/{wl.num_phys} K={K}")
    x, logits = W.make_inputs(wl)
    plan = M.Plan.from_workload(wl)
    cfg = oracle.Cfg.from_workload(wl)
    s = plan.sizes
    S = s.total_slots
    end = scale_region_end(H, wl.group_size)

    r = oracle.route(cfg, logits)
    assert r["dropped"] == 0
    got_r, _ = gpu_route(plan, wl, logits)
    compare_route(wl, got_r, r)
    log("  route bit-exact")

    slots_d, w_d = dev(r["slots"]), dev(r["topk_w"])
    dbuf = torch.full((S, s.slot_stride), SENTINEL, dtype=torch.uint8, device="cuda")
    plan.dispatch(dev_i16(x), slots_d, dbuf)
    y_q = torch.empty((T, H), dtype=torch.int16, device="cuda")
    plan.combine(dbuf, M.FMT_Q8, slots_d, w_d, y_q)
    pool = W.make_expert_out_bf16(31, POOL_ROWS, H)
    occ = torch.from_numpy(r["slots"][r["slots"] >= 0].astype(np.int64)).cuda()
    cbuf = torch.zeros((S, H), dtype=torch.int16, device="cuda")
    cbuf[occ] = dev_i16(pool)[occ % POOL_ROWS]
    del occ
    y_b = torch.empty((T, H), dtype=torch.int16, device="cuda")
    plan.combine(cbuf, M.FMT_BF16, slots_d, w_d, y_b)
    torch.cuda.synchronize()
    del cbuf
    check_dispatch_untouched(dbuf, r["slots"], H, group_size=wl.group_size)

    checked = 0
    for t0 in range(0, T, CHUNK):
        t1 = min(T, t0 + CHUNK)
        kept, remap = compact(r["slots"][t0:t1])
        ref = oracle.dispatch(cfg, x[t0:t1], remap, kept.size, s.slot_stride)
        got = dbuf[torch.from_numpy(kept).cuda(), :end].cpu().numpy()
        bad = np.nonzero((got != ref[:, :end]).any(axis=1))[0]
        assert bad.size == 0, f"dispatch: {bad.size} slots differ, first slot {kept[bad[0]]}"
        want = oracle.combine(cfg, ref, M.FMT_Q8, remap, r["topk_w"][t0:t1])
        gq = host_u16(y_q[t0:t1])
        assert np.array_equal(gq, want), f"Q8 combine: {(gq != want).any(1).sum()} tokens differ"
        want = oracle.combine(cfg, pool[kept % POOL_ROWS], M.FMT_BF16, remap,
                              r["topk_w"][t0:t1])
        gb = host_u16(y_b[t0:t1])
        assert np.array_equal(gb, want), f"BF16 combine: {(gb != want).any(1).sum()} tokens differ"
        checked += kept.size
    assert checked == T * K
    log(f"  {checked} slots and {T} tokens (Q8 and BF16 combine) bit-exact")
