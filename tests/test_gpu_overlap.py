"""The capped combine beside other work on the GPU: the decode pipeline of
the CloudMatrix384 article ("Micro-batch Decode Pipeline") gives the MoE
path a fixed share of the cores so that other work runs on the rest.  Here
moedc_combine_limited on 16 workgroups combines a 96-token decode batch on
one stream while the W8A8 expert layer of another batch (3000 tokens,
hidden 1152, 40 experts) runs on a second stream, both at the default
priority, several times over.  Both outputs must equal the oracle's: the
combine bit for bit, the expert rows bit for bit."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from combine_moedc_route_amd import moedc as M
from combine_moedc_route_amd import workloads as W

from gpu_common import dev, dev_i16, host_u16, log

pytestmark = pytest.mark.gpu


def test_capped_combine_beside_expert_layer_on_two_streams():
    # Stream A: the decode batch's combine (oracle inputs: route, dispatch, stand-in expert).
    wa = W.get("decode")
    xa, la = W.make_inputs(wa)
    pa, ca = M.Plan.from_workload(wa), oracle.Cfg.from_workload(wa)
    sa_ = pa.sizes
    ra = oracle.route(ca, la)
    da = oracle.dispatch(ca, xa, ra["slots"], sa_.total_slots, sa_.slot_stride)
    ea = oracle.expert_stub(ca, ra["counts"], da, sa_.slot_stride)
    want_a = oracle.combine(ca, ea, M.FMT_BF16, ra["slots"], ra["topk_w"])
    # Stream B: another batch's expert layer.
    wb = dataclasses.replace(W.with_tokens(W.get("ragged"), 3000),
                             capacity=np.full(40, 470, np.int32))
    xb, lb = W.make_inputs(wb)
    pb, cb = M.Plan.from_workload(wb), oracle.Cfg.from_workload(wb)
    sb_ = pb.sizes
    rb = oracle.route(cb, lb)
    db = oracle.dispatch(cb, xb, rb["slots"], sb_.total_slots, sb_.slot_stride)
    Wt, wsc = W.make_expert_weights(61, wb.num_phys, wb.hidden)
    want_b = oracle.expert_w8a8(cb, rb["counts"], db, sb_.slot_stride, Wt, wsc,
                                ebuf=np.full((sb_.total_slots, wb.hidden), 0x7FC1, np.uint16))
    log(f"[case] combine_limited(16) T={wa.tokens} beside expert_w8a8 T={wb.tokens} "
        f"H={wb.hidden} P={wb.num_phys}")

    ea_d, slots_a, w_a = dev_i16(ea), dev(ra["slots"]), dev(ra["topk_w"])
    ya = torch.full((wa.tokens, wa.hidden), -1, dtype=torch.int16, device="cuda")
    wsb = torch.empty(sb_.workspace_bytes, dtype=torch.uint8, device="cuda")
    pb.bind_workspace(wsb)
    db_d, cnt_b = dev(db), dev(rb["counts"])
    Wd, wsd = torch.from_numpy(Wt).cuda(), dev(wsc)
    eb = torch.full((sb_.total_slots, wb.hidden), 0x7FC1, dtype=torch.int16, device="cuda")
    torch.cuda.synchronize()

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority both
    for _ in range(4):
        with torch.cuda.stream(s2):
            pb.expert_w8a8(cnt_b, db_d, Wd, wsd, eb, wsb, stream=s2)
        with torch.cuda.stream(s1):
            for _ in range(3):
                pa.combine_limited(ea_d, M.FMT_BF16, slots_a, w_a, ya, 16, stream=s1)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(ya), want_a), "capped combine differs"
    assert np.array_equal(host_u16(eb), want_b), "expert rows differ"
    log("  both outputs bit-exact after 4 overlapped rounds")
