"""The trace build (libmoedc_trace.so, include/moedc_trace.h): dispatch with
per-wave phase stamps writes the same bytes as libmoedc.so, and on the
30720-token batch every wave leaves a complete, ordered record."""
import os
import sys

import numpy as np
import pytest
import torch

from combine_moedc_route_amd import build as B
from combine_moedc_route_amd import moedc as M
from combine_moedc_route_amd import workloads as W

from gpu_common import log

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

pytestmark = pytest.mark.gpu


def _dispatch_bytes(lib_path, wl, xd, logits, trace=False):
    """The dispatch buffer after route + dispatch with the library at
    `lib_path` (the trace build with tracing on when `trace`)."""
    import ctypes as C
    prev = M._lib
    M._lib = M.load_library(lib_path)
    try:
        plan = M.Plan.from_workload(wl)
        b = plan.alloc("cuda:0")
        b["dispatch_buf"].fill_(0x5A)
        plan.route(logits, b["topk_ids"], b["topk_w"], b["counts"], b["offsets"], b["slots"],
                   b["dropped"], b["workspace"])
        tr = None
        if trace:
            M._lib.moedc_trace_set.argtypes = [C.c_void_p, C.c_int64]
            tr = torch.zeros((wl.tokens * (-(-wl.hidden // 512)), 8), dtype=torch.int64,
                             device="cuda")
            torch.cuda.synchronize()
            assert M._lib.moedc_trace_set(tr.data_ptr(), tr.numel() * 8) == 0
        plan.dispatch(xd, b["slots"], b["dispatch_buf"])
        torch.cuda.synchronize()
        if trace:
            M._lib.moedc_trace_set(None, 0)
            assert (tr[:, 2] > 0).all(), "a wave left no record"
        out = b["dispatch_buf"].cpu().numpy()
        del plan, b, tr
    finally:
        M._lib = prev
    return out


@pytest.mark.parametrize("name", ["mid", "decode_pt"])
def test_trace_build_writes_the_same_bytes(name):
    wl = W.get(name)
    x, logits = W.make_inputs(wl)
    log(f"[case] trace build vs library, {name}")
    xd, lg = torch.from_numpy(x.view(np.int16)).cuda(), torch.from_numpy(logits).cuda()
    a = _dispatch_bytes(M.LIB_PATH, wl, xd, lg)
    b = _dispatch_bytes(B.TRACE_LIB, wl, xd, lg, trace=True)
    assert np.array_equal(a, b)


def test_dispatch_trace_records_every_wave():
    log("[case] dispatch trace, global batch")
    r = bench.dispatch_trace("global")
    assert r["records_complete"] and r["stamps_monotone"], r
    assert r["waves"] == 30720 * 14
    assert 0 < r["span_us"] < 5000
    log(f"  span {r['span_us']:.1f} us on {r['cus']} CUs, resident waves per CU "
        f"{r['resident_waves_per_cu_mean']:.1f}, loading+storing together "
        f"{r['frac_busy_cu_samples_loading_and_storing']:.2f}")
