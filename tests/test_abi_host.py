"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/moedc.h declares, and its host-side validation and sizing behave as
documented.  No call here reaches a kernel launch."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from combine_moedc_route_amd import moedc as M
from combine_moedc_route_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moedc.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moedc_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = M.lib()
    names = declared_functions()
    assert set(names) == set(M.EXPORTS), names
    for n in names:
        assert getattr(L, n) is not None


def test_ceiling_library_exports_every_declared_symbol():
    """libmoedc_ceiling.so (the benchmark's bandwidth-ceiling kernels) loads
    and exports what include/moedc_ceiling.h declares."""
    names = declared_functions(os.path.join(ROOT, "include", "moedc_ceiling.h"))
    assert names == ["moedc_ceiling_copy", "moedc_ceiling_gather", "moedc_ceiling_mfma",
                     "moedc_ceiling_read", "moedc_ceiling_scatter", "moedc_ceiling_write"]
    L = C.CDLL(os.path.join(ROOT, "combine_moedc_route_amd", "libmoedc_ceiling.so"))
    for n in names:
        assert getattr(L, n) is not None


def test_trace_library_exports_the_library_and_its_trace_call():
    """libmoedc_trace.so (dispatch with per-wave phase stamps) exports every
    symbol of include/moedc.h and moedc_trace_set (include/moedc_trace.h);
    libmoedc.so does not carry the trace call."""
    from combine_moedc_route_amd import build as B
    assert declared_functions(os.path.join(ROOT, "include", "moedc_trace.h")) == ["moedc_trace_set"]
    T = C.CDLL(B.TRACE_LIB)
    for n in declared_functions() + ["moedc_trace_set"]:
        assert getattr(T, n) is not None
    with pytest.raises(AttributeError):
        getattr(M.lib(), "moedc_trace_set")


def test_status_strings():
    for s in range(7):
        assert M.status_string(s)
    assert M.status_string(99) == "unknown status"


def plan_status(**kw):
    base = dict(max_tokens=64, hidden=256, group_size=128, num_logical=8, num_phys=8,
                top_k=2, num_shared=0, score_fn=1, capacity=[64] * 8, replica_table=None)
    base.update(kw)
    try:
        M.Plan(**base)
        return M.OK
    except M.MoedcError as e:
        return e.status


def test_plan_validation():
    assert plan_status() == M.OK
    assert plan_status(group_size=64) == M.ERR_UNSUPPORTED
    assert plan_status(group_size=256) == M.OK                      # one scale per token
    assert plan_status(hidden=200) == M.ERR_INVALID_ARG
    assert plan_status(hidden=8192 + 128) == M.ERR_UNSUPPORTED
    assert plan_status(top_k=0) == M.ERR_INVALID_ARG
    assert plan_status(top_k=9) == M.ERR_INVALID_ARG
    assert plan_status(num_shared=2) == M.ERR_INVALID_ARG
    assert plan_status(score_fn=7) == M.ERR_INVALID_ARG
    assert plan_status(capacity=[64] * 7 + [-1]) == M.ERR_INVALID_ARG
    assert plan_status(num_phys=7, capacity=[1] * 7) == M.ERR_INVALID_ARG  # E_phys < E_log
    assert plan_status(max_tokens=-1) == M.ERR_INVALID_ARG
    assert plan_status(num_logical=2000, num_phys=2000, capacity=[1] * 2000) == M.ERR_UNSUPPORTED
    assert plan_status(num_logical=20, num_phys=20, top_k=17,
                       capacity=[1] * 20) == M.ERR_UNSUPPORTED  # K > 16
    rep = np.array([[0, 8], [1, -1], [2, -1], [3, -1], [4, -1], [5, -1], [6, -1], [7, -1]])
    assert plan_status(num_phys=9, capacity=[4] * 9, replica_table=rep) == M.OK
    bad = rep.copy()
    bad[1, 1] = 8                                   # physical id owned twice
    assert plan_status(num_phys=9, capacity=[4] * 9, replica_table=bad) == M.ERR_INVALID_ARG
    bad = rep.copy()
    bad[2, 0] = 9                                   # out of range
    assert plan_status(num_phys=9, capacity=[4] * 9, replica_table=bad) == M.ERR_INVALID_ARG
    bad = rep.copy()
    bad[3, 1] = -2                                  # padding must be -1
    assert plan_status(num_phys=9, capacity=[4] * 9, replica_table=bad) == M.ERR_INVALID_ARG
    # shared expert must stay outside the routed range
    assert plan_status(num_phys=9, num_shared=1, capacity=[4] * 9, replica_table=rep) == \
        M.ERR_INVALID_ARG


def test_plan_sizes_match_page_slot_format():
    wl = W.get("global")
    p = M.Plan.from_workload(wl)
    s = p.sizes
    assert s.slot_stride == 7680                    # 7.5 KiB per INT8 token slot
    assert s.combine_slot_stride == 14336           # 14 KiB per BF16 token
    assert s.total_slots == 256 * 1920
    assert s.dispatch_buf_bytes == 256 * 1920 * 7680
    assert s.combine_buf_bytes == 256 * 1920 * 14336
    assert s.k == 8 and s.num_groups == 56
    assert s.workspace_bytes >= 4 * 256 * (30720 // 256)
    # The pages' per-die budget: 30720-slot windows of both buffers = 645 MiB.
    assert 30720 * (s.slot_stride + s.combine_slot_stride) == 645 * 2 ** 20
    s = M.Plan.from_workload(W.get("decode_pt")).sizes
    assert s.num_groups == 1 and s.slot_stride == 7680               # 7172 B -> 7.5 KiB
    for name in ("tiny", "ragged", "prefill", "skewed", "replica_shared"):
        wl = W.get(name)
        s = M.Plan.from_workload(wl).sizes
        G = wl.hidden // 128
        assert s.slot_stride % 512 == 0 and wl.hidden + 4 * G <= s.slot_stride < wl.hidden + 4 * G + 512
        assert s.total_slots == wl.total_slots and s.k == wl.K


def test_call_validation_returns_before_launch():
    L = M.lib()
    wl = W.get("tiny")
    p = M.Plan.from_workload(wl)
    h = p._h
    a16, a1 = 0x10000, 0x10001                      # never dereferenced
    st = L.moedc_route(h, 65, a16, a16, a16, a16, a16, a16, a16, a16, None)
    assert st == M.ERR_SHAPE
    st = L.moedc_route(h, -1, a16, a16, a16, a16, a16, a16, a16, a16, None)
    assert st == M.ERR_SHAPE
    st = L.moedc_route(h, 4, None, a16, a16, a16, a16, a16, a16, a16, None)
    assert st == M.ERR_INVALID_ARG
    st = L.moedc_route(h, 4, a1, a16, a16, a16, a16, a16, a16, a16, None)
    assert st == M.ERR_ALIGN
    st = L.moedc_route(None, 4, a16, a16, a16, a16, a16, a16, a16, a16, None)
    assert st == M.ERR_INVALID_ARG
    assert L.moedc_dispatch(h, 0, None, None, None, None) == M.OK       # empty: no-op
    assert L.moedc_dispatch(h, 65, a16, a16, a16, None) == M.ERR_SHAPE
    assert L.moedc_dispatch(h, 3, a1, a16, a16, None) == M.ERR_ALIGN
    assert L.moedc_dispatch(h, 3, a16, a16, a1 + 7, None) == M.ERR_ALIGN
    assert L.moedc_dispatch(h, 3, a16, None, a16, None) == M.ERR_INVALID_ARG
    assert L.moedc_combine(h, 0, None, M.FMT_BF16, None, None, None, None) == M.OK
    assert L.moedc_combine(h, 3, a16, 5, a16, a16, a16, None) == M.ERR_INVALID_ARG
    assert L.moedc_combine(h, 3, a16, M.FMT_Q8, a16, a16, a1, None) == M.ERR_ALIGN
    assert L.moedc_combine(h, 99, a16, M.FMT_Q8, a16, a16, a16, None) == M.ERR_SHAPE
    assert L.moedc_expert_stub(h, a16, a16, a16, None, None) == M.ERR_INVALID_ARG
    assert L.moedc_combine_limited(h, 3, a16, M.FMT_BF16, a16, a16, a16, 0, None) == \
        M.ERR_INVALID_ARG
    assert L.moedc_route_dispatch(h, 65, a16, a16, a16, a16, a16, a16, a16, a16, a16, a16,
                                  None) == M.ERR_SHAPE
    assert L.moedc_route_dispatch(h, 3, a16, a1, a16, a16, a16, a16, a16, a16, a16, a16,
                                  None) == M.ERR_ALIGN
    assert L.moedc_plan_bind_workspace(h, a1, None) == M.ERR_ALIGN
    # the workspace-free route validates like moedc_route
    assert L.moedc_route_noalloc(h, 65, a16, a16, a16, a16, a16, a16, a16, None) == M.ERR_SHAPE
    assert L.moedc_route_noalloc(h, 4, None, a16, a16, a16, a16, a16, a16, None) == \
        M.ERR_INVALID_ARG
    assert L.moedc_route_noalloc(h, 4, a1, a16, a16, a16, a16, a16, a16, None) == M.ERR_ALIGN
    assert L.moedc_route_noalloc(None, 4, a16, a16, a16, a16, a16, a16, a16, None) == \
        M.ERR_INVALID_ARG
    assert L.moedc_plan_sizes(None, None) == M.ERR_INVALID_ARG
    out = C.c_void_p(123)
    assert L.moedc_plan_create(None, C.byref(out)) == M.ERR_INVALID_ARG and not out.value
    L.moedc_plan_destroy(None)


def test_binding_refuses_undersized_or_mistyped_tensors():
    """The C ABI sees only addresses, so the binding checks each tensor's
    element size and extent against the plan before the call (the checks
    run before the device check, so CPU tensors exercise them)."""
    import torch
    wl = W.get("tiny")
    p = M.Plan.from_workload(wl)
    T, K, P, H, E = wl.tokens, wl.K, wl.num_phys, wl.hidden, wl.num_logical
    s = p.sizes
    i32, f32 = dict(dtype=torch.int32), dict(dtype=torch.float32)

    def route_args(**over):
        a = dict(logits=torch.empty((T, E), **f32), topk_ids=torch.empty((T, K), **i32),
                 topk_w=torch.empty((T, K), **f32), counts=torch.empty(P, **i32),
                 offsets=torch.empty(P + 1, **i32), slots=torch.empty((T, K), **i32),
                 dropped=torch.empty(1, **i32),
                 workspace=torch.empty(s.workspace_bytes, dtype=torch.uint8))
        a.update(over)
        return a

    with pytest.raises(ValueError, match="libmoedc takes device tensors"):
        p.route(**route_args())                  # sizes pass, then the device check
    for name, bad in [("offsets", torch.empty(P, **i32)),
                      ("slots", torch.empty((T, K - 1), **i32)),
                      ("workspace", torch.empty(s.workspace_bytes - 1, dtype=torch.uint8)),
                      ("topk_w", torch.empty((T, K), dtype=torch.float16))]:
        with pytest.raises(ValueError, match=name):
            p.route(**route_args(**{name: bad}))
    with pytest.raises(ValueError, match="dispatch_buf"):
        p.dispatch(torch.empty((T, H), dtype=torch.int16), torch.empty((T, K), **i32),
                   torch.empty(s.dispatch_buf_bytes - 512, dtype=torch.uint8))
    with pytest.raises(ValueError, match="expert_out"):
        p.combine(torch.empty(s.combine_buf_bytes - 2, dtype=torch.uint8), M.FMT_BF16,
                  torch.empty((T, K), **i32), torch.empty((T, K), **f32),
                  torch.empty((T, H), dtype=torch.int16))
    with pytest.raises(ValueError, match="^y: needs"):
        p.combine(torch.empty(s.combine_buf_bytes, dtype=torch.uint8), M.FMT_BF16,
                  torch.empty((T + 1, K), **i32), torch.empty((T + 1, K), **f32),
                  torch.empty((T, H), dtype=torch.int16), num_tokens=T + 1)


def test_product_path_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(M, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(M, "_lib", None)
    with pytest.raises(M.MoedcUnavailable):
        M.lib()


def test_product_package_does_not_import_oracle():
    pkg = os.path.join(ROOT, "combine_moedc_route_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "moedc_oracle" not in text, f


def test_route_noalloc_refuses_batches_beyond_its_array():
    """A batch whose per-block counts (4 B per 64 tokens and physical expert)
    exceed the static array (16 MiB minus 64 KiB of tables) is refused with
    UNSUPPORTED before any device call; the largest batch that fits is not."""
    L = M.lib()
    P = 1024
    p = M.Plan(max_tokens=1 << 24, hidden=128, num_logical=P, num_phys=P, top_k=2,
               capacity=np.full(P, 64, np.int32))
    a16 = 0x10000
    fits = ((16 << 20) - (64 << 10)) // (4 * P) * 64       # tokens whose counts just fit
    st = L.moedc_route_noalloc(p._h, fits + 64, a16, a16, a16, a16, a16, a16, a16, None)
    assert st == M.ERR_UNSUPPORTED
    st = L.moedc_route_noalloc(p._h, 1 << 24, a16, a16, a16, a16, a16, a16, a16, None)
    assert st == M.ERR_UNSUPPORTED
