"""Property test of plan validation and sizing through the C ABI (no GPU).

Hypothesis draws a valid layer description (shapes, scale groups, shared
expert, replica tables), then applies at most one documented violation.  A
valid description must give MOEDC_OK and the sizes moedc.h defines; each
single violation must give the status the header assigns to it and no plan.
"""
import ctypes as C

import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

from combine_moedc_route_amd import moedc as M

INT32_MAX = 2 ** 31 - 1


@st.composite
def valid_layer(draw):
    H = 128 * draw(st.integers(1, 64))
    gs = draw(st.sampled_from([128, H]))
    shared = draw(st.integers(0, 1))
    E = draw(st.integers(1, 200))
    R = draw(st.integers(1, 8))
    table = None
    extra = 0
    if R > 1 or draw(st.booleans()):
        # every logical expert gets 1..R copies on distinct physical ids
        copies = [draw(st.integers(1, R)) for _ in range(E)]
        ids = draw(st.permutations(list(range(sum(copies)))))
        table = np.full((E, R), -1, np.int32)
        pos = 0
        for e, c in enumerate(copies):
            table[e, :c] = ids[pos:pos + c]
            pos += c
        extra = sum(copies) - E
    P = E + extra + shared
    if P > 1024:
        return None
    KR = draw(st.integers(1, min(E, 16 - shared)))
    cap = draw(st.lists(st.integers(0, 5000), min_size=P, max_size=P))
    return dict(max_tokens=draw(st.integers(0, 1 << 24)), hidden=H, group_size=gs,
                num_logical=E, num_phys=P, top_k=KR, num_shared=shared,
                score_fn=draw(st.integers(0, 1)), max_replicas=R,
                capacity=np.array(cap, np.int32), replica_table=table)


# (name, how to break a valid layer, expected status)
MUTATIONS = [
    ("hidden not a multiple of 128", lambda d: d.update(hidden=d["hidden"] + 64), M.ERR_INVALID_ARG),
    ("hidden <= 0", lambda d: d.update(hidden=0), M.ERR_INVALID_ARG),
    ("group size 64", lambda d: d.update(group_size=64), M.ERR_UNSUPPORTED),
    ("negative max_tokens", lambda d: d.update(max_tokens=-1), M.ERR_INVALID_ARG),
    ("max_tokens above 2^24", lambda d: d.update(max_tokens=(1 << 24) + 1), M.ERR_UNSUPPORTED),
    ("two shared experts", lambda d: d.update(num_shared=2), M.ERR_INVALID_ARG),
    ("top_k 0", lambda d: d.update(top_k=0), M.ERR_INVALID_ARG),
    ("top_k above E_log", lambda d: d.update(top_k=d["num_logical"] + 1), M.ERR_INVALID_ARG),
    ("bad score function", lambda d: d.update(score_fn=2), M.ERR_INVALID_ARG),
    ("negative capacity", lambda d: d["capacity"].__setitem__(0, -1), M.ERR_INVALID_ARG),
    ("capacities past 2^31", lambda d: d["capacity"].__setitem__(slice(None), INT32_MAX // 2 + 1)
     if len(d["capacity"]) > 1 else d["capacity"].__setitem__(0, -1), None),
]


def status_of(d):
    cap = np.ascontiguousarray(d["capacity"], np.int32)
    tab = d["replica_table"]
    tab_p = (np.ascontiguousarray(tab, np.int32).ctypes.data_as(C.POINTER(C.c_int32))
             if tab is not None else None)
    R = d.get("max_replicas", 1 if tab is None else tab.shape[1])
    cfg = M.Config(d["max_tokens"], d["hidden"], d["group_size"], d["num_logical"],
                   d["num_phys"], d["top_k"], d["num_shared"], d["score_fn"], R,
                   cap.ctypes.data_as(C.POINTER(C.c_int32)), tab_p)
    h = C.c_void_p(12345)
    st_ = M.lib().moedc_plan_create(C.byref(cfg), C.byref(h))
    sizes = None
    if st_ == M.OK:
        sizes = M.Sizes()
        assert M.lib().moedc_plan_sizes(h, C.byref(sizes)) == M.OK
        M.lib().moedc_plan_destroy(h)
    else:
        assert not h.value, "a failed plan_create must leave *out NULL"
    return st_, sizes


@settings(max_examples=300, deadline=None)
@given(valid_layer(), st.integers(-1, len(MUTATIONS) - 1))
def test_plan_validation_and_sizes(layer, which):
    if layer is None:
        return
    d = dict(layer, capacity=layer["capacity"].copy())
    expected = M.OK
    if which >= 0:
        name, mutate, expected = MUTATIONS[which]
        mutate(d)
        if expected is None:  # sum of capacities past INT32_MAX, or the fallback above
            expected = (M.ERR_UNSUPPORTED if (d["capacity"] >= 0).all() else M.ERR_INVALID_ARG)
    st_, sz = status_of(d)
    assert st_ == expected, (MUTATIONS[which][0] if which >= 0 else "valid", st_)
    if st_ != M.OK:
        return
    H, G = d["hidden"], d["hidden"] // d["group_size"]
    total = int(d["capacity"].astype(np.int64).sum())
    stride = -(-(H + 4 * G) // 512) * 512
    assert sz.total_slots == total
    assert sz.slot_stride == stride and sz.combine_slot_stride == 2 * H
    assert sz.dispatch_buf_bytes == total * stride and sz.combine_buf_bytes == total * 2 * H
    assert sz.k == d["top_k"] + d["num_shared"] and sz.num_groups == G
    assert sz.workspace_bytes > 0 and sz.workspace_bytes % 256 == 0


@settings(max_examples=200, deadline=None)
@given(valid_layer(), st.data())
def test_replica_tables_that_break_the_rules_are_refused(layer, data):
    if layer is None or layer["replica_table"] is None:
        return
    d = dict(layer, capacity=layer["capacity"].copy())
    tab = layer["replica_table"].copy()
    E, R = tab.shape
    routed = d["num_phys"] - d["num_shared"]
    kind = data.draw(st.sampled_from(["id past routed", "repeated id", "hole", "empty row"]))
    e = data.draw(st.integers(0, E - 1))
    if kind == "id past routed":
        tab[e, 0] = routed
    elif kind == "repeated id":
        if E < 2:
            return
        f = (e + 1) % E
        tab[e, 0] = tab[f, 0]
    elif kind == "hole":  # -1 followed by a copy
        if R < 2:
            return
        tab[e, 0], tab[e, 1] = -1, tab[e, 0]
    else:
        tab[e, :] = -1
    d["replica_table"] = tab
    assert status_of(d)[0] == M.ERR_INVALID_ARG, kind
