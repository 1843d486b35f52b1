"""Pins for the CPU oracle, independent of the oracle's own code.

Each test checks the oracle against something it does not share: numbers
the pages print (tests/golden/page_facts.json), closed forms, library
routines (Python's sort, numpy float32 division and rint, torch's
float32->bfloat16 conversion), exact rational arithmetic within a proven
error bound, and invariants that determine the result uniquely.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from combine_moedc_route_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")
U = 2.0 ** -24  # unit roundoff of binary32


def facts():
    with open(GOLDEN) as f:
        return {d["name"]: d["value"] for d in json.load(f)["facts"]}


def bf16_to_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_bits_to_bf16_torch(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def slot_stride(H):
    # Slot format reading: payload H bytes, H/128 fp32 scales, padded to 512 B.
    return -(-(H + 4 * (H // 128)) // 512) * 512


# ---------------------------------------------------------------- page facts

def test_page_facts_token_bytes():
    f = facts()
    H = f["hidden"]
    assert H * 2 == f["bf16_token_kb"] * 1024            # 14 KB of BF16 per token
    algorithmic = H + 4 * (H // 128)                      # int8 payload + fp32 scales
    assert algorithmic == 7392 <= f["int8_token_kb_with_scale"] * 1024
    assert slot_stride(H) == f["int8_token_kb_with_scale"] * 1024 == 7680


def test_page_facts_static_buffer_budget():
    f = facts()
    H = f["hidden"]
    assert f["dies"] == f["routed_experts"] + f["shared_experts"] + f["redundant_experts"]
    assert f["global_batch"] == f["dies"] * f["local_batch"]
    # Separate dispatch (7.5 KiB) and combine (BF16, 14 KiB) slots for the
    # worst case where one die's expert receives the whole global batch.
    total = f["global_batch"] * (slot_stride(H) + 2 * H)
    assert total == 645 * 2 ** 20
    assert round(total / 2 ** 20) == f["static_buffers_mb_per_die"]


def test_oracle_slot_writes_exactly_payload_and_scales(orc):
    H, K = 7168, 2
    cfg = orc.Cfg(H, 4, 4, K, 0, orc.SCORE_SIGMOID_NORM, [3, 3, 3, 3])
    x = W.make_expert_out_bf16(5, 3, H)
    slots = np.array([[0, 4], [1, -1], [7, 8]], np.int32)
    sd = slot_stride(H)
    buf = np.full((12, sd), 0xA5, np.uint8)
    orc.dispatch(cfg, x, slots, 12, sd, buf=buf)
    used = {0, 4, 1, 7, 8}
    for s in range(12):
        if s in used:
            # Bytes past payload + scales keep the sentinel.
            assert (buf[s, 7392:] == 0xA5).all()
            assert (buf[s, :7392] != 0xA5).any()
        else:
            assert (buf[s] == 0xA5).all()
    # Both copies of token 0 are identical.
    assert (buf[0, :7392] == buf[4, :7392]).all()


# ---------------------------------------------------------------- top-k

def test_topk_against_python_sort(orc):
    rng = np.random.default_rng(100)
    menu = np.array([-1.0, -0.0, 0.0, 0.5, 1.0, 2.0, 1e-30, -1e-30], np.float32)
    for trial in range(3000):
        E = int(rng.integers(1, 25))
        K = int(rng.integers(1, E + 1))
        if trial % 2:
            row = menu[rng.integers(0, len(menu), E)]
        else:
            row = rng.standard_normal(E).astype(np.float32)
        want = sorted(range(E), key=lambda e: (-float(row[e]), e))[:K]
        got = orc.topk_row(row, K)
        assert list(got) == want, (row, K)


def test_topk_all_equal_rows_pick_lowest_ids(orc):
    for E, K in [(8, 2), (256, 8), (257, 9)]:
        assert list(orc.topk_row(np.zeros(E, np.float32), K)) == list(range(K))
        row = np.zeros(E, np.float32)
        row[::2] = -0.0
        assert list(orc.topk_row(row, K)) == list(range(K))


# ---------------------------------------------------------------- gates

def _route_one(orc, row, K, score_fn, shared=0):
    E = row.size
    P = E + shared
    cfg = orc.Cfg(128, E, P, K, shared, score_fn, [10] * P)
    return orc.route(cfg, row[None, :])


@pytest.mark.parametrize("seed", range(20))
def test_sigmoid_gates_closed_form(orc, seed):
    # sigmoid(ln a) = a / (1 + a), so with logits ln(a_k) the normalised gates
    # are (a_k/(1+a_k)) / sum_j (a_j/(1+a_j)).
    rng = np.random.default_rng(seed)
    E, K = 16, 5
    a = [Fraction(int(rng.integers(1, 50)), int(rng.integers(1, 50))) for _ in range(E)]
    row = np.array([math.log(float(v)) for v in a], np.float32)
    out = _route_one(orc, row, K, orc.SCORE_SIGMOID_NORM)
    ids, w = out["topk_ids"][0], out["topk_w"][0]
    s = [a[e] / (1 + a[e]) for e in ids]
    S = sum(s)
    for k in range(K):
        exact = float(s[k] / S)
        # logits carry a binary32 rounding of ln(a): relative gate error
        # <= 2*|ln a| * 2^-24, plus the final rounding.
        tol = (2 * 4.0 + 2) * U * exact
        assert abs(w[k] - exact) <= tol, (k, w[k], exact)
    assert abs(float(w.astype(np.float64).sum()) - 1.0) <= (K + 1) * U


@pytest.mark.parametrize("seed", range(20))
def test_softmax_gates_closed_form(orc, seed):
    # softmax over logits ln(n_e) is n_e / sum(n).
    rng = np.random.default_rng(1000 + seed)
    E, K = 12, 3
    n = [int(rng.integers(1, 100)) for _ in range(E)]
    row = np.array([math.log(v) for v in n], np.float32)
    out = _route_one(orc, row, K, orc.SCORE_SOFTMAX)
    ids, w = out["topk_ids"][0], out["topk_w"][0]
    tot = sum(n)
    for k in range(K):
        exact = n[ids[k]] / tot
        assert abs(w[k] - exact) <= 20 * U * exact, (k, w[k], exact)
    assert list(ids) == sorted(range(E), key=lambda e: (-n[e], e))[:K] or \
        sorted(n[e] for e in ids) == sorted(n)[-K:]


def test_gates_special_cases(orc):
    E = 16
    out = _route_one(orc, np.zeros(E, np.float32), 4, orc.SCORE_SIGMOID_NORM)
    assert (out["topk_w"][0] == np.float32(0.25)).all()
    out = _route_one(orc, np.zeros(E, np.float32), 4, orc.SCORE_SOFTMAX)
    assert (out["topk_w"][0] == np.float32(1 / 16)).all()
    out = _route_one(orc, np.full(E, 3.0, np.float32), 4, orc.SCORE_SIGMOID_NORM, shared=1)
    assert out["topk_ids"][0][-1] == E and out["topk_w"][0][-1] == 1.0
    assert list(out["topk_ids"][0][:4]) == [0, 1, 2, 3]
    # A single dominant logit under softmax takes (almost) all the mass.
    row = np.full(E, -50.0, np.float32)
    row[7] = 50.0
    out = _route_one(orc, row, 1, orc.SCORE_SOFTMAX)
    assert out["topk_ids"][0][0] == 7 and out["topk_w"][0][0] == 1.0


# ---------------------------------------------------------------- route layout

def check_route_invariants(wl, logits, out):
    """Properties that determine counts, offsets and the slot layout uniquely."""
    T, K, P = logits.shape[0], wl.K, wl.num_phys
    ids, slots = out["topk_ids"], out["slots"]
    counts, offsets = out["counts"], out["offsets"]
    cap = wl.capacity.astype(np.int64)
    assert ids.shape == (T, K) and slots.shape == (T, K)
    # Picks: brute-force top-k of the logical scores, then the replica copy.
    for t in range(T):
        row = logits[t]
        want = sorted(range(wl.num_logical), key=lambda e: (-float(row[e]), e))[:wl.top_k]
        for k, e in enumerate(want):
            if wl.replica_table is None:
                assert ids[t, k] == e
            else:
                copies = [p for p in wl.replica_table[e] if p >= 0]
                assert ids[t, k] == copies[t % len(copies)]
        if wl.num_shared:
            assert ids[t, K - 1] == P - 1
        assert len(set(ids[t].tolist())) == K
    # Histogram and its exclusive scan.
    assert (counts == np.bincount(ids.ravel(), minlength=P)).all()
    assert counts.sum() == T * K
    assert offsets[0] == 0 and (offsets[1:] == np.cumsum(counts)).all()
    # Slots: per expert, kept entries fill [base, base+min(count,cap)) in
    # ascending token order; the rest (highest tokens) are dropped.
    base = np.concatenate([[0], np.cumsum(cap)[:-1]])
    kept = slots >= 0
    assert len(set(slots[kept].tolist())) == int(kept.sum())
    total_drop = 0
    for p in range(P):
        tt, kk = np.nonzero(ids == p)          # row-major: ascending t
        n = len(tt)
        m = min(n, int(cap[p]))
        s = slots[tt, kk]
        assert (s[:m] == base[p] + np.arange(m)).all()
        assert (s[m:] == -1).all()
        total_drop += n - m
    assert out["dropped"] == total_drop == int(np.maximum(counts - cap, 0).sum())


@pytest.mark.parametrize("name,T", [("tiny", None), ("ragged", None), ("overflow", None),
                                    ("replica_shared", None), ("decode", None),
                                    ("global", 600), ("skewed", 500), ("prefill", 300)])
def test_route_invariants(orc, name, T):
    wl = W.get(name)
    _, logits = W.make_inputs(wl, T)
    out = orc.route(orc.Cfg.from_workload(wl), logits)
    check_route_invariants(wl, logits, out)
    if name == "overflow":
        assert out["dropped"] > 0


def test_route_empty(orc):
    wl = W.get("tiny")
    out = orc.route(orc.Cfg.from_workload(wl), np.zeros((0, 8), np.float32))
    assert out["counts"].sum() == 0 and out["dropped"] == 0
    assert (out["offsets"] == 0).all()


def test_route_rejects_bad_config_and_nonfinite(orc):
    assert orc.Cfg(100, 8, 8, 2, 0, 1, [4] * 8).check() != 0       # H % 128
    assert orc.Cfg(128, 8, 8, 9, 0, 1, [4] * 8).check() != 0       # K > E
    assert orc.Cfg(128, 8, 8, 2, 0, 1, [4] * 7 + [-1]).check() != 0
    dup = np.array([[0, 1], [1, -1]], np.int32)                    # phys 1 owned twice
    assert orc.Cfg(128, 2, 2, 1, 0, 1, [4, 4], dup).check() != 0
    cfg = orc.Cfg(128, 4, 4, 2, 0, 1, [4] * 4)
    with pytest.raises(ValueError):
        orc.route(cfg, np.array([[0, np.nan, 1, 2]], np.float32))


# ---------------------------------------------------------------- quantizer

def _numpy_quant(groups_bits):
    """numpy float32 division and rint: the library reference for one group."""
    x = bf16_to_f32(groups_bits)
    amax = np.abs(x).max(axis=1)
    s = amax / np.float32(127.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(x / s[:, None])
    q = np.where(s[:, None] == 0, 0, np.clip(r, -127, 127)).astype(np.int8)
    return q, s


def _all_positive_finite_bf16():
    return np.arange(0x0001, 0x7F80, dtype=np.uint16)


def test_quantizer_every_amax_sampled_x(orc):
    """Every positive finite BF16 amax, 126 sampled x with |x| <= amax."""
    rng = np.random.default_rng(7)
    amax = _all_positive_finite_bf16()
    n = amax.size
    g = np.empty((n, 128), np.uint16)
    g[:, 0] = amax
    g[:, 1] = amax | 0x8000                     # -amax
    mag = (rng.random((n, 126)) * (amax[:, None].astype(np.float64) + 1)).astype(np.uint16)
    sign = (rng.random((n, 126)) < 0.5).astype(np.uint16) << 15
    g[:, 2:] = np.minimum(mag, amax[:, None]) | sign
    q, s = orc.quantize_tokens(g)
    qn, sn = _numpy_quant(g)
    assert (s[:, 0].view(np.uint32) == sn.view(np.uint32)).all()
    assert (q == qn).all()
    # The element equal to +-amax always lands on +-127 (no flush of
    # subnormal scales).
    assert (q[:, 0] == 127).all() and (q[:, 1] == -127).all()
    # Reconstruction error bound: |q*s - x| <= s*(1/2 + 2^-16).
    x = bf16_to_f32(g).astype(np.float64)
    dq = (q.astype(np.float32) * s).astype(np.float64)
    assert (np.abs(dq - x) <= s.astype(np.float64) * (0.5 + 2.0 ** -16)).all()


@pytest.mark.parametrize("amax_bits", [0x0001, 0x0080, 0x3F80, 0x3F81, 0x4000, 0x42FE,
                                       0x0D00, 0x7F7F, 0x1234, 0x7A5A, 0x00FF, 0x3C01])
def test_quantizer_exhaustive_x_for_selected_amax(orc, amax_bits):
    """All BF16 x with |x| <= amax for selected amax values."""
    mags = np.arange(0, amax_bits + 1, dtype=np.uint32).astype(np.uint16)
    xs = np.concatenate([mags, mags | 0x8000])
    pad = (-xs.size) % 127
    xs = np.concatenate([xs, np.zeros(pad, np.uint16)]).reshape(-1, 127)
    g = np.concatenate([np.full((xs.shape[0], 1), amax_bits, np.uint16), xs], axis=1)
    q, s = orc.quantize_tokens(g)
    qn, sn = _numpy_quant(g)
    assert (s[:, 0].view(np.uint32) == sn.view(np.uint32)).all()
    assert (q == qn).all()


def test_quantizer_zero_and_nonfinite_groups(orc):
    z = np.zeros(128, np.uint16)
    z[::3] = 0x8000
    q, s = orc.quantize_group(z)
    assert s == 0 and (q == 0).all()
    bad = np.zeros(128, np.uint16)
    bad[5] = 0x7F80                             # +inf
    with pytest.raises(ValueError):
        orc.quantize_group(bad)


def test_quantizer_half_way_ties_round_to_even(orc):
    # amax = 127 -> scale exactly 1.0, so x = n + 0.5 is an exact tie.
    x = np.array([127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5] + [0.0] * 120, np.float32)
    g = f32_bits_to_bf16_torch(x)
    assert (bf16_to_f32(g) == x).all()
    q, s = orc.quantize_group(g)
    assert s == 1.0
    assert list(q[:8]) == [127, 0, 2, 2, 0, -2, -2, 126]


# ---------------------------------------------------------------- bf16 rounding

def test_f32_to_bf16_matches_torch(orc):
    hi = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000],
                    np.uint32)
    rng = np.random.default_rng(3)
    lows = np.concatenate([lows, rng.integers(0, 1 << 16, 8).astype(np.uint32)])
    bits = (hi[:, None] | lows[None, :]).ravel()
    f = bits.view(np.float32)
    ours = orc.f32_to_bf16(f)
    ref = f32_bits_to_bf16_torch(f)
    nan = np.isnan(f)
    assert (ours[~nan] == ref[~nan]).all()
    assert np.isnan(bf16_to_f32(ours[nan])).all()


# ---------------------------------------------------------------- combine

def _ulp_bf16(v):
    v = abs(v)
    if v < 2.0 ** -126:
        return 2.0 ** -133
    return 2.0 ** (math.floor(math.log2(v)) - 7)


@pytest.mark.parametrize("seed", range(6))
def test_combine_within_exact_error_bound(orc, seed):
    rng = np.random.default_rng(500 + seed)
    T, H, K, S = 24, 128, 5, 60
    cfg = orc.Cfg(H, 6, 6, K, 0, orc.SCORE_SIGMOID_NORM, [10] * 6)
    eout = W.make_expert_out_bf16(600 + seed, S, H)
    eout[:, ::7] ^= 0x8000                      # mixed signs
    eout[:, 3] = 0x8000                         # -0 column
    slots = rng.integers(0, S, (T, K)).astype(np.int32)
    slots[rng.random((T, K)) < 0.15] = -1
    slots[0, :] = -1                            # a token with every slot dropped
    w = W.make_gates(700 + seed, T, K)
    y = orc.combine(cfg, eout, orc.FMT_BF16, slots, w)
    yf = bf16_to_f32(y).astype(np.float64)
    ev = bf16_to_f32(eout)
    assert (y[0] == 0).all()                    # +0 when nothing is kept
    for t in range(T):
        for i in range(H):
            terms = [(Fraction(float(w[t, k])), Fraction(float(ev[slots[t, k], i])))
                     for k in range(K) if slots[t, k] >= 0]
            exact = sum((a * b for a, b in terms), Fraction(0))
            absum = float(sum((abs(a * b) for a, b in terms), Fraction(0)))
            bound = 0.5 * _ulp_bf16(max(abs(yf[t, i]), abs(float(exact)))) \
                + K * U * (1 + K * U) * absum
            assert abs(yf[t, i] - float(exact)) <= bound, (t, i)


def test_combine_identity_experts_recover_dequant(orc):
    """Dispatch then combine with identity experts and unit-sum weights gives
    dequant(quant(x)) exactly."""
    wl = W.get("tiny")
    H = wl.hidden
    x, _ = W.make_inputs(wl)
    T = x.shape[0]
    cfg = orc.Cfg(H, 4, 4, 2, 0, orc.SCORE_SIGMOID_NORM, [T, T, 0, 0])
    sd = slot_stride(H)
    slots = np.stack([np.arange(T), T + np.arange(T)], axis=1).astype(np.int32)
    dbuf = orc.dispatch(cfg, x, slots, 2 * T, sd)
    q, s = orc.quantize_tokens(x)
    dq = (q.astype(np.float32).reshape(T, H // 128, 128) * s[:, :, None]).reshape(T, H)
    want = f32_bits_to_bf16_torch(dq)
    cfg1 = orc.Cfg(H, 4, 4, 1, 0, orc.SCORE_SIGMOID_NORM, [T, T, 0, 0])
    y1 = orc.combine(cfg1, dbuf, orc.FMT_Q8, slots[:, :1], np.ones((T, 1), np.float32))
    assert (y1 == want).all()
    yh = orc.combine(cfg, dbuf, orc.FMT_Q8, slots, np.full((T, 2), 0.5, np.float32))
    assert (yh == want).all()
    y2 = orc.combine(cfg, dbuf, orc.FMT_Q8, slots, np.ones((T, 2), np.float32))
    assert (y2 == f32_bits_to_bf16_torch(2 * dq)).all()


def test_expert_stub_closed_form(orc):
    wl = W.get("ragged")
    H = wl.hidden
    x, logits = W.make_inputs(wl)
    cfg = orc.Cfg.from_workload(wl)
    r = orc.route(cfg, logits)
    sd = slot_stride(H)
    dbuf = orc.dispatch(cfg, x, r["slots"], wl.total_slots, sd)
    eb = orc.expert_stub(cfg, r["counts"], dbuf, sd)
    base = np.concatenate([[0], np.cumsum(wl.capacity)[:-1]])
    for p in range(wl.num_phys):
        m = np.float32(1.0) + np.float32(0.01) * np.float32(p)
        used = min(int(r["counts"][p]), int(wl.capacity[p]))
        for j in range(used):
            row = dbuf[base[p] + j]
            q = row[:H].view(np.int8).astype(np.float32)
            s = np.repeat(row[H:H + 4 * (H // 128)].view(np.float32), 128)
            want = f32_bits_to_bf16_torch((q * s) * m)
            assert (eb[base[p] + j] == want).all()


# ---------------------------------------------------------------- per-token scale

def test_page_facts_per_token_slot():
    f = facts()
    H = f["hidden"]
    assert H + 4 <= f["int8_token_kb_with_scale"] * 1024      # 7172 B
    assert -(-(H + 4) // 512) * 512 == 7680


@pytest.mark.parametrize("seed", range(4))
def test_quantizer_per_token_against_numpy(orc, seed):
    wl = W.get("decode_pt")
    x, _ = W.make_inputs(wl, 96)
    rng = np.random.default_rng(seed)
    x = x[rng.permutation(96)]
    x[3] = 0                                   # all-zero token
    x[4, :] = 0
    x[4, 17] = 0x0001                          # one subnormal element only
    q, s = orc.quantize_tokens(x, group_size=wl.hidden)
    qn, sn = _numpy_quant(x)                   # each row is one group
    assert s.shape == (96, 1)
    assert (s[:, 0].view(np.uint32) == sn.view(np.uint32)).all()
    assert (q == qn).all()
    assert s[3, 0] == 0 and (q[3] == 0).all()
    assert q[4, 17] == 127


def test_per_token_dispatch_combine_identity(orc):
    wl = W.get("decode_pt")
    H = wl.hidden
    x, _ = W.make_inputs(wl)
    T = x.shape[0]
    cfg = orc.Cfg(H, 4, 4, 1, 0, orc.SCORE_SIGMOID_NORM, [T, 0, 0, 0], group_size=H)
    sd = -(-(H + 4) // 512) * 512
    slots = np.arange(T, dtype=np.int32)[:, None]
    dbuf = orc.dispatch(cfg, x, slots, T, sd)
    q, s = orc.quantize_tokens(x, group_size=H)
    assert (dbuf[:, :H].view(np.int8) == q).all()
    assert (dbuf[:, H:H + 4].view(np.float32)[:, 0] == s[:, 0]).all()
    y = orc.combine(cfg, dbuf, orc.FMT_Q8, slots, np.ones((T, 1), np.float32))
    assert (y == f32_bits_to_bf16_torch(q.astype(np.float32) * s)).all()


# ---------------------------------------------------------------- expert W8A8 linear

def _expert_setup(orc, H, gs, T=20, P=3, seed=0):
    wl = W.Workload("e", "", T, H, P, P, 1, 0, W.SCORE_SIGMOID_NORM,
                    np.full(P, T, np.int32), None, seed, "normal", group_size=gs)
    cfg = orc.Cfg.from_workload(wl)
    x, _ = W.make_inputs(wl)
    sd = -(-(H + 4 * (H // gs)) // 512) * 512
    counts = np.array([T, T // 2, 0][:P], np.int32)
    slots = np.full((T, 1), -1, np.int32)
    slots[:, 0] = np.arange(T)                          # expert 0 window
    dbuf = orc.dispatch(cfg, x, slots, P * T, sd)
    if P > 1:
        dbuf[T:T + T // 2] = dbuf[:T // 2]              # expert 1 holds copies
    return cfg, x, dbuf, sd, counts


@pytest.mark.parametrize("H,gs", [(256, 128), (384, 384), (512, 128)])
def test_expert_w8a8_exact_bound(orc, H, gs):
    cfg, x, dbuf, sd, counts = _expert_setup(orc, H, gs)
    Wt, ws = W.make_expert_weights(3, 3, H)
    y = orc.expert_w8a8(cfg, counts, dbuf, sd, Wt, ws)
    G = H // gs
    T = x.shape[0]
    for p, base, n_rows in ((0, 0, counts[0]), (1, T, counts[1])):
        q = dbuf[base:base + n_rows, :H].view(np.int8).astype(np.int64)
        sx = dbuf[base:base + n_rows, H:H + 4 * G].view(np.float32).astype(np.float64)
        isum = np.stack([q[:, g * gs:(g + 1) * gs] @ Wt[p][:, g * gs:(g + 1) * gs].T.astype(np.int64)
                         for g in range(G)], axis=2)    # [rows][n][g], exact
        exact = (isum * sx[:, None, :]).sum(2) * ws[p].astype(np.float64)[None, :]
        mag = (np.abs(isum) * np.abs(sx[:, None, :])).sum(2) * ws[p][None, :]
        got = bf16_to_f32(y[base:base + n_rows]).astype(np.float64)
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(got), 1e-30))) - 7)
        assert (np.abs(got - exact) <= 0.5 * ulp + (G + 2) * U * mag + 1e-38).all()
    assert (y[2 * T:] == 0).all()                       # expert 2 has no tokens


def test_expert_w8a8_identity_weights_give_dequant(orc):
    H, gs = 256, 128
    cfg, x, dbuf, sd, counts = _expert_setup(orc, H, gs)
    Wt = np.zeros((3, H, H), np.int8)
    Wt[:, np.arange(H), np.arange(H)] = 1
    y = orc.expert_w8a8(cfg, counts, dbuf, sd, Wt, np.ones((3, H), np.float32))
    n = counts[0]
    q = dbuf[:n, :H].view(np.int8).astype(np.float32)
    s = np.repeat(dbuf[:n, H:H + 8].view(np.float32), gs, axis=1)
    assert (y[:n] == f32_bits_to_bf16_torch(q * s)).all()


def test_expert_w8a8_single_weight_picks_one_input(orc):
    H, gs = 256, 128
    cfg, x, dbuf, sd, counts = _expert_setup(orc, H, gs)
    Wt = np.zeros((3, H, H), np.int8)
    Wt[0, 7, 200] = 1                                   # out channel 7 <- input 200
    ws = np.full((3, H), 2.0, np.float32)
    y = orc.expert_w8a8(cfg, counts, dbuf, sd, Wt, ws)
    n = counts[0]
    q = dbuf[:n, 200].view(np.int8).astype(np.float32)
    s = dbuf[:n, H + 4:H + 8].view(np.float32)[:, 0]    # group 1 holds input 200
    assert (y[:n, 7] == f32_bits_to_bf16_torch((s * q) * np.float32(2.0))).all()
    assert (np.delete(y[:n], 7, axis=1) == 0).all()


def test_expert_w8a8_per_token_large_sum_rounds_like_float32(orc):
    H = 2048                                             # isum up to 33e6 > 2^24
    cfg, x, dbuf, sd, counts = _expert_setup(orc, H, H, T=4, P=1)
    dbuf[:, :H] = np.uint8(127)
    dbuf[1, 5] = np.uint8(126)                           # make the sums odd-ish
    dbuf[:, H:H + 4] = np.frombuffer(np.float32(0.75).tobytes(), np.uint8)
    Wt = np.full((1, H, H), 127, np.int8)
    Wt[0, 3, :9] = 125
    ws = np.full((1, H), 1.0 / 3, np.float32)
    y = orc.expert_w8a8(cfg, np.array([4], np.int32), dbuf, sd, Wt, ws)
    isum = dbuf[:4, :H].view(np.int8).astype(np.int64) @ Wt[0].T.astype(np.int64)
    want = f32_bits_to_bf16_torch((np.float32(0.75) * isum.astype(np.float32)) * ws[0][None, :])
    assert (y == want).all()


def test_expert_w8a8_per_token_random_large_sums(orc):
    H = 4096                                             # |isum| well beyond 2^24
    cfg, x, dbuf, sd, counts = _expert_setup(orc, H, H, T=6, P=1, seed=5)
    rng = np.random.default_rng(9)
    dbuf[:, :H] = rng.integers(100, 128, (6, H)).astype(np.int8).view(np.uint8)
    Wt = rng.integers(100, 128, (1, H, H)).astype(np.int8)
    ws = np.full((1, H), 0.001, np.float32)
    y = orc.expert_w8a8(cfg, np.array([6], np.int32), dbuf, sd, Wt, ws)
    isum = dbuf[:6, :H].view(np.int8).astype(np.int64) @ Wt[0].T.astype(np.int64)
    sx = dbuf[:6, H:H + 4].view(np.float32)
    want = f32_bits_to_bf16_torch((sx * isum.astype(np.float32)) * ws[0][None, :])
    assert (y == want).all()
