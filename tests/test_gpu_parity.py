"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Integer, index and byte outputs must match bit for bit;
gates within the derived fp32 tolerance; combine output within 1 BF16 ulp
(and is expected to be bit-identical: same operations, same order)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from combine_moedc_route_amd import moedc as M
from combine_moedc_route_amd import workloads as W

from gpu_common import (SENTINEL, U, assert_within_gate_bound, bf16_to_f32, check_dispatch_tokens,
                        check_dispatch_untouched, compare_route, dev, dev_i16,
                        expected_dispatch_buffer,
                        gpu_dispatch, gpu_route, host_u16, log,
                        ulp_diff_bf16)

pytestmark = pytest.mark.gpu

SMALL = ["tiny", "decode", "decode_pt", "mid", "ragged", "overflow", "replica_shared"]
FULL = ["global", "skewed", "prefill"]


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def setup(name, tokens=None):
    wl = W.get(name)
    log(f"[case] {name} T={wl.tokens if tokens is None else tokens} H={wl.hidden} "
        f"E={wl.num_logical}/{wl.num_phys} K={wl.K}")
    x, logits = W.make_inputs(wl, tokens)
    plan = M.Plan.from_workload(wl)
    cfg = oracle.Cfg.from_workload(wl)
    return wl, x, logits, plan, cfg


# ------------------------------------------------------------------ route

@pytest.mark.parametrize("name", SMALL + FULL)
def test_route_parity(name):
    wl, x, logits, plan, cfg = setup(name)
    want = oracle.route(cfg, logits)
    got, _ = gpu_route(plan, wl, logits)
    rel = compare_route(wl, got, want)
    log(f"  route bit-exact; max gate rel err {rel:.3g}; dropped {got['dropped']}")
    if name in FULL:
        assert want["dropped"] == 0


def test_route_empty_and_ragged_token_counts():
    wl, _, _, plan, cfg = setup("mid")
    got, _ = gpu_route(plan, wl, np.zeros((0, wl.num_logical), np.float32))
    assert (got["counts"] == 0).all() and (got["offsets"] == 0).all() and got["dropped"] == 0
    for T in (1, 63, 64, 65, 255, 256, 257, 999):
        _, logits = W.make_inputs(wl, T)
        compare_route(wl, gpu_route(plan, wl, logits)[0], oracle.route(cfg, logits))


@pytest.mark.parametrize("T", [700, 200])   # large- and small-batch route kernels
@pytest.mark.parametrize("score_fn", [W.SCORE_SOFTMAX, W.SCORE_SIGMOID_NORM])
def test_route_ties_signed_zeros_and_degenerate_rows(score_fn, T):
    rng = np.random.default_rng(77)
    E, K = 64, 8
    menu = np.array([-1.0, -0.0, 0.0, 0.25, 1.0, 2.0], np.float32)
    logits = menu[rng.integers(0, len(menu), (T, E))]
    logits[:50] = 0.0                          # all-equal rows -> ids 0..K-1
    logits[50:100] = -0.0
    logits[100:150, ::2] = -0.0                # +-0 mixed: equal keys
    wl = W.Workload("ties", "", T, 128, E, E, K, 0, score_fn,
                    np.full(E, T, np.int32), None, 0, "normal")
    plan = M.Plan.from_workload(wl)
    want = oracle.route(oracle.Cfg.from_workload(wl), logits)
    compare_route(wl, gpu_route(plan, wl, logits)[0], want)
    assert (want["topk_ids"][:100] == np.arange(K)).all()
    # one expert, top-1
    wl1 = W.Workload("one", "", 130, 128, 1, 1, 1, 0, score_fn,
                     np.array([100], np.int32), None, 0, "normal")
    lg = rng.standard_normal((130, 1)).astype(np.float32)
    want = oracle.route(oracle.Cfg.from_workload(wl1), lg)
    got = gpu_route(M.Plan.from_workload(wl1), wl1, lg)[0]
    compare_route(wl1, got, want)
    assert got["dropped"] == 30


def _near_tie_rows(T, E, K, seed):
    """Rows of E logits where picks share the packed key's high part: values
    that differ only in the low 8 bits of their order key (a few ulps apart),
    exactly equal values at several ids, and +-0 at the boundary.  Each row
    draws one case: 0 all K picks a few ulps apart; 1 the last pick decided
    among 3 near-equal values; 2 the last 4 picks decided among 6; 3 equal
    values at several ids across the boundary; 4 +0 and -0 across the
    boundary; 5 plain normal logits."""
    rng = np.random.default_rng(seed)
    lg = (0.1 * rng.standard_normal((T, E))).astype(np.float32)
    base = np.float32(2.0).view(np.uint32)
    case = rng.integers(0, 6, T)
    for t in range(T):
        cols = rng.permutation(E)
        c = case[t]
        if c == 0:
            d = rng.choice(256, K + 2, replace=False)
            lg[t, cols[:K + 2]] = (base + d).astype(np.uint32).view(np.float32)
        elif c in (1, 2):
            big = K - 1 if c == 1 else K - 4
            lg[t, cols[:big]] = 3.0 + np.arange(big, dtype=np.float32)
            n = 3 if c == 1 else 6
            d = rng.choice(256, n, replace=False)
            lg[t, cols[big:big + n]] = (base + d).astype(np.uint32).view(np.float32)
        elif c == 3:
            lg[t, cols[:K - 2]] = 3.0 + np.arange(K - 2, dtype=np.float32)
            lg[t, cols[K - 2:K + 3]] = 2.0
        elif c == 4:
            lg[t] = -np.abs(lg[t]) - 1.0
            lg[t, cols[:K - 3]] = 1.0 + np.arange(K - 3, dtype=np.float32)
            lg[t, cols[K - 3:K + 3:2]] = 0.0
            lg[t, cols[K - 2:K + 3:2]] = -0.0
    return lg


@pytest.mark.parametrize("T", [700, 300])
@pytest.mark.parametrize("score_fn", [W.SCORE_SOFTMAX, W.SCORE_SIGMOID_NORM])
def test_route_near_ties_on_256_expert_rows(score_fn, T):
    """Rows of 256 logits (the one-chunk rows of the large-batch route) with
    picks whose packed keys tie: the exact order is (value desc, id asc),
    and the sigmoid gates are normalised by the sum in that order."""
    E, K = 256, 8
    logits = _near_tie_rows(T, E, K, 31 + T)
    wl = W.Workload("near-ties", "", T, 128, E, E, K, 0, score_fn,
                    np.full(E, T, np.int32), None, 0, "normal")
    want = oracle.route(oracle.Cfg.from_workload(wl), logits)
    log(f"[case] near ties E=256 T={T} score_fn={score_fn}")
    compare_route(wl, gpu_route(M.Plan.from_workload(wl), wl, logits)[0], want)
    # with a shared expert and a replica table on the same rows
    P = E + 17
    rep = np.full((E, 2), -1, np.int32)
    rep[:, 0] = np.arange(E)
    rep[:16, 1] = E + np.arange(16)
    wl2 = W.Workload("near-ties-rep", "", T, 128, E, P, K, 1, score_fn,
                     np.full(P, T, np.int32), rep, 0, "normal")
    want = oracle.route(oracle.Cfg.from_workload(wl2), logits)
    compare_route(wl2, gpu_route(M.Plan.from_workload(wl2), wl2, logits)[0], want)


@pytest.mark.parametrize("T", [1, 77, 256, 300])
def test_route_widest_config(T):
    """1024 experts (16 logits per lane in the small-batch kernel), 15 routed
    picks + a shared expert, 3-copy replicas of the first 10 experts."""
    E, K, R = 1000, 15, 3
    rep = np.full((E, R), -1, np.int32)
    rep[:, 0] = np.arange(E)
    extra = E
    for e in range(10):
        rep[e, 1:] = [extra, extra + 1]
        extra += 2
    P = extra + 1                                   # + shared expert
    assert P <= 1024
    cap = np.full(P, max(4, T // 40), np.int32)     # some experts overflow
    cap[-1] = T
    wl = W.Workload("wide", "", T, 128, E, P, K, 1, W.SCORE_SIGMOID_NORM, cap, rep, 0, "normal")
    plan = M.Plan.from_workload(wl)
    logits = np.random.default_rng(5).standard_normal((T, E)).astype(np.float32)
    logits[0, :] = 0.5                              # an all-equal row
    want = oracle.route(oracle.Cfg.from_workload(wl), logits)
    got = gpu_route(plan, wl, logits)[0]
    compare_route(wl, got, want)
    assert (want["topk_ids"][0, :K] == [rep[e, 0] for e in range(K)]).all()


def test_route_deterministic():
    wl, x, logits, plan, cfg = setup("skewed")
    a, _ = gpu_route(plan, wl, logits)
    b, _ = gpu_route(plan, wl, logits)
    for k in a:
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k


# ------------------------------------------------------------------ dispatch

@pytest.mark.parametrize("name", SMALL)
def test_dispatch_parity(name):
    wl, x, logits, plan, cfg = setup(name)
    r = oracle.route(cfg, logits)
    dbuf = gpu_dispatch(plan, x, r["slots"])
    n = check_dispatch_tokens(dbuf, x, r["slots"], np.arange(x.shape[0]), wl.hidden,
                              wl.group_size)
    check_dispatch_untouched(dbuf, r["slots"], wl.hidden, group_size=wl.group_size)
    # Whole-buffer byte equality against the oracle's own dispatch (plus the
    # slot layout's zero padding after the scales).
    ref = expected_dispatch_buffer(cfg, x, r["slots"], plan.sizes)
    assert np.array_equal(dbuf.cpu().numpy(), ref)
    log(f"  {n} slots bit-exact")


# Full-size batches (every token and slot): tests/test_gpu_full_size.py.


# ------------------------------------------------------------------ combine

def _combine_inputs(wl, x, cfg, plan, r):
    s = plan.sizes
    dref = oracle.dispatch(cfg, x, r["slots"], s.total_slots, s.slot_stride)
    ebuf = oracle.expert_stub(cfg, r["counts"], dref, s.slot_stride)
    return dref, ebuf


@pytest.mark.parametrize("fmt", [M.FMT_BF16, M.FMT_Q8])
@pytest.mark.parametrize("name", SMALL)
def test_combine_parity(name, fmt):
    wl, x, logits, plan, cfg = setup(name)
    r = oracle.route(cfg, logits)
    dref, ebuf = _combine_inputs(wl, x, cfg, plan, r)
    src_host = ebuf if fmt == M.FMT_BF16 else dref
    want = oracle.combine(cfg, src_host, fmt, r["slots"], r["topk_w"])
    src = dev_i16(ebuf) if fmt == M.FMT_BF16 else dev(dref)
    y = torch.full((x.shape[0], wl.hidden), -1, dtype=torch.int16, device="cuda")
    plan.combine(src, fmt, dev(r["slots"]), dev(r["topk_w"]), y)
    got = host_u16(y)
    assert ulp_diff_bf16(got, want).max(initial=0) <= 1
    assert np.array_equal(got, want), f"{(got != want).sum()} elements differ by 1 ulp"


@pytest.mark.parametrize("T", [2047, 2048, 2051])
def test_dispatch_combine_around_split_threshold(T):
    """Token counts on both sides of the small-batch mapping (one wave per
    512-value chunk below 2048 tokens), ragged last workgroups, partial last
    chunk (H = 1152), capacity overflow."""
    cap = np.full(40, 400, np.int32)
    cap[0] = 200                                # one expert overflows
    wl = dataclasses.replace(W.get("ragged"), tokens=T, capacity=cap)
    log(f"[case] ragged T={T}")
    x, logits = W.make_inputs(wl)
    plan = M.Plan.from_workload(wl)
    cfg = oracle.Cfg.from_workload(wl)
    r = oracle.route(cfg, logits)
    dbuf = gpu_dispatch(plan, x, r["slots"])
    check_dispatch_tokens(dbuf, x, r["slots"], np.arange(T), wl.hidden)
    check_dispatch_untouched(dbuf, r["slots"], wl.hidden)
    _, ebuf = _combine_inputs(wl, x, cfg, plan, r)
    want = oracle.combine(cfg, ebuf, M.FMT_BF16, r["slots"], r["topk_w"])
    y = torch.full((T, wl.hidden), -1, dtype=torch.int16, device="cuda")
    plan.combine(dev_i16(ebuf), M.FMT_BF16, dev(r["slots"]), dev(r["topk_w"]), y)
    assert np.array_equal(host_u16(y), want)
    log(f"  dropped {r['dropped']}; dispatch and combine bit-exact")


def test_dispatch_store_kinds_agree_at_the_input_size_threshold():
    """Dispatch writes the payload with non-temporal stores while the batch's
    BF16 input is at most 256 MiB and with ordinary stores above.  At hidden
    8192, 16384 tokens are exactly 256 MiB and 16385 tokens one row more:
    a token's slot depends only on the tokens before it, so both calls must
    leave identical bytes in every slot but the extra token's, and both
    agree with the oracle on a sample of tokens (the extra one included)."""
    T, H, E, K = 16385, 8192, 256, 8
    cap = np.full(E, 2 * T * K // E, np.int32)
    wl = W.Workload("thr", "", T, H, E, E, K, 0, W.SCORE_SIGMOID_NORM, cap, None, 77, "normal")
    log(f"[case] dispatch at the input-size threshold: T={T - 1} and {T}, H={H}")
    x, logits = W.make_inputs(wl)
    plan = M.Plan.from_workload(wl)
    cfg = oracle.Cfg.from_workload(wl)
    r = oracle.route(cfg, logits)
    assert r["dropped"] == 0
    assert (T - 1) * 2 * H == 256 << 20
    a = gpu_dispatch(plan, x[:T - 1], r["slots"][:T - 1])      # non-temporal payload stores
    b = gpu_dispatch(plan, x, r["slots"])                       # ordinary payload stores
    last = torch.tensor([int(sl) for sl in r["slots"][T - 1] if sl >= 0], device="cuda",
                        dtype=torch.long)
    b[last] = SENTINEL
    assert torch.equal(a, b), "the two store kinds left different bytes"
    del a
    b = gpu_dispatch(plan, x, r["slots"])
    sample = np.concatenate([np.arange(0, T - 1, 997), [T - 1]])
    check_dispatch_tokens(b, x, r["slots"], sample, H)
    log(f"  identical slots below the extra token; {sample.size} tokens bit-exact against the oracle")


def test_combine_dropped_entries_and_signed_zero():
    rng = np.random.default_rng(91)
    T, H, K, S = 300, 640, 4, 500
    wl = W.Workload("c", "", T, H, 8, 8, K, 0, 1, np.array([S // 8 + 1] * 7 + [S - 7 * (S // 8 + 1)],
                    np.int32), None, 0, "normal")
    plan = M.Plan.from_workload(wl)
    cfg = oracle.Cfg.from_workload(wl)
    S = plan.sizes.total_slots
    ebuf = W.make_expert_out_bf16(92, S, H)
    ebuf[:, ::5] = 0x8000                       # -0 values
    ebuf[:, 1::7] ^= 0x8000
    slots = rng.integers(0, S, (T, K)).astype(np.int32)
    slots[rng.random((T, K)) < 0.2] = -1
    slots[:3] = -1                              # tokens with nothing kept -> +0
    w = W.make_gates(93, T, K)
    w[5] = 0.0
    want = oracle.combine(cfg, ebuf, M.FMT_BF16, slots, w)
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    plan.combine(dev_i16(ebuf), M.FMT_BF16, dev(slots), dev(w), y)
    got = host_u16(y)
    assert np.array_equal(got, want)
    assert (got[:3] == 0).all()


@pytest.mark.parametrize("fmt", [M.FMT_BF16, M.FMT_Q8])
@pytest.mark.parametrize("T,cap", [(300, None), (2500, None), (300, 2), (2500, 3)])
def test_combine_skipped_entry_after_negative_zero(T, cap, fmt):
    """A product that underflows to -0 leaves acc = -0; a later skipped entry
    (slot -1 or outside the buffer) must leave it there (fmaf(w, y, +0) with
    w * y in (-2^-150, 0) is -0, and the oracle skips the entry).  Rows:
    entry 0 = the smallest negative subnormal times a gate that underflows it,
    entry 1 skipped, entry 2 (some rows) a zero weight on a -0 value.  Small
    and large batches, with and without a workgroup cap."""
    K, H = 3, 640
    wl = W.Workload("negzero", "", T, H, 4, 4, K, 0, W.SCORE_SIGMOID_NORM,
                    np.full(4, T, np.int32), None, 0, "normal")
    log(f"[case] negative zero T={T} cap={cap} fmt={fmt}")
    plan = M.Plan.from_workload(wl)
    cfg = oracle.Cfg.from_workload(wl)
    s = plan.sizes
    S = s.total_slots
    rng = np.random.default_rng(98)
    slots = np.stack([np.arange(T), np.full(T, -1), T + np.arange(T)], axis=1).astype(np.int32)
    slots[1::3, 1] = S + 2                               # outside the buffer: skipped too
    slots[2::5, 2] = -1
    w = np.zeros((T, K), np.float32)
    w[:, 0] = np.float32(1e-6)
    w[::4, 0] = np.float32(0.5)                          # 0.5 * denorm_min: a tie, rounds to -0
    w[:, 1] = rng.random(T, dtype=np.float32)
    if fmt == M.FMT_BF16:
        eout = W.make_expert_out_bf16(99, S, H)
        eout[:T] = 0x8001                                # smallest negative BF16 subnormal
        eout[T:2 * T] = 0x8000
        src = dev_i16(eout)
    else:
        G = H // 128
        eout = np.zeros((S, s.slot_stride), np.uint8)
        eout[:, :H] = 0xFF                               # q = -1 everywhere
        sc = np.full((S, G), np.float32(1.4e-45))        # the smallest subnormal scale
        eout[:, H:H + 4 * G] = sc.view(np.uint8)
        eout[T:2 * T, :H] = 0                            # q = 0 with scale -0: (float)0 * -0 = -0
        eout[T:2 * T, H:H + 4 * G] = np.full((T, G), np.float32(-0.0)).view(np.uint8)
        src = dev(eout)
    clean = np.where((slots >= 0) & (slots < S), slots, -1).astype(np.int32)  # the oracle's view
    want = oracle.combine(cfg, eout, fmt, clean, w)
    assert (want[:, : H] == 0x8000).mean() > 0.5          # the case is exercised
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    if cap is None:
        plan.combine(src, fmt, dev(slots), dev(w), y)
    else:
        plan.combine_limited(src, fmt, dev(slots), dev(w), y, cap)
    assert np.array_equal(host_u16(y), want)


@pytest.mark.parametrize("T", [300, 2500])     # chunk-unit and token-unit kernels
def test_slots_outside_the_buffer_are_skipped(T):
    """Entries outside [0, total_slots) are skipped like -1 by dispatch and
    combine: buffers get a guard region past total_slots that stays untouched
    and unread.  Expected values: the oracle with those entries set to -1."""
    wl = W.Workload("guard", "", T, 640, 8, 8, 4, 0, W.SCORE_SIGMOID_NORM,
                    np.full(8, T, np.int32), None, 95, "normal")
    log(f"[case] out-of-range slots T={T}")
    plan = M.Plan.from_workload(wl)
    cfg = oracle.Cfg.from_workload(wl)
    s = plan.sizes
    S, H, G, K = s.total_slots, wl.hidden, wl.hidden // 128, wl.K
    x, logits = W.make_inputs(wl)
    clean = oracle.route(cfg, logits)["slots"]
    bad = clean.copy()
    rng = np.random.default_rng(96)
    pick = rng.random(bad.shape) < 0.25
    menu = np.array([S, S + 1, S + 3, -2, -(2 ** 31)], np.int64)
    bad[pick] = menu[rng.integers(0, len(menu), int(pick.sum()))].astype(np.int32)
    clean[pick] = -1
    guard = 4

    dbuf = torch.full((S + guard, s.slot_stride), SENTINEL, dtype=torch.uint8, device="cuda")
    plan.dispatch(dev_i16(x), dev(bad), dbuf)
    torch.cuda.synchronize()
    check_dispatch_tokens(dbuf, x, clean, np.arange(T), H)
    check_dispatch_untouched(dbuf[:S], clean, H)
    assert bool((dbuf[S:] == SENTINEL).all()), "dispatch wrote past total_slots"

    dref = oracle.dispatch(cfg, x, clean, S, s.slot_stride)
    ebuf = oracle.expert_stub(cfg, oracle.route(cfg, logits)["counts"], dref, s.slot_stride)
    w = W.make_gates(97, T, K)
    for fmt, src in ((M.FMT_BF16, ebuf), (M.FMT_Q8, dref)):
        ref = oracle.combine(cfg, src, fmt, clean, w)
        # guard rows that would change y if read: BF16 1.0, or q = 63 with scales ~0.75
        junk = np.full((guard,) + src.shape[1:], 0x3F80 if src.dtype == np.uint16 else 0x3F,
                       src.dtype)
        full = np.concatenate([src, junk])
        y = torch.empty((T, H), dtype=torch.int16, device="cuda")
        plan.combine(dev_i16(full) if fmt == M.FMT_BF16 else dev(full), fmt, dev(bad), dev(w), y)
        assert np.array_equal(host_u16(y), ref), f"fmt {fmt}"


def test_bf16_rounding_every_upper_half_and_rounding_class():
    """The device's fp32 -> BF16 rounding, reached through the Q8 combine with
    payload q = 1, gate 1.0 and one entry per token: every output is
    bf16(fma(1, s, +0)) of its group's fp32 scale s.  The scales take every
    one of the 2^16 upper halves (each sign, exponent -- zero, subnormal,
    normal, Inf, NaN -- and upper mantissa) with eight lower halves (0, 1,
    0x4000, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF), which covers every case
    of round-to-nearest-even: below, at and above the halfway point, with an
    even or odd kept bit.  Expected values are the oracle's, whose rounding
    is defined by exact distances, not bit tricks.  Rows after y stay
    untouched."""
    H, G = 8192, 64
    lows = np.array([0x0000, 0x0001, 0x4000, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF], np.uint32)
    x = ((np.arange(1 << 16, dtype=np.uint32)[:, None] << 16) | lows[None, :]).ravel()
    T = x.size // G                                              # 8192 tokens
    wl = W.Workload("bf16", "", T, H, 1, 1, 1, 0, W.SCORE_SIGMOID_NORM,
                    np.array([T], np.int32), None, 0, "normal")
    log(f"[case] bf16 rounding over {x.size} scales")
    plan = M.Plan.from_workload(wl)
    cfg = oracle.Cfg.from_workload(wl)
    s = plan.sizes
    dbuf = np.zeros((s.total_slots, s.slot_stride), np.uint8)
    dbuf[:, :H] = 1                                              # q = 1 everywhere
    dbuf[:T, H:H + 4 * G] = x.reshape(T, G).view(np.uint8)
    slots = np.arange(T, dtype=np.int32).reshape(T, 1)
    w = np.ones((T, 1), np.float32)
    want = oracle.combine(cfg, dbuf, M.FMT_Q8, slots, w)
    guard = 16
    ybuf = torch.full((T + guard, H), 0x5A5A, dtype=torch.int16, device="cuda")
    plan.combine(dev(dbuf), M.FMT_Q8, dev(slots), dev(w), ybuf[:T])
    torch.cuda.synchronize()
    got = host_u16(ybuf[:T])
    assert np.array_equal(got, want)
    assert bool((ybuf[T:] == 0x5A5A).all()), "combine wrote past y"
    # every group's 128 outputs are the rounding of one scale: spot-check the layout
    assert np.array_equal(got[:, ::128].ravel(), want[:, ::128].ravel())


def test_expert_layers_on_an_empty_batch_write_nothing():
    """All counts zero (the route of an empty batch): the expert layer's tile
    list is empty and neither it nor the stand-in writes anything."""
    wl, x, logits, plan, cfg = setup("tiny")
    s = plan.sizes
    ws = torch.empty(s.workspace_bytes, dtype=torch.uint8, device="cuda")
    plan.bind_workspace(ws)
    i32 = dict(dtype=torch.int32, device="cuda")
    counts, offsets = torch.full((wl.num_phys,), -7, **i32), torch.full((wl.num_phys + 1,), -7, **i32)
    dropped = torch.full((1,), -7, **i32)
    empty = torch.empty((0, wl.K), **i32)
    plan.route(torch.empty((0, wl.num_logical), dtype=torch.float32, device="cuda"), empty,
               torch.empty((0, wl.K), dtype=torch.float32, device="cuda"), counts, offsets,
               empty, dropped, ws, num_tokens=0)
    torch.cuda.synchronize()
    assert (counts.cpu().numpy() == 0).all() and int(dropped.item()) == 0
    dbuf = torch.zeros(s.dispatch_buf_bytes, dtype=torch.uint8, device="cuda")
    out = torch.full((s.total_slots, wl.hidden), 0x7FC1, dtype=torch.int16, device="cuda")
    Wt, wsc = W.make_expert_weights(3, wl.num_phys, wl.hidden)
    plan.expert_w8a8(counts, dbuf, torch.from_numpy(Wt).cuda(), dev(wsc), out, ws)
    plan.expert_stub(counts, dbuf, out, ws)
    torch.cuda.synchronize()
    assert bool((out == 0x7FC1).all())


# ------------------------------------------------------------------ expert stand-in

@pytest.mark.parametrize("name", ["decode", "decode_pt", "ragged", "replica_shared", "overflow"])
def test_expert_stub_parity(name):
    wl, x, logits, plan, cfg = setup(name)
    r = oracle.route(cfg, logits)
    dref, ebuf = _combine_inputs(wl, x, cfg, plan, r)
    ws = torch.empty(plan.sizes.workspace_bytes, dtype=torch.uint8, device="cuda")
    plan.bind_workspace(ws)
    out = torch.zeros((plan.sizes.total_slots, wl.hidden), dtype=torch.int16, device="cuda")
    plan.expert_stub(dev(r["counts"]), dev(dref), out, ws)
    assert np.array_equal(host_u16(out), ebuf)


# ------------------------------------------------------------------ end to end

def _e2e(name):
    wl, x, logits, plan, cfg = setup(name)
    T, H, K = x.shape[0], wl.hidden, wl.K
    b = plan.alloc()
    lg, xd = dev(logits), dev_i16(x)
    plan.route(lg, b["topk_ids"], b["topk_w"], b["counts"], b["offsets"], b["slots"],
               b["dropped"], b["workspace"])
    b["dispatch_buf"].fill_(SENTINEL)
    plan.dispatch(xd, b["slots"], b["dispatch_buf"])
    identity = wl.expert == "identity"
    if identity:
        src, fmt = b["dispatch_buf"], M.FMT_Q8
    else:
        plan.expert_stub(b["counts"], b["dispatch_buf"], b["combine_buf"], b["workspace"])
        src, fmt = b["combine_buf"], M.FMT_BF16
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    plan.combine(src, fmt, b["slots"], b["topk_w"], y)
    torch.cuda.synchronize()
    r = oracle.route(cfg, logits)
    got_r = {k: b[k].cpu().numpy() for k in ("topk_ids", "topk_w", "counts", "offsets", "slots")}
    got_r["dropped"] = int(b["dropped"].item())
    compare_route(wl, got_r, r)
    s = plan.sizes
    check_dispatch_tokens(b["dispatch_buf"].view(s.total_slots, s.slot_stride), x, r["slots"],
                          np.arange(T), H, wl.group_size)
    # Final output: GPU gates differ from the oracle's by the gate tolerance,
    # so the bound is 1 BF16 ulp + sum_k |dw_k||y_k| + 2K u sum_k |w_k y_k|.
    dref = oracle.dispatch(cfg, x, r["slots"], s.total_slots, s.slot_stride)
    eref = dref if identity else oracle.expert_stub(cfg, r["counts"], dref, s.slot_stride)
    want = oracle.combine(cfg, eref, fmt, r["slots"], r["topk_w"])
    gs = wl.group_size

    def rows_f64(idx):
        if identity:
            q = dref[idx, :H].view(np.int8).astype(np.float32)             # [n][K][H]
            sc = np.repeat(dref[idx, H:H + 4 * (H // gs)].view(np.float32), gs, axis=2)
            return (q * sc).astype(np.float64)
        return bf16_to_f32(eref[idx]).astype(np.float64)

    assert_within_gate_bound(host_u16(y), want, r["slots"], got_r["topk_w"], r["topk_w"],
                             rows_f64)
    return wl


@pytest.mark.parametrize("name", SMALL + ["global"])
def test_end_to_end(name):
    _e2e(name)


# ------------------------------------------------------------------ fused route + dispatch

def _fused_case(wl, logits, x):
    plan = M.Plan.from_workload(wl)
    cfg = oracle.Cfg.from_workload(wl)
    T, K, P = x.shape[0], wl.K, wl.num_phys
    s = plan.sizes
    ws = torch.empty(s.workspace_bytes, dtype=torch.uint8, device="cuda")
    plan.bind_workspace(ws)
    i32 = dict(dtype=torch.int32, device="cuda")
    out = dict(topk_ids=torch.full((T, K), -7, **i32),
               topk_w=torch.full((T, K), -7.0, dtype=torch.float32, device="cuda"),
               counts=torch.full((P,), -7, **i32), offsets=torch.full((P + 1,), -7, **i32),
               slots=torch.full((T, K), -7, **i32), dropped=torch.full((1,), -7, **i32))
    dbuf = torch.full((s.total_slots, s.slot_stride), SENTINEL, dtype=torch.uint8, device="cuda")
    plan.route_dispatch(dev(logits), dev_i16(x), out["topk_ids"], out["topk_w"], out["counts"],
                        out["offsets"], out["slots"], out["dropped"], dbuf, ws)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    got["dropped"] = int(got["dropped"][0])
    want = oracle.route(cfg, logits)
    compare_route(wl, got, want)
    ref = expected_dispatch_buffer(cfg, x, want["slots"], s)
    assert np.array_equal(dbuf.cpu().numpy(), ref)
    return got


@pytest.mark.parametrize("name", ["tiny", "decode", "decode_pt", "mid", "replica_shared"])
def test_route_dispatch_fused_parity(name):
    wl, x, logits, plan, cfg = setup(name)
    _fused_case(wl, logits, x)


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 128, 129, 200, 256])
@pytest.mark.parametrize("variant", ["softmax40", "sigmoid_shared_rep", "drops_pertoken"])
def test_route_dispatch_fused_sizes(T, variant):
    base = W.get({"softmax40": "ragged", "sigmoid_shared_rep": "replica_shared",
                  "drops_pertoken": "overflow"}[variant])
    wl = W.with_tokens(base, T)
    if variant == "drops_pertoken":
        wl = W.Workload("d", "", T, 512, 16, 16, 4, 0, W.SCORE_SIGMOID_NORM,
                        np.full(16, max(1, T // 8), np.int32), None, 13, "zipf",
                        ("fraction", 0.05, 1000.0), group_size=512)
    log(f"[case] fused {variant} T={T}")
    x, logits = W.make_inputs(wl, T)
    got = _fused_case(wl, logits, x)
    if variant == "drops_pertoken" and T >= 64:
        assert got["dropped"] > 0


@pytest.mark.parametrize("workgroups", [1, 3, 16, 10 ** 6])
@pytest.mark.parametrize("fmt", [M.FMT_BF16, M.FMT_Q8])
def test_combine_limited_matches_combine(workgroups, fmt):
    wl, x, logits, plan, cfg = setup("decode_pt" if fmt == M.FMT_Q8 else "decode")
    r = oracle.route(cfg, logits)
    dref, ebuf = _combine_inputs(wl, x, cfg, plan, r)
    src = dev_i16(ebuf) if fmt == M.FMT_BF16 else dev(dref)
    want = oracle.combine(cfg, ebuf if fmt == M.FMT_BF16 else dref, fmt, r["slots"], r["topk_w"])
    y = torch.full((x.shape[0], wl.hidden), -1, dtype=torch.int16, device="cuda")
    plan.combine_limited(src, fmt, dev(r["slots"]), dev(r["topk_w"]), y, workgroups)
    assert np.array_equal(host_u16(y), want)


@pytest.mark.parametrize("H,K", [(1152, 5), (640, 3), (1152, 15), (8192, 16), (128, 1), (4096, 13)])
@pytest.mark.parametrize("T", [37, 300, 2100, 3000])   # 2048+: 16-wave workgroups
def test_combine_limited_unit_shapes(H, K, T):
    """Capped combine: multi-chunk units (a ragged last unit when the chunk
    count is odd), single-chunk units from K = 14, dropped entries; both
    formats against the oracle."""
    rng = np.random.default_rng(H + 17 * K + T)
    S = 97
    wl = W.Workload("cl", "", T, H, K, K, K, 0, W.SCORE_SIGMOID_NORM,
                    np.full(K, S, np.int32), None, 3, "normal")
    log(f"[case] combine_limited H={H} K={K} T={T}")
    plan = M.Plan.from_workload(wl)
    cfg = oracle.Cfg.from_workload(wl)
    s = plan.sizes
    ebuf = W.make_expert_out_bf16(H + K, s.total_slots, H)
    xq = W.make_expert_out_bf16(H + K + 1, T, H)                 # BF16 rows to quantize
    qslots = np.arange(T, dtype=np.int32).reshape(T, 1) % s.total_slots
    dref = oracle.dispatch(oracle.Cfg(H, 1, 1, 1, 0, 1, [s.total_slots]), xq, qslots,
                           s.total_slots, s.slot_stride)
    slots = rng.integers(0, s.total_slots, (T, K)).astype(np.int32)
    slots[rng.random((T, K)) < 0.15] = -1
    w = W.make_gates(H + K + 2, T, K)
    for fmt, src_host in ((M.FMT_BF16, ebuf), (M.FMT_Q8, dref)):
        want = oracle.combine(cfg, src_host, fmt, slots, w)
        src = dev_i16(src_host) if fmt == M.FMT_BF16 else dev(src_host)
        for wgs in (1, 7):
            y = torch.full((T, H), -1, dtype=torch.int16, device="cuda")
            plan.combine_limited(src, fmt, dev(slots), dev(w), y, wgs)
            assert np.array_equal(host_u16(y), want), (fmt, wgs)


# ------------------------------------------------------------------ expert W8A8 GEMM

def _gemm_case(wl, x, logits, seed=21):
    plan = M.Plan.from_workload(wl)
    cfg = oracle.Cfg.from_workload(wl)
    s = plan.sizes
    r = oracle.route(cfg, logits)
    dref = oracle.dispatch(cfg, x, r["slots"], s.total_slots, s.slot_stride)
    Wt, ws = W.make_expert_weights(seed, wl.num_phys, wl.hidden)
    want = oracle.expert_w8a8(cfg, r["counts"], dref, s.slot_stride, Wt, ws,
                              ebuf=np.full((s.total_slots, wl.hidden), 0x7FC1, np.uint16))
    wsp = torch.empty(s.workspace_bytes, dtype=torch.uint8, device="cuda")
    plan.bind_workspace(wsp)
    out = torch.full((s.total_slots, wl.hidden), 0x7FC1, dtype=torch.int16, device="cuda")
    plan.expert_w8a8(dev(r["counts"]), dev(dref), torch.from_numpy(Wt).cuda(), dev(ws), out, wsp)
    got = host_u16(out)
    assert np.array_equal(got, want), f"{(got != want).any(axis=1).sum()} rows differ"


@pytest.mark.parametrize("name", ["tiny", "ragged", "overflow", "replica_shared"])
def test_expert_w8a8_parity(name):
    wl, x, logits, plan, cfg = setup(name)
    _gemm_case(wl, x, logits)


# 150 and 70 tokens: one partial tile per expert; 1500 and 1300 tokens:
# experts of ~560 and ~490 rows span two or three 256-row tiles with a
# ragged last one, and H = 1152 ends in a 128-channel tile.  H = 384 and
# 256: three and two K steps (the two wave groups' first and last phases
# meet), H = 384 with a 128-channel last tile.
@pytest.mark.parametrize("H,T", [(1024, 150), (2048, 70), (1024, 1500), (1152, 1300),
                                 (384, 300), (256, 900)])
def test_expert_w8a8_parity_per_token(H, T):
    wl = W.Workload("pt", "", T, H, 8, 8, 3, 0, W.SCORE_SIGMOID_NORM,
                    np.full(8, T, np.int32), None, 31, "normal", ("fraction", 0.05, 50.0),
                    group_size=H)
    log(f"[case] expert gemm per-token H={H} T={T}")
    x, logits = W.make_inputs(wl)
    _gemm_case(wl, x, logits)


@pytest.mark.parametrize("group", [128, 7168])   # 128 x 256 tiles; 256 x 256 (one scale per token)
def test_expert_w8a8_full_size_sampled(group):
    wl, x, logits, plan, cfg = setup("global")
    if group != wl.group_size:
        wl = dataclasses.replace(wl, group_size=group)
        plan, cfg = M.Plan.from_workload(wl), oracle.Cfg.from_workload(wl)
    log(f"[case] expert layer, global batch, group {group}")
    s = plan.sizes
    H, P = wl.hidden, wl.num_phys
    r = oracle.route(cfg, logits)
    b = plan.alloc()
    plan.dispatch(dev_i16(x), dev(r["slots"]), b["dispatch_buf"])
    gen = torch.Generator(device="cuda").manual_seed(41)
    Wd = torch.randint(-127, 128, (P, H, H), dtype=torch.int8, device="cuda", generator=gen)
    wsd = (torch.rand((P, H), device="cuda", generator=gen) + 0.5) / (127.0 * H ** 0.5)
    plan.expert_w8a8(dev(r["counts"]), b["dispatch_buf"], Wd, wsd, b["combine_buf"],
                     b["workspace"])
    torch.cuda.synchronize()
    base = np.concatenate([[0], np.cumsum(wl.capacity)[:-1]])
    owner = np.full(s.total_slots, -1, np.int64)          # slot -> token
    kept = r["slots"] >= 0
    owner[r["slots"][kept]] = np.nonzero(kept)[0]
    for p in (0, 77, 200, 255):
        n_p = min(int(r["counts"][p]), int(wl.capacity[p]))
        rows = np.unique(np.concatenate([[0, n_p - 1], np.arange(0, n_p, 97)]))
        sl = base[p] + rows
        # The sampled rows as the oracle's own dispatch writes them (one
        # entry per token, slot i for the i-th sampled row).
        one = oracle.Cfg(H, 1, 1, 1, 0, 1, [len(rows)], group_size=wl.group_size)
        d = oracle.dispatch(one, x[owner[sl]], np.arange(len(rows), dtype=np.int32)[:, None],
                            len(rows), s.slot_stride)
        want = oracle.expert_w8a8(one, np.array([len(rows)], np.int32), d, s.slot_stride,
                                  Wd[p:p + 1].cpu().numpy(), wsd[p:p + 1].cpu().numpy())
        got = host_u16(b["combine_buf"][torch.from_numpy(sl).cuda()])
        assert np.array_equal(got, want), p


@pytest.mark.parametrize("T", [5, 100, 700])   # one-launch, two-launch and large-batch routes
def test_route_one_copy_table_that_is_not_the_identity(T):
    """A one-column replica table may still place logical expert e on another
    physical id; every route path must follow it."""
    E, P = 32, 40
    table = ((7 * np.arange(E) + 3) % P).astype(np.int32).reshape(E, 1)
    assert len(set(table[:, 0])) == E and (table[:, 0] != np.arange(E)).any()
    wl = W.Workload("perm", "", T, 256, E, P, 6, 0, W.SCORE_SIGMOID_NORM,
                    np.full(P, T, np.int32), table, 77, "normal")
    log(f"[case] permuted one-copy table T={T}")
    x, logits = W.make_inputs(wl)
    plan = M.Plan.from_workload(wl)
    want = oracle.route(oracle.Cfg.from_workload(wl), logits)
    assert set(np.unique(want["topk_ids"])) <= set(table[:, 0])
    got, ws = gpu_route(plan, wl, logits)
    compare_route(wl, got, want)
    dbuf = gpu_dispatch(plan, x, want["slots"])
    fbuf = torch.full_like(dbuf, SENTINEL)
    i32 = dict(dtype=torch.int32, device="cuda")
    o = [torch.empty((T, wl.K), **i32), torch.empty((T, wl.K), device="cuda"),
         torch.empty(P, **i32), torch.empty(P + 1, **i32), torch.empty((T, wl.K), **i32),
         torch.empty(1, **i32)]
    plan.route_dispatch(dev(logits), dev_i16(x), *o, fbuf, ws)
    torch.cuda.synchronize()
    assert np.array_equal(o[0].cpu().numpy(), want["topk_ids"])
    assert np.array_equal(o[4].cpu().numpy(), want["slots"])
    assert torch.equal(fbuf, dbuf)


def test_route_eight_copy_replicas():
    """Replica rows of up to 8 copies (the layout the load-proportional
    placement produces), on the skewed logits."""
    base = W.get("skewed")
    E, R = base.num_logical, 8
    table = np.full((E, R), -1, np.int32)
    table[:, 0] = np.arange(E)
    nxt = E
    for e, copies in ((0, 8), (1, 4), (2, 3), (3, 2), (5, 2)):
        for c in range(1, copies):
            table[e, c] = nxt
            nxt += 1
    P = nxt
    wl = W.Workload("rep8", "", 3000, 256, E, P, 8, 0, W.SCORE_SIGMOID_NORM,
                    np.full(P, 3000, np.int32), table, base.seed, "zipf")
    log(f"[case] 8-copy replicas P={P}")
    x, logits = W.make_inputs(wl)
    want = oracle.route(oracle.Cfg.from_workload(wl), logits)
    compare_route(wl, gpu_route(M.Plan.from_workload(wl), wl, logits)[0], want)
    assert (np.bincount(want["topk_ids"].ravel(), minlength=P)[E:] > 0).all()
