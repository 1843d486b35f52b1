"""Helpers shared by the GPU parity tests: run the HIP path through the
C-ABI binding and compare with the CPU oracle on the same seeded inputs."""
import numpy as np
import torch

import oracle
from combine_moedc_route_amd import moedc as M
from combine_moedc_route_amd import workloads as W

U = 2.0 ** -24
SENTINEL = 0xA5


def log(msg):
    print(msg, flush=True)


def dev_i16(bits_u16):
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).cuda()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_u16(t):
    return t.cpu().numpy().view(np.uint16)


def bf16_to_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def gate_rel_tol(wl):
    """Relative gate tolerance derived from fp32 evaluation:
    softmax: E exponentials (<= 2u each after argument rounding), an E-term
    positive sum and one division; sigmoid-normalised: exp, 1+e, reciprocal,
    a K-term positive sum and one division, plus the reference's rounding."""
    if wl.score_fn == W.SCORE_SOFTMAX:
        return (wl.num_logical + 32) * U
    return (wl.top_k + 16) * U


def gpu_route(plan, wl, logits):
    T = logits.shape[0]
    K, P = plan.K, plan.num_phys
    ws = torch.empty(max(plan.sizes.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    plan.bind_workspace(ws)
    out = dict(
        topk_ids=torch.full((T, K), -7, dtype=torch.int32, device="cuda"),
        topk_w=torch.full((T, K), -7.0, dtype=torch.float32, device="cuda"),
        counts=torch.full((P,), -7, dtype=torch.int32, device="cuda"),
        offsets=torch.full((P + 1,), -7, dtype=torch.int32, device="cuda"),
        slots=torch.full((T, K), -7, dtype=torch.int32, device="cuda"),
        dropped=torch.full((1,), -7, dtype=torch.int32, device="cuda"),
    )
    lg = dev(logits) if T else torch.empty((0, wl.num_logical), dtype=torch.float32, device="cuda")
    plan.route(lg, out["topk_ids"], out["topk_w"], out["counts"], out["offsets"],
               out["slots"], out["dropped"], ws, num_tokens=T)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res["dropped"] = int(res["dropped"][0])
    return res, ws


def compare_route(wl, got, want):
    assert np.array_equal(got["topk_ids"], want["topk_ids"]), "topk_ids differ"
    assert np.array_equal(got["counts"], want["counts"]), "counts differ"
    assert np.array_equal(got["offsets"], want["offsets"]), "offsets differ"
    assert np.array_equal(got["slots"], want["slots"]), "slots differ"
    assert got["dropped"] == want["dropped"]
    gw, ow = got["topk_w"].astype(np.float64), want["topk_w"].astype(np.float64)
    err = np.abs(gw - ow)
    tol = gate_rel_tol(wl) * np.abs(ow)
    bad = err > tol
    assert not bad.any(), f"gates: {bad.sum()} out of tolerance, max rel {(err / np.abs(ow)).max():.3g}"
    if wl.num_shared:
        assert (got["topk_w"][:, -1] == 1.0).all()
    return float((err / np.maximum(np.abs(ow), 1e-30)).max()) if err.size else 0.0


def gpu_dispatch(plan, x_bits, slots, sentinel=SENTINEL):
    s = plan.sizes
    dbuf = torch.full((s.total_slots, s.slot_stride), sentinel, dtype=torch.uint8, device="cuda")
    T = x_bits.shape[0]
    plan.dispatch(dev_i16(x_bits), dev(slots), dbuf, num_tokens=T)
    torch.cuda.synchronize()
    return dbuf


def check_dispatch_tokens(dbuf, x_bits, slots, tokens, H, group_size=128):
    """Bit-exact payload + scales of every kept slot of the given tokens."""
    G = H // group_size
    q, s = oracle.quantize_tokens(x_bits[tokens], group_size)
    want = np.concatenate([q.view(np.uint8), s.view(np.uint8)], axis=1)   # [n][H+4G]
    rows, owner = [], []
    for i, t in enumerate(tokens):
        for sl in slots[t]:
            if sl >= 0:
                rows.append(int(sl))
                owner.append(i)
    if not rows:
        return 0
    got = dbuf[torch.tensor(rows, device="cuda", dtype=torch.long), : H + 4 * G].cpu().numpy()
    exp = want[np.array(owner)]
    bad = np.nonzero((got != exp).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} slots differ, first slot {rows[bad[0]]} token {tokens[owner[bad[0]]]}"
    return len(rows)


def scale_region_end(H, group_size=128):
    """End of the bytes dispatch writes in a slot: the G scales, then zero
    bytes up to the next multiple of 128 (the slot layout in moedc.h)."""
    G = H // group_size
    return H + 4 * (-(-G // 32) * 32)


def expected_dispatch_buffer(cfg, x, slots, sizes, fill=SENTINEL):
    """The whole dispatch buffer a call on a `fill`-initialised buffer must
    leave: the oracle's payload and scales (the method's bytes) in every
    occupied slot, the layout's zero padding after the scales, and `fill`
    everywhere else."""
    ref = np.full((sizes.total_slots, sizes.slot_stride), fill, np.uint8)
    oracle.dispatch(cfg, x, slots, sizes.total_slots, sizes.slot_stride, buf=ref)
    H, G = cfg.hidden, cfg.hidden // cfg.group_size
    occupied = np.unique(slots[(slots >= 0) & (slots < sizes.total_slots)])
    ref[occupied, H + 4 * G:scale_region_end(H, cfg.group_size)] = 0
    return ref


def check_dispatch_untouched(dbuf, slots, H, sentinel=SENTINEL, group_size=128):
    """Unoccupied slots keep the sentinel.  In an occupied slot the bytes
    after the G scales are zero up to the next multiple of 128 (the header's
    layout: H + 4 * round_up(G, 32)) and the rest keeps the sentinel."""
    G = H // group_size
    end = scale_region_end(H, group_size)
    assert end % 128 == 0 and end - (H + 4 * G) < 128
    S = dbuf.shape[0]
    occ = torch.zeros(S, dtype=torch.bool, device="cuda")
    sl = torch.from_numpy(slots[slots >= 0].astype(np.int64)).cuda()
    occ[sl] = True
    assert bool((dbuf[~occ] == sentinel).all()), "unoccupied slot written"
    assert bool((dbuf[occ, H + 4 * G:end] == 0).all()), "scale padding not zero"
    assert bool((dbuf[occ, end:] == sentinel).all()), "slot tail written"


def ulp_diff_bf16(a_bits, b_bits):
    """|a - b| in BF16 ulps via the ordered integer mapping (+0 == -0)."""
    def ordered(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def sample_tokens(T, n, seed):
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    pick = rng.choice(T, size=n - 2, replace=False)
    return np.unique(np.concatenate([[0, T - 1], pick]))


def assert_within_gate_bound(got, want, slots, gw, ow, rows_f64, chunk=512):
    """End-to-end combine check when the device's gates feed its combine:
    |got - want| <= 1 BF16 ulp + sum_k |dw_k| |y_k| + 2K u sum_k |w_k y_k|
    per value, with want the oracle's combine on the oracle's gates ow, gw
    the device's gates, and rows_f64(idx) the expert output rows at slot
    indices idx ([n][K]) as float64 [n][K][H].  Every token is checked."""
    T, K = slots.shape
    gw = gw.astype(np.float64)
    ow = ow.astype(np.float64)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        sl = slots[t0:t1]
        keep = sl >= 0
        yk = rows_f64(np.where(keep, sl, 0))
        yk[~keep] = 0.0
        a = bf16_to_f32(got[t0:t1]).astype(np.float64)
        b = bf16_to_f32(want[t0:t1]).astype(np.float64)
        mag = np.maximum(np.abs(a), np.abs(b))
        ulp = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-38))) - 7), 2.0 ** -133)
        bound = ulp + (np.abs(gw[t0:t1] - ow[t0:t1])[:, :, None] * np.abs(yk)).sum(1) \
            + 2 * K * U * (np.abs(ow[t0:t1])[:, :, None] * np.abs(yk)).sum(1)
        bad = np.nonzero((np.abs(a - b) > bound).any(axis=1))[0]
        assert bad.size == 0, f"token {t0 + bad[0]} outside the end-to-end bound"
