"""Benchmark of the MoE route -> INT8 dispatch -> combine path on one MI355X.

One step = moedc_route + moedc_dispatch + moedc_combine over the 30720-token
global decode batch (hidden 7168, 256 experts, top-8, INT8 groups of 128,
capacity 1920 per expert, BF16 expert outputs), alternating two static
dispatch/combine buffer sets.  The stand-in expert fills both combine sets
once before timing; it is not part of the path and is not timed.

Prints ONE JSON line.  Per-kernel durations come from HIP events recorded
on the stream the library launches on (torch's current stream).

Extra modes (measurement plumbing, not the product path):
  --calib-copy            time a plain device copy of known size (the
                          reference kernel for scaling rocprofv3 byte counters)
  --summarize-rocprof DIR write a text summary of rocprofv3 CSV output
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
INT8_PEAK_TOPS = 5000.0  # MI355X dense int8 MFMA
METRIC = ("dispatch+combine µs and tokens/s at 30720×7168 top-8/256; "
          "% of HBM peak GB/s")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
# Every source a kernel is compiled from: its .hip file and the headers it
# includes (moedc.h through internal.hpp).
_CSRC = "combine_moedc_route_amd/csrc/"
_COMMON = (_CSRC + "device.hpp", _CSRC + "internal.hpp", "include/moedc.h")
KERNEL_SOURCES = {
    "combine": (_CSRC + "combine.hip",) + _COMMON,
    "dispatch": (_CSRC + "dispatch.hip", _CSRC + "quant.hpp") + _COMMON,
    "route": (_CSRC + "route.hip",) + _COMMON,
    "expert_gemm": (_CSRC + "expert_gemm.hip",) + _COMMON,
}


def algorithmic_bytes(T, H, K, E):
    """Bytes the method must move (padding, unoccupied slots excluded)."""
    G = H // 128
    return dict(
        route=4 * T * E + 12 * T * K,
        dispatch=2 * T * H + 4 * T * K + T * K * (H + 4 * G),
        combine=2 * T * K * H + 8 * T * K + 2 * T * H,
        combine_q8=T * K * (H + 4 * G) + 8 * T * K + 2 * T * H,
    )


def code_text(src):
    """C/C++ source without comments and with whitespace runs collapsed:
    what the compiler sees, so editing a comment keeps recorded counters."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            i = src.find("\n", i)
            i = n if i < 0 else i
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":  # string or character literal, kept verbatim
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_sha(rels):
    """Hash of the code (comments and whitespace removed) of the files
    `rels` (one path or several)."""
    h = hashlib.sha256()
    for rel in ([rels] if isinstance(rels, str) else rels):
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode() + b"\0")
    return h.hexdigest()[:16]


def progress(msg):
    """One line on stderr when a leg of the benchmark ends (the JSON line
    alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(kernel, workload="global"):
    """HBM bytes per launch of `kernel` on `workload` from committed PMC
    runs, or None if none were taken on that workload or the kernel's
    source changed since (the bytes of a launch depend on its code and
    shape)."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)[workload][kernel]
    except (OSError, KeyError, ValueError, TypeError):
        return None
    if d.get("source_sha") != source_sha(KERNEL_SOURCES[kernel]):
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(tokens=30720, reps=3, keep=None):
    """The oracle, single-threaded and pinned to one host core, on the same
    workload recipe (`tokens` tokens, seed and capacity as on the GPU when
    tokens = 30720).  Route, dispatch and combine are each timed `reps`
    times and the per-step medians summed; the stand-in expert fills the
    combine buffer once, untimed, as on the GPU."""
    import numpy as np

    import oracle
    from combine_moedc_route_amd import workloads as W
    wl = W.get("global")
    if tokens == wl.tokens:
        sub = wl
    else:
        cap = 2 * tokens * wl.K // wl.num_phys
        sub = W.Workload("global-prefix", "", tokens, wl.hidden, wl.num_logical, wl.num_phys,
                         wl.top_k, 0, wl.score_fn, np.full(wl.num_phys, cap, np.int32), None,
                         wl.seed, wl.logits_kind)
    x, logits = W.make_inputs(sub)
    cfg = oracle.Cfg.from_workload(sub)
    H, G = sub.hidden, sub.hidden // 128
    sd = -(-(H + 4 * G) // 512) * 512
    S = int(np.sum(sub.capacity))
    # Buffers are allocated and touched before timing, as the GPU's are
    # resident before its timed region (first-touch page faults excluded).
    dbuf = np.zeros((S, sd), np.uint8)
    dbuf.fill(0)
    y = np.empty((tokens, H), np.uint16)
    y.fill(0)
    old = os.sched_getaffinity(0)
    core = min(old)
    os.sched_setaffinity(0, {core})
    try:
        t_r, t_d, t_c = [], [], []
        ebuf = None
        for _ in range(reps):
            t0 = time.perf_counter()
            r = oracle.route(cfg, logits)
            t1 = time.perf_counter()
            oracle.dispatch(cfg, x, r["slots"], S, sd, buf=dbuf)
            t2 = time.perf_counter()
            if ebuf is None:
                ebuf = oracle.expert_stub(cfg, r["counts"], dbuf, sd)  # writes every row combine reads
            t3 = time.perf_counter()
            oracle.combine(cfg, ebuf, oracle.FMT_BF16, r["slots"], r["topk_w"], out=y)
            t4 = time.perf_counter()
            t_r.append(t1 - t0)
            t_d.append(t2 - t1)
            t_c.append(t4 - t3)
    finally:
        os.sched_setaffinity(0, old)
    med = [statistics.median(v) for v in (t_r, t_d, t_c)]
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    sec = sum(med)
    if keep is not None:  # the oracle's outputs, for the parity check of the timed GPU step
        keep.update(route=r, dbuf=dbuf, y=y, slot_stride=sd)
    return {"value": tokens / sec, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{tokens} tokens of the {wl.tokens}-token workload recipe "
                      f"(capacity {int(sub.capacity[0])}/expert), 1 core ({model}, core {core}); "
                      f"median of {reps} "
                      f"runs per step: route {1e3 * med[0]:.1f} ms, dispatch {1e3 * med[1]:.1f} ms, "
                      f"combine {1e3 * med[2]:.1f} ms (single thread, "
                      f"{sum(t_r) + sum(t_d) + sum(t_c):.1f} s timed in all)"}


def gpu_snapshot(st):
    """Host copies of what the last timed step left on the GPU: route
    outputs, the dispatch buffer (both sets hold the same slots) and y."""
    out = {k: st[k].cpu().numpy() for k in ("slots", "w")}
    out.update({k: v.cpu().numpy() for k, v in st["route_out"].items()})
    out["dbuf"] = st["sets"][0][0].cpu().numpy()
    out["y"] = st["y"].cpu().numpy().view("uint16")
    return out


def parity(gpu, orc):
    """The timed step's GPU outputs against the oracle on the same inputs:
    route integers and INT8 slot bytes bit for bit, gates and BF16 outputs
    as the largest difference in units in the last place."""
    import numpy as np
    r = orc["route"]
    occ = r["slots"][r["slots"] >= 0]
    sd = orc["slot_stride"]
    H = gpu["y"].shape[1]
    nbytes = H + 4 * (H // 128)
    dg = gpu["dbuf"].reshape(-1, sd)
    dispatch_exact = bool(np.array_equal(dg[occ, :nbytes], orc["dbuf"][occ, :nbytes]))
    wg = gpu["w"].astype(np.float32).view(np.int32).astype(np.int64)
    wo = r["topk_w"].astype(np.float32).view(np.int32).astype(np.int64)
    yd = np.abs(gpu["y"].astype(np.int32) - orc["y"].astype(np.int32))
    return {"route_ids_slots_counts_exact": bool(
                np.array_equal(gpu["topk_ids"], r["topk_ids"]) and
                np.array_equal(gpu["slots"], r["slots"]) and
                np.array_equal(gpu["counts"], r["counts"]) and
                np.array_equal(gpu["offsets"], r["offsets"]) and
                int(gpu["dropped"][0]) == int(r["dropped"])),
            "gates_max_ulp": int(np.abs(wg - wo).max()),
            "dispatch_slot_bytes_exact": dispatch_exact,
            "combine_max_bf16_ulp": int(yd.max()),
            "combine_tokens_not_bit_identical": int((yd.max(axis=1) > 0).sum()),
            "what": f"every token of the timed step ({gpu['y'].shape[0]}): route outputs, bytes "
                    f"[0, {nbytes}) of all {len(occ)} occupied slots, y; against the oracle "
                    "outputs of the cpu_baseline leg (same inputs)"}


def measure_path(wl, steps, warmup, fmt_name="bf16"):
    """Time route + dispatch + combine on workload `wl` over `steps` steps
    (after `warmup`), alternating two static dispatch/combine buffer sets;
    the stand-in expert fills both combine sets once, untimed.  Returns the
    numbers and the state the other legs reuse."""
    import numpy as np
    import torch

    from combine_moedc_route_amd import moedc as M
    from combine_moedc_route_amd import workloads as W

    T, H, K, E = wl.tokens, wl.hidden, wl.K, wl.num_logical
    dev = "cuda:0"
    plan = M.Plan.from_workload(wl)
    s = plan.sizes
    x, logits = W.make_inputs(wl)
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    lg = torch.from_numpy(logits).to(dev)
    del x, logits
    ws = torch.empty(s.workspace_bytes, dtype=torch.uint8, device=dev)
    plan.bind_workspace(ws)
    i32 = dict(dtype=torch.int32, device=dev)
    ids = torch.empty((T, K), **i32)
    w = torch.empty((T, K), dtype=torch.float32, device=dev)
    counts = torch.empty(wl.num_phys, **i32)
    offsets = torch.empty(wl.num_phys + 1, **i32)
    slots = torch.empty((T, K), **i32)
    dropped = torch.empty(1, **i32)
    sets = []
    for _ in range(2):  # double-buffered static dispatch/combine buffers
        sets.append((torch.empty(s.dispatch_buf_bytes, dtype=torch.uint8, device=dev),
                     torch.empty((s.total_slots, H), dtype=torch.int16, device=dev)))
    y = torch.empty((T, H), dtype=torch.int16, device=dev)
    fmt = M.FMT_Q8 if fmt_name == "q8" else M.FMT_BF16

    def route():
        plan.route(lg, ids, w, counts, offsets, slots, dropped, ws)

    for dbuf, cbuf in sets:  # fill combine inputs once (untimed)
        route()
        plan.dispatch(xd, slots, dbuf)
        plan.expert_stub(counts, dbuf, cbuf, ws)
    torch.cuda.synchronize()
    assert int(dropped.item()) == 0

    def step(i, ev=None):
        dbuf, cbuf = sets[i & 1]
        src = dbuf if fmt == M.FMT_Q8 else cbuf
        if ev:
            ev[0].record()
        route()
        if ev:
            ev[1].record()
        plan.dispatch(xd, slots, dbuf)
        if ev:
            ev[2].record()
        plan.combine(src, fmt, slots, w, y)
        if ev:
            ev[3].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(steps):
        step(i, evs[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = start.elapsed_time(stop) / steps
    r_us = [1e3 * e[0].elapsed_time(e[1]) for e in evs]
    d_us = [1e3 * e[1].elapsed_time(e[2]) for e in evs]
    c_us = [1e3 * e[2].elapsed_time(e[3]) for e in evs]
    mean = statistics.fmean
    ab = algorithmic_bytes(T, H, K, E)
    cb = ab["combine_q8"] if fmt == M.FMT_Q8 else ab["combine"]
    dc_us = mean(d_us) + mean(c_us)
    comb_gbps = cb / (mean(c_us) * 1e-6) / 1e9
    disp_gbps = ab["dispatch"] / (mean(d_us) * 1e-6) / 1e9
    dc_gbps = (ab["dispatch"] + cb) / (dc_us * 1e-6) / 1e9
    out = {
        "ms_per_step": ms_per_step,
        "tokens_per_s": T / (ms_per_step * 1e-3),
        "route_us": mean(r_us),
        "dispatch_us": mean(d_us),
        "combine_us": mean(c_us),
        "dispatch_us_median": statistics.median(d_us),
        "combine_us_median": statistics.median(c_us),
        "dispatch_us_min": min(d_us),
        "combine_us_min": min(c_us),
        "dispatch_plus_combine_us": dc_us,
        "dispatch_plus_combine_tokens_per_s": T / (dc_us * 1e-6),
        "dispatch_GBps": disp_gbps,
        "combine_GBps": comb_gbps,
        "dispatch_plus_combine_GBps": dc_gbps,
        "dispatch_plus_combine_frac_of_hbm_peak": dc_gbps / HBM_PEAK_GBPS,
        "dispatch_frac_of_hbm_peak": disp_gbps / HBM_PEAK_GBPS,
        "combine_frac_of_hbm_peak": comb_gbps / HBM_PEAK_GBPS,
        "route_GBps": ab["route"] / (mean(r_us) * 1e-6) / 1e9,
        "route_frac_of_hbm_peak": ab["route"] / (mean(r_us) * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        "algorithmic_bytes": {"dispatch": ab["dispatch"], "combine": cb, "route": ab["route"]},
        "wall_s_timed": wall,
    }
    state = dict(plan=plan, wl=wl, counts=counts, sets=sets, ws=ws, xd=xd, slots=slots, w=w,
                 y=y, fmt=fmt, ab=ab, cb=cb,
                 route_out=dict(topk_ids=ids, counts=counts, offsets=offsets, dropped=dropped))
    return out, state


def run(args):
    import torch

    from combine_moedc_route_amd import moedc as M
    from combine_moedc_route_amd import workloads as W

    wl = W.get(args.workload)
    T, H, K = wl.tokens, wl.hidden, wl.K
    torch.cuda.set_device(0)
    m, st = measure_path(wl, args.steps, args.warmup, args.combine_fmt)
    progress(f"{wl.name}: {m['ms_per_step']:.4f} ms per step")
    # The timed step's outputs, for the parity check against the oracle
    # (taken now: later legs reuse these buffers).
    snap = (gpu_snapshot(st) if args.workload == "global" and args.cpu_tokens == wl.tokens
            and args.combine_fmt == "bf16" and not args.no_cpu_baseline else None)
    fmt, ab, cb = st["fmt"], st["ab"], st["cb"]
    plan, sets, slots, w, y = st["plan"], st["sets"], st["slots"], st["w"], st["y"]
    # Dominant kernel: the one with the larger mean duration.
    dom = "combine" if m["combine_us"] >= m["dispatch_us"] else "dispatch"
    dom_bytes, dom_gbps = ((cb, m["combine_GBps"]) if dom == "combine"
                           else (ab["dispatch"], m["dispatch_GBps"]))
    traffic = measured_traffic(dom, wl.name) if fmt == M.FMT_BF16 else None
    res = {
        "metric": METRIC,
        "value": m["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in/out, int8 payload + fp32 scales, fp32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: {wl.description}",
            "tokens": T, "hidden": H, "experts": wl.num_phys, "top_k": K,
            "group": 128, "capacity_per_expert": int(wl.capacity[0]),
            "combine_input": "bf16" if fmt == M.FMT_BF16 else "q8",
            "step": "route + dispatch + combine, buffer sets alternating",
        },
    }
    res.update({k: v for k, v in m.items() if k not in ("ms_per_step", "tokens_per_s")})
    res["roofline"] = {
        "kernel": dom,
        "bound": "hbm",
        "achieved": dom_gbps,
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": dom_gbps / HBM_PEAK_GBPS,
        "traffic": traffic,
    }
    if fmt == M.FMT_BF16:
        # The same combine reading the INT8 dispatch slots (identity experts /
        # quantized return), timed over the two dispatch buffer sets.
        cq = []
        for i in range(args.warmup + args.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            plan.combine(sets[i & 1][0], M.FMT_Q8, slots, w, y)
            e1.record()
            if i >= args.warmup:
                cq.append((e0, e1))
        torch.cuda.synchronize()
        q_us = [1e3 * e0.elapsed_time(e1) for e0, e1 in cq]
        mean = statistics.fmean
        q_gbps = ab["combine_q8"] / (mean(q_us) * 1e-6) / 1e9
        res["combine_q8"] = {"us": mean(q_us), "us_median": statistics.median(q_us),
                             "GBps": q_gbps, "frac_of_hbm_peak": q_gbps / HBM_PEAK_GBPS,
                             "algorithmic_bytes": ab["combine_q8"]}
    if args.workload == "global" and not args.no_ceilings:
        res["ceilings"] = ceilings(st, m)
        progress("ceilings")
    if args.workload == "global" and not args.no_expert:
        res["expert_gemm"] = expert_gemm(plan, wl, st["counts"], sets[0][0], sets[0][1],
                                         st["ws"], st["xd"], slots)
        progress("expert_gemm")
    del st, sets
    torch.cuda.empty_cache()
    if args.workload == "global" and not args.no_workloads:
        # The other large configurations, each on its own buffers.
        for name in ("skewed", "prefill"):
            sub, sst = measure_path(W.get(name), max(10, args.steps // 4), 5)
            sub["workload"] = f"{name}: {W.get(name).description}"
            sub["roofline_traffic"] = {k: measured_traffic(k, name) for k in ("dispatch", "combine")}
            res[name] = sub
            progress(f"{name}: {sub['ms_per_step']:.4f} ms per step")
            del sst
            torch.cuda.empty_cache()
    if args.workload == "global" and not args.no_expert and not args.no_lpt:
        res["expert_lpt"] = expert_lpt()
        progress("expert_lpt")
        torch.cuda.empty_cache()
    if args.workload == "global" and not args.no_decode:
        res["decode_latency"] = decode_latency()
        # Batches of one token per wave or fewer take the one-launch route.
        res["decode_latency"]["small_batches"] = {
            str(n): decode_latency(tokens=n, which=("route", "route_dispatch_fused", "fused_step"))
            for n in (1, 16)}
        progress("decode_latency")
        res["overlap"] = overlap()
        progress("overlap")
    if args.workload == "global" and not args.no_placement:
        res["placement"] = placement()
        progress("placement")
    if not args.no_cpu_baseline:
        orc = {} if snap is not None else None
        res["cpu_baseline"] = cpu_baseline(args.cpu_tokens, keep=orc)
        if snap is not None:
            res["parity"] = parity(snap, orc)
            progress(f"parity {res['parity']}")
            del snap, orc
    print(json.dumps(res), flush=True)


def decode_latency(reps=50, per_graph=20, tokens=None, which=None):
    """Latency of one die's decode batch (96 tokens, hidden 7168, 256 experts,
    top-8).  Each figure is the mean device time per call when `per_graph`
    calls run back to back from one captured HIP graph, replayed `reps`
    times: no host launch cost and no per-call event overhead, as in a
    serving loop.  The two-step path (route, dispatch, combine) and the
    route+dispatch entry are timed alone and as whole steps; the replayed
    step's outputs are checked bit for bit against an eager run.  `tokens`
    replaces the batch size (same capacities), `which` restricts the calls
    timed."""
    import dataclasses

    import numpy as np
    import torch

    from combine_moedc_route_amd import moedc as M
    from combine_moedc_route_amd import workloads as W
    wl = W.get("decode")
    if tokens is not None:
        wl = dataclasses.replace(wl, tokens=tokens)
    T, H, K = wl.tokens, wl.hidden, wl.K
    plan = M.Plan.from_workload(wl)
    b = plan.alloc("cuda:0")
    x, logits = W.make_inputs(wl)
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    lg = torch.from_numpy(logits).cuda()
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    rargs = (b["topk_ids"], b["topk_w"], b["counts"], b["offsets"], b["slots"], b["dropped"])
    route = lambda: plan.route(lg, *rargs, b["workspace"])
    dispatch = lambda: plan.dispatch(xd, b["slots"], b["dispatch_buf"])
    fused = lambda: plan.route_dispatch(lg, xd, *rargs, b["dispatch_buf"], b["workspace"])
    combine = lambda: plan.combine(b["combine_buf"], M.FMT_BF16, b["slots"], b["topk_w"], y)
    route()
    dispatch()
    plan.expert_stub(b["counts"], b["dispatch_buf"], b["combine_buf"], b["workspace"])
    combine()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in (("y", y), ("slots", b["slots"]), ("w", b["topk_w"]))}
    calls = {
        "route": route,
        "dispatch": dispatch,
        "route_dispatch_fused": fused,
        "combine": combine,
        "combine_16wg": lambda: plan.combine_limited(b["combine_buf"], M.FMT_BF16, b["slots"],
                                                     b["topk_w"], y, 16),
        "two_step": lambda: (route(), dispatch(), combine()),
        "fused_step": lambda: (fused(), combine()),
        "launch_floor": lambda: y[:1, :8].fill_(1),  # one tiny torch kernel
    }
    res = {}
    for name, f in calls.items():
        if which is not None and name not in which:
            continue
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                f()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                f()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        res[name + "_us"] = 1e3 * e0.elapsed_time(e1) / (reps * per_graph)
        if name in ("two_step", "fused_step"):
            ok = all(bool(torch.equal(ref[k], v)) for k, v in
                     (("y", y), ("slots", b["slots"]), ("w", b["topk_w"])))
            res[name + "_replay_matches_eager"] = ok
        del g
    res["timing"] = f"HIP graph of {per_graph} back-to-back calls, {reps} replays"
    res["workload"] = f"decode: {wl.description}" if tokens is None else f"decode with {T} tokens"
    return res


def expert_gemm(plan, wl, counts, dbuf, cbuf, ws, xd, slots, iters=5):
    """The W8A8 expert layer (hidden -> hidden per physical expert) over the
    global batch's occupied slots, against the int8 MFMA roofline: with the
    workload's 128-value activation groups, and again with one scale per
    token (the slots re-dispatched with per-token scales)."""
    import dataclasses

    import torch

    from combine_moedc_route_amd import moedc as M
    H, P = wl.hidden, wl.num_phys
    gen = torch.Generator(device="cuda").manual_seed(41)
    Wd = torch.randint(-127, 128, (P, H, H), dtype=torch.int8, device="cuda", generator=gen)
    wsd = (torch.rand((P, H), device="cuda", generator=gen) + 0.5) / (127.0 * H ** 0.5)
    used = torch.minimum(counts, torch.from_numpy(wl.capacity).cuda()).sum().item()
    ops = 2.0 * used * H * H

    def timed(p, w):
        p.expert_w8a8(counts, dbuf, Wd, wsd, cbuf, w)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            p.expert_w8a8(counts, dbuf, Wd, wsd, cbuf, w)
        e1.record()
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / iters

    us = timed(plan, ws)
    # Per-token scales: same slots, payload and weights; one fold per tile.
    plan_pt = M.Plan.from_workload(dataclasses.replace(wl, group_size=H))
    ws_pt = torch.empty(plan_pt.sizes.workspace_bytes, dtype=torch.uint8, device="cuda")
    plan_pt.bind_workspace(ws_pt)
    plan_pt.dispatch(xd, slots, dbuf)
    us_pt = timed(plan_pt, ws_pt)
    lib_us = library_int8_gemm(wl, counts, dbuf, Wd, plan.sizes.slot_stride, iters)
    floor = mfma_floor(ops)
    del Wd
    torch.cuda.empty_cache()
    tops, tops_pt = ops / (us * 1e-6) / 1e12, ops / (us_pt * 1e-6) / 1e12
    return {"kernel": "expert_w8a8", "us": us, "rows": int(used), "TOPs": tops,
            "roofline": {"bound": "mfma", "achieved": tops, "peak": INT8_PEAK_TOPS,
                         "unit": "TOP/s (int8)", "frac": tops / INT8_PEAK_TOPS,
                         "traffic": measured_traffic("expert_gemm")},
            "weight_GBps": P * H * H / (us * 1e-6) / 1e9,
            "per_token_scales": {"us": us_pt, "TOPs": tops_pt, "frac": tops_pt / INT8_PEAK_TOPS,
                                 "frac_of_compute_floor": floor["per_token_us"] / us_pt},
            "compute_floor": floor,
            "frac_of_compute_floor": floor["groups_us"] / us,
            "library_int8_gemm": {
                "what": "torch._int_mm (hipBLASLt) once per expert on the same rows and weights, "
                        "int32 out, no scales: context, not part of the path",
                "us": lib_us, "frac": ops / (lib_us * 1e-6) / 1e12 / INT8_PEAK_TOPS}}


def mfma_floor(ops, iters=3):
    """The expert layer's compute floor on this part (libmoedc_ceiling's
    MFMA kernel): the layer's int8 MACs as v_mfma_i32_16x16x64_i8 from
    registers, two waves per SIMD, no memory traffic; with the 128-input
    groups' fold after every 32 MFMAs per wave, and without (one scale per
    token)."""
    import torch
    L = _ceiling_lib()
    cs = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    n = int(ops // (2 * 16 * 16 * 64))

    def run(fold):
        rc = L.moedc_ceiling_mfma(n, fold, sink.data_ptr(), cs)
        if rc:
            raise RuntimeError(f"ceiling kernel failed: hip error {rc}")

    res = {"mfma": n, "what": "the layer's MACs as 16x16x64 int8 MFMAs from registers, "
                              "2 waves per SIMD, no memory; groups: plus the per-group fold"}
    for key, fold in (("per_token_us", 0), ("groups_us", 1)):
        res[key] = _time_us(lambda: run(fold), iters=iters, warm=1)
    res["per_token_frac_of_int8_peak"] = ops / (res["per_token_us"] * 1e-6) / 1e12 / INT8_PEAK_TOPS
    res["groups_frac_of_int8_peak"] = ops / (res["groups_us"] * 1e-6) / 1e12 / INT8_PEAK_TOPS
    return res


def library_int8_gemm(wl, counts, dbuf, Wd, slot_stride, iters):
    """The library's int8 GEMM on the expert layer's shapes: for each physical
    expert, its occupied rows (INT8 payload copied out of the dispatch slots,
    untimed) times its weight matrix, as 256 back-to-back torch._int_mm
    calls."""
    import numpy as np
    import torch
    H = wl.hidden
    n = np.minimum(counts.cpu().numpy(), wl.capacity)
    base = np.concatenate([[0], np.cumsum(wl.capacity)[:-1]])
    rows = torch.from_numpy(np.concatenate([base[p] + np.arange(n[p]) for p in range(len(n))])).cuda()
    xq = dbuf.view(-1, slot_stride)[rows, :H].contiguous()  # [used][H] int8
    xq = xq.view(torch.int8)
    out = torch.empty((xq.shape[0], H), dtype=torch.int32, device="cuda")
    starts = np.concatenate([[0], np.cumsum(n)])
    parts = [(xq[starts[p]:starts[p + 1]], Wd[p].t(), out[starts[p]:starts[p + 1]])
             for p in range(len(n)) if n[p] > 16]

    def run():
        for a, b, o in parts:
            torch._int_mm(a, b, out=o)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        run()
    e1.record()
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / iters


def _ceiling_lib():
    import ctypes as C
    L = C.CDLL(os.path.join(ROOT, "combine_moedc_route_amd", "libmoedc_ceiling.so"))
    P, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
    L.moedc_ceiling_read.argtypes = [P, i64, P, P]
    L.moedc_ceiling_write.argtypes = [P, i64, P]
    L.moedc_ceiling_copy.argtypes = [P, P, i64, P]
    L.moedc_ceiling_scatter.argtypes = [P, i32, i32, P, i64, i32, P]
    L.moedc_ceiling_gather.argtypes = [P, P, i32, i32, i64, i32, P, P]
    L.moedc_ceiling_mfma.argtypes = [i64, i32, P, P]
    for f in ("read", "write", "copy", "scatter", "gather", "mfma"):
        getattr(L, "moedc_ceiling_" + f).restype = i32
    return L


def _time_us(fn, iters=10, warm=3):
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / iters


def ceilings(st, m, stream_bytes=4 << 30):
    """What the memory system gives (libmoedc_ceiling kernels, on the
    current stream): 4 GiB streaming read, write and copy, and the exact
    access patterns of the global batch's dispatch (stores of each token's
    K slots, 7424 bytes each, without reading x or quantizing) and combine
    (each token's K BF16 rows read, one row written, without arithmetic).
    Dispatch and combine are read against these as well as 8 TB/s."""
    import torch
    L = _ceiling_lib()
    wl, plan, slots = st["wl"], st["plan"], st["slots"]
    T, H, K = wl.tokens, wl.hidden, wl.K
    sz = plan.sizes
    cs = torch.cuda.current_stream().cuda_stream
    a = torch.empty(stream_bytes, dtype=torch.uint8, device="cuda")
    b = torch.empty(stream_bytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    a.fill_(1)

    def ok(rc):
        if rc:
            raise RuntimeError(f"ceiling kernel failed: hip error {rc}")

    res = {}
    us = _time_us(lambda: ok(L.moedc_ceiling_read(a.data_ptr(), stream_bytes, sink.data_ptr(), cs)))
    res["read"] = {"bytes": stream_bytes, "us": us, "GBps": stream_bytes / us / 1e3}
    us = _time_us(lambda: ok(L.moedc_ceiling_write(b.data_ptr(), stream_bytes, cs)))
    res["write"] = {"bytes": stream_bytes, "us": us, "GBps": stream_bytes / us / 1e3}
    us = _time_us(lambda: ok(L.moedc_ceiling_copy(b.data_ptr(), a.data_ptr(), stream_bytes, cs)))
    res["copy"] = {"bytes": 2 * stream_bytes, "us": us, "GBps": 2 * stream_bytes / us / 1e3}
    del a, b
    torch.cuda.empty_cache()
    G = H // 128
    row = H + 4 * (-(-G // 32) * 32)            # the bytes dispatch writes per slot (padding included)
    dbuf, cbuf = st["sets"][0]
    kept = int((slots >= 0).sum().item())
    us = _time_us(lambda: ok(L.moedc_ceiling_scatter(slots.data_ptr(), T, K, dbuf.data_ptr(),
                                                     sz.slot_stride, row, cs)))
    res["dispatch_scatter"] = {"bytes": kept * row, "us": us, "GBps": kept * row / us / 1e3,
                               "what": "dispatch's stores alone (each token's K slots, "
                                       f"{row} B each), no x read, no quantization"}
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    gb = kept * 2 * H + 2 * T * H
    us = _time_us(lambda: ok(L.moedc_ceiling_gather(cbuf.data_ptr(), slots.data_ptr(), T, K,
                                                    2 * H, 2 * H, out.data_ptr(), cs)))
    res["combine_gather"] = {"bytes": gb, "us": us, "GBps": gb / us / 1e3,
                             "what": "combine's BF16 row reads and output writes alone, "
                                     "no weights, no arithmetic"}
    # The path's kernels against these ceilings (algorithmic bytes / time).
    res["dispatch_frac_of_scatter_plus_read"] = None
    res["combine_frac_of_gather"] = m["combine_GBps"] / res["combine_gather"]["GBps"]
    # dispatch = its stores + reading x: against the scatter pattern plus a
    # streaming read of x at the read ceiling.
    t_ideal = res["dispatch_scatter"]["us"] + 2 * T * H / res["read"]["GBps"] / 1e3
    res["dispatch_frac_of_scatter_plus_read"] = t_ideal / m["dispatch_us"]
    res["dispatch_frac_of_copy"] = m["dispatch_GBps"] / res["copy"]["GBps"]
    res["combine_frac_of_copy"] = m["combine_GBps"] / res["copy"]["GBps"]
    return res


def expert_lpt(iters=5):
    """The expert layer on the skewed batch (Zipf(1.1), 256 logical experts,
    30720 tokens, top-8, hidden 7168) with the bands of its work dealt to
    the 8 XCDs round-robin and by the device-built LPT schedule, under two
    replica tables: the workload's own (the 32 most popular experts get one
    extra copy) and one from moedc_place_replicas on the batch's loads.
    Tiles per XCD are the device's own schedule (xcd_tiles output)."""
    import dataclasses

    import numpy as np
    import torch

    from combine_moedc_route_amd import moedc as M
    from combine_moedc_route_amd import workloads as W
    base = W.get("skewed")
    T, H, E = base.tokens, base.hidden, base.num_logical
    x, logits = W.make_inputs(base)
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    lg = torch.from_numpy(logits).cuda()
    del x
    P = base.num_phys
    gen = torch.Generator(device="cuda").manual_seed(71)
    Wd = torch.randint(-127, 128, (P, H, H), dtype=torch.int8, device="cuda", generator=gen)
    wsd = (torch.rand((P, H), device="cuda", generator=gen) + 0.5) / (127.0 * H ** 0.5)

    def route_counts(wl):
        plan = M.Plan.from_workload(dataclasses.replace(wl, hidden=128))
        b = plan.alloc("cuda:0")
        plan.route(lg, b["topk_ids"], b["topk_w"], b["counts"], b["offsets"], b["slots"],
                   b["dropped"], b["workspace"])
        return b["counts"].cpu().numpy()

    ident = dataclasses.replace(base, num_phys=E, capacity=np.full(E, T, np.int32),
                                replica_table=None)
    load = route_counts(ident).astype(np.float64)
    table = M.place_replicas(load, P - E, 8)
    planned = dataclasses.replace(base, capacity=np.full(P, T, np.int32), replica_table=table)
    cnt = route_counts(planned)
    planned.capacity = ((cnt + 64 + 63) // 64 * 64).astype(np.int32)
    res = {"workload": f"skewed: {base.description}", "weights": "int8 U[-127,127], torch seed 71",
           "what": "expert_w8a8 over every occupied slot; bands of 4 x 256 channels x all rows "
                   "of one expert dealt to the 8 XCDs"}
    for tname, wl in (("fixed_table", base), ("planned_table", planned)):
        plan = M.Plan.from_workload(wl)
        b = plan.alloc("cuda:0")
        plan.route(lg, b["topk_ids"], b["topk_w"], b["counts"], b["offsets"], b["slots"],
                   b["dropped"], b["workspace"])
        plan.dispatch(xd, b["slots"], b["dispatch_buf"])
        torch.cuda.synchronize()
        assert int(b["dropped"].item()) == 0
        used = torch.minimum(b["counts"], torch.from_numpy(wl.capacity).cuda()).sum().item()
        ops = 2.0 * used * H * H
        sub = {"rows": int(used), "largest_copy_rows": int(b["counts"].max().item())}
        outs = {}
        for dname, deal in (("round_robin", M.DEAL_ROUND_ROBIN), ("lpt", M.DEAL_LPT)):
            xt = torch.zeros(8, dtype=torch.int32, device="cuda")
            f = lambda: plan.expert_w8a8_dealt(b["counts"], b["dispatch_buf"], Wd, wsd,
                                               b["combine_buf"], b["workspace"], deal, xt)
            us = _time_us(f, iters=iters, warm=1)
            tiles = xt.cpu().numpy()
            outs[dname] = b["combine_buf"].clone() if dname == "round_robin" else None
            sub[dname] = {"us": us, "TOPs": ops / (us * 1e-6) / 1e12,
                          "frac_of_int8_peak": ops / (us * 1e-6) / 1e12 / INT8_PEAK_TOPS,
                          "xcd_tiles": tiles.tolist(),
                          "max_over_mean": float(tiles.max() / tiles.mean())}
        sub["outputs_identical"] = bool(torch.equal(outs["round_robin"], b["combine_buf"]))
        sub["lpt_gain"] = sub["round_robin"]["us"] / sub["lpt"]["us"] - 1.0
        res[tname] = sub
        del plan, b, outs
        torch.cuda.empty_cache()
    del Wd
    torch.cuda.empty_cache()
    return res


def overlap(rounds=20):
    """moedc_combine_limited on 16 workgroups (the 96-token decode batch,
    BF16 expert outputs) beside the expert layer of another batch (3000
    tokens, hidden 1152, 40 experts) on a second stream, both at the default
    priority: one round run serially on one stream, and with the two on two
    streams; also with the uncapped combine.  Mean device time per round
    between events on the launching stream."""
    import dataclasses

    import numpy as np
    import torch

    from combine_moedc_route_amd import moedc as M
    from combine_moedc_route_amd import workloads as W
    wa = W.get("decode")
    pa = M.Plan.from_workload(wa)
    ba = pa.alloc("cuda:0")
    xa, la = W.make_inputs(wa)
    pa.route(torch.from_numpy(la).cuda(), ba["topk_ids"], ba["topk_w"], ba["counts"],
             ba["offsets"], ba["slots"], ba["dropped"], ba["workspace"])
    pa.dispatch(torch.from_numpy(xa.view(np.int16)).cuda(), ba["slots"], ba["dispatch_buf"])
    pa.expert_stub(ba["counts"], ba["dispatch_buf"], ba["combine_buf"], ba["workspace"])
    ya = torch.empty((wa.tokens, wa.hidden), dtype=torch.int16, device="cuda")
    wb = dataclasses.replace(W.with_tokens(W.get("ragged"), 3000),
                             capacity=np.full(40, 470, np.int32))
    pb = M.Plan.from_workload(wb)
    bb = pb.alloc("cuda:0")
    xb, lb = W.make_inputs(wb)
    pb.route(torch.from_numpy(lb).cuda(), bb["topk_ids"], bb["topk_w"], bb["counts"],
             bb["offsets"], bb["slots"], bb["dropped"], bb["workspace"])
    pb.dispatch(torch.from_numpy(xb.view(np.int16)).cuda(), bb["slots"], bb["dispatch_buf"])
    Wt, wsc = W.make_expert_weights(61, wb.num_phys, wb.hidden)
    Wd, wsd = torch.from_numpy(Wt).cuda(), torch.from_numpy(wsc).cuda()
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()

    def comb(stream, cap):
        if cap:
            pa.combine_limited(ba["combine_buf"], M.FMT_BF16, ba["slots"], ba["topk_w"], ya, 16,
                               stream=stream)
        else:
            pa.combine(ba["combine_buf"], M.FMT_BF16, ba["slots"], ba["topk_w"], ya,
                       stream=stream)

    def expert(stream):
        pb.expert_w8a8(bb["counts"], bb["dispatch_buf"], Wd, wsd, bb["combine_buf"],
                       bb["workspace"], stream=stream)

    def timed(body):
        """Mean us per round of `body(rounds)`, which issues all rounds."""
        body(3)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(main)
        body(rounds)
        e1.record(main)
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / rounds

    def serial(cap, n):
        for _ in range(n):
            comb(main, cap)
            expert(main)

    def parallel(cap, n):
        # every round's combine on one stream, every expert layer on the
        # other, joined once at the end
        s1.wait_stream(main)
        s2.wait_stream(main)
        for _ in range(n):
            comb(s1, cap)
        for _ in range(n):
            expert(s2)
        main.wait_stream(s1)
        main.wait_stream(s2)

    res = {"what": "combine of the 96-token decode batch beside the expert layer of a "
                   "3000-token batch (hidden 1152, 40 experts); mean us per round over "
                   f"{rounds} rounds issued back to back (two streams joined once)",
           "combine_16wg_alone_us": timed(lambda n: [comb(main, True) for _ in range(n)]),
           "combine_alone_us": timed(lambda n: [comb(main, False) for _ in range(n)]),
           "expert_alone_us": timed(lambda n: [expert(main) for _ in range(n)])}
    for cap, name in ((True, "capped_16wg"), (False, "uncapped")):
        res[name] = {"serial_us": timed(lambda n: serial(cap, n)),
                     "two_streams_us": timed(lambda n: parallel(cap, n))}
        res[name]["saved_us"] = res[name]["serial_us"] - res[name]["two_streams_us"]
    return res


def dispatch_trace(workload="global", sample_us=0.5):
    """One moedc_dispatch of `workload` run by the trace build
    (libmoedc_trace.so, per-wave phase stamps on the 100 MHz constant
    clock): per-phase durations over all waves, and per CU, at every
    `sample_us` of the launch, how many of its resident waves are loading
    (start -> chunk loaded), quantizing (-> quantized) or storing (-> stores
    complete) -- whether the load -> quantize -> write pipeline of the
    token stream overlaps on each CU."""
    import numpy as np
    import torch

    from combine_moedc_route_amd import build as B
    from combine_moedc_route_amd import moedc as M
    from combine_moedc_route_amd import workloads as W
    import ctypes as C
    wl = W.get(workload)
    T, H = wl.tokens, wl.hidden
    nw = -(-H // 512)
    prev = M._lib
    M._lib = M.load_library(B.TRACE_LIB)
    try:
        L = M._lib
        L.moedc_trace_set.argtypes = [C.c_void_p, C.c_int64]
        L.moedc_trace_set.restype = C.c_int32
        plan = M.Plan.from_workload(wl)
        b = plan.alloc("cuda:0")
        x, logits = W.make_inputs(wl)
        xd = torch.from_numpy(x.view(np.int16)).cuda()
        del x
        plan.route(torch.from_numpy(logits).cuda(), b["topk_ids"], b["topk_w"], b["counts"],
                   b["offsets"], b["slots"], b["dropped"], b["workspace"])
        for _ in range(3):
            plan.dispatch(xd, b["slots"], b["dispatch_buf"])
        tr = torch.zeros((T * nw, 8), dtype=torch.int64, device="cuda")
        torch.cuda.synchronize()
        if L.moedc_trace_set(tr.data_ptr(), tr.numel() * 8):
            raise RuntimeError("moedc_trace_set failed")
        plan.dispatch(xd, b["slots"], b["dispatch_buf"])
        torch.cuda.synchronize()
        L.moedc_trace_set(None, 0)
        rec = tr.cpu().numpy().view(np.uint64)
        del plan, b, xd, tr
        torch.cuda.empty_cache()
    finally:
        M._lib = prev
    return {"workload": f"{workload}: {wl.description}",
            **trace_summary(rec, T, nw, sample_us)}


def trace_summary(rec, T, nw, sample_us=0.5):
    """Decode dispatch trace records (uint64 [T * nw][8], the layout of
    include/moedc_trace.h) into per-phase durations and the per-CU phase
    overlap over the launch."""
    import numpy as np
    tok, wave = (rec[:, 0] >> np.uint64(32)).astype(np.int64), (rec[:, 0] & np.uint64(0xFFFF)).astype(np.int64)
    idx = np.arange(T * nw)
    written = bool(np.array_equal(tok * nw + wave, idx) and (rec[:, 2] > 0).all())
    ts = rec[:, 2:].astype(np.int64)
    ts = (ts - ts[:, 0].min()) * 1e-2  # us (10 ns ticks)
    monotone = bool((np.diff(ts, axis=1) >= 0).all())
    hw = rec[:, 1]
    cu = ((hw >> np.uint64(32)) << np.uint64(8)) | ((hw >> np.uint64(8)) & np.uint64(0xFF))
    names = ["load", "scales", "quantize", "store issue", "store complete"]
    d = np.diff(ts, axis=1)
    phases = {n: {"median_us": float(np.median(d[:, k])), "p90_us": float(np.percentile(d[:, k], 90)),
                  "max_us": float(d[:, k].max())} for k, n in enumerate(names)}
    span = float(ts[:, 5].max())
    grid = np.arange(0.0, span, sample_us)
    ucu, inv = np.unique(cu, return_inverse=True)
    # per (CU, sample): waves in each phase
    counts = np.zeros((3, len(ucu), len(grid)), np.int32)
    bounds = [(0, 1), (1, 3), (3, 5)]  # load, quantize (scales + quantize), store
    for k, (lo, hi) in enumerate(bounds):
        a = np.searchsorted(grid, ts[:, lo], side="left")
        z = np.searchsorted(grid, ts[:, hi], side="left")
        diff = np.zeros((len(ucu), len(grid) + 1), np.int32)
        np.add.at(diff, (inv, a), 1)
        np.add.at(diff, (inv, z), -1)
        counts[k] = np.cumsum(diff, axis=1)[:, :-1]
    busy = counts.sum(0) > 0
    both = (counts[0] > 0) & (counts[2] > 0)
    three = (counts[0] > 0) & (counts[1] > 0) & (counts[2] > 0)
    return {"waves": int(T * nw), "cus": int(len(ucu)),
            "records_complete": written, "stamps_monotone": monotone,
            "span_us": span, "phase_us": phases,
            "resident_waves_per_cu_mean": float(counts.sum(0)[busy].mean()),
            "frac_busy_cu_samples_loading_and_storing": float(both[busy].mean()),
            "frac_busy_cu_samples_all_three_phases": float(three[busy].mean()),
            "sample_us": sample_us,
            "what": "per CU and time sample: waves between start and chunk loaded (loading), "
                    "chunk loaded and quantized (quantizing), quantized and stores complete "
                    "(storing)"}


def placement(workers=8, redundant=32, max_replicas=8):
    """Load balancing on the skewed workload (Zipf(1.1) popularity over 256
    experts, top-8, 30720 tokens): per-expert loads from the device route,
    a redundant-copy table from moedc_place_replicas, the device route again
    with the workload's fixed table and with the planned one (largest token
    count per physical copy), and the expert layer's 128 x 256 tiles per
    copy assigned to `workers` devices by moedc_lpt_partition vs round-robin."""
    import numpy as np
    import torch

    from combine_moedc_route_amd import moedc as M
    from combine_moedc_route_amd import workloads as W
    wl = W.get("skewed")
    T, E, KR, H = wl.tokens, wl.num_logical, wl.top_k, wl.hidden
    _, logits = W.make_inputs(wl)
    lg = torch.from_numpy(logits).cuda()

    def route_counts(P, table):
        plan = M.Plan(max_tokens=T, hidden=128, num_logical=E, num_phys=P, top_k=KR,
                      capacity=np.full(P, T, np.int32), replica_table=table)
        i32 = dict(dtype=torch.int32, device="cuda")
        ws = torch.empty(plan.sizes.workspace_bytes, dtype=torch.uint8, device="cuda")
        plan.bind_workspace(ws)
        counts = torch.empty(P, **i32)
        plan.route(lg, torch.empty((T, KR), **i32), torch.empty((T, KR), device="cuda"), counts,
                   torch.empty(P + 1, **i32), torch.empty((T, KR), **i32), torch.empty(1, **i32), ws)
        return counts.cpu().numpy().astype(np.int64)

    load = route_counts(E, None)
    t0 = time.perf_counter()
    table = M.place_replicas(load.astype(np.float64), redundant, max_replicas)
    t_place = time.perf_counter() - t0
    fixed = route_counts(E + redundant, wl.replica_table)
    planned = route_counts(E + redundant, table)
    tiles = np.ceil(planned / 128.0) * (H // 256)
    t0 = time.perf_counter()
    assign, makespan = M.lpt_partition(tiles, workers)
    t_lpt = time.perf_counter() - t0
    rr = np.bincount(np.arange(tiles.size) % workers, weights=tiles, minlength=workers).max()
    return {"workload": f"skewed: {wl.description}",
            "max_tokens_per_copy": {"no_replicas": int(load.max()), "fixed_table": int(fixed.max()),
                                    "planned_table": int(planned.max()),
                                    "mean_per_copy": T * KR / (E + redundant)},
            "experts_replicated": int(((table >= 0).sum(axis=1) > 1).sum()),
            "max_copies": int((table >= 0).sum(axis=1).max()),
            "place_replicas_us": 1e6 * t_place,
            f"expert_tiles_on_{workers}_devices": {"lower_bound": float(tiles.sum() / workers),
                                                  "round_robin": float(rr), "lpt": float(makespan)},
            "lpt_partition_us": 1e6 * t_lpt}


def calib_copy(args):
    """A plain device-to-device copy of a known byte count (reads N, writes N)."""
    import torch
    n = args.calib_bytes
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / args.steps
    print(json.dumps({"calib_copy_bytes": n, "us_per_copy": us,
                      "GBps_read_plus_write": 2 * n / (us * 1e-6) / 1e9}), flush=True)


def summarize_rocprof(d, out):
    """Condense rocprofv3 CSV output (kernel stats and/or counters) to text."""
    import csv
    lines = []
    for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        lines.append(f"# kernel stats: {os.path.relpath(path, d)}")
        with open(path) as f:
            rows = list(csv.DictReader(f))
        lines.append(f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel")
        for r in rows:
            lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                         f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                         f"{float(r['Percentage']):6.2f}  {r['Name'][:110]}")
        # Kernels launched with several grid sizes (one kernel serving the
        # global and the decode batch): one row per launch shape, from the trace.
        trace = path.replace("kernel_stats.csv", "kernel_trace.csv")
        if os.path.exists(trace):
            shapes = {}
            with open(trace) as f:
                for r in csv.DictReader(f):
                    key = (r["Kernel_Name"], int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
                    shapes.setdefault(key, []).append(
                        (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            names = {}
            for (k, g, w) in shapes:
                names[k] = names.get(k, 0) + 1
            multi = sorted(key for key in shapes if names[key[0]] > 1 and "moedc::" in key[0])
            if multi:
                lines.append("# per launch shape (kernels launched with several grid sizes): "
                             + os.path.relpath(trace, d))
                lines.append(f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} "
                             f"{'threads':>10} {'wg':>5}  kernel")
                for (k, g, w) in multi:
                    v = shapes[(k, g, w)]
                    lines.append(f"{len(v):6d} {statistics.fmean(v):10.2f} {min(v):10.2f} "
                                 f"{max(v):10.2f} {g:10d} {w:5d}  {k[:110]}")
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        lines.append(f"# counters: {os.path.relpath(path, d)}")
        agg = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                key = (r.get("Kernel_Name", "")[:110], r.get("Counter_Name", ""))
                agg.setdefault(key, []).append(float(r.get("Counter_Value", "nan")))
        lines.append(f"{'n':>5} {'mean_per_dispatch':>20} {'counter':>14}  kernel")
        for (k, c), v in sorted(agg.items()):
            lines.append(f"{len(v):5d} {statistics.fmean(v):20.1f} {c:>14}  {k}")
    text = "\n".join(lines) + "\n"
    if out:
        with open(out, "w") as f:
            f.write(text)
    print(text)


# Kernel of each path step in a one-workload bench run (name patterns):
# combine on BF16 expert outputs, dispatch with a workgroup per token, the
# route's top-k kernel and the expert layer's GEMM.
TRAFFIC_TAGS = {"combine": r"combine_kernel<\d+, false,", "dispatch": r"dispatch_token_block<false, true>",
                "route": r"route_topk<", "expert_gemm": r"expert_gemm_groups\("}


def record_traffic(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_bytes):
    """Per-launch HBM bytes of each kernel of one workload's bench run from
    its FETCH_SIZE and WRITE_SIZE runs, each counter scaled by what it reads
    for a plain copy of known size; merged into the committed table under
    the workload's name."""
    import csv

    def per_kernel(d, counter):
        agg = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if r.get("Counter_Name") == counter:
                        agg.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: statistics.fmean(v) * 1024 for k, v in agg.items()}  # KiB -> B

    def copy_factor(d, counter):
        v = [b for k, b in per_kernel(d, counter).items() if "copyBuffer" in k]
        return copy_bytes / max(v)

    ff = copy_factor(copy_fetch_dir, "FETCH_SIZE")
    fw = copy_factor(copy_write_dir, "WRITE_SIZE")
    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    entry = {}
    for key, tag in TRAFFIC_TAGS.items():
        kf = [k for k in fetch if re.search(tag, k)]
        kw = [k for k in write if re.search(tag, k)]
        if len(kf) != 1 or len(kw) != 1:
            if kf or kw:
                raise SystemExit(f"record_traffic: {key}: expected one kernel matching {tag!r}, "
                                 f"found {kf} / {kw}; nothing written")
            continue
        entry[key] = {"source_sha": source_sha(KERNEL_SOURCES[key]), "kernel": kf[0][:120],
                      "fetch_bytes": fetch[kf[0]] * ff, "write_bytes": write[kw[0]] * fw,
                      "bytes_per_launch": fetch[kf[0]] * ff + write[kw[0]] * fw}
    if "combine" not in entry or "dispatch" not in entry:
        raise SystemExit(f"record_traffic: no combine/dispatch counter rows in {fetch_dir} / "
                         f"{write_dir}; nothing written")
    try:
        with open(TRAFFIC_FILE) as f:
            out = json.load(f)
    except (OSError, ValueError):
        out = {}
    out = {k: v for k, v in out.items() if isinstance(v, dict) and "source_sha" not in v}
    out["_about"] = ("HBM bytes per launch, by workload and kernel, from rocprofv3 FETCH_SIZE "
                     "and WRITE_SIZE runs scaled by what each counter reads for a plain "
                     f"{copy_bytes}-byte copy; an entry is valid while its source_sha matches.")
    out[workload] = {"fetch_scale": ff, "write_scale": fw, **entry}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out[workload], indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="global")
    ap.add_argument("--combine-fmt", choices=["bf16", "q8"], default="bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-expert", action="store_true")
    ap.add_argument("--no-placement", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--no-workloads", action="store_true")
    ap.add_argument("--no-lpt", action="store_true")
    ap.add_argument("--decode-only", action="store_true")
    ap.add_argument("--dispatch-trace", metavar="WORKLOAD")
    ap.add_argument("--cpu-tokens", type=int, default=30720)
    ap.add_argument("--calib-copy", action="store_true")
    ap.add_argument("--calib-bytes", type=int, default=4 << 30)
    ap.add_argument("--summarize-rocprof", metavar="DIR")
    ap.add_argument("--record-traffic", nargs=5,
                    metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"))
    ap.add_argument("--out")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(*args.record_traffic, copy_bytes=args.calib_bytes)
        return
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof, args.out)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: libmoedc runs on exactly one GPU (the MoE path's simulated "
              "expert-parallel ranks are partitions of one GPU's HBM); --gpus must be 1.",
              file=sys.stderr, flush=True)
        sys.exit(2)
    if args.calib_copy:
        calib_copy(args)
        return
    if args.dispatch_trace:
        print(json.dumps(dispatch_trace(args.dispatch_trace)), flush=True)
        return
    if args.decode_only:
        res = decode_latency()
        res["small_batches"] = {
            str(n): decode_latency(tokens=n, which=("route", "route_dispatch_fused", "fused_step"))
            for n in (1, 16)}
        print(json.dumps(res), flush=True)
        return
    run(args)


if __name__ == "__main__":
    main()
