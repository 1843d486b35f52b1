"""Host planning algorithms (no GPU): redundant-expert placement and the
LPT list scheduler, checked against brute-force optima and Graham's bound."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from combine_moedc_route_amd import moedc as M
from combine_moedc_route_amd import workloads as W


def max_per_copy(load, table):
    copies = (table >= 0).sum(axis=1)
    return max(Fraction(int(l)) / int(c) for l, c in zip(load, copies))


@pytest.mark.parametrize("seed", range(40))
def test_place_replicas_is_minmax_optimal(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 6))
    R = int(rng.integers(1, 4))
    N = int(rng.integers(0, E * (R - 1) + 1))
    load = rng.integers(0, 50, E)
    table = M.place_replicas(load, N, R)
    # Layout: row e starts with e; extra ids E..E+N-1 each once; -1 padding.
    assert (table[:, 0] == np.arange(E)).all()
    extra = table[:, 1:][table[:, 1:] >= 0]
    assert sorted(extra.tolist()) == list(range(E, E + N))
    for row in table:
        k = (row >= 0).sum()
        assert (row[k:] == -1).all()
    best = None
    for r in itertools.product(range(1, R + 1), repeat=E):
        if sum(r) - E != N:
            continue
        v = max(Fraction(int(l)) / c for l, c in zip(load, r))
        best = v if best is None else min(best, v)
    assert max_per_copy(load, table) == best


def test_place_replicas_rejects_bad_input():
    with pytest.raises(M.MoedcError):
        M.place_replicas([1.0, 2.0], 3, 2)           # only 2 extra copies fit
    with pytest.raises(M.MoedcError):
        M.place_replicas([1.0, -2.0], 1, 2)
    with pytest.raises(M.MoedcError):
        M.place_replicas([1.0, float("nan")], 1, 2)


def test_place_replicas_on_zipf_loads_beats_fixed_table():
    wl = W.get("skewed")
    E = wl.num_logical
    p = np.arange(1, E + 1, dtype=np.float64) ** -wl.zipf_s
    p /= p.sum()
    # Expected load with sampling K of E without replacement is at most T;
    # use the empirical counts of the workload's own logits as the load.
    _, logits = W.make_inputs(wl, 4096)
    top = np.argsort(-logits, axis=1, kind="stable")[:, :wl.top_k]
    load = np.bincount(top.ravel(), minlength=E).astype(np.float64)
    greedy = M.place_replicas(load, 32, 8)
    fixed = wl.replica_table
    fixed8 = np.full((E, 8), -1, np.int32)
    fixed8[:, :2] = fixed
    assert max_per_copy(load, greedy) <= max_per_copy(load, fixed8)
    # The table is a valid layer description.
    cap = np.full(E + 32, 4096, np.int32)
    M.Plan(max_tokens=4096, hidden=256, num_logical=E, num_phys=E + 32, top_k=8,
           capacity=cap, replica_table=greedy)


def brute_makespan(cost, workers, group=None, cap=0):
    best = None
    for a in itertools.product(range(workers), repeat=len(cost)):
        if cap and group is not None:
            ok = all(len({a[u] for u in range(len(cost)) if group[u] == g}) <= cap
                     for g in set(group))
            if not ok:
                continue
        loads = [0] * workers
        for u, w in enumerate(a):
            loads[w] += cost[u]
        m = max(loads)
        best = m if best is None else min(best, m)
    return best


@pytest.mark.parametrize("seed", range(40))
def test_lpt_within_graham_bound(seed):
    rng = np.random.default_rng(100 + seed)
    U = int(rng.integers(1, 8))
    Wk = int(rng.integers(1, 4))
    cost = rng.integers(1, 20, U).astype(np.float64)
    assign, ms = M.lpt_partition(cost, Wk)
    assert ((assign >= 0) & (assign < Wk)).all()
    loads = np.bincount(assign, weights=cost, minlength=Wk)
    assert ms == loads.max()
    opt = brute_makespan(cost.tolist(), Wk)
    assert opt <= ms <= (4 / 3 - 1 / (3 * Wk)) * opt + 1e-9


def test_lpt_tight_instance():
    # Graham's example: LPT gives 7 on two workers where 6 is optimal.
    assign, ms = M.lpt_partition([3, 3, 2, 2, 2], 2)
    assert ms == 7 and brute_makespan([3, 3, 2, 2, 2], 2) == 6
    assert assign.tolist() == [0, 1, 0, 1, 0]


@pytest.mark.parametrize("seed", range(20))
def test_lpt_fanout_cap_respected(seed):
    rng = np.random.default_rng(200 + seed)
    U, Wk, G = 7, 3, 3
    cost = rng.integers(1, 20, U).astype(np.float64)
    group = rng.integers(0, G, U)
    cap = int(rng.integers(1, 3))
    assign, ms = M.lpt_partition(cost, Wk, group, G, cap)
    for g in range(G):
        assert len(set(assign[group == g].tolist())) <= cap
    assert ms >= brute_makespan(cost.tolist(), Wk, group.tolist(), cap)


def test_lpt_empty_and_errors():
    assign, ms = M.lpt_partition([], 4)
    assert assign.size == 0 and ms == 0.0
    with pytest.raises(M.MoedcError):
        M.lpt_partition([1.0, -1.0], 2)
    with pytest.raises(M.MoedcError):
        M.lpt_partition([1.0, 2.0], 2, [0, 5], 2, 1)
