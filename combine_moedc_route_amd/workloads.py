"""Seeded synthetic workloads for MoE route / dispatch / combine.

This module only draws inputs and describes shapes; it holds none of the
method's arithmetic (no routing, quantization or reduction).  Both the HIP
path's tests/benchmark and the CPU oracle take their inputs from here.

Shapes follow the pages' decode deployment ("CloudMatrix384: Co-Designing
Supernodes for Trillion-Parameter LLM Inference", section "Decode Phase":
hidden 7168, 256 routed experts, top-8, 96 tokens per die, 30,720 tokens
globally, plus shared and redundant experts) and the StrataCL analysis
(section 4.1: hidden 7168, top-8 dispatch/combine microbenchmark).  No
public dataset is involved: activations and router logits are synthetic.

Recipe (numpy PCG64 ``default_rng(seed)``; draw order x, logits, extras):
  * x: standard normal float32, optional whole-row outlier scaling in fp32,
    then rounded to BF16 by torch's float32->bfloat16 conversion.
  * logits: float32 N(0,1), U[0,1), or Zipf(1.1) popularity via
    ``ln p_e + Gumbel(0,1)`` (Gumbel-top-k = sampling without replacement).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SCORE_SOFTMAX = 0
SCORE_SIGMOID_NORM = 1


@dataclasses.dataclass
class Workload:
    name: str
    description: str
    tokens: int
    hidden: int
    num_logical: int
    num_phys: int
    top_k: int
    num_shared: int
    score_fn: int
    capacity: np.ndarray                    # int32 [num_phys]
    replica_table: Optional[np.ndarray]     # int32 [num_logical][R] or None
    seed: int
    logits_kind: str                        # "normal" | "uniform" | "zipf"
    outliers: Optional[tuple] = None        # ("per_group", group, rows, factor) | ("fraction", frac, factor)
    expert: str = "stub"                    # "identity" (combine reads dispatch slots) | "stub"
    zipf_s: float = 1.1
    group_size: int = 128                   # values per fp32 scale: 128, or hidden (per token)

    @property
    def K(self) -> int:
        return self.top_k + self.num_shared

    @property
    def total_slots(self) -> int:
        return int(self.capacity.astype(np.int64).sum())


def _uniform_caps(P, cap):
    return np.full(P, cap, dtype=np.int32)


def _skewed():
    E, R_hot = 256, 32
    table = np.full((E, 2), -1, dtype=np.int32)
    table[:, 0] = np.arange(E)
    table[:R_hot, 1] = E + np.arange(R_hot)
    P = E + R_hot
    cap = np.full(P, 1728, dtype=np.int32)       # round_up(2*T*K/288, 64)
    cap[:R_hot] = 15360                          # hot primaries: T/2
    cap[E:] = 15360                              # their replicas
    return Workload(
        "skewed", "30720 tokens, hidden 7168, 256 logical experts with Zipf(1.1) "
        "popularity + 32 redundant replicas (288 physical), top-8; 8 of every 96 "
        "rows scaled x50", 30720, 7168, E, P, 8, 0, SCORE_SIGMOID_NORM, cap, table,
        4, "zipf", ("per_group", 96, 8, 50.0))


def _prefill():
    E = 256
    cap = np.full(E + 1, 4096, dtype=np.int32)
    cap[E] = 65536
    return Workload(
        "prefill", "65536 tokens, hidden 7168, 256 routed + 1 shared expert "
        "(top-8+1), 1% rows scaled x100", 65536, 7168, E, E + 1, 8, 1,
        SCORE_SIGMOID_NORM, cap, None, 5, "normal", ("fraction", 0.01, 100.0))


def _make_all():
    w = {}
    w["tiny"] = Workload(
        "tiny", "64 tokens, hidden 256, 8 experts, top-2 softmax gates, "
        "identity experts", 64, 256, 8, 8, 2, 0, SCORE_SOFTMAX,
        _uniform_caps(8, 64), None, 1, "normal", None, "identity")
    w["decode"] = Workload(
        "decode", "96 tokens (one die's decode batch), hidden 7168, 256 experts, "
        "top-8 sigmoid-normalised", 96, 7168, 256, 256, 8, 0, SCORE_SIGMOID_NORM,
        _uniform_caps(256, 96), None, 2, "normal")
    w["decode_pt"] = dataclasses.replace(
        w["decode"], name="decode_pt", description="96 tokens, hidden 7168, 256 experts, "
        "top-8 sigmoid-normalised, one INT8 scale per token", seed=6, group_size=7168,
        outliers=("per_group", 96, 8, 50.0))
    w["global"] = Workload(
        "global", "30720 tokens (global decode batch), hidden 7168, 256 experts, "
        "top-8 from U[0,1) logits, capacity 1920 per expert", 30720, 7168, 256,
        256, 8, 0, SCORE_SIGMOID_NORM, _uniform_caps(256, 1920), None, 3,
        "uniform")
    w["skewed"] = _skewed()
    w["prefill"] = _prefill()
    # Parity-only cases: several tiles plus ragged tails, and edge cases.
    w["mid"] = Workload(
        "mid", "1000 tokens, hidden 7168, 256 experts, top-8 (ragged token tail)",
        1000, 7168, 256, 256, 8, 0, SCORE_SIGMOID_NORM, _uniform_caps(256, 64),
        None, 11, "normal")
    w["ragged"] = Workload(
        "ragged", "333 tokens, hidden 1152 (9 groups), 40 experts, top-6 softmax",
        333, 1152, 40, 40, 6, 0, SCORE_SOFTMAX, _uniform_caps(40, 60), None, 12,
        "normal")
    w["overflow"] = Workload(
        "overflow", "700 tokens, hidden 512, 16 experts, top-4, capacity 100 "
        "(drops)", 700, 512, 16, 16, 4, 0, SCORE_SIGMOID_NORM,
        _uniform_caps(16, 100), None, 13, "zipf", ("fraction", 0.05, 1000.0))
    rep = np.full((12, 3), -1, dtype=np.int32)
    rep[:, 0] = np.arange(12)
    rep[0, 1:] = [12, 13]
    rep[1, 1] = 14
    w["replica_shared"] = Workload(
        "replica_shared", "517 tokens, hidden 384, 12 logical experts, 3 replicas "
        "(16 physical incl. 1 shared), top-3+1", 517, 384, 12, 16, 3, 1,
        SCORE_SIGMOID_NORM, np.array([300] * 15 + [517], np.int32), rep, 14,
        "zipf", ("fraction", 0.02, 100.0))
    return w


WORKLOADS = _make_all()


def get(name: str) -> Workload:
    return WORKLOADS[name]


def with_tokens(wl: Workload, tokens: int) -> Workload:
    """Same workload, fewer tokens (capacities unchanged)."""
    return dataclasses.replace(wl, tokens=tokens)


def _to_bf16_bits(f32: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make_inputs(wl: Workload, tokens: Optional[int] = None):
    """Return (x_bits uint16 [T][H], logits float32 [T][E_log]) for ``wl``.

    ``tokens`` draws only the first rows of the same stream layout (a prefix
    is not bitwise the same as the full draw; each T is its own input set).
    """
    T = wl.tokens if tokens is None else tokens
    rng = np.random.default_rng(wl.seed)
    x = rng.standard_normal((T, wl.hidden), dtype=np.float32)
    E = wl.num_logical
    if wl.logits_kind == "normal":
        logits = rng.standard_normal((T, E), dtype=np.float32)
    elif wl.logits_kind == "uniform":
        logits = rng.random((T, E), dtype=np.float32)
    elif wl.logits_kind == "zipf":
        p = (np.arange(1, E + 1, dtype=np.float64)) ** (-wl.zipf_s)
        p /= p.sum()
        g = rng.gumbel(size=(T, E))
        logits = (np.log(p)[None, :] + g).astype(np.float32)
    else:
        raise ValueError(wl.logits_kind)
    if wl.outliers is not None:
        if wl.outliers[0] == "per_group":
            _, group, rows, factor = wl.outliers
            for g0 in range(0, T, group):
                n = min(group, T - g0)
                pick = rng.choice(n, size=min(rows, n), replace=False)
                x[g0 + pick] *= np.float32(factor)
        else:
            _, frac, factor = wl.outliers
            n = max(1, int(frac * T)) if T else 0
            pick = rng.choice(T, size=n, replace=False) if n else []
            x[pick] *= np.float32(factor)
    return _to_bf16_bits(x), np.ascontiguousarray(logits)


def make_expert_out_bf16(seed: int, rows: int, hidden: int) -> np.ndarray:
    """Random BF16 expert outputs (N(0,1)) for combine-only cases."""
    rng = np.random.default_rng(seed)
    return _to_bf16_bits(rng.standard_normal((rows, hidden), dtype=np.float32))


def make_expert_weights(seed: int, num_phys: int, hidden: int):
    """Synthetic W8A8 expert weights: int8 [P][H][H] uniform in [-127, 127]
    and per-output-channel fp32 scales ~ U[0.5, 1.5) / (127 * sqrt(H))."""
    rng = np.random.default_rng(seed)
    W = rng.integers(-127, 128, size=(num_phys, hidden, hidden), dtype=np.int8)
    ws = (rng.random((num_phys, hidden), dtype=np.float32) + np.float32(0.5)) / \
        np.float32(127.0 * np.sqrt(hidden))
    return W, ws.astype(np.float32)


def make_gates(seed: int, T: int, K: int) -> np.ndarray:
    """Random positive fp32 gate weights for combine-only cases."""
    rng = np.random.default_rng(seed)
    return rng.random((T, K), dtype=np.float32)
