"""CPU oracle for MoE route / INT8 dispatch / combine -- TEST INFRASTRUCTURE.

Only ``tests/``, the smoke entry point and the benchmark's CPU-baseline leg
may import this package.  The product path (``combine_moedc_route_amd``)
never does; it fails loudly when its HIP library is missing instead.

This module is a ctypes wrapper over ``moedc_oracle.c`` taking and returning
numpy arrays.  It holds no arithmetic of the method itself.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

SCORE_SOFTMAX = 0
SCORE_SIGMOID_NORM = 1
FMT_BF16 = 0
FMT_Q8 = 1

_lib = None


class OrcCfg(C.Structure):
    _fields_ = [
        ("hidden", C.c_int32),
        ("group_size", C.c_int32),
        ("num_logical", C.c_int32),
        ("num_phys", C.c_int32),
        ("top_k", C.c_int32),
        ("num_shared", C.c_int32),
        ("score_fn", C.c_int32),
        ("max_replicas", C.c_int32),
        ("replica_table", C.POINTER(C.c_int32)),
        ("capacity", C.POINTER(C.c_int32)),
    ]


def lib():
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        L = C.CDLL(path)
        P = C.c_void_p
        i32, i64 = C.c_int32, C.c_int64
        L.orc_check_cfg.argtypes = [C.POINTER(OrcCfg)]
        L.orc_topk_row.argtypes = [i32, i32, P, P]
        L.orc_f32_to_bf16.argtypes = [C.c_float]
        L.orc_f32_to_bf16.restype = C.c_uint16
        L.orc_f32_to_bf16_array.argtypes = [i64, P, P]
        L.orc_f32_to_bf16_array.restype = None
        L.orc_route.argtypes = [C.POINTER(OrcCfg), i32, P, P, P, P, P, P, P]
        L.orc_quantize_group.argtypes = [i32, P, P, P]
        L.orc_quantize_token.argtypes = [i32, i32, P, P, P]
        L.orc_dispatch.argtypes = [C.POINTER(OrcCfg), i32, P, P, P, i64]
        L.orc_expert_stub.argtypes = [C.POINTER(OrcCfg), P, P, i64, P, i64]
        L.orc_combine.argtypes = [C.POINTER(OrcCfg), i32, P, i32, i64, P, P, P]
        L.orc_expert_w8a8.argtypes = [C.POINTER(OrcCfg), P, P, i64, P, P, P, i64]
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(C.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


class Cfg:
    """Holds the numpy arrays a ``OrcCfg`` points into, keeping them alive."""

    def __init__(self, hidden, num_logical, num_phys, top_k, num_shared,
                 score_fn, capacity, replica_table=None, group_size=128):
        self.capacity = np.ascontiguousarray(capacity, dtype=np.int32)
        self.replica_table = (None if replica_table is None else
                              np.ascontiguousarray(replica_table, dtype=np.int32))
        R = 1 if self.replica_table is None else self.replica_table.shape[1]
        self.c = OrcCfg(
            hidden, group_size, num_logical, num_phys, top_k, num_shared, score_fn, R,
            (None if self.replica_table is None else
             self.replica_table.ctypes.data_as(C.POINTER(C.c_int32))),
            self.capacity.ctypes.data_as(C.POINTER(C.c_int32)))
        self.hidden = hidden
        self.group_size = group_size
        self.num_phys = num_phys
        self.K = top_k + num_shared

    @classmethod
    def from_workload(cls, wl):
        return cls(wl.hidden, wl.num_logical, wl.num_phys, wl.top_k,
                   wl.num_shared, wl.score_fn, wl.capacity, wl.replica_table,
                   getattr(wl, "group_size", 128))

    def check(self):
        return lib().orc_check_cfg(C.byref(self.c))


def topk_row(row, k):
    row = np.ascontiguousarray(row, dtype=np.float32)
    out = np.empty(k, dtype=np.int32)
    _check(lib().orc_topk_row(row.size, k, _p(row), _p(out)), "topk_row")
    return out


def f32_to_bf16(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().orc_f32_to_bf16_array(a.size, _p(a), _p(out))
    return out


def route(cfg: Cfg, logits):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T = logits.shape[0]
    K, P = cfg.K, cfg.num_phys
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    counts = np.empty(P, np.int32)
    offsets = np.empty(P + 1, np.int32)
    slots = np.empty((T, K), np.int32)
    dropped = np.zeros(1, np.int32)
    _check(lib().orc_route(C.byref(cfg.c), T, _p(logits), _p(ids), _p(w),
                           _p(counts), _p(offsets), _p(slots), _p(dropped)),
           "route")
    return dict(topk_ids=ids, topk_w=w, counts=counts, offsets=offsets,
                slots=slots, dropped=int(dropped[0]))


def quantize_group(x_bits):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    q = np.empty(x.size, np.int8)
    s = np.empty(1, np.float32)
    _check(lib().orc_quantize_group(x.size, _p(x), _p(q), _p(s)), "quantize_group")
    return q, s[0]


def quantize_tokens(x_bits, group_size=128):
    """Quantize rows of a [T][H] uint16 BF16 array in groups of group_size
    -> (q [T][H] int8, s [T][H/group_size] f32)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x.shape
    q = np.empty((T, H), np.int8)
    s = np.empty((T, H // group_size), np.float32)
    for t in range(T):
        _check(lib().orc_quantize_token(H, group_size, _p(x[t]), _p(q[t]), _p(s[t])),
               "quantize_token")
    return q, s


def dispatch(cfg: Cfg, x_bits, slots, total_slots, slot_stride, buf=None):
    """Dispatch into ``buf`` ([total_slots][slot_stride] uint8, zero-filled if None)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    slots = np.ascontiguousarray(slots, dtype=np.int32)
    if buf is None:
        buf = np.zeros((total_slots, slot_stride), np.uint8)
    assert buf.shape == (total_slots, slot_stride) and buf.dtype == np.uint8
    assert buf.flags.c_contiguous
    _check(lib().orc_dispatch(C.byref(cfg.c), x.shape[0], _p(x), _p(slots),
                              _p(buf), slot_stride), "dispatch")
    return buf


def expert_stub(cfg: Cfg, counts, dbuf, slot_stride):
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    S = dbuf.shape[0]
    H = cfg.hidden
    ebuf = np.zeros((S, H), np.uint16)
    _check(lib().orc_expert_stub(C.byref(cfg.c), _p(counts), _p(dbuf),
                                 slot_stride, _p(ebuf), 2 * H), "expert_stub")
    return ebuf


def expert_w8a8(cfg: Cfg, counts, dbuf, slot_stride, W, w_scale, ebuf=None):
    """One W8A8 linear layer per physical expert over the occupied slots.
    W: int8 [P][H][H]; w_scale: fp32 [P][H]; returns ebuf uint16 [S][H]."""
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    W = np.ascontiguousarray(W, dtype=np.int8)
    w_scale = np.ascontiguousarray(w_scale, dtype=np.float32)
    H = cfg.hidden
    if ebuf is None:
        ebuf = np.zeros((dbuf.shape[0], H), np.uint16)
    _check(lib().orc_expert_w8a8(C.byref(cfg.c), _p(counts), _p(dbuf), slot_stride,
                                 _p(W), _p(w_scale), _p(ebuf), 2 * H), "expert_w8a8")
    return ebuf


def combine(cfg: Cfg, eout, fmt, slots, topk_w, out=None):
    """eout: [S][H] uint16 (FMT_BF16) or [S][slot_stride] uint8 (FMT_Q8);
    the result goes to ``out`` ([T][H] uint16) when given."""
    eout = np.ascontiguousarray(eout)
    slots = np.ascontiguousarray(slots, dtype=np.int32)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    T = slots.shape[0]
    if out is None:
        out = np.empty((T, cfg.hidden), np.uint16)
    assert out.shape == (T, cfg.hidden) and out.dtype == np.uint16 and out.flags.c_contiguous
    y = out
    stride = eout.strides[0]
    _check(lib().orc_combine(C.byref(cfg.c), T, _p(eout), fmt, stride,
                             _p(slots), _p(w), _p(y)), "combine")
    return y
