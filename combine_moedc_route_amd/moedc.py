"""Thin ctypes binding over libmoedc (argument marshalling only).

Every step of route / dispatch / combine runs in the library's HIP kernels;
this module only turns torch tensors into device pointers and the current
HIP stream, and raises on a non-OK status.  There is no fallback: a missing
library raises ``MoedcUnavailable``.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoedc.so")

OK, ERR_INVALID_ARG, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_HIP, ERR_NO_MEMORY = range(7)
SCORE_SOFTMAX, SCORE_SIGMOID_NORM = 0, 1
FMT_BF16, FMT_Q8 = 0, 1
DEAL_LPT, DEAL_ROUND_ROBIN = 0, 1

# Every symbol include/moedc.h declares.
EXPORTS = (
    "moedc_plan_create", "moedc_plan_destroy", "moedc_plan_sizes",
    "moedc_plan_bind_workspace", "moedc_route", "moedc_dispatch",
    "moedc_combine", "moedc_route_dispatch", "moedc_combine_limited",
    "moedc_expert_stub", "moedc_expert_w8a8", "moedc_place_replicas",
    "moedc_lpt_partition", "moedc_status_string", "moedc_last_hip_error",
    "moedc_route_noalloc", "moedc_expert_w8a8_dealt",
)


class MoedcUnavailable(RuntimeError):
    pass


class MoedcError(RuntimeError):
    def __init__(self, status: int, what: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{what}: {status_string(status)} (status {status}"
        msg += f", hip error {hip_error})" if status == ERR_HIP else ")"
        super().__init__(msg)


class Config(C.Structure):
    _fields_ = [
        ("max_tokens", C.c_int32),
        ("hidden", C.c_int32),
        ("group_size", C.c_int32),
        ("num_logical_experts", C.c_int32),
        ("num_phys_experts", C.c_int32),
        ("top_k", C.c_int32),
        ("num_shared", C.c_int32),
        ("score_fn", C.c_int32),
        ("max_replicas", C.c_int32),
        ("capacity", C.POINTER(C.c_int32)),
        ("replica_table", C.POINTER(C.c_int32)),
    ]


class Sizes(C.Structure):
    _fields_ = [
        ("workspace_bytes", C.c_int64),
        ("dispatch_buf_bytes", C.c_int64),
        ("combine_buf_bytes", C.c_int64),
        ("slot_stride", C.c_int64),
        ("combine_slot_stride", C.c_int64),
        ("total_slots", C.c_int64),
        ("k", C.c_int32),
        ("num_groups", C.c_int32),
    ]


_lib = None


def lib():
    """Load libmoedc.so from the package directory (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoedcUnavailable(
                f"{LIB_PATH} is missing; build it with __graft_entry__.build() "
                "or python combine_moedc_route_amd/build.py")
        _lib = load_library(LIB_PATH)
    return _lib


def load_library(path):
    """dlopen a libmoedc build and declare its C signatures."""
    L = C.CDLL(path)
    P, i32 = C.c_void_p, C.c_int32
    L.moedc_plan_create.argtypes = [C.POINTER(Config), C.POINTER(C.c_void_p)]
    L.moedc_plan_create.restype = i32
    L.moedc_plan_destroy.argtypes = [P]
    L.moedc_plan_destroy.restype = None
    L.moedc_plan_sizes.argtypes = [P, C.POINTER(Sizes)]
    L.moedc_plan_sizes.restype = i32
    L.moedc_plan_bind_workspace.argtypes = [P, P, P]
    L.moedc_plan_bind_workspace.restype = i32
    L.moedc_route.argtypes = [P, i32, P, P, P, P, P, P, P, P, P]
    L.moedc_route.restype = i32
    L.moedc_dispatch.argtypes = [P, i32, P, P, P, P]
    L.moedc_dispatch.restype = i32
    L.moedc_combine.argtypes = [P, i32, P, i32, P, P, P, P]
    L.moedc_combine.restype = i32
    L.moedc_route_dispatch.argtypes = [P, i32, P, P, P, P, P, P, P, P, P, P, P]
    L.moedc_route_dispatch.restype = i32
    L.moedc_combine_limited.argtypes = [P, i32, P, i32, P, P, P, i32, P]
    L.moedc_combine_limited.restype = i32
    L.moedc_expert_w8a8.argtypes = [P, P, P, P, P, P, P, P]
    L.moedc_expert_w8a8.restype = i32
    L.moedc_expert_w8a8_dealt.argtypes = [P, P, P, P, P, P, P, i32, P, P]
    L.moedc_expert_w8a8_dealt.restype = i32
    L.moedc_expert_stub.argtypes = [P, P, P, P, P, P]
    L.moedc_expert_stub.restype = i32
    L.moedc_place_replicas.argtypes = [i32, P, i32, i32, P]
    L.moedc_place_replicas.restype = i32
    L.moedc_lpt_partition.argtypes = [i32, P, P, i32, i32, i32, P, C.POINTER(C.c_double)]
    L.moedc_lpt_partition.restype = i32
    L.moedc_route_noalloc.argtypes = [P, i32, P, P, P, P, P, P, P, P]
    L.moedc_route_noalloc.restype = i32
    L.moedc_status_string.argtypes = [i32]
    L.moedc_status_string.restype = C.c_char_p
    L.moedc_last_hip_error.argtypes = []
    L.moedc_last_hip_error.restype = i32
    return L


def status_string(status: int) -> str:
    return lib().moedc_status_string(status).decode()


def _check(status: int, what: str):
    if status != OK:
        raise MoedcError(status, what, lib().moedc_last_hip_error() if status == ERR_HIP else 0)


def _ptr(t) -> Optional[int]:
    """Device address of a torch tensor (None for None)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmoedc takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmoedc takes contiguous tensors")
    return t.data_ptr()


def _need(t, what: str, n: int = 0, nbytes: int = 0, itemsize: int = 0):
    """Refuse a tensor that is too small for what the call will write or read
    (the C ABI sees only its address), or of the wrong element size."""
    if itemsize and t.element_size() != itemsize:
        raise ValueError(f"{what}: {itemsize}-byte elements expected, got {t.dtype}")
    if n and t.numel() < n:
        raise ValueError(f"{what}: needs {n} elements, has {t.numel()}")
    if nbytes and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{what}: needs {nbytes} bytes, has {t.numel() * t.element_size()}")


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def place_replicas(load, num_redundant: int, max_replicas: int) -> np.ndarray:
    """Replica table [E][max_replicas] from expected per-expert loads."""
    load = np.ascontiguousarray(load, dtype=np.float64)
    table = np.empty((load.size, max_replicas), np.int32)
    _check(lib().moedc_place_replicas(load.size, load.ctypes.data_as(C.c_void_p), num_redundant,
                                      max_replicas, table.ctypes.data_as(C.c_void_p)),
           "moedc_place_replicas")
    return table


def lpt_partition(cost, num_workers: int, group=None, num_groups: int = 0,
                  fanout_cap: int = 0):
    """(assign [U] int32, makespan) of the LPT list schedule."""
    cost = np.ascontiguousarray(cost, dtype=np.float64)
    g = None if group is None else np.ascontiguousarray(group, dtype=np.int32)
    assign = np.empty(cost.size, np.int32)
    ms = C.c_double()
    _check(lib().moedc_lpt_partition(cost.size, cost.ctypes.data_as(C.c_void_p),
                                     None if g is None else g.ctypes.data_as(C.c_void_p),
                                     num_groups, num_workers, fanout_cap,
                                     assign.ctypes.data_as(C.c_void_p), C.byref(ms)),
           "moedc_lpt_partition")
    return assign, ms.value


class Plan:
    """A validated layer description (host-only; owns no device memory)."""

    def __init__(self, *, max_tokens: int, hidden: int, num_logical: int,
                 num_phys: int, top_k: int, num_shared: int = 0,
                 score_fn: int = SCORE_SIGMOID_NORM, capacity,
                 replica_table=None, group_size: int = 128):
        self._cap = np.ascontiguousarray(capacity, dtype=np.int32)
        self._rep = (None if replica_table is None
                     else np.ascontiguousarray(replica_table, dtype=np.int32))
        R = 1 if self._rep is None else int(self._rep.shape[1])
        cfg = Config(max_tokens, hidden, group_size, num_logical, num_phys, top_k,
                     num_shared, score_fn, R,
                     self._cap.ctypes.data_as(C.POINTER(C.c_int32)),
                     (None if self._rep is None else
                      self._rep.ctypes.data_as(C.POINTER(C.c_int32))))
        h = C.c_void_p()
        self._h = None
        _check(lib().moedc_plan_create(C.byref(cfg), C.byref(h)), "moedc_plan_create")
        self._h = h
        s = Sizes()
        _check(lib().moedc_plan_sizes(self._h, C.byref(s)), "moedc_plan_sizes")
        self.sizes = s
        self.max_tokens, self.hidden, self.K = max_tokens, hidden, s.k
        self.num_logical, self.num_phys = num_logical, num_phys

    @classmethod
    def from_workload(cls, wl, max_tokens: Optional[int] = None):
        return cls(max_tokens=wl.tokens if max_tokens is None else max_tokens,
                   hidden=wl.hidden, num_logical=wl.num_logical,
                   num_phys=wl.num_phys, top_k=wl.top_k, num_shared=wl.num_shared,
                   score_fn=wl.score_fn, capacity=wl.capacity,
                   replica_table=wl.replica_table,
                   group_size=getattr(wl, "group_size", 128))

    def close(self):
        if self._h is not None:
            lib().moedc_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- device buffers (caller-owned, allocated through torch) ----------
    def alloc(self, device="cuda"):
        """Allocate workspace, route outputs and one dispatch/combine set."""
        import torch
        T, K, P = self.max_tokens, self.K, self.num_phys
        s = self.sizes
        u8 = dict(dtype=torch.uint8, device=device)
        i32 = dict(dtype=torch.int32, device=device)
        bufs = dict(
            workspace=torch.empty(max(s.workspace_bytes, 16), **u8),
            topk_ids=torch.empty((T, K), **i32),
            topk_w=torch.empty((T, K), dtype=torch.float32, device=device),
            counts=torch.empty(P, **i32),
            offsets=torch.empty(P + 1, **i32),
            slots=torch.empty((T, K), **i32),
            dropped=torch.empty(1, **i32),
            dispatch_buf=torch.empty(max(s.dispatch_buf_bytes, 16), **u8),
            combine_buf=torch.empty((max(s.total_slots, 1), self.hidden),
                                    dtype=torch.int16, device=device),
        )
        self.bind_workspace(bufs["workspace"])
        return bufs

    def _route_bufs(self, T, topk_ids, topk_w, counts, offsets, slots, dropped, workspace):
        K, P = self.K, self.num_phys
        _need(topk_ids, "topk_ids", T * K, itemsize=4)
        _need(topk_w, "topk_w", T * K, itemsize=4)
        _need(counts, "counts", P, itemsize=4)
        _need(offsets, "offsets", P + 1, itemsize=4)
        _need(slots, "slots", T * K, itemsize=4)
        _need(dropped, "dropped", 1, itemsize=4)
        _need(workspace, "workspace", nbytes=self.sizes.workspace_bytes)

    def _combine_bufs(self, T, expert_out, fmt, slots, topk_w, y):
        s = self.sizes
        _need(expert_out, "expert_out",
              nbytes=s.dispatch_buf_bytes if fmt == FMT_Q8 else s.combine_buf_bytes)
        _need(slots, "slots", T * self.K, itemsize=4)
        _need(topk_w, "topk_w", T * self.K, itemsize=4)
        _need(y, "y", T * self.hidden, itemsize=2)

    def bind_workspace(self, ws, stream=None):
        _need(ws, "workspace", nbytes=self.sizes.workspace_bytes)
        _check(lib().moedc_plan_bind_workspace(self._h, _ptr(ws), _stream(stream)),
               "moedc_plan_bind_workspace")

    def route(self, logits, topk_ids, topk_w, counts, offsets, slots, dropped,
              workspace, num_tokens: Optional[int] = None, stream=None):
        T = logits.shape[0] if num_tokens is None else num_tokens
        _need(logits, "logits", T * self.num_logical, itemsize=4)
        self._route_bufs(T, topk_ids, topk_w, counts, offsets, slots, dropped, workspace)
        _check(lib().moedc_route(self._h, T, _ptr(logits), _ptr(topk_ids), _ptr(topk_w),
                                 _ptr(counts), _ptr(offsets), _ptr(slots), _ptr(dropped),
                                 _ptr(workspace), _stream(stream)), "moedc_route")

    def route_noalloc(self, logits, topk_ids, topk_w, counts, offsets, slots, dropped,
                      num_tokens: Optional[int] = None, stream=None):
        """moedc_route on the library's static scratch array (no workspace)."""
        T = logits.shape[0] if num_tokens is None else num_tokens
        K, P = self.K, self.num_phys
        _need(logits, "logits", T * self.num_logical, itemsize=4)
        for t, what, n in ((topk_ids, "topk_ids", T * K), (topk_w, "topk_w", T * K),
                           (counts, "counts", P), (offsets, "offsets", P + 1),
                           (slots, "slots", T * K), (dropped, "dropped", 1)):
            _need(t, what, n, itemsize=4)
        _check(lib().moedc_route_noalloc(self._h, T, _ptr(logits), _ptr(topk_ids),
                                         _ptr(topk_w), _ptr(counts), _ptr(offsets),
                                         _ptr(slots), _ptr(dropped), _stream(stream)),
               "moedc_route_noalloc")

    def dispatch(self, x, slots, dispatch_buf, num_tokens: Optional[int] = None,
                 stream=None):
        T = x.shape[0] if num_tokens is None else num_tokens
        _need(x, "x", T * self.hidden, itemsize=2)
        _need(slots, "slots", T * self.K, itemsize=4)
        _need(dispatch_buf, "dispatch_buf", nbytes=self.sizes.dispatch_buf_bytes)
        _check(lib().moedc_dispatch(self._h, T, _ptr(x), _ptr(slots), _ptr(dispatch_buf),
                                    _stream(stream)), "moedc_dispatch")

    def combine(self, expert_out, fmt: int, slots, topk_w, y,
                num_tokens: Optional[int] = None, stream=None):
        T = y.shape[0] if num_tokens is None else num_tokens
        self._combine_bufs(T, expert_out, fmt, slots, topk_w, y)
        _check(lib().moedc_combine(self._h, T, _ptr(expert_out), fmt, _ptr(slots),
                                   _ptr(topk_w), _ptr(y), _stream(stream)), "moedc_combine")

    def route_dispatch(self, logits, x, topk_ids, topk_w, counts, offsets, slots, dropped,
                       dispatch_buf, workspace, num_tokens: Optional[int] = None, stream=None):
        T = logits.shape[0] if num_tokens is None else num_tokens
        _need(logits, "logits", T * self.num_logical, itemsize=4)
        _need(x, "x", T * self.hidden, itemsize=2)
        _need(dispatch_buf, "dispatch_buf", nbytes=self.sizes.dispatch_buf_bytes)
        self._route_bufs(T, topk_ids, topk_w, counts, offsets, slots, dropped, workspace)
        _check(lib().moedc_route_dispatch(
            self._h, T, _ptr(logits), _ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(counts),
            _ptr(offsets), _ptr(slots), _ptr(dropped), _ptr(dispatch_buf), _ptr(workspace),
            _stream(stream)), "moedc_route_dispatch")

    def combine_limited(self, expert_out, fmt: int, slots, topk_w, y, max_workgroups: int,
                        num_tokens: Optional[int] = None, stream=None):
        T = y.shape[0] if num_tokens is None else num_tokens
        self._combine_bufs(T, expert_out, fmt, slots, topk_w, y)
        _check(lib().moedc_combine_limited(self._h, T, _ptr(expert_out), fmt, _ptr(slots),
                                           _ptr(topk_w), _ptr(y), max_workgroups,
                                           _stream(stream)), "moedc_combine_limited")

    def expert_w8a8(self, counts, dispatch_buf, weights, w_scale, combine_buf, workspace,
                    stream=None):
        s, H, P = self.sizes, self.hidden, self.num_phys
        _need(counts, "counts", P, itemsize=4)
        _need(dispatch_buf, "dispatch_buf", nbytes=s.dispatch_buf_bytes)
        _need(weights, "weights", P * H * H, itemsize=1)
        _need(w_scale, "w_scale", P * H, itemsize=4)
        _need(combine_buf, "combine_buf", nbytes=s.combine_buf_bytes)
        _need(workspace, "workspace", nbytes=s.workspace_bytes)
        _check(lib().moedc_expert_w8a8(self._h, _ptr(counts), _ptr(dispatch_buf), _ptr(weights),
                                       _ptr(w_scale), _ptr(combine_buf), _ptr(workspace),
                                       _stream(stream)), "moedc_expert_w8a8")

    def expert_w8a8_dealt(self, counts, dispatch_buf, weights, w_scale, combine_buf, workspace,
                          dealing: int, xcd_tiles=None, stream=None):
        """moedc_expert_w8a8 with the band dealing chosen; xcd_tiles (int32
        [8] on the device, optional) receives the tiles dealt to each die."""
        s, H, P = self.sizes, self.hidden, self.num_phys
        _need(counts, "counts", P, itemsize=4)
        _need(dispatch_buf, "dispatch_buf", nbytes=s.dispatch_buf_bytes)
        _need(weights, "weights", P * H * H, itemsize=1)
        _need(w_scale, "w_scale", P * H, itemsize=4)
        _need(combine_buf, "combine_buf", nbytes=s.combine_buf_bytes)
        _need(workspace, "workspace", nbytes=s.workspace_bytes)
        if xcd_tiles is not None:
            _need(xcd_tiles, "xcd_tiles", 8, itemsize=4)
        _check(lib().moedc_expert_w8a8_dealt(self._h, _ptr(counts), _ptr(dispatch_buf),
                                             _ptr(weights), _ptr(w_scale), _ptr(combine_buf),
                                             _ptr(workspace), dealing, _ptr(xcd_tiles),
                                             _stream(stream)), "moedc_expert_w8a8_dealt")

    def expert_stub(self, counts, dispatch_buf, combine_buf, workspace, stream=None):
        s = self.sizes
        _need(counts, "counts", self.num_phys, itemsize=4)
        _need(dispatch_buf, "dispatch_buf", nbytes=s.dispatch_buf_bytes)
        _need(combine_buf, "combine_buf", nbytes=s.combine_buf_bytes)
        _need(workspace, "workspace", nbytes=s.workspace_bytes)
        _check(lib().moedc_expert_stub(self._h, _ptr(counts), _ptr(dispatch_buf),
                                       _ptr(combine_buf), _ptr(workspace),
                                       _stream(stream)), "moedc_expert_stub")
