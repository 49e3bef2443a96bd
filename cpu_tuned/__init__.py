"""ctypes binding of the tuned CPU comparator (libk3cpu.so): the routed-expert MoE layer
for bf16 tokens on the host cores, equal to the plain fp64 definition bit for bit."""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libk3cpu.so")
_lib = None
_NAMES = ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")


class _Expert(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _NAMES]


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB)
        L.k3cpu_layer_forward.restype = ctypes.c_int
        L.k3cpu_layer_forward.argtypes = [ctypes.c_int32] * 5 + [ctypes.c_void_p] * 7
        L.k3cpu_layer_route.restype = ctypes.c_int
        L.k3cpu_layer_route.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 5
        L.k3cpu_simd.restype = ctypes.c_int
        _lib = L
    return _lib


def simd() -> bool:
    return bool(lib().k3cpu_simd())


def layer_forward(x, w_router, bias, experts, d, f, E, k):
    """x: bf16 bits uint16 [T][d]; w_router uint16 [d][E]; bias float32 [E] or None;
    experts: {id: {name: uint8 array}} holding at least the selected experts.
    Returns (y fp64 [T][d], ids int32 [T][k], gates fp64 [T][k])."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w_router, dtype=np.uint16)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    T = x.shape[0]
    table = (_Expert * E)()
    keep = []
    for e, tens in experts.items():
        for n in _NAMES:
            a = np.ascontiguousarray(tens[n], dtype=np.uint8)
            keep.append(a)
            setattr(table[int(e)], n, a.ctypes.data)
    y = np.empty((T, d), dtype=np.float64)
    ids = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float64)
    rc = lib().k3cpu_layer_forward(T, d, f, E, k, x.ctypes.data, w.ctypes.data,
                                   None if b is None else b.ctypes.data,
                                   ctypes.cast(table, ctypes.c_void_p), y.ctypes.data,
                                   ids.ctypes.data, gates.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"k3cpu_layer_forward failed ({rc})")
    return y, ids, gates


def layer_route(x, w_router, bias, k):
    """Routing only: (ids int32 [T][k], gates fp64 [T][k])."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w_router, dtype=np.uint16)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    T, d = x.shape
    E = w.shape[1]
    ids = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float64)
    rc = lib().k3cpu_layer_route(T, d, E, k, x.ctypes.data, w.ctypes.data,
                                 None if b is None else b.ctypes.data, ids.ctypes.data,
                                 gates.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"k3cpu_layer_route failed ({rc})")
    return ids, gates
