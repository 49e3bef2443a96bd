"""fp64 CPU oracle of the routed-expert MoE layer — Python binding.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The GPU library
and its Python binding never import it; they share no code with it.

The arithmetic lives in ``k3oracle.c`` (plain fp64 loops, sums in index order);
this file only marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# K3ORACLE_LIB lets the mutation tests load a deliberately broken copy.
LIB = os.environ.get("K3ORACLE_LIB") or os.path.join(_HERE, "libk3oracle.so")

BF16, F32, F64 = 0, 1, 2

_lib = None


class _Expert(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")]


class _Block(ctypes.Structure):
    _fields_ = [("gamma", ctypes.c_void_p), ("eps", ctypes.c_double),
                ("sh_gate", ctypes.c_void_p), ("sh_up", ctypes.c_void_p),
                ("sh_down", ctypes.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.k3o_e2m1.restype = dbl
        L.k3o_e2m1.argtypes = [ctypes.c_uint32]
        L.k3o_e8m0.restype = dbl
        L.k3o_e8m0.argtypes = [ctypes.c_uint32]
        L.k3o_bf16.restype = dbl
        L.k3o_bf16.argtypes = [ctypes.c_uint16]
        L.k3o_nibble.restype = ctypes.c_uint32
        L.k3o_nibble.argtypes = [vp, i64]
        L.k3o_mx_row.argtypes = [vp, vp, i32, vp]
        L.k3o_mx_dot.restype = dbl
        L.k3o_mx_dot.argtypes = [vp, vp, i32, vp]
        L.k3o_mx_dot_blockscaled.restype = dbl
        L.k3o_mx_dot_blockscaled.argtypes = [vp, vp, i32, vp]
        L.k3o_load_x.argtypes = [i64, vp, i32, vp]
        L.k3o_router_logits.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.k3o_softmax.argtypes = [i32, vp, vp]
        L.k3o_topk.argtypes = [i32, i32, vp, vp]
        L.k3o_route.argtypes = [i32, i32, i32, vp, vp, vp]
        L.k3o_bucket.restype = ctypes.c_int
        L.k3o_bucket.argtypes = [i32, i32, i32, vp, vp, vp]
        L.k3o_expert_ffn.argtypes = [i32, i32, vp, ctypes.POINTER(_Expert), vp, vp]
        L.k3o_moe_combine.restype = ctypes.c_int
        L.k3o_moe_combine.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp,
                                      ctypes.POINTER(_Expert), vp]
        L.k3o_rmsnorm.argtypes = [i32, vp, vp, dbl, vp]
        L.k3o_dense_swiglu.argtypes = [i32, i32, vp, vp, vp, vp, vp]
        L.k3o_layer_route.restype = ctypes.c_int
        L.k3o_layer_route.argtypes = [i32, i32, i32, i32, vp, i32, vp, vp,
                                      ctypes.POINTER(_Block), vp, vp, vp, vp]
        L.k3o_layer_forward.restype = ctypes.c_int
        L.k3o_layer_forward.argtypes = [i32, i32, i32, i32, i32, vp, i32, vp, vp,
                                        ctypes.POINTER(_Expert), ctypes.POINTER(_Block), vp,
                                        vp, vp]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- element decoding ------------------------------------------------------
def e2m1(code: int) -> float:
    return float(lib().k3o_e2m1(code))


def e8m0(s: int) -> float:
    return float(lib().k3o_e8m0(s))


def bf16(bits: int) -> float:
    return float(lib().k3o_bf16(bits))


def nibble(q: np.ndarray, k: int) -> int:
    q = _c(q, np.uint8)
    return int(lib().k3o_nibble(q.ctypes.data, k))


def mx_row(q: np.ndarray, s: np.ndarray, K: int) -> np.ndarray:
    q, s = _c(q, np.uint8), _c(s, np.uint8)
    out = np.empty(K, dtype=np.float64)
    lib().k3o_mx_row(q.ctypes.data, s.ctypes.data, K, out.ctypes.data)
    return out


def mx_dot(q, s, x, blockscaled=False) -> float:
    q, s, x = _c(q, np.uint8), _c(s, np.uint8), _c(x, np.float64)
    fn = lib().k3o_mx_dot_blockscaled if blockscaled else lib().k3o_mx_dot
    return float(fn(q.ctypes.data, s.ctypes.data, x.shape[0], x.ctypes.data))


def load_x(x: np.ndarray) -> np.ndarray:
    """Exact fp64 values of bf16 (uint16 bits) / fp32 / fp64 activations."""
    dt = {np.dtype(np.uint16): BF16, np.dtype(np.float32): F32,
          np.dtype(np.float64): F64}[x.dtype]
    x = np.ascontiguousarray(x)
    out = np.empty(x.shape, dtype=np.float64)
    lib().k3o_load_x(x.size, x.ctypes.data, dt, out.ctypes.data)
    return out


# ---- routing ---------------------------------------------------------------
def router_logits(x: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray]) -> np.ndarray:
    x = _c(x, np.float64)
    w = _c(w, np.uint16)
    T, d = x.shape
    E = w.shape[1]
    assert w.shape[0] == d
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((T, E), dtype=np.float64)
    lib().k3o_router_logits(T, d, E, x.ctypes.data, w.ctypes.data, _p(b), out.ctypes.data)
    return out


def softmax(l: np.ndarray) -> np.ndarray:
    l = _c(l, np.float64)
    p = np.empty_like(l)
    lib().k3o_softmax(l.shape[0], l.ctypes.data, p.ctypes.data)
    return p


def topk(l: np.ndarray, k: int) -> np.ndarray:
    l = _c(l, np.float64)
    ids = np.empty(k, dtype=np.int32)
    lib().k3o_topk(l.shape[0], k, l.ctypes.data, ids.ctypes.data)
    return ids


def route(logits: np.ndarray, k: int):
    logits = _c(logits, np.float64)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float64)
    lib().k3o_route(T, E, k, logits.ctypes.data, ids.ctypes.data, gates.ctypes.data)
    return ids, gates


def bucket(ids: np.ndarray, E: int):
    ids = _c(ids, np.int32)
    T, k = ids.shape
    offsets = np.empty(E + 1, dtype=np.int32)
    rows = np.empty(T * k, dtype=np.int32)
    rc = lib().k3o_bucket(T, E, k, ids.ctypes.data, offsets.ctypes.data, rows.ctypes.data)
    if rc != 0:
        raise ValueError("expert id out of range")
    return offsets, rows


# ---- experts ------------------------------------------------------------------
def _expert_struct(ex: Dict[str, np.ndarray], keep: list) -> _Expert:
    s = _Expert()
    for n in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s"):
        a = _c(ex[n], np.uint8)
        keep.append(a)
        setattr(s, n, a.ctypes.data)
    return s


def expert_ffn(x: np.ndarray, ex: Dict[str, np.ndarray], d: int, f: int):
    keep: list = []
    x = _c(x, np.float64)
    st = _expert_struct(ex, keep)
    h = np.empty(f, dtype=np.float64)
    out = np.empty(d, dtype=np.float64)
    lib().k3o_expert_ffn(d, f, x.ctypes.data, ctypes.byref(st), h.ctypes.data,
                         out.ctypes.data)
    return h, out


def _expert_table(experts: Dict[int, Dict[str, np.ndarray]], E: int, keep: list):
    table = (_Expert * E)()
    for e, ex in experts.items():
        table[e] = _expert_struct(ex, keep)
    return table


def moe_combine(x, ids, gates, experts, d, f, E):
    keep: list = []
    x = _c(x, np.float64)
    ids = _c(ids, np.int32)
    gates = _c(gates, np.float64)
    T, k = ids.shape
    table = _expert_table(experts, E, keep)
    y = np.empty((T, d), dtype=np.float64)
    rc = lib().k3o_moe_combine(T, d, f, E, k, x.ctypes.data, ids.ctypes.data,
                               gates.ctypes.data, table, y.ctypes.data)
    if rc != 0:
        raise ValueError("a selected expert was not supplied")
    return y


# ---- block extras ----------------------------------------------------------------
def rmsnorm(h: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    h = _c(h, np.float64)
    gamma = _c(gamma, np.uint16)
    out = np.empty_like(h)
    lib().k3o_rmsnorm(h.shape[0], h.ctypes.data, gamma.ctypes.data, eps, out.ctypes.data)
    return out


def dense_swiglu(x, wg, wu, wd) -> np.ndarray:
    x = _c(x, np.float64)
    wg, wu, wd = _c(wg, np.uint16), _c(wu, np.uint16), _c(wd, np.uint16)
    f, d = wg.shape
    out = np.empty(d, dtype=np.float64)
    lib().k3o_dense_swiglu(d, f, x.ctypes.data, wg.ctypes.data, wu.ctypes.data,
                           wd.ctypes.data, out.ctypes.data)
    return out


def _block_struct(block: Optional[dict], keep: list):
    if block is None:
        return None
    b = _Block()
    for n in ("gamma", "sh_gate", "sh_up", "sh_down"):
        a = _c(block[n], np.uint16)
        keep.append(a)
        setattr(b, n, a.ctypes.data)
    b.eps = float(block.get("eps", 1e-6))
    return ctypes.byref(b)


def _xdtype(x: np.ndarray) -> int:
    return {np.dtype(np.uint16): BF16, np.dtype(np.float32): F32,
            np.dtype(np.float64): F64}[x.dtype]


# ---- whole layer -------------------------------------------------------------------
def layer_route(x, w_router, bias, k, block=None):
    """Router + softmax + top-k (after RMSNorm in block mode).

    Returns (ids [T][k] int32, gates [T][k] fp64, logits [T][E] fp64, xin [T][d] fp64)."""
    keep: list = []
    x = np.ascontiguousarray(x)
    w = _c(w_router, np.uint16)
    T, d = x.shape
    E = w.shape[1]
    b = None if bias is None else _c(bias, np.float32)
    ids = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float64)
    logits = np.empty((T, E), dtype=np.float64)
    xin = np.empty((T, d), dtype=np.float64)
    rc = lib().k3o_layer_route(T, d, E, k, x.ctypes.data, _xdtype(x), w.ctypes.data, _p(b),
                               _block_struct(block, keep), ids.ctypes.data, gates.ctypes.data,
                               logits.ctypes.data, xin.ctypes.data)
    if rc != 0:
        raise ValueError("bad arguments")
    return ids, gates, logits, xin


def layer_forward(x, w_router, bias, experts, d, f, E, k, block=None):
    """Full layer: y [T][d] fp64 (block mode: h_out), ids, gates."""
    keep: list = []
    x = np.ascontiguousarray(x)
    w = _c(w_router, np.uint16)
    T = x.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    table = _expert_table(experts, E, keep)
    y = np.empty((T, d), dtype=np.float64)
    ids = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float64)
    rc = lib().k3o_layer_forward(T, d, f, E, k, x.ctypes.data, _xdtype(x), w.ctypes.data,
                                 _p(b), table, _block_struct(block, keep), y.ctypes.data,
                                 ids.ctypes.data, gates.ctypes.data)
    if rc != 0:
        raise ValueError("a selected expert was not supplied or arguments are bad")
    return y, ids, gates
