"""Seeded synthetic-input generator (SplitMix64 counter form) — Python binding.

This package only draws inputs; it holds none of the MoE method's arithmetic.
Both the CPU oracle harness and the GPU tests/bench take their inputs from it.
The C sources next to this file define every draw (see ``k3gen.h``).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libk3gen.so")
DEV_LIB = os.path.join(_HERE, "libk3gen_dev.so")

MASTER_SEED = 0x4B334D4F45
MASK64 = (1 << 64) - 1

T_X, T_WROUTER, T_ZIPF = 1, 2, 3
T_GATE_Q, T_GATE_S, T_UP_Q, T_UP_S, T_DOWN_Q, T_DOWN_S = 4, 5, 6, 7, 8, 9
T_GAMMA, T_SH_GATE, T_SH_UP, T_SH_DOWN, T_RESID = 10, 11, 12, 13, 14

_host = None
_dev = None


def _load_host():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        u64, i32, dbl = ctypes.c_uint64, ctypes.c_int32, ctypes.c_double
        lib.k3gen_at.restype = u64
        lib.k3gen_at.argtypes = [u64, u64]
        lib.k3gen_key.restype = u64
        lib.k3gen_key.argtypes = [u64, u64, u64, u64]
        lib.k3gen_bytes.argtypes = [u64, u64, u64, ctypes.c_void_p]
        lib.k3gen_e8m0.argtypes = [u64, u64, u64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.k3gen_normal_f64.restype = dbl
        lib.k3gen_normal_f64.argtypes = [u64, u64]
        lib.k3gen_f64_to_bf16.restype = ctypes.c_uint16
        lib.k3gen_f64_to_bf16.argtypes = [dbl]
        lib.k3gen_normal_bf16.argtypes = [u64, u64, u64, dbl, dbl, ctypes.c_void_p]
        lib.k3gen_normal_f32.argtypes = [u64, u64, u64, dbl, dbl, ctypes.c_void_p]
        lib.k3gen_zipf_bias.argtypes = [u64, i32, dbl, ctypes.c_void_p, ctypes.c_void_p]
        _host = lib
    return _host


def _load_dev():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEV_LIB)
        u64 = ctypes.c_uint64
        lib.k3gen_dev_fill_bytes.restype = ctypes.c_int
        lib.k3gen_dev_fill_bytes.argtypes = [u64, u64, u64, ctypes.c_int32, u64,
                                             ctypes.c_void_p, ctypes.c_void_p]
        lib.k3gen_dev_fill_e8m0.restype = ctypes.c_int
        lib.k3gen_dev_fill_e8m0.argtypes = [u64, u64, u64, ctypes.c_int32, u64, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        _dev = lib
    return _dev


def at(key: int, i: int) -> int:
    return int(_load_host().k3gen_at(key & MASK64, i & MASK64))


def key(seed: int, a: int, b: int, c: int) -> int:
    return int(_load_host().k3gen_key(seed & MASK64, a, b, c))


def host_bytes(k: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    if n:
        _load_host().k3gen_bytes(k & MASK64, start, n, out.ctypes.data)
    return out


def host_e8m0(k: int, n: int, lo: int, count: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    if n:
        _load_host().k3gen_e8m0(k & MASK64, start, n, lo, count, out.ctypes.data)
    return out


def host_normal_bf16(k: int, n: int, mean: float, sd: float, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    if n:
        _load_host().k3gen_normal_bf16(k & MASK64, start, n, mean, sd, out.ctypes.data)
    return out


def host_normal_f32(k: int, n: int, mean: float, sd: float, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    if n:
        _load_host().k3gen_normal_f32(k & MASK64, start, n, mean, sd, out.ctypes.data)
    return out


def normal_f64(k: int, j: int) -> float:
    return float(_load_host().k3gen_normal_f64(k & MASK64, j))


def f64_to_bf16(v: float) -> int:
    return int(_load_host().k3gen_f64_to_bf16(v))


def zipf_bias(k: int, E: int, alpha: float):
    ranks = np.empty(E, dtype=np.int32)
    bias = np.empty(E, dtype=np.float32)
    _load_host().k3gen_zipf_bias(k & MASK64, E, alpha, ranks.ctypes.data, bias.ctypes.data)
    return ranks, bias


def dev_fill_bytes(seed: int, layer: int, tag: int, E: int, per_expert: int, ptr: int,
                   stream: int) -> None:
    rc = _load_dev().k3gen_dev_fill_bytes(seed & MASK64, layer, tag, E, per_expert, ptr, stream)
    if rc != 0:
        raise RuntimeError(f"k3gen_dev_fill_bytes failed ({rc})")


def dev_fill_e8m0(seed: int, layer: int, tag: int, E: int, per_expert: int, lo: int,
                  count: int, ptr: int, stream: int) -> None:
    rc = _load_dev().k3gen_dev_fill_e8m0(seed & MASK64, layer, tag, E, per_expert, lo, count,
                                         ptr, stream)
    if rc != 0:
        raise RuntimeError(f"k3gen_dev_fill_e8m0 failed ({rc})")
