"""MI355X routed-expert MoE FFN on MXFP4 weights — Python binding of libk3moe.so.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, then their device pointers and torch's current HIP stream are
passed to the C ABI declared in ``include/k3moe.h``. Every step of the layer
runs in the library's gfx950 kernels; there is no fallback. If the library is
missing, every call raises.
"""
from __future__ import annotations

import atexit
import ctypes
import dataclasses
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libk3moe.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
BF16, F32 = 0, 1
KERNEL_ROUTER, KERNEL_GATE_UP, KERNEL_DOWN = 1, 2, 3


class K3MoEError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"k3moe error {code}: {msg}")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32)]


class _MxExperts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")]


class _Block(ctypes.Structure):
    _fields_ = [("rms_gamma", ctypes.c_void_p), ("rms_eps", ctypes.c_float),
                ("sh_gate", ctypes.c_void_p), ("sh_up", ctypes.c_void_p),
                ("sh_down", ctypes.c_void_p)]


class PackedBytes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")]


class CacheStats(ctypes.Structure):
    _fields_ = [("hits", ctypes.c_int64), ("misses", ctypes.c_int64),
                ("bytes_copied", ctypes.c_int64), ("distinct", ctypes.c_int32)]


@dataclasses.dataclass
class MxExperts:
    """One layer of routed experts: uint8 device tensors, stacked over experts.

    gate_q/up_q [E][d_ff][d_model/2], gate_s/up_s [E][d_ff][d_model/32],
    down_q [E][d_model][d_ff/2], down_s [E][d_model][d_ff/32]."""
    gate_q: torch.Tensor
    gate_s: torch.Tensor
    up_q: torch.Tensor
    up_s: torch.Tensor
    down_q: torch.Tensor
    down_s: torch.Tensor


@dataclasses.dataclass
class BlockWeights:
    """Extras of a full block: bf16 RMSNorm gain and shared SwiGLU expert."""
    rms_gamma: torch.Tensor  # [d_model] bf16
    sh_gate: torch.Tensor    # [d_ff][d_model] bf16
    sh_up: torch.Tensor      # [d_ff][d_model] bf16
    sh_down: torch.Tensor    # [d_model][d_ff] bf16
    rms_eps: float = 1e-6


_lib = None


def lib() -> ctypes.CDLL:
    """Load libk3moe.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        D = ctypes.POINTER(Dims)
        L.k3moe_version.restype = ctypes.c_int
        L.k3moe_last_error.restype = ctypes.c_char_p
        L.k3moe_workspace_bytes.restype = sz
        L.k3moe_workspace_bytes.argtypes = [D, i32]
        L.k3moe_router.restype = ctypes.c_int
        L.k3moe_router.argtypes = [D, i32, vp, ctypes.c_int, vp, vp, vp, vp, vp, sz, vp]
        L.k3moe_route_bucket.restype = ctypes.c_int
        L.k3moe_route_bucket.argtypes = [D, i32, vp, vp, vp, vp, sz, vp]
        L.k3moe_expert_ffn.restype = ctypes.c_int
        L.k3moe_expert_ffn.argtypes = [D, i32, vp, ctypes.c_int, ctypes.POINTER(_MxExperts), vp,
                                       vp, vp, vp, vp, sz, vp]
        L.k3moe_time_next_kernel.restype = ctypes.c_int
        L.k3moe_time_next_kernel.argtypes = [ctypes.c_int, vp, vp]
        L.k3moe_layer_forward.restype = ctypes.c_int
        L.k3moe_layer_forward.argtypes = [D, i32, vp, ctypes.c_int, vp, vp,
                                          ctypes.POINTER(_MxExperts), ctypes.POINTER(_Block),
                                          vp, vp, vp, vp, vp, sz, vp]
        L.k3moe_cache_state_bytes.restype = sz
        L.k3moe_cache_state_bytes.argtypes = [i32, i32, i32]
        L.k3moe_cache_init.restype = ctypes.c_int
        L.k3moe_cache_init.argtypes = [vp, sz, i32, i32, i32]
        L.k3moe_cache_plan.restype = ctypes.c_int
        L.k3moe_cache_plan.argtypes = [vp, i32, vp, vp, vp, ctypes.POINTER(i32)]
        L.k3moe_cache_stats_get.restype = ctypes.c_int
        L.k3moe_cache_stats_get.argtypes = [vp, ctypes.POINTER(CacheStats)]
        L.k3moe_layer_forward_cached.restype = ctypes.c_int
        L.k3moe_layer_forward_cached.argtypes = [D, i32, vp, ctypes.c_int, vp, vp,
                                                 ctypes.POINTER(_MxExperts),
                                                 ctypes.POINTER(_MxExperts), vp, vp, vp, vp, vp,
                                                 ctypes.POINTER(CacheStats), vp, sz, vp]
        L.k3moe_layer_forward_noalloc.restype = ctypes.c_int
        L.k3moe_layer_forward_noalloc.argtypes = [D, i32, vp, ctypes.c_int, vp, vp,
                                                  ctypes.POINTER(_MxExperts),
                                                  ctypes.POINTER(_Block), vp, vp, vp, vp, vp]
        L.k3moe_packed_expert_bytes.restype = ctypes.c_int
        L.k3moe_packed_expert_bytes.argtypes = [D, ctypes.POINTER(PackedBytes)]
        L.k3moe_pack_experts.restype = ctypes.c_int
        L.k3moe_pack_experts.argtypes = [D, ctypes.POINTER(_MxExperts),
                                         ctypes.POINTER(_MxExperts), vp]
        L.k3moe_layer_forward_packed.restype = ctypes.c_int
        L.k3moe_layer_forward_packed.argtypes = [D, i32, vp, ctypes.c_int, vp, vp,
                                                 ctypes.POINTER(_MxExperts),
                                                 ctypes.POINTER(_Block), vp, vp, vp, vp, vp, sz,
                                                 vp]
        L.k3moe_release.restype = ctypes.c_int
        L.k3moe_release.argtypes = []
        L.k3moe_set_hot_tokens.restype = ctypes.c_int
        L.k3moe_set_hot_tokens.argtypes = [i32]
        L.k3moe_hot_tokens.restype = i32
        L.k3moe_hot_tokens.argtypes = []
        _lib = L
        # streams and events the library keeps are released while the HIP runtime is
        # still up (Python's exit handlers run before the runtime's own finalisers)
        atexit.register(L.k3moe_release)
    return _lib


def _check(rc: int) -> None:
    if rc != OK:
        raise K3MoEError(rc, lib().k3moe_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _x_dtype(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return BF16
    if x.dtype == torch.float32:
        return F32
    raise ValueError(f"x must be bf16 or fp32, got {x.dtype}")


def set_hot_tokens(n: int) -> None:
    """k3moe_set_hot_tokens: experts with fewer than n tokens in a call read their weights
    non-temporally in the grouped kernels (0 <= n <= 16)."""
    _check(lib().k3moe_set_hot_tokens(int(n)))


def hot_tokens() -> int:
    return int(lib().k3moe_hot_tokens())


def time_next_kernel(which: int, ev_start, ev_stop) -> None:
    """Arm the one-shot probe: the next call launching kernel `which` records the two
    hipEvent_t handles around that launch (diagnostics for live kernel timing)."""
    _check(lib().k3moe_time_next_kernel(which, ev_start, ev_stop))


def make_dims(d_model: int, d_ff: int, n_experts: int, top_k: int) -> Dims:
    return Dims(d_model, d_ff, n_experts, top_k)


def workspace_bytes(dims: Dims, max_tokens: int) -> int:
    return int(lib().k3moe_workspace_bytes(ctypes.byref(dims), max_tokens))


def make_workspace(dims: Dims, max_tokens: int, device="cuda") -> torch.Tensor:
    n = workspace_bytes(dims, max_tokens)
    if n == 0:
        raise ValueError("invalid dims")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _experts_struct(dims: Dims, ex: MxExperts, packed: bool = False) -> _MxExperts:
    E, d, f = dims.n_experts, dims.d_model, dims.d_ff
    if packed:
        pb = packed_expert_bytes(dims)
        sizes = {n: E * pb[n] for n in pb}
    else:
        sizes = {"gate_q": E * f * (d // 2), "gate_s": E * f * (d // 32),
                 "up_q": E * f * (d // 2), "up_s": E * f * (d // 32),
                 "down_q": E * d * (f // 2), "down_s": E * d * (f // 32)}
    s = _MxExperts()
    for n, size in sizes.items():
        t = _dev(getattr(ex, n), f"experts.{n}", torch.uint8)
        if t.numel() != size:
            raise ValueError(f"experts.{n} has {t.numel()} bytes, expected {size}")
        setattr(s, n, t.data_ptr())
    return s


def packed_expert_bytes(dims: Dims) -> dict:
    """Per-expert bytes of each tensor in the packed tile layout (k3moe_packed_expert_bytes)."""
    pb = PackedBytes()
    _check(lib().k3moe_packed_expert_bytes(ctypes.byref(dims), ctypes.byref(pb)))
    return {n: int(getattr(pb, n)) for n, _ in PackedBytes._fields_}


def pack_experts(dims: Dims, experts: MxExperts, stream=None) -> MxExperts:
    """Packed copy (k3moe_pack_experts) of row-major experts, as new uint8 device tensors of
    shape [E][bytes per expert]; enqueued on the stream."""
    pb = packed_expert_bytes(dims)
    dev = experts.gate_q.device
    out = MxExperts(**{n: torch.empty((dims.n_experts, pb[n]), dtype=torch.uint8, device=dev)
                       for n in pb})
    src = _experts_struct(dims, experts)
    dst = _experts_struct(dims, out, packed=True)
    _check(lib().k3moe_pack_experts(ctypes.byref(dims), ctypes.byref(src), ctypes.byref(dst),
                                    _stream(stream)))
    return out


def _ws(dims: Dims, T: int, ws: Optional[torch.Tensor], device) -> torch.Tensor:
    if ws is None:
        return make_workspace(dims, T, device)
    return _dev(ws, "ws", torch.uint8)


def router(dims: Dims, x: torch.Tensor, w_router: torch.Tensor,
           logit_bias: Optional[torch.Tensor] = None, *, ids: Optional[torch.Tensor] = None,
           gates: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
           stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    T = x.shape[0]
    d, E, k = dims.d_model, dims.n_experts, dims.top_k
    _dev(x, "x", (torch.bfloat16, torch.float32), (T, d))
    _dev(w_router, "w_router", (torch.bfloat16, torch.int16), (d, E))
    if logit_bias is not None:
        _dev(logit_bias, "logit_bias", torch.float32, (E,))
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device) if ids is None else \
        _dev(ids, "ids", torch.int32, (T, k))
    gates = torch.empty((T, k), dtype=torch.float32, device=x.device) if gates is None else \
        _dev(gates, "gates", torch.float32, (T, k))
    w = _ws(dims, T, ws, x.device)
    _check(lib().k3moe_router(ctypes.byref(dims), T, _ptr(x), _x_dtype(x), _ptr(w_router),
                              _ptr(logit_bias), _ptr(ids), _ptr(gates), _ptr(w), w.numel(),
                              _stream(stream)))
    return ids, gates


def route_bucket(dims: Dims, ids: torch.Tensor, *, offsets: Optional[torch.Tensor] = None,
                 rows: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                 stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    T = ids.shape[0]
    E, k = dims.n_experts, dims.top_k
    _dev(ids, "ids", torch.int32, (T, k))
    offsets = torch.empty(E + 1, dtype=torch.int32, device=ids.device) if offsets is None else \
        _dev(offsets, "offsets", torch.int32, (E + 1,))
    rows = torch.empty(T * k, dtype=torch.int32, device=ids.device) if rows is None else \
        _dev(rows, "rows", torch.int32, (T * k,))
    w = _ws(dims, T, ws, ids.device)
    _check(lib().k3moe_route_bucket(ctypes.byref(dims), T, _ptr(ids), _ptr(offsets), _ptr(rows),
                                    _ptr(w), w.numel(), _stream(stream)))
    return offsets, rows


def expert_ffn(dims: Dims, x: torch.Tensor, experts: MxExperts, offsets: torch.Tensor,
               rows: torch.Tensor, gates: torch.Tensor, *, y: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    T = x.shape[0]
    d, E, k = dims.d_model, dims.n_experts, dims.top_k
    _dev(x, "x", (torch.bfloat16, torch.float32), (T, d))
    _dev(offsets, "offsets", torch.int32, (E + 1,))
    _dev(rows, "rows", torch.int32, (T * k,))
    _dev(gates, "gates", torch.float32, (T, k))
    y = torch.empty((T, d), dtype=torch.float32, device=x.device) if y is None else \
        _dev(y, "y", torch.float32, (T, d))
    es = _experts_struct(dims, experts)
    w = _ws(dims, T, ws, x.device)
    _check(lib().k3moe_expert_ffn(ctypes.byref(dims), T, _ptr(x), _x_dtype(x), ctypes.byref(es),
                                  _ptr(offsets), _ptr(rows), _ptr(gates), _ptr(y), _ptr(w),
                                  w.numel(), _stream(stream)))
    return y


def _block_struct(dims: Dims, block: Optional[BlockWeights]):
    """ctypes reference to a k3moe_block for ``block`` (None for no block mode)."""
    if block is None:
        return None
    d, f = dims.d_model, dims.d_ff
    _dev(block.rms_gamma, "rms_gamma", (torch.bfloat16, torch.int16), (d,))
    _dev(block.sh_gate, "sh_gate", (torch.bfloat16, torch.int16), (f, d))
    _dev(block.sh_up, "sh_up", (torch.bfloat16, torch.int16), (f, d))
    _dev(block.sh_down, "sh_down", (torch.bfloat16, torch.int16), (d, f))
    b = _Block(block.rms_gamma.data_ptr(), float(block.rms_eps), block.sh_gate.data_ptr(),
               block.sh_up.data_ptr(), block.sh_down.data_ptr())
    return ctypes.byref(b)


def layer_forward(dims: Dims, x: torch.Tensor, w_router: torch.Tensor,
                  logit_bias: Optional[torch.Tensor], experts: MxExperts,
                  block: Optional[BlockWeights] = None, *, y: Optional[torch.Tensor] = None,
                  y_bf16: Optional[torch.Tensor] = None, ids: Optional[torch.Tensor] = None,
                  gates: Optional[torch.Tensor] = None, ws=None,
                  stream=None) -> torch.Tensor:
    """y = MoE(x) (or, with ``block``, h + S(RMSNorm(h)) + MoE(RMSNorm(h)) for fp32 h).

    ``y_bf16``/``ids``/``gates``, when given, are filled in as well. ``ws``: a device
    workspace of at least workspace_bytes(dims, T) bytes, None to allocate one, or False for
    the allocation-free entry point (see layer_forward_noalloc)."""
    T = x.shape[0]
    d, E, k, f = dims.d_model, dims.n_experts, dims.top_k, dims.d_ff
    _dev(x, "x", (torch.bfloat16, torch.float32), (T, d))
    _dev(w_router, "w_router", (torch.bfloat16, torch.int16), (d, E))
    if logit_bias is not None:
        _dev(logit_bias, "logit_bias", torch.float32, (E,))
    y = torch.empty((T, d), dtype=torch.float32, device=x.device) if y is None else \
        _dev(y, "y", torch.float32, (T, d))
    if y_bf16 is not None:
        _dev(y_bf16, "y_bf16", (torch.bfloat16, torch.int16), (T, d))
    if ids is not None:
        _dev(ids, "ids", torch.int32, (T, k))
    if gates is not None:
        _dev(gates, "gates", torch.float32, (T, k))
    blk_ref = _block_struct(dims, block)
    es = _experts_struct(dims, experts)
    if ws is False:  # the allocation-free entry point: static device scratch
        _check(lib().k3moe_layer_forward_noalloc(ctypes.byref(dims), T, _ptr(x), _x_dtype(x),
                                                 _ptr(w_router), _ptr(logit_bias),
                                                 ctypes.byref(es), blk_ref, _ptr(y),
                                                 _ptr(y_bf16), _ptr(ids), _ptr(gates),
                                                 _stream(stream)))
        return y
    w = _ws(dims, T, ws, x.device)
    _check(lib().k3moe_layer_forward(ctypes.byref(dims), T, _ptr(x), _x_dtype(x), _ptr(w_router),
                                     _ptr(logit_bias), ctypes.byref(es), blk_ref, _ptr(y),
                                     _ptr(y_bf16), _ptr(ids), _ptr(gates), _ptr(w), w.numel(),
                                     _stream(stream)))
    return y


def layer_forward_packed(dims: Dims, x: torch.Tensor, w_router: torch.Tensor,
                         logit_bias: Optional[torch.Tensor], experts: MxExperts,
                         block: Optional[BlockWeights] = None, *,
                         y: Optional[torch.Tensor] = None,
                         y_bf16: Optional[torch.Tensor] = None,
                         ids: Optional[torch.Tensor] = None,
                         gates: Optional[torch.Tensor] = None, ws=None,
                         stream=None) -> torch.Tensor:
    """layer_forward with `experts` in the packed tile layout (pack_experts). fp32 tokens
    and ``block`` only for one token (the library refuses them otherwise)."""
    T = x.shape[0]
    d, E, k, f = dims.d_model, dims.n_experts, dims.top_k, dims.d_ff
    _dev(x, "x", (torch.bfloat16, torch.float32), (T, d))
    _dev(w_router, "w_router", (torch.bfloat16, torch.int16), (d, E))
    if logit_bias is not None:
        _dev(logit_bias, "logit_bias", torch.float32, (E,))
    y = torch.empty((T, d), dtype=torch.float32, device=x.device) if y is None else \
        _dev(y, "y", torch.float32, (T, d))
    if y_bf16 is not None:
        _dev(y_bf16, "y_bf16", (torch.bfloat16, torch.int16), (T, d))
    if ids is not None:
        _dev(ids, "ids", torch.int32, (T, k))
    if gates is not None:
        _dev(gates, "gates", torch.float32, (T, k))
    blk_ref = _block_struct(dims, block)
    es = _experts_struct(dims, experts, packed=True)
    w = _ws(dims, T, ws, x.device)
    _check(lib().k3moe_layer_forward_packed(ctypes.byref(dims), T, _ptr(x), _x_dtype(x),
                                            _ptr(w_router), _ptr(logit_bias), ctypes.byref(es),
                                            blk_ref, _ptr(y), _ptr(y_bf16), _ptr(ids),
                                            _ptr(gates), _ptr(w), w.numel(), _stream(stream)))
    return y


def layer_forward_noalloc(dims: Dims, x: torch.Tensor, w_router: torch.Tensor,
                          logit_bias: Optional[torch.Tensor], experts: MxExperts,
                          block: Optional[BlockWeights] = None, *, y: torch.Tensor,
                          y_bf16: Optional[torch.Tensor] = None,
                          ids: Optional[torch.Tensor] = None,
                          gates: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """layer_forward through k3moe_layer_forward_noalloc: no workspace, nothing allocated
    (y must be given); the library's static per-GPU scratch is used instead, so calls on one
    GPU must not overlap."""
    if y is None:
        raise ValueError("layer_forward_noalloc needs y (it allocates nothing)")
    return layer_forward(dims, x, w_router, logit_bias, experts, block, y=y, y_bf16=y_bf16,
                         ids=ids, gates=gates, ws=False, stream=stream)


# ---- routed experts beyond HBM: the slot cache -------------------------------------------
class ExpertCache:
    """Host state of an HBM slot cache over host-resident experts (k3moe_cache_*): which
    expert sits in which of `n_slots` slots, least recently used evicted first. Held in a
    host buffer owned here; `max_ids` bounds T * top_k per call."""

    def __init__(self, n_experts: int, n_slots: int, max_ids: int):
        import numpy as np
        n = int(lib().k3moe_cache_state_bytes(n_experts, n_slots, max_ids))
        if n == 0:
            raise ValueError(f"invalid cache shape E={n_experts} slots={n_slots} "
                             f"max_ids={max_ids}")
        self._buf = np.zeros((n + 7) // 8, dtype=np.uint64)  # 8-byte aligned
        self.n_experts, self.n_slots, self.max_ids = n_experts, n_slots, max_ids
        _check(lib().k3moe_cache_init(self.ptr, self._buf.nbytes, n_experts, n_slots, max_ids))

    @property
    def ptr(self) -> ctypes.c_void_p:
        return ctypes.c_void_p(self._buf.ctypes.data)

    def plan(self, ids):
        """Host-side plan for routed ids: returns (slot of each id, [(expert, slot) per miss])."""
        import numpy as np
        a = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).reshape(-1))
        slots = np.empty_like(a)
        fetch = np.empty(2 * self.n_slots, dtype=np.int32)
        nf = ctypes.c_int32(0)
        _check(lib().k3moe_cache_plan(self.ptr, a.size, ctypes.c_void_p(a.ctypes.data),
                                      ctypes.c_void_p(slots.ctypes.data),
                                      ctypes.c_void_p(fetch.ctypes.data), ctypes.byref(nf)))
        return slots, [(int(fetch[2 * i]), int(fetch[2 * i + 1])) for i in range(nf.value)]

    def stats(self) -> CacheStats:
        st = CacheStats()
        _check(lib().k3moe_cache_stats_get(self.ptr, ctypes.byref(st)))
        return st


def _host_experts_struct(dims: Dims, ex: MxExperts) -> _MxExperts:
    E, d, f = dims.n_experts, dims.d_model, dims.d_ff
    shapes = {"gate_q": f * d // 2, "gate_s": f * d // 32, "up_q": f * d // 2,
              "up_s": f * d // 32, "down_q": d * f // 2, "down_s": d * f // 32}
    s = _MxExperts()
    for n, per in shapes.items():
        t = getattr(ex, n)
        if t.is_cuda or not t.is_contiguous() or t.dtype != torch.uint8:
            raise ValueError(f"host experts.{n} must be a contiguous uint8 host tensor")
        if t.numel() != E * per:
            raise ValueError(f"host experts.{n} has {t.numel()} bytes, expected {E * per}")
        setattr(s, n, t.data_ptr())
    return s


def layer_forward_cached(dims: Dims, x: torch.Tensor, w_router: torch.Tensor,
                         logit_bias: Optional[torch.Tensor], host_experts: MxExperts,
                         slot_experts: MxExperts, cache: ExpertCache, *,
                         y: Optional[torch.Tensor] = None, y_bf16: Optional[torch.Tensor] = None,
                         ids: Optional[torch.Tensor] = None, gates: Optional[torch.Tensor] = None,
                         ws: Optional[torch.Tensor] = None, stream=None):
    """y = MoE(x) with the experts in host memory and `cache.n_slots` of them in HBM
    (k3moe_layer_forward_cached; synchronises the stream once to read the routed ids).
    Returns (y, this call's CacheStats)."""
    T = x.shape[0]
    d, E, k = dims.d_model, dims.n_experts, dims.top_k
    _dev(x, "x", (torch.bfloat16, torch.float32), (T, d))
    _dev(w_router, "w_router", (torch.bfloat16, torch.int16), (d, E))
    if logit_bias is not None:
        _dev(logit_bias, "logit_bias", torch.float32, (E,))
    y = torch.empty((T, d), dtype=torch.float32, device=x.device) if y is None else \
        _dev(y, "y", torch.float32, (T, d))
    if y_bf16 is not None:
        _dev(y_bf16, "y_bf16", (torch.bfloat16, torch.int16), (T, d))
    if ids is not None:
        _dev(ids, "ids", torch.int32, (T, k))
    if gates is not None:
        _dev(gates, "gates", torch.float32, (T, k))
    hs = _host_experts_struct(dims, host_experts)
    sdims = Dims(dims.d_model, dims.d_ff, cache.n_slots, dims.top_k)
    ss = _experts_struct(sdims, slot_experts)
    w = _ws(dims, T, ws, x.device)
    st = CacheStats()
    _check(lib().k3moe_layer_forward_cached(ctypes.byref(dims), T, _ptr(x), _x_dtype(x),
                                            _ptr(w_router), _ptr(logit_bias), ctypes.byref(hs),
                                            ctypes.byref(ss), cache.ptr, _ptr(y), _ptr(y_bf16),
                                            _ptr(ids), _ptr(gates), ctypes.byref(st), _ptr(w),
                                            w.numel(), _stream(stream)))
    return y, st
