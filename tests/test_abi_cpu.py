"""C ABI checks that need no GPU: the library loads, exports every declared entry
point, sizes workspaces, and rejects bad arguments before enqueuing anything.

Only argument combinations that fail validation are passed here, so no HIP call
is ever made (validation runs on the host before any launch)."""
import ctypes
import os
import re

import numpy as np
import pytest

import mxfp4_expert_matmul_k3moe_amd as k3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "k3moe.h")

K3 = k3.make_dims(7168, 1536, 896, 16)
FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails validation first


def declared_functions():
    src = open(HEADER).read()
    return re.findall(r"K3MOE_API\s+[\w\s\*]+?\b(k3moe_\w+)\s*\(", src)


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == {"k3moe_version", "k3moe_workspace_bytes", "k3moe_router",
                          "k3moe_route_bucket", "k3moe_expert_ffn", "k3moe_layer_forward",
                          "k3moe_last_error", "k3moe_time_next_kernel",
                          "k3moe_cache_state_bytes", "k3moe_cache_init", "k3moe_cache_plan",
                          "k3moe_cache_stats_get", "k3moe_layer_forward_cached",
                          "k3moe_release", "k3moe_layer_forward_noalloc",
                          "k3moe_packed_expert_bytes", "k3moe_pack_experts",
                          "k3moe_layer_forward_packed", "k3moe_set_hot_tokens",
                          "k3moe_hot_tokens"}
    L = k3.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.k3moe_version() == 1
    assert L.k3moe_time_next_kernel(99, None, None) == k3.EINVAL
    assert L.k3moe_time_next_kernel(k3.KERNEL_GATE_UP, None, None) == k3.OK  # disarm
    # nothing created yet: release touches no HIP state and succeeds
    assert L.k3moe_release() == k3.OK


def test_hot_tokens_setting_range():
    """The grouped kernels' cache-policy threshold: default 16, settable in [0, 16], anything
    else rejected with the setting unchanged (host state only, no GPU)."""
    L = k3.lib()
    assert L.k3moe_hot_tokens() == 16
    try:
        for n in (0, 1, 15, 16):
            assert L.k3moe_set_hot_tokens(n) == k3.OK and L.k3moe_hot_tokens() == n
        for n in (-1, 17, 1 << 30):
            assert L.k3moe_set_hot_tokens(n) == k3.EINVAL
            assert b"hot_tokens" in L.k3moe_last_error()
            assert L.k3moe_hot_tokens() == 16
    finally:
        assert L.k3moe_set_hot_tokens(16) == k3.OK


def test_workspace_bytes_monotone_and_zero_for_bad_dims():
    prev = 0
    for T in (1, 2, 16, 32, 63, 64, 65, 128, 2048):
        n = k3.workspace_bytes(K3, T)
        assert n >= prev > -1
        prev = n
    # dominant terms at T=2048: z = P*d*4, h = P*f*4 with P = T*k
    P = 2048 * 16
    assert k3.workspace_bytes(K3, 2048) >= P * 7168 * 4 + P * 1536 * 4
    assert k3.workspace_bytes(k3.make_dims(33, 1536, 896, 16), 1) == 0
    assert k3.workspace_bytes(k3.make_dims(7168, 1536, 896, 0), 1) == 0
    assert k3.workspace_bytes(K3, -1) == 0


def _router(dims, T=1, x=FAKE, dt=0, w=FAKE, ids=FAKE, gates=FAKE, ws=FAKE, nbytes=1 << 40):
    return k3.lib().k3moe_router(ctypes.byref(dims), T, x, dt, w, None, ids, gates, ws, nbytes,
                                 None)


@pytest.mark.parametrize("dims,code", [
    (k3.make_dims(7168 + 16, 1536, 896, 16), k3.EINVAL),
    (k3.make_dims(0, 1536, 896, 16), k3.EINVAL),
    (k3.make_dims(7168, 1537, 896, 16), k3.EINVAL),
    (k3.make_dims(7168, 1536, 0, 1), k3.EINVAL),
    (k3.make_dims(7168, 1536, 896, 0), k3.EINVAL),
    (k3.make_dims(7168, 1536, 896, 33), k3.EINVAL),
    (k3.make_dims(7168, 1536, 8, 9), k3.EINVAL),
    (k3.make_dims(7168, 1536, 5000, 16), k3.EUNSUPPORTED),
    (k3.make_dims(32768, 1536, 896, 16), k3.EUNSUPPORTED),
])
def test_bad_dims_rejected(dims, code):
    assert _router(dims) == code
    assert k3.lib().k3moe_last_error()


def test_bad_scalars_and_pointers_rejected():
    assert _router(K3, T=-1) == k3.EINVAL
    assert _router(K3, T=(1 << 20) + 1) == k3.EUNSUPPORTED
    assert _router(K3, dt=7) == k3.EINVAL
    assert _router(K3, x=None) == k3.EINVAL
    assert _router(K3, x=ctypes.c_void_p(0x100008)) == k3.EINVAL  # x rows need 16 bytes
    assert _router(K3, w=None) == k3.EINVAL
    assert _router(K3, ids=None) == k3.EINVAL
    assert _router(K3, nbytes=16) == k3.EWORKSPACE
    assert b"workspace" in k3.lib().k3moe_last_error()
    assert _router(K3, ws=None) == k3.EINVAL
    assert _router(K3, T=0) == k3.OK  # no-op


def test_layer_forward_validation():
    L = k3.lib()
    ex = k3._MxExperts(*(0x100000 for _ in range(6)))
    blk = k3._Block(0x100000, 1e-6, 0x100000, 0x100000, 0x100000)

    def call(dims=K3, x=FAKE, dt=0, experts=ex, block=None, y=FAKE, nbytes=1 << 40):
        return L.k3moe_layer_forward(ctypes.byref(dims), 1, x, dt, FAKE, None,
                                     ctypes.byref(experts) if experts is not None else None,
                                     ctypes.byref(block) if block is not None else None, y, None,
                                     None, None, FAKE, nbytes, None)

    assert call(x=ctypes.c_void_p(0x100001)) == k3.EINVAL  # misaligned activations
    assert call(y=None) == k3.EINVAL
    assert call(experts=None) == k3.EINVAL
    bad = k3._MxExperts(0x100000, 0x100000, 0x100008, 0x100000, 0x100000, 0x100000)
    assert call(experts=bad) == k3.EINVAL  # up_q not 16-byte aligned
    assert call(block=blk, dt=0) == k3.EINVAL  # block mode needs fp32 residual
    blk_bad = k3._Block(0x100000, -1.0, 0x100000, 0x100000, 0x100000)
    assert call(block=blk_bad, dt=1) == k3.EINVAL
    assert call(nbytes=100) == k3.EWORKSPACE
    # d_ff/32 = 7 needs 7 blocks per lane in the down projection: not implemented
    assert call(dims=k3.make_dims(7168, 224, 896, 16)) == k3.EUNSUPPORTED


def test_expert_ffn_and_bucket_validation():
    L = k3.lib()
    ex = k3._MxExperts(*(0x100000 for _ in range(6)))
    assert L.k3moe_expert_ffn(ctypes.byref(K3), 1, FAKE, 0, ctypes.byref(ex), None, FAKE, FAKE,
                              FAKE, FAKE, 1 << 40, None) == k3.EINVAL
    assert L.k3moe_expert_ffn(ctypes.byref(K3), 1, FAKE, 0, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                              1 << 40, None) == k3.EINVAL
    assert L.k3moe_route_bucket(ctypes.byref(K3), 1, None, FAKE, FAKE, FAKE, 1 << 40,
                                None) == k3.EINVAL
    assert L.k3moe_route_bucket(ctypes.byref(K3), 4, FAKE, FAKE, FAKE, FAKE, 8,
                                None) == k3.EWORKSPACE
    assert L.k3moe_route_bucket(ctypes.byref(K3), 0, None, None, None, None, 0, None) == k3.OK


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(1, 7168, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        k3.router(K3, x, torch.zeros(7168, 896, dtype=torch.bfloat16))


def test_layer_forward_cached_validation():
    """Everything the cached layer rejects is rejected on the host, before any GPU work."""
    L = k3.lib()
    ex = k3._MxExperts(*(0x100000 for _ in range(6)))
    cache = k3.ExpertCache(896, 32, 16)  # room for one token of top-16

    def call(dims=K3, T=1, state=cache.ptr, host=ex, slots=ex, nbytes=1 << 40):
        return L.k3moe_layer_forward_cached(ctypes.byref(dims), T, FAKE, 0, FAKE, None,
                                            ctypes.byref(host) if host is not None else None,
                                            ctypes.byref(slots) if slots is not None else None,
                                            state, FAKE, None, None, None, None, FAKE, nbytes,
                                            None)

    assert call(T=0) == k3.OK  # no-op
    assert call(state=None) == k3.EINVAL
    junk = np.zeros(64, dtype=np.uint64)
    assert call(state=ctypes.c_void_p(junk.ctypes.data)) == k3.EINVAL  # not a cache state
    assert call(host=None) == k3.EINVAL
    assert call(slots=None) == k3.EINVAL
    assert call(dims=k3.make_dims(7168, 1536, 895, 16)) == k3.EINVAL  # E differs from the state
    assert call(T=2) == k3.EUNSUPPORTED  # T * top_k above max_ids
    small = k3.ExpertCache(896, 8, 16)
    assert call(state=small.ptr) == k3.EUNSUPPORTED  # top_k above n_slots
    assert call(nbytes=100) == k3.EWORKSPACE


def test_noalloc_rejects_beyond_its_scratch():
    """T whose workspace exceeds the static scratch: EUNSUPPORTED on the host, before any
    HIP call (the K3 layer needs more than 64 MiB from about 96 tokens on)."""
    L = k3.lib()
    assert k3.workspace_bytes(K3, 64) <= 64 << 20 < k3.workspace_bytes(K3, 128)
    es = k3._MxExperts(*([FAKE.value] * 6))
    rc = L.k3moe_layer_forward_noalloc(ctypes.byref(K3), 128, FAKE, 0, FAKE, None,
                                       ctypes.byref(es), None, FAKE, None, None, None, None)
    assert rc == k3.EUNSUPPORTED
    assert b"static scratch" in L.k3moe_last_error()
    # invalid arguments are still rejected first, and T = 0 is a no-op
    assert L.k3moe_layer_forward_noalloc(ctypes.byref(K3), -1, FAKE, 0, FAKE, None,
                                         ctypes.byref(es), None, FAKE, None, None, None,
                                         None) == k3.EINVAL
    assert L.k3moe_layer_forward_noalloc(ctypes.byref(K3), 0, None, 0, None, None, None, None,
                                         None, None, None, None, None) == k3.OK


def test_packed_sizes_and_shape_checks():
    """Packed sizes are host arithmetic: codes keep R K / 2 bytes, scales are padded to whole
    chunks of 8 K steps (16 rows x 64 lanes x 8 bytes per chunk and tile)."""
    pb = k3.packed_expert_bytes(K3)
    assert pb["gate_q"] == pb["up_q"] == 1536 * 7168 // 2
    assert pb["down_q"] == 7168 * 1536 // 2
    assert pb["gate_s"] == pb["up_s"] == (1536 // 16) * 7 * 512 == 1536 * 7168 // 32
    assert pb["down_s"] == (7168 // 16) * 2 * 512  # 12 steps -> 2 chunks (4 steps of padding)
    with pytest.raises(k3.K3MoEError) as ei:
        k3.packed_expert_bytes(k3.make_dims(512, 256, 32, 4))  # d_model not a multiple of 1024
    assert ei.value.code == k3.EUNSUPPORTED
