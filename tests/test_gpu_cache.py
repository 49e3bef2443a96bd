"""Routed experts beyond HBM (k3moe_layer_forward_cached): the layer with its experts in
pinned host memory and a few HBM slots must give the resident layer's routing and output
bit for bit, over a stream of token sets that forces evictions; one step is also held to
the oracle."""
import numpy as np
import pytest
import torch

import mxfp4_expert_matmul_k3moe_amd as k3
from k3gen import device as gdev
from k3gen.workloads import TOY, Workload
from oracle import harness

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def say(msg):
    print(f"[case] {msg}", flush=True)


def _slot_experts(w: Workload, C: int, dev) -> k3.MxExperts:
    shp = {n: (C,) + tuple(w.tensor_shape(n)) for n in
           ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")}
    # filled with junk so that a slot read before its copy would show
    return k3.MxExperts(**{n: torch.full(s, 0x5A, dtype=torch.uint8, device=dev)
                           for n, s in shp.items()})


@pytest.mark.parametrize("w,C", [
    (TOY.with_(T=1, name="toy_t1"), 6),       # T = 1: decode kernels on slots, evictions
    (TOY.with_(T=3, name="toy_t3"), 12),      # few tokens: GEMV kernels
    (TOY.with_(T=20, name="toy_t20"), 32),    # grouped MFMA GEMMs on slots
    (Workload("k3w_cache", 31, d=7168, f=1536, E=40, k=16, T=1), 20),  # K3 widths, MFMA down
    # the limits: 4096 experts, 32 slots a token, and no more cache slots than one call's
    # pairs (T * k = 64), so almost every step evicts
    (Workload("e4096_cache", 32, d=256, f=128, E=4096, k=32, T=2), 64),
])
def test_cached_layer_equals_resident(dev, w, C):
    say(f"cached layer {w.name} d={w.d} f={w.f} E={w.E} k={w.k} T={w.T} slots={C}")
    dims = k3.make_dims(w.d, w.f, w.E, w.k)
    ex_dev = gdev.experts(w, 0, dev)
    host = k3.MxExperts(**{n: t.cpu().pin_memory() for n, t in ex_dev.items()})
    resident = k3.MxExperts(**ex_dev)
    slots = _slot_experts(w, C, dev)
    cache = k3.ExpertCache(w.E, C, w.T * w.k)
    wr, b = gdev.router_w(w, 0, dev), gdev.bias(w, 0, dev)
    ws = k3.make_workspace(dims, w.T, dev)
    misses = hits = 0
    for step in range(8):
        x = gdev.x_bf16(w, token_set=step % 5, device=dev)  # token sets come back: hits
        ids_r = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
        g_r = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
        ybf_r = torch.empty((w.T, w.d), dtype=torch.bfloat16, device=dev)
        y_r = k3.layer_forward(dims, x, wr, b, resident, y_bf16=ybf_r, ids=ids_r, gates=g_r)
        ids_c = torch.empty_like(ids_r)
        g_c = torch.empty_like(g_r)
        ybf_c = torch.empty_like(ybf_r)
        y_c, st = k3.layer_forward_cached(dims, x, wr, b, host, slots, cache, y_bf16=ybf_c,
                                          ids=ids_c, gates=g_c, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(ids_c, ids_r) and torch.equal(g_c, g_r)
        assert torch.equal(y_c, y_r), f"step {step}: cached output differs from resident"
        assert torch.equal(ybf_c, ybf_r)
        distinct = len(set(ids_r.cpu().numpy().reshape(-1).tolist()))
        assert st.distinct == distinct and st.hits + st.misses == distinct
        assert st.bytes_copied == st.misses * w.expert_bytes
        misses += st.misses
        hits += st.hits
        if step == 0:
            ref = harness.run_layer(w, w.x_bf16(0))
            assert np.array_equal(ids_c.cpu().numpy(), ref["ids"])
            yc = y_c.cpu().double().numpy()
            err = np.linalg.norm(yc - ref["y"], axis=1) / np.linalg.norm(ref["y"], axis=1)
            assert err.max() < 1e-4
    tot = cache.stats()
    assert (tot.hits, tot.misses) == (hits, misses) and hits > 0 and misses > 0
