"""The allocation-free entry point (k3moe_layer_forward_noalloc) against k3moe_layer_forward
with a workspace: same kernels, so the same routing and outputs bit for bit. Two calls in a
row on the shared static scratch, the second with fewer tokens, for each path (grouped MFMA,
per-expert GEMV, one-token decode kernels, block mode)."""
import numpy as np
import pytest
import torch

import mxfp4_expert_matmul_k3moe_amd as k3
from k3gen import device as gdev
from k3gen.workloads import Workload

pytestmark = pytest.mark.gpu

K3W = Workload("k3w_noalloc", 51, d=7168, f=1536, E=40, k=16, T=32)
SMALL = Workload("small_noalloc", 52, d=512, f=256, E=24, k=4, T=20)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _run(fn, w, x, ex, wr, blk, dev):
    T = x.shape[0]
    y = torch.empty((T, w.d), dtype=torch.float32, device=dev)
    ybf = torch.empty((T, w.d), dtype=torch.bfloat16, device=dev)
    ids = torch.empty((T, w.k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, w.k), dtype=torch.float32, device=dev)
    fn(k3.make_dims(w.d, w.f, w.E, w.k), x, wr, gdev.bias(w, 0, dev), ex, blk, y=y, y_bf16=ybf,
       ids=ids, gates=gates)
    torch.cuda.synchronize()
    return y, ybf, ids, gates


@pytest.mark.parametrize("w,Ts", [(K3W, (32, 17)), (K3W, (5, 1)), (SMALL, (20, 3)),
                                  (SMALL, (64, 1))],
                         ids=["k3w_grouped_then_smaller", "k3w_gemv_then_decode",
                              "small_grouped_then_gemv", "small_64_then_1"])
def test_noalloc_equals_workspace_entry_point(dev, w, Ts):
    ex = k3.MxExperts(**gdev.experts(w, 0, dev))
    wr = gdev.router_w(w, 0, dev)
    for T in Ts:  # the second call has fewer tokens and reuses the scratch
        print(f"[case] noalloc vs workspace: {w.name} T={T}", flush=True)
        x = gdev.bf16_tensor(w.x_bf16(token_set=T, T=T), dev)
        a = _run(k3.layer_forward, w, x, ex, wr, None, dev)
        b = _run(k3.layer_forward_noalloc, w, x, ex, wr, None, dev)
        for u, v in zip(a, b):
            assert torch.equal(u, v)


def test_noalloc_block_mode_equals_workspace_entry_point(dev):
    w = SMALL.with_(block=True, layers=1, name="small_noalloc_block")
    ex = k3.MxExperts(**gdev.experts(w, 0, dev))
    wr = gdev.router_w(w, 0, dev)
    b = gdev.block_extras(w, 0, dev)
    blk = k3.BlockWeights(b["rms_gamma"], b["sh_gate"], b["sh_up"], b["sh_down"], 1e-6)
    for T in (9, 2):
        print(f"[case] noalloc vs workspace, block mode: T={T}", flush=True)
        h = torch.from_numpy(w.resid0(token_set=T, T=T)).to(dev)
        a = _run(k3.layer_forward, w, h, ex, wr, blk, dev)
        c = _run(k3.layer_forward_noalloc, w, h, ex, wr, blk, dev)
        for u, v in zip(a, c):
            assert torch.equal(u, v)


def test_noalloc_beyond_scratch_is_an_error(dev):
    w = K3W
    dims = k3.make_dims(w.d, w.f, w.E, w.k)
    T = 128  # needs about 85 MiB of scratch
    x = torch.zeros((T, w.d), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T, w.d), dtype=torch.float32, device=dev)
    ex = k3.MxExperts(**{n: torch.empty((w.E,) + w.tensor_shape(n), dtype=torch.uint8, device=dev)
                         for n in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")})
    with pytest.raises(k3.K3MoEError) as ei:
        k3.layer_forward_noalloc(dims, x, gdev.router_w(w, 0, dev), None, ex, y=y)
    assert ei.value.code == k3.EUNSUPPORTED
