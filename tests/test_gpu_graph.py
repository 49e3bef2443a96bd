"""GPU: the layer and block calls captured into a HIP graph (torch.cuda.CUDAGraph on the
caller's stream) and replayed several times, with eager work and synchronisations of the
program between replays; every replay must equal the eager result for the same input bit
for bit. Covers the single-token decode kernels, the block-mode side stream (it joins the
capture through the fork event) and the many-token grouped-GEMM path with its bucketing."""
import pytest
import torch

import mxfp4_expert_matmul_k3moe_amd as k3
from k3gen import device as gdev
from k3gen.workloads import TOY

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def say(msg):
    print(f"[case] {msg}", flush=True)


def capture(fn):
    """Capture fn() into a graph after one eager run of it on the capture stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def chain_setup(w, dev, block):
    dims = k3.make_dims(w.d, w.f, w.E, w.k)
    layers = []
    for l in range(w.layers):
        blk = None
        if block:
            b = gdev.block_extras(w, l, dev)
            blk = k3.BlockWeights(b["rms_gamma"], b["sh_gate"], b["sh_up"], b["sh_down"], 1e-6)
        layers.append((gdev.router_w(w, l, dev), gdev.bias(w, l, dev),
                       k3.MxExperts(**gdev.experts(w, l, dev)), blk))
    return dims, layers


def make_inputs(w, dev, block, n):
    if block:
        return [torch.from_numpy(w.resid0(token_set=i)).to(dev) for i in range(n)]
    return [gdev.x_bf16(w, token_set=i, device=dev) for i in range(n)]


def run_chain(w, dims, layers, x_in, outs, ids, gates, ws):
    h = x_in
    for l, (wr, bias, ex, blk) in enumerate(layers):
        k3.layer_forward(dims, h, wr, bias, ex, blk, y=outs[l], ids=ids[l], gates=gates[l], ws=ws)
        h = outs[l]


@pytest.mark.parametrize("case", ["decode_layer", "block_chain", "grouped_t32"])
def test_graph_replay_matches_eager(dev, case):
    if case == "decode_layer":
        w, block = TOY.with_(name="toy_graph"), False
    elif case == "block_chain":
        w, block = TOY.with_(block=True, layers=2, name="toy_block_graph"), True
    else:
        w, block = TOY.with_(T=32, name="toy_t32_graph"), False
    say(f"graph capture and replay: {case} (T={w.T}, layers={w.layers})")
    dims, layers = chain_setup(w, dev, block)
    xs = make_inputs(w, dev, block, 3)
    ws = k3.make_workspace(dims, w.T, dev)
    L = len(layers)

    def buffers():
        outs = [torch.empty((w.T, w.d), dtype=torch.float32, device=dev) for _ in range(L)]
        ids = [torch.empty((w.T, w.k), dtype=torch.int32, device=dev) for _ in range(L)]
        gates = [torch.empty((w.T, w.k), dtype=torch.float32, device=dev) for _ in range(L)]
        return outs, ids, gates

    # eager results for each input
    eager = []
    for x in xs:
        outs, ids, gates = buffers()
        run_chain(w, dims, layers, x, outs, ids, gates, ws)
        torch.cuda.synchronize()
        eager.append(([o.clone() for o in outs], [i.clone() for i in ids], [g.clone() for g in gates]))

    x_static = xs[0].clone()
    outs, ids, gates = buffers()
    g = capture(lambda: run_chain(w, dims, layers, x_static, outs, ids, gates, ws))
    for rep, sel in enumerate((0, 1, 2, 1, 0)):
        x_static.copy_(xs[sel])
        g.replay()
        torch.cuda.synchronize()
        eo, ei, eg = eager[sel]
        for l in range(L):
            assert torch.equal(ids[l], ei[l]), f"replay {rep}: ids differ at layer {l}"
            assert torch.equal(gates[l], eg[l]), f"replay {rep}: gates differ at layer {l}"
            assert torch.equal(outs[l], eo[l]), f"replay {rep}: output differs at layer {l}"
        # eager work of the program between replays (other buffers, same workspace)
        o2, i2, g2 = buffers()
        run_chain(w, dims, layers, xs[(sel + 1) % 3], o2, i2, g2, ws)
        torch.cuda.synchronize()
        assert torch.equal(o2[-1], eager[(sel + 1) % 3][0][-1])
    print(f"    5 replays equal to eager", flush=True)
