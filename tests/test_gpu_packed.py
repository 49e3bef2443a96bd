"""The packed tile layout of the expert weights (k3moe_pack_experts) and the layer on it
(k3moe_layer_forward_packed), through the C ABI.

- The pack call is checked byte for byte against the layout as include/k3moe.h states it,
  built here with numpy index arithmetic (a permutation: no arithmetic of the method).
- The layer on packed experts is checked against the fp64 oracle with the bars of
  test_gpu_parity.py (routing bit-exact, per-token relative L2 and element bounds), on small
  ragged shapes (16-, 32- and 64-row tiles, partial row slices, experts with one to many
  subtiles; one-token cases on the decode kernels) and on the K3 layer: two single tokens,
  every token of the 32-token batch, and routing-chosen tile edges of the 2048-token prefill
  chunk; and at the API's limits (d_model 16384, d_ff 8192, 4096 experts with 32 slots, block
  mode at d_model 16384).
"""
import numpy as np
import pytest
import torch

import mxfp4_expert_matmul_k3moe_amd as k3
import oracle
from k3gen import device as gdev
from k3gen.workloads import BATCHED, DECODE, PREFILL, STACK8, Workload
from oracle import harness

from test_gpu_parity import ELEM_FACTOR, K3_TOL, TOL, check_routing, rel_elem, rel_l2, \
    run_gpu_layer, tile_probe_tokens

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def say(msg):
    print(f"[case] {msg}", flush=True)


def pack_reference(q: np.ndarray, s: np.ndarray, R: int, K: int):
    """The packed layout of one [R][K] matrix, from the row-major codes q [R][K/2] and
    scales s [R][K/32], by index arithmetic."""
    nk, nch = K // 128, (K // 128 + 7) // 8
    # codes: (t, step, lane = i + 16 g) -> 16 bytes of row 16 t + i at 64 step + 16 g
    qr = q.reshape(R // 16, 16, nk, 4, 16)               # [t][i][step][g][16 B]
    pq = qr.transpose(0, 2, 3, 1, 4).reshape(-1)         # [t][step][g][i][16 B]
    # scales: (t, c, lane) byte j -> block 4 (8 c + j) + g of row 16 t + i, 0 past nk
    sp = np.zeros((R // 16, 16, nch * 8, 4), dtype=np.uint8)  # [t][i][step][g]
    sp[:, :, :nk, :] = s.reshape(R // 16, 16, nk, 4)
    ps = sp.reshape(R // 16, 16, nch, 8, 4).transpose(0, 2, 4, 1, 3).reshape(-1)
    return pq, ps


SMALL = [
    # one 8-step chunk of d, f = 512 (4 down steps), mixed 16/32/64-row tiles
    Workload("pk_d1024", 61, d=1024, f=512, E=12, k=3, T=40, zipf_alpha=0.6),
    # three chunks of d, down with 12 steps (f = 1536), hot experts over several M tiles
    Workload("pk_mixed", 62, d=3072, f=1536, E=24, k=4, T=150, zipf_alpha=0.9),
    # f = 1024 (8 down steps), one token (the one-token kernels: a wave per slot tile of
    # G and U, decode down on whole tiles), two tokens (grouped GEMMs)
    Workload("pk_t1", 63, d=2048, f=1024, E=16, k=4, T=1),
    Workload("pk_t2", 64, d=2048, f=1024, E=16, k=4, T=2),
    # one token: three 8-step chunks of d and 12 down steps with 16 slots; one chunk of d
    # (the scale prefetch clamps at once) with two slots
    Workload("pk_t1_k16", 65, d=3072, f=1536, E=40, k=16, T=1),
    Workload("pk_t1_d1024", 66, d=1024, f=512, E=8, k=2, T=1),
]


# the API's limits on the packed layout (d_model % 1024 == 0, d_ff % 512 == 0)
LIMITS = [
    # d_model = 16384: one token on the one-token kernels with 16 waves (one per 1024 of
    # d_model, 1024 threads), and 20 tokens on the grouped GEMMs (16 scale chunks)
    Workload("pk_d16384_t1", 69, d=16384, f=512, E=8, k=2, T=1),
    Workload("pk_d16384_t20", 70, d=16384, f=512, E=8, k=2, T=20),
    # d_ff = 8192: one token with d_ff above 1536 runs the grouped GEMMs (64 down K steps)
    Workload("pk_f8192_t1", 71, d=1024, f=8192, E=6, k=2, T=1),
    Workload("pk_f8192_t20", 72, d=1024, f=8192, E=6, k=2, T=20),
    # 4096 experts with 32 slots: one token (more than 16 slots: grouped GEMMs, 32 experts
    # of one row each) and 24 tokens (about 700 experts)
    Workload("pk_e4096_k32_t1", 73, d=1024, f=512, E=4096, k=32, T=1),
    Workload("pk_e4096_k32_t24", 74, d=1024, f=512, E=4096, k=32, T=24),
]


def test_pack_matches_layout(dev):
    for w in SMALL[:2]:
        say(f"pack {w.name} d={w.d} f={w.f} E={w.E}")
        dims = k3.make_dims(w.d, w.f, w.E, w.k)
        ex = gdev.experts(w, 0, dev)
        pk = k3.pack_experts(dims, k3.MxExperts(**ex))
        torch.cuda.synchronize()
        for e in (0, w.E - 1):
            h = w.expert_host(0, e)
            for name, R, K in (("gate", w.f, w.d), ("up", w.f, w.d), ("down", w.d, w.f)):
                pq, ps = pack_reference(h[name + "_q"], h[name + "_s"], R, K)
                assert np.array_equal(getattr(pk, name + "_q")[e].cpu().numpy(), pq), (name, e)
                assert np.array_equal(getattr(pk, name + "_s")[e].cpu().numpy(), ps), (name, e)


def run_packed(w: Workload, x_np, dev, packed):
    dims = k3.make_dims(w.d, w.f, w.E, w.k)
    x = gdev.bf16_tensor(x_np, dev)
    T = x.shape[0]
    ids = torch.empty((T, w.k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, w.k), dtype=torch.float32, device=dev)
    ybf = torch.empty((T, w.d), dtype=torch.bfloat16, device=dev)
    y = k3.layer_forward_packed(dims, x, gdev.router_w(w, 0, dev), gdev.bias(w, 0, dev), packed,
                                y_bf16=ybf, ids=ids, gates=gates)
    torch.cuda.synchronize()
    return {"y": y, "ybf": ybf, "ids": ids.cpu().numpy(), "gates": gates.cpu().numpy()}


def check(g, ref, rows=None, tol=TOL):
    ids_g, gates_g = g["ids"], g["gates"]
    yg = g["y"].cpu().double().numpy()
    if rows is not None:
        ids_g, gates_g, yg = ids_g[rows], gates_g[rows], yg[rows]
    check_routing(ids_g, gates_g, ref["ids"], ref["gates"])
    assert np.isfinite(yg).all()
    err, el = rel_l2(yg, ref["y"]), rel_elem(yg, ref["y"])
    print(f"    max rel L2 err {err.max():.3e}, max elem err / row rms {el.max():.3e}  "
          f"(tokens {len(err)})", flush=True)
    assert err.max() <= tol and el.max() <= ELEM_FACTOR * tol
    assert torch.equal(g["ybf"], g["y"].to(torch.bfloat16))


@pytest.mark.parametrize("w", SMALL, ids=[s.name for s in SMALL])
def test_packed_layer_matches_oracle(dev, w):
    say(f"packed layer {w.name} d={w.d} f={w.f} E={w.E} k={w.k} T={w.T}")
    dims = k3.make_dims(w.d, w.f, w.E, w.k)
    packed = k3.pack_experts(dims, k3.MxExperts(**gdev.experts(w, 0, dev)))
    x = w.x_bf16()
    g = run_packed(w, x, dev, packed)
    check(g, harness.run_layer(w, x), tol=1e-4)


@pytest.mark.parametrize("w", LIMITS, ids=[s.name for s in LIMITS])
def test_packed_layer_at_api_limits(dev, w):
    say(f"packed layer at the limits {w.name} d={w.d} f={w.f} E={w.E} k={w.k} T={w.T}")
    dims = k3.make_dims(w.d, w.f, w.E, w.k)
    packed = k3.pack_experts(dims, k3.MxExperts(**gdev.experts(w, 0, dev)))
    x = w.x_bf16()
    g = run_packed(w, x, dev, packed)
    check(g, harness.run_layer(w, x), tol=K3_TOL)
    del packed
    torch.cuda.empty_cache()


def test_packed_repeat_runs_bit_identical(dev):
    w = SMALL[1]
    say(f"packed determinism {w.name}")
    dims = k3.make_dims(w.d, w.f, w.E, w.k)
    packed = k3.pack_experts(dims, k3.MxExperts(**gdev.experts(w, 0, dev)))
    x = w.x_bf16()
    a = run_packed(w, x, dev, packed)
    b = run_packed(w, x, dev, packed)
    assert torch.equal(a["y"], b["y"]) and np.array_equal(a["ids"], b["ids"])


def test_packed_decode_k3(dev):
    w = DECODE
    say("packed decode: d=7168 f=1536 E=896 k=16 T=1, two tokens")
    dims = k3.make_dims(w.d, w.f, w.E, w.k)
    ex = gdev.experts(w, 0, dev)
    packed = k3.pack_experts(dims, k3.MxExperts(**ex))
    del ex
    for ts in (0, 1):
        x = w.x_bf16(token_set=ts)
        g = run_packed(w, x, dev, packed)
        check(g, harness.run_layer(w, x), tol=K3_TOL)
        g2 = run_packed(w, x, dev, packed)
        assert torch.equal(g["y"], g2["y"])
    del packed
    torch.cuda.empty_cache()


def test_hot_tokens_policy_keeps_results(dev):
    """The cache policy of the grouped kernels' weight reads (experts below the threshold
    read non-temporally) changes no result: both layouts, bit for bit, with the threshold at
    0 (every expert normal), 16 (the default) and 9, on a skewed batch that has experts
    below and above every threshold."""
    w = SMALL[1]  # pk_mixed: Zipf(0.9), T=150, experts with 2 to 115 tokens
    say(f"cache policy invariance {w.name}")
    dims = k3.make_dims(w.d, w.f, w.E, w.k)
    ex = gdev.experts(w, 0, dev)
    packed = k3.pack_experts(dims, k3.MxExperts(**ex))
    x = w.x_bf16()
    got = {}
    try:
        for n in (0, 16, 9):
            k3.set_hot_tokens(n)
            got[n] = (run_gpu_layer(w, x, dev, experts=ex)["y"], run_packed(w, x, dev, packed)["y"])
    finally:
        k3.set_hot_tokens(16)
    for n in (16, 9):
        assert torch.equal(got[n][0], got[0][0]) and torch.equal(got[n][1], got[0][1]), n


def run_packed_block(w: Workload, h: torch.Tensor, layer: int, packed, dev):
    """One block (RMSNorm -> routed MoE on packed experts + shared expert -> residual) on the
    fp32 residual h [1][d]."""
    dims = k3.make_dims(w.d, w.f, w.E, w.k)
    b = gdev.block_extras(w, layer, dev)
    blk = k3.BlockWeights(b["rms_gamma"], b["sh_gate"], b["sh_up"], b["sh_down"], 1e-6)
    ids = torch.empty((1, w.k), dtype=torch.int32, device=dev)
    y = k3.layer_forward_packed(dims, h, gdev.router_w(w, layer, dev), gdev.bias(w, layer, dev),
                                packed, blk, ids=ids)
    torch.cuda.synchronize()
    return y, ids.cpu().numpy()


def packed_layer(w: Workload, layer: int, dev):
    """Layer `layer`'s experts in the packed layout (the row-major copy freed)."""
    dims = k3.make_dims(w.d, w.f, w.E, w.k)
    ex = gdev.experts(w, layer, dev)
    pk = k3.pack_experts(dims, k3.MxExperts(**ex))
    torch.cuda.synchronize()
    del ex
    return pk


def test_packed_block_mode_small_chain(dev):
    """Block mode on packed experts (one token, fp32 residual): three chained blocks with
    packed-layout shapes (two 8-step chunks of d, 8 down steps) against the oracle's stack."""
    w = Workload("pk_block", 67, d=2048, f=1024, E=16, k=4, T=1, layers=3, block=True)
    say("packed block mode, 3 chained blocks d=2048 f=1024")
    h0 = w.resid0()
    ref = harness.run_stack(w, h0)
    h = torch.from_numpy(h0).to(dev)
    for layer in range(w.layers):
        h, ids = run_packed_block(w, h, layer, packed_layer(w, layer, dev), dev)
        assert np.array_equal(ids, ref["ids"][layer]), f"routing differs at layer {layer}"
    yg = h.cpu().double().numpy()
    err, el = rel_l2(yg, ref["y"]), rel_elem(yg, ref["y"])
    print(f"    max rel L2 err {err.max():.3e}, max elem err / rms {el.max():.3e}", flush=True)
    assert err.max() <= 1e-4 and el.max() <= ELEM_FACTOR * 1e-4


def test_packed_block_mode_widest_rows(dev):
    """Block mode on packed experts at d_model = 16384: the two-pass RMSNorm (rows above
    8192), the shared expert on its own launches, and the fp32 one-token gate/up with 16
    waves of 4 KB token chunks in LDS; two chained blocks against the oracle's stack."""
    w = Workload("pk_block_d16384", 75, d=16384, f=512, E=8, k=2, T=1, layers=2, block=True)
    say(f"packed block mode, 2 chained blocks d={w.d} f={w.f}")
    h0 = w.resid0()
    ref = harness.run_stack(w, h0)
    h = torch.from_numpy(h0).to(dev)
    for layer in range(w.layers):
        h, ids = run_packed_block(w, h, layer, packed_layer(w, layer, dev), dev)
        assert np.array_equal(ids, ref["ids"][layer]), f"routing differs at layer {layer}"
    yg = h.cpu().double().numpy()
    err, el = rel_l2(yg, ref["y"]), rel_elem(yg, ref["y"])
    print(f"    max rel L2 err {err.max():.3e}, max elem err / rms {el.max():.3e}", flush=True)
    assert err.max() <= 1e-4 and el.max() <= ELEM_FACTOR * 1e-4


@pytest.mark.parametrize("E", [320, 1032])
def test_packed_block_mode_wide_router_chain(dev, E):
    """Block mode on packed experts with more than 256 experts (the shared gate/up rides in
    the top-k launch, the shared down in the expert gate/up launch; E = 1032: five keys per
    top-k thread): three chained blocks against the oracle."""
    w = Workload(f"pk_block_e{E}", 68, d=2048, f=1024, E=E, k=4, T=1, layers=3, block=True)
    say(f"packed block mode, 3 chained blocks d=2048 f=1024 E={E}")
    h0 = w.resid0()
    ref = harness.run_stack(w, h0)
    h = torch.from_numpy(h0).to(dev)
    for layer in range(w.layers):
        h, ids = run_packed_block(w, h, layer, packed_layer(w, layer, dev), dev)
        assert np.array_equal(ids, ref["ids"][layer]), f"routing differs at layer {layer}"
    yg = h.cpu().double().numpy()
    err, el = rel_l2(yg, ref["y"]), rel_elem(yg, ref["y"])
    print(f"    max rel L2 err {err.max():.3e}, max elem err / rms {el.max():.3e}", flush=True)
    assert err.max() <= 1e-4 and el.max() <= ELEM_FACTOR * 1e-4


def test_packed_stack8_k3(dev):
    """The 8-block K3 stack on packed experts (fp32 tokens on the one-token kernels), one
    token, routed exactly as the oracle at every block; the final residual within the K3 bar
    in L2 and element-wise."""
    w = STACK8
    say("packed 8 stacked blocks, T=1, ~126 GB of packed MXFP4 experts resident")
    h0 = w.resid0()
    ref = harness.run_stack(w, h0)
    layers = [packed_layer(w, l, dev) for l in range(w.layers)]
    torch.cuda.empty_cache()
    h = torch.from_numpy(h0).to(dev)
    for l in range(w.layers):
        h, ids = run_packed_block(w, h, l, layers[l], dev)
        assert np.array_equal(ids, ref["ids"][l]), f"routing differs at layer {l}"
    yg = h.cpu().double().numpy()
    err, el = rel_l2(yg, ref["y"]), rel_elem(yg, ref["y"])
    print(f"    max rel L2 err after 8 blocks {err.max():.3e}, max elem err / rms {el.max():.3e}",
          flush=True)
    assert err.max() <= K3_TOL and el.max() <= ELEM_FACTOR * K3_TOL
    del layers
    torch.cuda.empty_cache()


def test_packed_batched_k3(dev):
    w = BATCHED
    say("packed batched decode: T=32, every token")
    dims = k3.make_dims(w.d, w.f, w.E, w.k)
    ex = gdev.experts(w, 0, dev)
    packed = k3.pack_experts(dims, k3.MxExperts(**ex))
    del ex
    x = w.x_bf16()
    g = run_packed(w, x, dev, packed)
    check(g, harness.run_layer(w, x), tol=K3_TOL)
    del packed
    torch.cuda.empty_cache()


def test_packed_prefill_k3(dev):
    w = PREFILL
    say("packed prefill: T=2048 with Zipf(1.1) logit bias")
    dims = k3.make_dims(w.d, w.f, w.E, w.k)
    ex = gdev.experts(w, 0, dev)
    packed = k3.pack_experts(dims, k3.MxExperts(**ex))
    del ex
    x = w.x_bf16()
    g = run_packed(w, x, dev, packed)
    ids_all, gates_all, _, _ = oracle.layer_route(x, w.router_w(0), w.bias(0), w.k)
    check_routing(g["ids"], g["gates"], ids_all, gates_all)
    rows = tile_probe_tokens(ids_all, w.E, seed=2)
    check(g, harness.run_layer(w, x, tokens=rows), rows=rows, tol=K3_TOL)
    del packed
    torch.cuda.empty_cache()
