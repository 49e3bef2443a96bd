"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars (the oracle is the reference):
  - routing: expert ids and their order bit-exact; gates within 2 fp32 ulps;
  - bucketing: offsets and rows bit-exact;
  - layer output: max over tokens of ||y_gpu - y_ref||_2 / ||y_ref||_2 <= 2e-3 on the
    fp32 output (the 2e-3 relative bound, read per token in the L2 norm), and per element
    max_i |y_gpu[t,i] - y_ref[t,i]| / rms(y_ref[t]) <= 5 x the L2 bar (the largest of d
    roughly normal errors stays within about 5 of their standard deviations; relative to
    the row rms, since single outputs can sit arbitrarily close to zero);
  - K3-width layers are also held to 5e-4 in L2 (about 10 x the 2e-5 .. 6e-5 the FP8-term
    MFMA paths measure), so a single wrong tile row or N slice cannot hide under 2e-3;
  - the bf16 copy equals round-to-nearest-even of the fp32 output;
  - repeated runs are bit-identical.
Every case prints its name before touching the GPU.
"""
import numpy as np
import pytest
import torch

import mxfp4_expert_matmul_k3moe_amd as k3
import oracle
from k3gen import device as gdev
from k3gen.workloads import BATCHED, DECODE, PREFILL, STACK8, TINY, TOY, Workload
from oracle import harness

pytestmark = pytest.mark.gpu
TOL = 2e-3
K3_TOL = 5e-4
ELEM_FACTOR = 5.0


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def say(msg):
    print(f"[case] {msg}", flush=True)


def dims_of(w: Workload):
    return k3.make_dims(w.d, w.f, w.E, w.k)


def rel_l2(yg: np.ndarray, yr: np.ndarray) -> np.ndarray:
    return np.linalg.norm(yg - yr, axis=1) / np.maximum(np.linalg.norm(yr, axis=1), 1e-300)


def check_routing(ids_g, gates_g, ids_r, gates_r):
    assert np.array_equal(ids_g, ids_r), "expert ids/order differ from the oracle"
    g32 = gates_r.astype(np.float32)
    ulp = np.spacing(np.abs(g32))
    assert np.all(np.abs(gates_g - g32) <= 2 * ulp), "gates differ by more than 2 ulp"


def run_gpu_layer(w: Workload, x_np, dev, layer=0, experts=None, block=False, x_dtype="bf16"):
    dims = dims_of(w)
    ex = k3.MxExperts(**(experts if experts is not None else gdev.experts(w, layer, dev)))
    if x_dtype == "bf16":
        x = gdev.bf16_tensor(x_np, dev)
    else:
        x = torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).to(dev)
    T = x.shape[0]
    ids = torch.empty((T, w.k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, w.k), dtype=torch.float32, device=dev)
    ybf = torch.empty((T, w.d), dtype=torch.bfloat16, device=dev)
    blk = None
    if block:
        b = gdev.block_extras(w, layer, dev)
        blk = k3.BlockWeights(b["rms_gamma"], b["sh_gate"], b["sh_up"], b["sh_down"], 1e-6)
    y = k3.layer_forward(dims, x, gdev.router_w(w, layer, dev), gdev.bias(w, layer, dev), ex,
                         blk, y_bf16=ybf, ids=ids, gates=gates)
    torch.cuda.synchronize()
    return {"y": y, "ybf": ybf, "ids": ids.cpu().numpy(), "gates": gates.cpu().numpy()}


def rel_elem(yg: np.ndarray, yr: np.ndarray) -> np.ndarray:
    """Per token: the largest element error relative to the reference row's rms."""
    rms = np.sqrt(np.mean(yr * yr, axis=1))
    return np.max(np.abs(yg - yr), axis=1) / np.maximum(rms, 1e-300)


def assert_layer(w: Workload, g, ref, rows=None, tol=TOL):
    ids_g, gates_g = g["ids"], g["gates"]
    yg = g["y"].cpu().double().numpy()
    if rows is not None:
        ids_g, gates_g, yg = ids_g[rows], gates_g[rows], yg[rows]
    check_routing(ids_g, gates_g, ref["ids"], ref["gates"])
    assert np.isfinite(yg).all() and np.isfinite(ref["y"]).all()
    err = rel_l2(yg, ref["y"])
    el = rel_elem(yg, ref["y"])
    print(f"    max rel L2 err {err.max():.3e}, max elem err / row rms {el.max():.3e}  "
          f"(tokens {len(err)})", flush=True)
    assert err.max() <= tol
    assert el.max() <= ELEM_FACTOR * tol, f"element error {el.max():.3e} of the row rms"
    assert torch.equal(g["ybf"], g["y"].to(torch.bfloat16)), "bf16 copy is not RNE(fp32)"
    return err


def tile_probe_tokens(ids: np.ndarray, E: int, want: int = 40, seed: int = 0) -> list:
    """Tokens whose (token, expert) pairs sit where the grouped GEMM's tiling has edges.

    Bucket rows of an expert run in ascending token order; an expert with n tokens takes one
    16-row tile (n <= 16), one 32-row tile (n <= 32) or ceil(n / 64) tiles of 64 rows. Taken:
    the first and last row of several 64-row tiles of the two hottest experts and of their
    final partial tiles, the first and last row of experts on 16-, 32- and single partial
    64-row tiles, tokens 0 and T-1, then random tokens up to `want`."""
    T, k = ids.shape
    members = [[] for _ in range(E)]
    for t in range(T):
        for e in ids[t]:
            members[int(e)].append(t)
    counts = np.array([len(m) for m in members])
    pick = {0, T - 1}

    def rows_of(e, rows):
        for r in rows:
            if 0 <= r < counts[e]:
                pick.add(members[e][r])

    for e in np.argsort(-counts, kind="stable")[:2]:
        n = int(counts[e])
        nt = (n + 63) // 64
        tiles = sorted({0, 1, nt // 2, nt - 2, nt - 1} & set(range(nt)))
        for m in tiles:
            rows_of(e, [64 * m, 64 * m + 63, min(64 * m + 63, n - 1)])
    for lo, hi in ((1, 16), (17, 32), (33, 64), (65, 128)):
        cand = [e for e in range(E) if lo <= counts[e] <= hi]
        # the fullest and the emptiest tile of each kind
        cand.sort(key=lambda e: (-counts[e], e))
        for e in cand[:1] + cand[-1:]:
            rows_of(e, [0, counts[e] - 1, counts[e] // 2])
    rng = np.random.default_rng(seed)
    rest = [t for t in rng.permutation(T) if t not in pick]
    while len(pick) < want and rest:
        pick.add(int(rest.pop()))
    return sorted(int(t) for t in pick)


# ---- generator ----------------------------------------------------------------------------
def test_device_generator_matches_host(dev):
    say("device generator vs host generator")
    for w, es in [(TOY, range(TOY.E)), (DECODE.with_(E=3), range(3))]:
        d = gdev.experts(w, 0, dev)
        for e in es:
            h = w.expert_host(0, e)
            for n, t in d.items():
                assert np.array_equal(t[e].cpu().numpy(), h[n]), (w.name, e, n)


# ---- small layers -------------------------------------------------------------------------
SHAPES = [
    TINY,                                                   # T=3, multi-token GEMV path
    TOY,                                                    # the toy layer, T=1
    Workload("ragged1", 11, d=96, f=64, E=13, k=3, T=37),   # 3 blocks/row, ragged tails
    Workload("k_eq_e", 12, d=160, f=96, E=5, k=5, T=1),     # k = E
    Workload("prefill_small", 13, d=512, f=256, E=40, k=8, T=70, zipf_alpha=1.1),
    Workload("one_expert", 14, d=64, f=32, E=1, k=1, T=4),
    Workload("k3_widths", 15, d=7168, f=1536, E=24, k=4, T=5),
    Workload("k3_widths_t1", 16, d=7168, f=1536, E=40, k=16, T=1),
    Workload("many_tokens", 17, d=256, f=128, E=16, k=2, T=130),
    # grouped MFMA GEMMs with 16-, 32- and 64-row tiles, several M tiles per hot expert
    # and partial N slices (f = 384 of 2 x 256 rows, d = 384 of 512)
    Workload("mfma_mixed", 18, d=384, f=384, E=24, k=3, T=150, zipf_alpha=0.6),
    # more than 64 tokens with d not a multiple of 128: per-expert GEMV path
    Workload("gemv_many", 19, d=224, f=64, E=12, k=3, T=70),
    # the smallest token count that takes the grouped MFMA path; d and f multiples of 512
    # (scales fetched 4 steps at a time)
    Workload("mfma_t16", 20, d=512, f=512, E=10, k=3, T=16),
    # one token with more than 16 slots: the fp32-FMA down kernel instead of the MFMA one
    Workload("k20_t1", 21, d=512, f=256, E=40, k=20, T=1),
    # one token on the MFMA down kernel with 6 K steps (f = 768)
    Workload("mfma_t1_f768", 22, d=384, f=768, E=12, k=5, T=1),
    # one token with 9 MXFP4 blocks of a row per lane (d = 288: 1 lane x 9 blocks;
    # d = 2304: 8 lanes x 9 blocks): the GEMV gate/up, which walks rows in groups of 8
    Workload("d288_t1", 23, d=288, f=64, E=12, k=3, T=1),
    Workload("d2304_t1", 24, d=2304, f=256, E=16, k=4, T=1),
    Workload("d4608_t1", 25, d=4608, f=128, E=9, k=2, T=1),
    # the register-fed grouped gate/up (d a multiple of 1024): one scale chunk of 8 K steps
    # (d = 1024), and three chunks with 16-, 32- and 64-row tiles, several M tiles per hot
    # expert and a half-full second N slice (d = 3072, f = 384)
    Workload("mfma_rw_d1024", 26, d=1024, f=256, E=12, k=3, T=40, zipf_alpha=0.6),
    Workload("mfma_rw_mixed", 27, d=3072, f=384, E=24, k=3, T=150, zipf_alpha=0.6),
]


@pytest.mark.parametrize("w", SHAPES, ids=[s.name for s in SHAPES])
def test_layer_matches_oracle(dev, w):
    say(f"layer {w.name} d={w.d} f={w.f} E={w.E} k={w.k} T={w.T}")
    x = w.x_bf16()
    g = run_gpu_layer(w, x, dev)
    ref = harness.run_layer(w, x)
    err = assert_layer(w, g, ref)
    assert err.max() < 1e-4  # fp32 accumulation throughout these GEMV paths


LIMIT_SHAPES = [
    # 4096 experts and 32 slots: one token (fp32-FMA down, more than 16 slots), and 40
    # tokens on the grouped MFMA GEMMs (about 1100 experts, each on a 16-row tile)
    Workload("e4096_k32_t1", 28, d=256, f=64, E=4096, k=32, T=1),
    Workload("e4096_k32_t40", 29, d=256, f=128, E=4096, k=32, T=40),
    # d_model = 16384: 16 scale chunks of the register-fed gate/up, 64 down N slices
    Workload("d16384_t1", 30, d=16384, f=128, E=8, k=2, T=1),
    Workload("d16384_t20", 31, d=16384, f=128, E=8, k=2, T=20),
    # d_ff = 8192, the widest the expert kernels take (256 scale blocks a row, 4 per lane)
    Workload("f8192_t1", 32, d=256, f=8192, E=6, k=2, T=1),
    Workload("f8192_t20", 33, d=256, f=8192, E=6, k=2, T=20),
]


@pytest.mark.parametrize("w", LIMIT_SHAPES, ids=[s.name for s in LIMIT_SHAPES])
def test_layer_at_api_limits(dev, w):
    say(f"layer at the limits {w.name} d={w.d} f={w.f} E={w.E} k={w.k} T={w.T}")
    x = w.x_bf16()
    g = run_gpu_layer(w, x, dev)
    ref = harness.run_layer(w, x)
    assert_layer(w, g, ref, tol=K3_TOL)


def test_block_mode_widest_rows(dev):
    """Block mode at d_model = 16384, above the rows the RMSNorm keeps in registers (8192):
    the two-pass norm that reads h again, two chained blocks of three tokens."""
    w = Workload("block_d16384", 34, d=16384, f=128, E=8, k=2, T=3, layers=2, block=True)
    say(f"block mode, 2 chained blocks, d={w.d}, T={w.T}")
    h0 = w.resid0()
    ref = harness.run_stack(w, h0)
    h = torch.from_numpy(h0).to(dev)
    for layer in range(w.layers):
        g = run_gpu_layer(w, h.cpu().numpy(), dev, layer=layer, block=True, x_dtype="f32")
        assert np.array_equal(g["ids"], ref["ids"][layer]), f"routing differs at layer {layer}"
        h = g["y"]
    err = rel_l2(h.cpu().double().numpy(), ref["y"])
    print(f"    max rel L2 err {err.max():.3e}", flush=True)
    assert err.max() < 1e-4


def test_entry_points_separately(dev):
    w = TOY.with_(T=9, name="toy9")
    say("router / route_bucket / expert_ffn separately on toy T=9")
    dims = dims_of(w)
    xh = w.x_bf16()
    x = gdev.bf16_tensor(xh, dev)
    ids, gates = k3.router(dims, x, gdev.router_w(w, 0, dev))
    ref = harness.run_layer(w, xh)
    torch.cuda.synchronize()
    check_routing(ids.cpu().numpy(), gates.cpu().numpy(), ref["ids"], ref["gates"])
    offs, rows = k3.route_bucket(dims, ids)
    ro, rr = oracle.bucket(ref["ids"], w.E)
    assert np.array_equal(offs.cpu().numpy(), ro) and np.array_equal(rows.cpu().numpy(), rr)
    ex = k3.MxExperts(**gdev.experts(w, 0, dev))
    y = k3.expert_ffn(dims, x, ex, offs, rows, gates)
    torch.cuda.synchronize()
    assert rel_l2(y.cpu().double().numpy(), ref["y"]).max() < 1e-4
    # the same with a single token (fused down + combine path)
    y1 = k3.expert_ffn(dims, x[:1].contiguous(), ex, *k3.route_bucket(dims, ids[:1].contiguous()),
                       gates[:1].contiguous())
    torch.cuda.synchronize()
    assert rel_l2(y1.cpu().double().numpy(), ref["y"][:1]).max() < 1e-4


def test_bucket_large_T_exact(dev):
    say("route_bucket T=300 (multi-block) vs oracle")
    rng = np.random.default_rng(9)
    E, k, T = 50, 6, 300
    ids_np = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    dims = k3.make_dims(64, 32, E, k)
    offs, rows = k3.route_bucket(dims, torch.from_numpy(ids_np).to(dev))
    torch.cuda.synchronize()
    ro, rr = oracle.bucket(ids_np, E)
    assert np.array_equal(offs.cpu().numpy(), ro) and np.array_equal(rows.cpu().numpy(), rr)


def test_zero_input_routes_first_k(dev):
    w = TOY.with_(T=2, name="toy_zero")
    say("x = 0")
    x = np.zeros((2, w.d), dtype=np.uint16)
    g = run_gpu_layer(w, x, dev)
    assert g["ids"].tolist() == [list(range(w.k))] * 2
    assert np.all(g["gates"] == np.float32(1.0 / w.E))
    ref = harness.run_layer(w, x)
    assert_layer(w, g, ref)


@pytest.mark.parametrize("E,k,T", [(32, 4, 1), (896, 16, 1), (896, 16, 80),
                                   (4096, 32, 1), (4096, 32, 80)])
def test_router_near_ties_below_upper_key_bits(dev, E, k, T):
    # x = 0, so every logit is exactly its fp32 bias. Clusters of biases that differ only
    # in the last fp32 mantissa bits share the upper 32 bits of their fp64 order keys, so
    # the threshold cannot separate them and the exact ranking on full keys must.
    say(f"router near-ties in the low key bits: E={E} k={k} T={T}")
    rng = np.random.default_rng(E + k + T)
    perm = rng.permutation(E)
    bias = rng.uniform(-2.0, -1.0, E).astype(np.float32)
    for c, base in enumerate((1.0, 0.5, 0.25)):
        idx = perm[8 * c:8 * c + 8]
        bias[idx] = (np.float32(base) + rng.permutation(8).astype(np.float32) *
                     np.float32(base * 2.0 ** -23)).astype(np.float32)
    d = 512
    dims = k3.make_dims(d, 256, E, k)
    x = torch.zeros((T, d), dtype=torch.bfloat16, device=dev)
    wr = torch.zeros((d, E), dtype=torch.bfloat16, device=dev)
    ids, gates = k3.router(dims, x, wr, torch.from_numpy(bias).to(dev))
    torch.cuda.synchronize()
    ids_r, gates_r = oracle.route(np.tile(bias.astype(np.float64), (T, 1)), k)
    check_routing(ids.cpu().numpy(), gates.cpu().numpy(), ids_r, gates_r)


def test_nan_scale_propagates(dev):
    w = TOY
    say("E8M0 255 in one down row of a selected expert")
    x = w.x_bf16()
    ref0 = harness.run_layer(w, x)
    e = int(ref0["ids"][0, 0])
    ex = gdev.experts(w, 0, dev)
    ex["down_s"][e, 5, 0] = 255
    g = run_gpu_layer(w, x, dev, experts=ex)
    over = w.expert_host(0, e)
    over["down_s"][5, 0] = 255
    ref = harness.run_layer(w, x, expert_override={e: over})
    yg = g["y"].cpu().numpy()[0]
    assert np.array_equal(np.isnan(yg), np.isnan(ref["y"][0]))
    assert np.isnan(yg[5]) and np.isfinite(np.delete(yg, 5)).all()


def test_nan_scales_propagate_grouped_gemm(dev):
    """E8M0 255 on the grouped-GEMM path: a gate scale makes h NaN for the expert's pairs
    (NaN through the FP8 terms of h into down: every output of those tokens), a down scale
    makes one output row NaN. The NaN pattern must be the oracle's."""
    w = next(s for s in SHAPES if s.name == "mfma_t16")
    x = w.x_bf16()
    ref0 = harness.run_layer(w, x)
    e = int(ref0["ids"][0, 0])
    for name, row, blk in (("gate_s", 7, 0), ("down_s", 5, 1)):
        say(f"E8M0 255 in {name}[{e}, {row}, {blk}] ({w.name}, T={w.T})")
        ex = gdev.experts(w, 0, dev)
        ex[name][e, row, blk] = 255
        g = run_gpu_layer(w, x, dev, experts=ex)
        over = w.expert_host(0, e)
        over[name][row, blk] = 255
        ref = harness.run_layer(w, x, expert_override={e: over})
        yg = g["y"].cpu().numpy()
        nan_ref = np.isnan(ref["y"])
        assert nan_ref.any() and not nan_ref.all()
        assert np.array_equal(np.isnan(yg), nan_ref)
        ok = ~nan_ref.any(axis=1)  # tokens that did not pick e stay within tolerance
        assert rel_l2(yg[ok].astype(np.float64), ref["y"][ok]).max() <= TOL


def test_unaligned_scales_take_the_gemv_kernels(dev):
    """Scale arrays starting at an odd address: the MFMA kernels read scales as dwords, so
    one token (down) and 20 tokens (grouped GEMMs) must fall back to the byte-reading GEMV
    kernels and still match the oracle."""
    for w in (TOY, TOY.with_(T=20, name="toy20")):
        say(f"odd-address scale arrays ({w.name}, T={w.T})")
        x = w.x_bf16()
        ex = gdev.experts(w, 0, dev)
        for name in ("gate_s", "up_s", "down_s"):
            t = ex[name]
            buf = torch.empty(t.numel() + 1, dtype=torch.uint8, device=dev)
            v = buf[1:].view(t.shape)
            v.copy_(t)
            assert v.data_ptr() % 2 == 1
            ex[name] = v
        g = run_gpu_layer(w, x, dev, experts=ex)
        ref = harness.run_layer(w, x)
        err = assert_layer(w, g, ref)
        assert err.max() < 1e-4


def test_down_scale_plus_one_doubles_exactly(dev):
    for w in (TOY, TINY):
        say(f"down scales +1 doubles y exactly ({w.name})")
        x = w.x_bf16()
        ex = gdev.experts(w, 0, dev)
        y1 = run_gpu_layer(w, x, dev, experts=ex)["y"].clone()
        ex["down_s"] += 1
        y2 = run_gpu_layer(w, x, dev, experts=ex)["y"]
        assert torch.equal(y2, 2 * y1)


def test_repeat_runs_bit_identical(dev):
    for w in (TOY, TINY, SHAPES[4]):
        say(f"determinism {w.name}")
        x = w.x_bf16()
        ex = gdev.experts(w, 0, dev)
        a = run_gpu_layer(w, x, dev, experts=ex)
        b = run_gpu_layer(w, x, dev, experts=ex)
        assert torch.equal(a["y"], b["y"]) and np.array_equal(a["ids"], b["ids"])
        assert np.array_equal(a["gates"], b["gates"])


@pytest.mark.parametrize("d,E,k,T,xdt", [
    (7168, 896, 16, 9, "bf16"),    # last token count on the 4-token-group GEMV
    (7168, 896, 16, 10, "bf16"),   # first one on the in-lane-reduction kernel
    (7008, 896, 16, 33, "bf16"),   # last 512-row chunk ragged (352 rows), ragged token group
    (1024, 40, 8, 13, "bf16"),     # one column slab with 5 of 64 lanes in use
    (2080, 520, 16, 64, "f32"),    # last chunk 32 rows (one wave), second slab one lane wide
    (7168, 896, 16, 64, "f32"),
    # more than 64 tokens: the fp64 MFMA router (64 x 64 tiles, K split into chunks)
    (7168, 896, 16, 100, "bf16"),  # 8 K chunks of 896, second token tile 36 rows
    (7008, 896, 16, 300, "bf16"),  # 8 K chunks, the last 736 deep; last token tile 44 rows
    (2080, 520, 16, 130, "f32"),   # fp32 tokens, 5 K chunks of 416, last expert tile 8 wide
    (1024, 44, 8, 70, "bf16"),     # E % 8 != 0: router weights read element by element
    # the API's limits: 4096 experts (16 keys per top-k thread), 32 slots, d_model = 16384
    (512, 4096, 32, 1, "bf16"),    # one token: the 1024-thread logit block, then top-32
    (512, 4096, 32, 40, "bf16"),   # one logit block per token
    (1024, 4096, 32, 100, "bf16"), # fp64 MFMA router, 256-thread top-k with 16 keys each
    (512, 4095, 32, 3, "f32"),     # E % 8 != 0 at 16 keys per thread, last thread short
    (16384, 128, 8, 1, "bf16"),    # widest d_model: 32 K chunks of 512 rows
    (16384, 128, 8, 100, "f32"),   # widest d_model on the MFMA router
])
def test_router_multi_token_shapes(dev, d, E, k, T, xdt):
    say(f"router, several tokens: d={d} E={E} k={k} T={T} x={xdt}")
    from k3gen import host_normal_bf16, host_normal_f32
    key = d * 7919 + E * 31 + T
    xh = (host_normal_bf16(key, T * d, 0.0, 1.0) if xdt == "bf16"
          else host_normal_f32(key, T * d, 0.0, 1.0)).reshape(T, d)
    wh = host_normal_bf16(key + 1, d * E, 0.0, 0.02).reshape(d, E)
    dims = k3.make_dims(d, 256, E, k)
    x = gdev.bf16_tensor(xh, dev) if xdt == "bf16" else torch.from_numpy(xh).to(dev)
    ids, gates = k3.router(dims, x, gdev.bf16_tensor(wh, dev))
    torch.cuda.synchronize()
    ids_r, gates_r = oracle.route(oracle.router_logits(oracle.load_x(xh), wh, None), k)
    check_routing(ids.cpu().numpy(), gates.cpu().numpy(), ids_r, gates_r)


@pytest.mark.parametrize("T", [3, 100])
def test_fp32_activations(dev, T):
    # T = 100: the many-token fp64 MFMA router reading fp32 activations
    w = TOY.with_(T=T, name=f"toy_f32_t{T}")
    say(f"fp32 activations T={T}")
    x = w.resid0()
    g = run_gpu_layer(w, x, dev, x_dtype="f32")
    ref = harness.run_layer(w, x)
    assert_layer(w, g, ref)


def test_block_mode_small_chain(dev):
    w = TINY.with_(block=True, layers=3, T=2, name="tiny_block")
    say("block mode, 3 chained tiny blocks")
    h0 = w.resid0()
    ref = harness.run_stack(w, h0)
    h = torch.from_numpy(h0).to(dev)
    for layer in range(w.layers):
        g = run_gpu_layer(w, h.cpu().numpy(), dev, layer=layer, block=True, x_dtype="f32")
        assert np.array_equal(g["ids"], ref["ids"][layer]), f"routing differs at layer {layer}"
        h = g["y"]
    err = rel_l2(h.cpu().double().numpy(), ref["y"])
    print(f"    max rel L2 err {err.max():.3e}", flush=True)
    assert err.max() < 1e-4


@pytest.mark.parametrize("E,k", [(264, 4), (1032, 4), (4096, 32)])
def test_block_mode_wide_router_chain(dev, E, k):
    """Block mode with more than 256 experts at one token, where the shared expert's GEMVs
    ride in the router and top-k launches (E = 1032: five keys per top-k thread; E = 4096:
    sixteen, with 32 slots): three chained blocks against the oracle's stack, routed exactly
    as the oracle at every block."""
    w = Workload(f"block_e{E}", 23, d=512, f=256, E=E, k=k, T=1, layers=3, block=True)
    say(f"block mode, 3 chained blocks, E={E}, k={k}, T=1")
    h0 = w.resid0()
    ref = harness.run_stack(w, h0)
    h = torch.from_numpy(h0).to(dev)
    for layer in range(w.layers):
        g = run_gpu_layer(w, h.cpu().numpy(), dev, layer=layer, block=True, x_dtype="f32")
        assert np.array_equal(g["ids"], ref["ids"][layer]), f"routing differs at layer {layer}"
        h = g["y"]
    err = rel_l2(h.cpu().double().numpy(), ref["y"])
    print(f"    max rel L2 err {err.max():.3e}", flush=True)
    assert err.max() < 1e-4


def test_workspace_too_small_reports(dev):
    w = TOY
    dims = dims_of(w)
    small = torch.empty(64, dtype=torch.uint8, device=dev)
    with pytest.raises(k3.K3MoEError) as ei:
        k3.router(dims, gdev.x_bf16(w, device=dev), gdev.router_w(w, 0, dev), ws=small)
    assert ei.value.code == k3.EWORKSPACE


# ---- K3-shaped workloads ------------------------------------------------------------------
@pytest.fixture(scope="module")
def k3_decode_layer(dev):
    ex = gdev.experts(DECODE, 0, dev)
    yield ex
    del ex
    torch.cuda.empty_cache()


def test_decode_k3(dev, k3_decode_layer):
    w = DECODE
    say("decode: d=7168 f=1536 E=896 k=16 T=1")
    for ts in (0, 1):
        x = w.x_bf16(token_set=ts)
        g = run_gpu_layer(w, x, dev, experts=k3_decode_layer)
        ref = harness.run_layer(w, x)
        assert_layer(w, g, ref, tol=K3_TOL)
        g2 = run_gpu_layer(w, x, dev, experts=k3_decode_layer)
        assert torch.equal(g["y"], g2["y"])


def test_batched_k3(dev):
    """All 32 tokens of the batched-decode workload against the oracle (grouped GEMMs with
    16- and 32-row tiles at K3 widths)."""
    w = BATCHED
    say("batched decode: T=32, every token")
    x = w.x_bf16()
    ex = gdev.experts(w, 0, dev)
    g = run_gpu_layer(w, x, dev, experts=ex)
    ref = harness.run_layer(w, x)
    assert_layer(w, g, ref, tol=K3_TOL)
    del ex
    torch.cuda.empty_cache()


def test_prefill_k3(dev):
    w = PREFILL
    say("prefill: T=2048 with Zipf(1.1) logit bias")
    x = w.x_bf16()
    ex = gdev.experts(w, 0, dev)
    g = run_gpu_layer(w, x, dev, experts=ex)
    ids_all, gates_all, _, _ = oracle.layer_route(x, w.router_w(0), w.bias(0), w.k)
    check_routing(g["ids"], g["gates"], ids_all, gates_all)
    counts = np.bincount(ids_all.ravel(), minlength=w.E)
    print(f"    touched experts {int((counts > 0).sum())}, max load {counts.max()}", flush=True)
    rows = tile_probe_tokens(ids_all, w.E)
    assert len(rows) >= 32
    ref = harness.run_layer(w, x, tokens=rows)
    assert_layer(w, g, ref, rows=rows, tol=K3_TOL)
    del ex
    torch.cuda.empty_cache()


def test_prefill_k3_t8192(dev):
    """The largest chunk of the prefill sweep that the oracle routes in seconds: 8192 tokens,
    the hottest experts spread over a hundred and more 64-row tiles."""
    w = PREFILL.with_(T=8192, name="prefill_t8192")
    say("prefill: T=8192 with Zipf(1.1) logit bias")
    x = w.x_bf16()
    ex = gdev.experts(w, 0, dev)
    g = run_gpu_layer(w, x, dev, experts=ex)
    ids_all, gates_all, _, _ = oracle.layer_route(x, w.router_w(0), w.bias(0), w.k)
    check_routing(g["ids"], g["gates"], ids_all, gates_all)
    counts = np.bincount(ids_all.ravel(), minlength=w.E)
    print(f"    touched experts {int((counts > 0).sum())}, max load {counts.max()}", flush=True)
    assert counts.max() > 64 * 64  # some expert spans more than 64 full tiles
    rows = tile_probe_tokens(ids_all, w.E, seed=1)
    assert len(rows) >= 32
    ref = harness.run_layer(w, x, tokens=rows)
    assert_layer(w, g, ref, rows=rows, tol=K3_TOL)
    del ex
    torch.cuda.empty_cache()


def test_tokens_past_65536(dev):
    """70,000 tokens on a small layer (grouped GEMMs, fp64 MFMA router with 1094 token tiles):
    every routed id against the oracle, outputs at tile edges and at tokens 65535, 65536 and
    T-1, past the 65536 blocks the device reports for its second and third grid dimensions."""
    w = Workload("t70000", 35, d=256, f=128, E=16, k=2, T=70000)
    say(f"{w.T} tokens d={w.d} f={w.f} E={w.E} k={w.k}")
    x = w.x_bf16()
    g = run_gpu_layer(w, x, dev)
    ids_all, gates_all, _, _ = oracle.layer_route(x, w.router_w(0), w.bias(0), w.k)
    check_routing(g["ids"], g["gates"], ids_all, gates_all)
    rows = sorted(set(tile_probe_tokens(ids_all, w.E)) | {65535, 65536, w.T - 1})
    ref = harness.run_layer(w, x, tokens=rows)
    assert_layer(w, g, ref, rows=rows, tol=K3_TOL)


def test_stack8_k3(dev):
    w = STACK8
    say("8 stacked blocks, T=1, ~126 GB of MXFP4 experts resident")
    h0 = w.resid0()
    ref = harness.run_stack(w, h0)
    layers = [gdev.experts(w, l, dev) for l in range(w.layers)]
    h = h0
    for l in range(w.layers):
        g = run_gpu_layer(w, h, dev, layer=l, experts=layers[l], block=True, x_dtype="f32")
        assert np.array_equal(g["ids"], ref["ids"][l]), f"routing differs at layer {l}"
        h = g["y"].cpu().numpy()
    err = rel_l2(h.astype(np.float64), ref["y"])
    el = rel_elem(h.astype(np.float64), ref["y"])
    print(f"    max rel L2 err after 8 blocks {err.max():.3e}, max elem err / rms {el.max():.3e}",
          flush=True)
    assert err.max() <= K3_TOL
    assert el.max() <= ELEM_FACTOR * K3_TOL
    del layers
    torch.cuda.empty_cache()
