"""Pins of the fp64 oracle against things other than itself.

Each test ties an oracle function to a fixture from a specification or the
pages, a closed form, an invariant, a special case that reduces to a library
routine, or brute force on tiny inputs. The mutation tests
(test_oracle_mutants.py) rerun this file against deliberately broken oracle
builds and require a failure for each planted mistake.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import k3gen
import oracle
from k3gen.workloads import DECODE, TINY, TOY, Workload
from oracle import harness

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1_FIX = json.load(open(os.path.join(GOLDEN, "e2m1_ocp_mx.json")))
FACTS = json.load(open(os.path.join(GOLDEN, "format_facts.json")))
E2M1_TABLE = np.array([E2M1_FIX["values"][str(c)] for c in range(16)], dtype=np.float64)


# ---- independent reference pieces (fixture table + library routines) ----------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def np_decode(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Dense fp64 matrix from packed rows, via the OCP fixture table."""
    codes = np.stack([q & 15, q >> 4], axis=-1).reshape(q.shape[0], -1)
    vals = E2M1_TABLE[codes]
    scale = np.where(s == 255, np.nan, np.ldexp(1.0, s.astype(np.int64) - 127))
    return vals * np.repeat(scale, 32, axis=1)


def np_silu(z):
    return z / (1.0 + np.exp(-z))


def np_expert(x, ex):
    G = np_decode(ex["gate_q"], ex["gate_s"])
    U = np_decode(ex["up_q"], ex["up_s"])
    D = np_decode(ex["down_q"], ex["down_s"])
    return D @ (np_silu(G @ x) * (U @ x))


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---- P1: element decoding ------------------------------------------------------------------
def test_e2m1_matches_ocp_fixture_exhaustively():
    for c in range(16):
        v = oracle.e2m1(c)
        ref = E2M1_FIX["values"][str(c)]
        assert v == ref and math.copysign(1, v) == math.copysign(1, ref), c


def test_e8m0_all_codes():
    for s in range(255):
        assert oracle.e8m0(s) == 2.0 ** (s - E2M1_FIX["e8m0"]["bias"]), s
    assert math.isnan(oracle.e8m0(E2M1_FIX["e8m0"]["nan_code"]))


def test_workload_values_exact_in_bf16():
    for s in range(120, 129):
        for c in range(16):
            v = oracle.e2m1(c) * oracle.e8m0(s)
            assert oracle.bf16(k3gen.f64_to_bf16(v)) == v


# ---- P2: packing, block direction, byte counts ------------------------------------------------
def test_nibble_order_low_first():
    q = np.array([0x21, 0xF7], dtype=np.uint8)
    assert [oracle.nibble(q, k) for k in range(4)] == [1, 2, 7, 15]
    w = oracle.mx_row(np.concatenate([q, np.zeros(14, np.uint8)]), np.array([127], np.uint8), 32)
    assert w[:4].tolist() == [0.5, 1.0, 6.0, -6.0]


def test_every_byte_roundtrips():
    q = np.arange(256, dtype=np.uint8)
    for b in range(256):
        assert oracle.nibble(q, 2 * b) == b & 15
        assert oracle.nibble(q, 2 * b + 1) == b >> 4


def test_scale_blocks_run_along_k():
    K = 96
    q = np.full(K // 2, 0x22, dtype=np.uint8)  # every element code 2 = 1.0
    s = np.array([127, 128, 125], dtype=np.uint8)
    for k, want in [(0, 1.0), (31, 1.0), (32, 2.0), (63, 2.0), (64, 0.25), (95, 0.25)]:
        x = np.zeros(K)
        x[k] = 1.0
        assert oracle.mx_dot(q, s, x) == want, k


def test_bytes_per_weight_closed_form():
    for K in (32, 64, 1536, 7168):
        assert (K / 2 + K / 32) / K == FACTS["bytes_per_weight"]["value"]
    w = TOY
    for name, (r, c) in [("gate_q", (w.f, w.d // 2)), ("down_s", (w.d, w.f // 32))]:
        assert w.tensor_shape(name) == (r, c)


def test_k3_expert_size_matches_pages_store():
    d, f = FACTS["layer_shape"]["d_model"], FACTS["layer_shape"]["d_ff"]
    assert (DECODE.d, DECODE.f) == (d, f)
    assert DECODE.expert_bytes == 3 * d * f * 17 // 32 == 17_547_264
    assert 16 * DECODE.expert_bytes == 280_756_224
    st = FACTS["routed_store"]
    assert st["moe_layers"] * st["experts_per_layer"] == st["experts"]
    total_tb = st["experts"] * DECODE.expert_bytes / 1e12
    assert abs(total_tb - st["terabytes"]) / st["terabytes"] < 5e-4
    assert FACTS["routing"]["experts"] == DECODE.E and FACTS["routing"]["top_k"] == DECODE.k


# ---- P3: router ---------------------------------------------------------------------------------
def test_router_integer_inputs_exact():
    rng = np.random.default_rng(1)
    T, d, E = 3, 40, 7  # d != E: a transposed read gives wrong values
    x = rng.integers(-8, 9, (T, d)).astype(np.float64)
    wi = rng.integers(-16, 17, (d, E))
    w = np.array([[k3gen.f64_to_bf16(float(v)) for v in row] for row in wi], dtype=np.uint16)
    bias = rng.integers(-3, 4, E).astype(np.float32)
    got = oracle.router_logits(x, w, bias)
    want = x.astype(np.int64) @ wi + bias.astype(np.int64)
    assert np.array_equal(got, want.astype(np.float64))


def test_router_random_vs_exact_sum():
    w = TINY
    x = oracle.load_x(w.x_bf16())
    wr = w.router_w()
    got = oracle.router_logits(x, wr, None)
    W = bf16_to_f64(wr)
    for t in range(w.T):
        for e in range(w.E):
            exact = math.fsum(x[t, k] * W[k, e] for k in range(w.d))
            bound = w.d * 2.0 ** -53 * np.sum(np.abs(x[t] * W[:, e]))
            assert abs(got[t, e] - exact) <= bound


# ---- P4: softmax and top-k ------------------------------------------------------------------------
def test_softmax_vs_library_and_sum():
    rng = np.random.default_rng(2)
    for scale in (1.0, 30.0, 1000.0):
        l = rng.standard_normal(896) * scale
        p = oracle.softmax(l)
        assert abs(p.sum() - 1.0) < 1e-14
        assert np.max(np.abs(p - sp_softmax(l))) < 1e-15 + 1e-13 * np.max(p)


def _brute_topk(l, k):
    order = sorted(range(len(l)), key=lambda e: (math.isnan(l[e]), -l[e] if not math.isnan(l[e]) else 0, e))
    return order[:k]


@pytest.mark.parametrize("kind", ["random", "ties", "allequal", "nan", "signed_zero"])
def test_topk_brute_force(kind):
    rng = np.random.default_rng(3)
    for trial in range(20):
        E = int(rng.integers(2, 60))
        k = int(rng.integers(1, E + 1))
        if kind == "random":
            l = rng.standard_normal(E)
        elif kind == "ties":
            l = rng.integers(-2, 3, E).astype(np.float64)
        elif kind == "allequal":
            l = np.full(E, 0.25)
        elif kind == "nan":
            l = rng.standard_normal(E)
            l[rng.integers(0, E, 3)] = np.nan
        else:
            l = np.where(rng.random(E) < 0.5, 0.0, -0.0)
        assert oracle.topk(l, k).tolist() == _brute_topk(l.tolist(), k), (kind, trial)


def test_zero_input_routes_to_first_k_uniform():
    w = TINY
    x = np.zeros((1, w.d), dtype=np.float32)
    ids, gates, _, _ = oracle.layer_route(x, w.router_w(), None, w.k)
    assert ids.tolist() == [list(range(w.k))]
    assert np.all(gates == 1.0 / w.E)


def test_k_equals_e_takes_all_and_gates_sum_to_one():
    w = TINY
    x = w.x_bf16()
    ids, gates, logits, _ = oracle.layer_route(x, w.router_w(), None, w.E)
    for t in range(w.T):
        assert sorted(ids[t].tolist()) == list(range(w.E))
        assert abs(gates[t].sum() - 1.0) < 1e-14
        assert np.all(np.diff(logits[t][ids[t]]) <= 0)


def test_doubling_router_keeps_order():
    w = TOY
    x = w.x_bf16(T=8)
    wr = w.router_w()
    w2 = np.array([k3gen.f64_to_bf16(2 * v) for v in bf16_to_f64(wr).ravel()],
                  dtype=np.uint16).reshape(wr.shape)
    ids1, _, l1, _ = oracle.layer_route(x, wr, None, w.k)
    ids2, _, l2, _ = oracle.layer_route(x, w2, None, w.k)
    assert np.array_equal(ids1, ids2)
    assert np.array_equal(l2, 2 * l1)


def test_permuting_experts_permutes_ids():
    w = TOY
    x = w.x_bf16(T=8)
    wr = w.router_w()
    perm = np.random.default_rng(4).permutation(w.E)  # new column j = old column perm[j]
    ids1, g1, _, _ = oracle.layer_route(x, wr, None, w.k)
    ids2, g2, _, _ = oracle.layer_route(x, np.ascontiguousarray(wr[:, perm]), None, w.k)
    assert np.array_equal(perm[ids2], ids1)
    # the softmax denominator is summed in a different order: equal up to rounding
    assert np.allclose(g1, g2, rtol=1e-14, atol=0)


def test_bucket_vs_stable_sort():
    rng = np.random.default_rng(5)
    for T, E, k in [(1, 8, 2), (37, 16, 4), (64, 896, 16), (5, 3, 3)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        off, rows = oracle.bucket(ids, E)
        pairs = sorted(range(T * k), key=lambda p: (ids.ravel()[p], p))
        assert rows.tolist() == pairs
        assert off.tolist() == [int(np.sum(ids < e)) for e in range(E + 1)]


# ---- P5: experts ----------------------------------------------------------------------------------
def test_single_expert_is_dense_swiglu():
    w = TINY.with_(E=1, k=1)
    x = w.x_bf16()
    ex = w.expert_host(0, 0)
    y, ids, gates = oracle.layer_forward(x, w.router_w(), None, {0: ex}, w.d, w.f, 1, 1)
    assert np.all(ids == 0) and np.all(gates == 1.0)
    xf = bf16_to_f64(x)
    for t in range(w.T):
        assert rel(y[t], np_expert(xf[t], ex)) < 1e-13


def test_tiny_layer_brute_force():
    w = TINY
    x = w.x_bf16()
    wr = w.router_w()
    experts = {e: w.expert_host(0, e) for e in range(w.E)}
    y, ids, gates = oracle.layer_forward(x, wr, None, experts, w.d, w.f, w.E, w.k)
    xf = bf16_to_f64(x)
    L = xf @ bf16_to_f64(wr)
    P = sp_softmax(L, axis=1)
    for t in range(w.T):
        want_ids = np.argsort(-L[t], kind="stable")[: w.k]
        assert ids[t].tolist() == want_ids.tolist()
        assert np.allclose(gates[t], P[t][want_ids], rtol=1e-14, atol=0)
        want = sum(P[t][e] * np_expert(xf[t], experts[e]) for e in want_ids)
        assert rel(y[t], want) < 1e-13


def test_toy_layer_vs_dense_numpy():
    w = TOY.with_(T=2)
    x = w.x_bf16()
    r = harness.run_layer(w, x)
    xf = bf16_to_f64(x)
    for t in range(w.T):
        want = sum(g * np_expert(xf[t], w.expert_host(0, int(e)))
                   for e, g in zip(r["ids"][t], r["gates"][t]))
        assert rel(r["y"][t], want) < 1e-13


def test_silu_saturates_without_nan():
    d, f = 64, 32
    ex = {"gate_q": np.full((f, d // 2), 0xFF, np.uint8), "gate_s": np.full((f, d // 32), 140, np.uint8),
          "up_q": np.full((f, d // 2), 0x77, np.uint8), "up_s": np.full((f, d // 32), 127, np.uint8),
          "down_q": np.full((d, f // 2), 0x22, np.uint8), "down_s": np.full((d, f // 32), 127, np.uint8)}
    x = np.full(d, 100.0)
    h, out = oracle.expert_ffn(x, ex, d, f)
    assert np.all(np.isfinite(h)) and np.all(h == 0.0) and np.all(out == 0.0)
    h2, out2 = oracle.expert_ffn(-x, ex, d, f)  # u -> +huge: silu(u) = u exactly
    u = d * (-6.0 * 2.0 ** 13) * -100.0
    v = d * 6.0 * -100.0
    assert np.all(np.isfinite(out2)) and np.all(h2 == u * v)


def test_nan_scale_propagates():
    w = TINY
    x = oracle.load_x(w.x_bf16()[0])
    ex = w.expert_host(0, 0)
    ex["down_s"] = ex["down_s"].copy()
    ex["down_s"][3, 0] = 255
    _, out = oracle.expert_ffn(x, ex, w.d, w.f)
    assert np.isnan(out[3]) and np.all(np.isfinite(np.delete(out, 3)))


# ---- P6, P7, P9: block scaling, linearity, batch invariance ---------------------------------------
def test_block_scaled_accumulation_equals_elementwise():
    rng = np.random.default_rng(6)
    K = 7168
    for _ in range(5):
        q = rng.integers(0, 256, K // 2).astype(np.uint8)
        s = rng.integers(100, 151, K // 32).astype(np.uint8)
        xb = np.array([k3gen.f64_to_bf16(v) for v in rng.standard_normal(K)], dtype=np.uint16)
        x = bf16_to_f64(xb)
        a = oracle.mx_dot(q, s, x)
        b = oracle.mx_dot(q, s, x, blockscaled=True)
        wx = np.abs(np_decode(q[None, :], s[None, :])[0] * x).sum()
        assert abs(a - b) <= 2 * K * 2.0 ** -53 * wx  # two summation orders, each within K*u
        # power-of-two scaling commutes with each block's sum: one block is bit-exact
        assert oracle.mx_dot(q[:16], s[:1], x[:32]) == oracle.mx_dot(q[:16], s[:1], x[:32], True)


def test_down_scale_plus_one_doubles_output_exactly():
    w = TOY
    x = w.x_bf16()
    r0 = harness.run_layer(w, x)
    over = {}
    for e in np.unique(r0["ids"]):
        ex = w.expert_host(0, int(e))
        ex["down_s"] = (ex["down_s"] + 1).astype(np.uint8)
        over[int(e)] = ex
    r1 = harness.run_layer(w, x, expert_override=over)
    assert np.array_equal(r1["y"], 2.0 * r0["y"])


def test_batch_invariance_bitwise():
    w = TOY.with_(T=5)
    x = w.x_bf16()
    full = harness.run_layer(w, x)
    for t in range(w.T):
        one = harness.run_layer(w, x, tokens=[t])
        assert np.array_equal(one["y"][0], full["y"][t])
        assert np.array_equal(one["ids"][0], full["ids"][t])


# ---- block extras ------------------------------------------------------------------------------
def test_rmsnorm_closed_form():
    d = 48
    gamma = np.array([k3gen.f64_to_bf16(1.0 + 0.01 * i) for i in range(d)], dtype=np.uint16)
    for c, eps in [(3.0, 1e-6), (-0.5, 1e-6), (2.0, 0.0)]:
        out = oracle.rmsnorm(np.full(d, c), gamma, eps)
        want = c / math.sqrt(c * c + eps) * bf16_to_f64(gamma)
        assert np.allclose(out, want, rtol=1e-15, atol=0)


def test_rmsnorm_scale_invariant_without_eps():
    rng = np.random.default_rng(7)
    h = rng.standard_normal(100)
    g = np.full(100, 0x3F80, np.uint16)
    a = oracle.rmsnorm(h, g, 0.0)
    b = oracle.rmsnorm(h * 1024.0, g, 0.0)
    assert np.array_equal(a, b)
    assert abs(np.mean(a * a) - 1.0) < 1e-14


def test_dense_swiglu_vs_numpy():
    w = TINY.with_(block=True)
    sh = w.shared(0)
    x = oracle.load_x(w.x_bf16()[0])
    got = oracle.dense_swiglu(x, sh["sh_gate"], sh["sh_up"], sh["sh_down"])
    G, U, D = (bf16_to_f64(sh[n]) for n in ("sh_gate", "sh_up", "sh_down"))
    assert rel(got, D @ (np_silu(G @ x) * (U @ x))) < 1e-13


def test_block_layer_composition():
    w = TINY.with_(block=True, T=2)
    h = w.resid0()
    blk = harness.block_params(w, 0)
    experts = {e: w.expert_host(0, e) for e in range(w.E)}
    out, ids, gates = oracle.layer_forward(h, w.router_w(), None, experts, w.d, w.f, w.E, w.k,
                                           blk)
    hf = h.astype(np.float64)
    for t in range(w.T):
        xh = hf[t] / math.sqrt(np.mean(hf[t] ** 2) + blk["eps"]) * bf16_to_f64(blk["gamma"])
        L = xh @ bf16_to_f64(w.router_w())
        P = sp_softmax(L)
        sel = np.argsort(-L, kind="stable")[: w.k]
        assert ids[t].tolist() == sel.tolist()
        y = sum(P[e] * np_expert(xh, experts[e]) for e in sel)
        G, U, D = (bf16_to_f64(blk[n]) for n in ("sh_gate", "sh_up", "sh_down"))
        s = D @ (np_silu(G @ xh) * (U @ xh))
        assert rel(out[t], hf[t] + s + y) < 1e-12


def test_stack_chains_layers():
    w = TINY.with_(block=True, layers=3, T=1)
    h0 = w.resid0()
    r = harness.run_stack(w, h0)
    h = h0.astype(np.float64)
    for layer in range(3):
        h = harness.run_layer(w, h, layer)["y"]
    assert np.array_equal(r["y"], h)
