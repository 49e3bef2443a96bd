"""The tuned CPU comparator (cpu_tuned/) against the oracle: same ids, same gates and the
same fp64 output, bit for bit, on the toy layer, ragged small layers and K3-width experts
(its vector lanes run across independent outputs, never along a sum). No GPU."""
import numpy as np
import pytest

import cpu_tuned
import oracle
from k3gen.workloads import TOY, Workload


def _check(w: Workload, token_sets=(0,)):
    wr = w.router_w(0)
    bias = w.bias(0)
    for ts in token_sets:
        x = w.x_bf16(token_set=ts)
        ids, _, _, _ = oracle.layer_route(x, wr, bias, w.k)
        experts = {int(e): w.expert_host(0, int(e)) for e in np.unique(ids)}
        y_o, ids_o, g_o = oracle.layer_forward(x, wr, bias, experts, w.d, w.f, w.E, w.k)
        y_c, ids_c, g_c = cpu_tuned.layer_forward(x, wr, bias, experts, w.d, w.f, w.E, w.k)
        assert np.array_equal(ids_c, ids_o)
        assert np.array_equal(g_c, g_o)
        ids_r, g_r = cpu_tuned.layer_route(x, wr, bias, w.k)
        assert np.array_equal(ids_r, ids_o) and np.array_equal(g_r, g_o)
        assert np.array_equal(y_c, y_o), f"{w.name} set {ts}: max diff {np.abs(y_c - y_o).max()}"


@pytest.mark.parametrize("w", [
    TOY,
    TOY.with_(T=3, name="toy_t3"),
    Workload("ragged_e", 41, d=96, f=64, E=13, k=3, T=2),            # E not a multiple of 4
    Workload("zipf_bias", 42, d=512, f=256, E=40, k=8, T=2, zipf_alpha=1.1),  # router bias
    Workload("k3_widths", 43, d=7168, f=1536, E=18, k=2, T=1),
])
def test_tuned_cpu_equals_oracle_bit_for_bit(w):
    _check(w, token_sets=(0, 1))


def test_reports_simd():
    assert cpu_tuned.simd() in (True, False)
