"""Run the fp64 oracle on a synthetic workload (TEST INFRASTRUCTURE ONLY).

Draws the inputs of a :class:`k3gen.workloads.Workload` with the seeded
generator, routes with the oracle, regenerates only the experts the oracle
selected, and runs the oracle layer. The arithmetic is all in ``k3oracle.c``.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

import oracle
from k3gen.workloads import Workload

RMS_EPS = 1e-6


def block_params(w: Workload, layer: int) -> Optional[dict]:
    if not w.block:
        return None
    p = {"gamma": w.gamma(layer), "eps": RMS_EPS}
    p.update(w.shared(layer))
    return p


def run_layer(w: Workload, x: np.ndarray, layer: int = 0,
              tokens: Optional[Sequence[int]] = None,
              expert_override: Optional[Dict[int, dict]] = None) -> dict:
    """Oracle output of one layer on x ([T][d] bf16 bits as uint16, or fp32).

    ``tokens`` restricts the run to a subset of rows (sampled parity).
    ``expert_override`` replaces the generated tensors of some experts.
    Returns y ([T'][d] fp64), ids, gates, logits."""
    if tokens is not None:
        x = np.ascontiguousarray(x[np.asarray(tokens)])
    wr = w.router_w(layer)
    bias = w.bias(layer)
    blk = block_params(w, layer)
    ids, gates, logits, _ = oracle.layer_route(x, wr, bias, w.k, blk)
    experts = {}
    for e in np.unique(ids):
        e = int(e)
        if expert_override and e in expert_override:
            experts[e] = expert_override[e]
        else:
            experts[e] = w.expert_host(layer, e)
    y, ids2, gates2 = oracle.layer_forward(x, wr, bias, experts, w.d, w.f, w.E, w.k, blk)
    assert np.array_equal(ids, ids2)
    return {"y": y, "ids": ids, "gates": gates, "logits": logits}


def run_stack(w: Workload, h0: np.ndarray, layers: Optional[int] = None) -> dict:
    """Chain ``layers`` blocks of a block-mode workload starting from residual h0 (fp32).

    Each block's output feeds the next one in fp64; returns the final residual
    and the per-layer routing."""
    L = w.layers if layers is None else layers
    h = np.ascontiguousarray(h0, dtype=np.float64)
    ids_all, gates_all = [], []
    for layer in range(L):
        r = run_layer(w, h, layer)
        h = r["y"]
        ids_all.append(r["ids"])
        gates_all.append(r["gates"])
    return {"y": h, "ids": ids_all, "gates": gates_all}
