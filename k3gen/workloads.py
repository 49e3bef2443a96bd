"""Synthetic workloads: shapes, value distributions and stream keys.

Nothing here computes any part of the MoE layer; it only says which numbers
go in. The named workloads are:

  toy      d=512,  f=256,  E=32,  k=4,  T=1
  decode   d=7168, f=1536, E=896, k=16, T=1
  batched  same layer, T=32 independent tokens
  prefill  same layer, T=2048, Zipf(1.1) logit bias
  batched_zipf  same layer, T=32, Zipf(1.1) logit bias (a hot set of experts that every
           step routes to again; about 165 distinct experts per step)
  stack8   8 blocks (RMSNorm -> routed MoE + bf16 shared SwiGLU -> residual), T=1

Value distributions (all workloads): x ~ bf16(N(0,1)); router weight
~ bf16(N(0, 0.02)) (standard deviation 0.02); MXFP4 nibbles uniform over the
16 E2M1 codes; E8M0 scale bytes uniform in [120, 128]. stack8 adds
gamma ~ bf16(1 + 0.1 N(0,1)), shared-expert weights ~ bf16(N(0,1)) and an fp32
N(0,1) residual entering the first block.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from . import (MASTER_SEED, T_DOWN_Q, T_DOWN_S, T_GAMMA, T_GATE_Q, T_GATE_S, T_RESID,
               T_SH_DOWN, T_SH_GATE, T_SH_UP, T_UP_Q, T_UP_S, T_WROUTER, T_X, T_ZIPF, at,
               host_bytes, host_e8m0, host_normal_bf16, host_normal_f32, key, zipf_bias)

EXPERT_TENSORS = ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")
_TAGS = {"gate_q": T_GATE_Q, "gate_s": T_GATE_S, "up_q": T_UP_Q, "up_s": T_UP_S,
         "down_q": T_DOWN_Q, "down_s": T_DOWN_S}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    d: int
    f: int
    E: int
    k: int
    T: int
    zipf_alpha: Optional[float] = None
    layers: int = 1
    block: bool = False
    scale_lo: int = 120
    scale_count: int = 9
    router_sd: float = 0.02
    x_sd: float = 1.0

    # ---- derived sizes -------------------------------------------------
    def tensor_shape(self, name: str):
        d, f = self.d, self.f
        return {"gate_q": (f, d // 2), "gate_s": (f, d // 32), "up_q": (f, d // 2),
                "up_s": (f, d // 32), "down_q": (d, f // 2), "down_s": (d, f // 32)}[name]

    def per_expert(self, name: str) -> int:
        a, b = self.tensor_shape(name)
        return a * b

    @property
    def expert_bytes(self) -> int:
        return sum(self.per_expert(n) for n in EXPERT_TENSORS)

    # ---- keys ------------------------------------------------------------
    @property
    def seed(self) -> int:
        return at(MASTER_SEED, self.cfg_id)

    def key(self, layer: int, tag: int, c: int = 0) -> int:
        return key(self.seed, layer, tag, c)

    def tag(self, name: str) -> int:
        return _TAGS[name]

    # ---- host draws ------------------------------------------------------
    def x_bf16(self, token_set: int = 0, T: Optional[int] = None) -> np.ndarray:
        T = self.T if T is None else T
        return host_normal_bf16(self.key(0, T_X, token_set), T * self.d, 0.0,
                                self.x_sd).reshape(T, self.d)

    def router_w(self, layer: int = 0) -> np.ndarray:
        return host_normal_bf16(self.key(layer, T_WROUTER), self.d * self.E, 0.0,
                                self.router_sd).reshape(self.d, self.E)

    def bias(self, layer: int = 0) -> Optional[np.ndarray]:
        if self.zipf_alpha is None:
            return None
        return zipf_bias(self.key(layer, T_ZIPF), self.E, self.zipf_alpha)[1]

    def expert_tensor(self, layer: int, e: int, name: str) -> np.ndarray:
        k = self.key(layer, _TAGS[name], e)
        n = self.per_expert(name)
        if name.endswith("_q"):
            a = host_bytes(k, n)
        else:
            a = host_e8m0(k, n, self.scale_lo, self.scale_count)
        return a.reshape(self.tensor_shape(name))

    def expert_host(self, layer: int, e: int) -> dict:
        return {n: self.expert_tensor(layer, e, n) for n in EXPERT_TENSORS}

    def gamma(self, layer: int) -> np.ndarray:
        return host_normal_bf16(self.key(layer, T_GAMMA), self.d, 1.0, 0.1)

    def shared(self, layer: int) -> dict:
        d, f = self.d, self.f
        return {
            "sh_gate": host_normal_bf16(self.key(layer, T_SH_GATE), f * d, 0.0, 1.0).reshape(f, d),
            "sh_up": host_normal_bf16(self.key(layer, T_SH_UP), f * d, 0.0, 1.0).reshape(f, d),
            "sh_down": host_normal_bf16(self.key(layer, T_SH_DOWN), d * f, 0.0, 1.0).reshape(d, f),
        }

    def resid0(self, token_set: int = 0, T: Optional[int] = None) -> np.ndarray:
        T = self.T if T is None else T
        return host_normal_f32(self.key(0, T_RESID, token_set), T * self.d, 0.0,
                               1.0).reshape(T, self.d)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


TOY = Workload("toy", 1, d=512, f=256, E=32, k=4, T=1)
DECODE = Workload("decode", 2, d=7168, f=1536, E=896, k=16, T=1)
BATCHED = Workload("batched", 3, d=7168, f=1536, E=896, k=16, T=32)
PREFILL = Workload("prefill", 4, d=7168, f=1536, E=896, k=16, T=2048, zipf_alpha=1.1)
STACK8 = Workload("stack8", 5, d=7168, f=1536, E=896, k=16, T=1, layers=8, block=True)
TINY = Workload("tiny", 6, d=64, f=32, E=8, k=2, T=3)
BATCHED_ZIPF = Workload("batched_zipf", 7, d=7168, f=1536, E=896, k=16, T=32, zipf_alpha=1.1)

WORKLOADS = {w.name: w for w in (TOY, DECODE, BATCHED, PREFILL, STACK8, TINY, BATCHED_ZIPF)}
