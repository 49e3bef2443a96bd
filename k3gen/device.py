"""Device copies of a workload's inputs (input drawing only, no layer arithmetic).

Packed MXFP4 tensors are filled directly in HBM by the device generator; bf16
normals (router, shared expert, gamma, activations) are drawn on the host and
copied. Both sides draw from the same SplitMix64 streams, so the device tensors
equal what :mod:`k3gen.workloads` produces on the host.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import dev_fill_bytes, dev_fill_e8m0
from .workloads import EXPERT_TENSORS, Workload


def experts(w: Workload, layer: int, device="cuda") -> Dict[str, torch.Tensor]:
    """All E experts of one layer, uint8 [E][rows][cols] per tensor, on the device."""
    out = {}
    stream = torch.cuda.current_stream(device).cuda_stream
    for name in EXPERT_TENSORS:
        a, b = w.tensor_shape(name)
        t = torch.empty((w.E, a, b), dtype=torch.uint8, device=device)
        if name.endswith("_q"):
            dev_fill_bytes(w.seed, layer, w.tag(name), w.E, a * b, t.data_ptr(), stream)
        else:
            dev_fill_e8m0(w.seed, layer, w.tag(name), w.E, a * b, w.scale_lo, w.scale_count,
                          t.data_ptr(), stream)
        out[name] = t
    return out


def bf16_tensor(a: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bits on the host -> torch.bfloat16 on the device."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def router_w(w: Workload, layer: int, device="cuda") -> torch.Tensor:
    return bf16_tensor(w.router_w(layer), device)


def bias(w: Workload, layer: int, device="cuda") -> Optional[torch.Tensor]:
    b = w.bias(layer)
    return None if b is None else torch.from_numpy(b).to(device)


def x_bf16(w: Workload, token_set: int = 0, T: Optional[int] = None, device="cuda"):
    return bf16_tensor(w.x_bf16(token_set, T), device)


def block_extras(w: Workload, layer: int, device="cuda") -> Dict[str, torch.Tensor]:
    sh = w.shared(layer)
    return {"rms_gamma": bf16_tensor(w.gamma(layer), device),
            "sh_gate": bf16_tensor(sh["sh_gate"], device),
            "sh_up": bf16_tensor(sh["sh_up"], device),
            "sh_down": bf16_tensor(sh["sh_down"], device)}
