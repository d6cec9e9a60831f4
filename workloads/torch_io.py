"""Copy a seeded numpy layer (``workloads.make_layer``) to torch tensors.

Plumbing only: bf16 bit patterns become torch.bfloat16 tensors bit for bit."""
from __future__ import annotations

import numpy as np
import torch


def to_torch(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def layer_to_torch(L: dict, device) -> dict:
    out = {}
    for name in ("x", "gamma", "w_router", "router_bias", "w_gate", "w_up", "w_down", "a_gsp", "a_rcr"):
        v = L.get(name)
        out[name] = None if v is None else to_torch(v, device)
    return out


def from_torch(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy (bf16 returned as uint16 bit patterns)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
