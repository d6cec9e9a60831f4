"""Seeded synthetic layers drawn on the device with torch's generator.

For the layers whose host draw would take minutes (the GLM-4.5-Air-shaped
layer: 4.4 GB of bf16 expert weights; the 48-layer stack: 58 GB).  Same
recipe as ``make_layer``: x ~ N(0,1), gamma ~ U(0.5,1.5), router and expert
weights ~ N(0, std), the Zipf router prior b_e = -s*ln(r_e) over a seeded
permutation r of 1..E, and lognormal(0, sigma) tables; bf16 tensors are the
float32 draws rounded to nearest-even.  Only the random stream differs: each
tensor has its own ``torch.Generator(device)`` seeded from
``SeedSequence([seed, cfg_id, layer, tensor_id, step])``.

Like the rest of this package it draws numbers only (no layer arithmetic).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import (A_GSP, A_RCR, GAMMA, ROUTER_BIAS, W_DOWN, W_GATE, W_ROUTER, W_UP, X, LayerShape)


def _gen(device, seed: int, cfg_id: int, layer: int, tensor_id: int, step: int = 0) -> torch.Generator:
    s = np.random.SeedSequence([int(seed), int(cfg_id), int(layer), int(tensor_id), int(step)])
    g = torch.Generator(device=device)
    g.manual_seed(int(s.generate_state(1, dtype=np.uint64)[0] >> np.uint64(1)))
    return g


def _dtype(S: LayerShape):
    return torch.bfloat16 if S.dtype == "bf16" else torch.float32


def _normal(shape, std, g, device, out_dtype):
    """N(0, std) float32 draw, stored in out_dtype (rounded to nearest-even for bf16)."""
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t if out_dtype == torch.float32 else t.to(out_dtype)


def make_tokens_device(S: LayerShape, device, seed: int = 0, layer: int = 0, step: int = 0, T: int | None = None):
    T = S.T if T is None else T
    return _normal((T, S.H), 1.0, _gen(device, seed, S.cfg_id, layer, X, step), device, _dtype(S))


def make_layer_device(S: LayerShape, device, seed: int = 0, layer: int = 0, with_x: bool = True) -> dict:
    """Parameters of one layer (and its input batch x) as device tensors, in
    the layouts of ``make_layer``."""
    dt = _dtype(S)
    d = {"shape": S, "seed": seed, "layer": layer}
    d["x"] = make_tokens_device(S, device, seed, layer) if with_x else None
    g = _gen(device, seed, S.cfg_id, layer, GAMMA)
    d["gamma"] = torch.rand(S.H, generator=g, device=device, dtype=torch.float32).add_(0.5)
    d["w_router"] = _normal((S.E, S.H), S.router_std, _gen(device, seed, S.cfg_id, layer, W_ROUTER), device,
                            torch.float32)
    if S.zipf_s > 0:
        g = _gen(device, seed, S.cfg_id, layer, ROUTER_BIAS)
        r = (torch.randperm(S.E, generator=g, device=device) + 1).cpu().tolist()
        d["router_bias"] = torch.tensor([-S.zipf_s * math.log(float(v)) for v in r], dtype=torch.float32,
                                        device=device)
    else:
        d["router_bias"] = None
    for name, tid, shape in (("w_gate", W_GATE, (S.E, S.I, S.H)), ("w_up", W_UP, (S.E, S.I, S.H)),
                             ("w_down", W_DOWN, (S.E, S.H, S.I))):
        d[name] = _normal(shape, S.expert_std, _gen(device, seed, S.cfg_id, layer, tid), device, dt)
    for name, tid in (("a_gsp", A_GSP), ("a_rcr", A_RCR)):
        g = _gen(device, seed, S.cfg_id, layer, tid)
        d[name] = torch.randn(S.E, generator=g, device=device, dtype=torch.float32).mul_(S.table_sigma).exp_()
    return d


def to_host(d: dict) -> dict:
    """The same layer as numpy arrays (bf16 as uint16 bit patterns), the form
    ``make_layer`` returns."""
    from .torch_io import from_torch
    out = {}
    for k, v in d.items():
        out[k] = from_torch(v) if isinstance(v, torch.Tensor) else v
    return out
