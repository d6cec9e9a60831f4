"""Seeded synthetic inputs for the routed SwiGLU MoE layer.

This module only draws and stores numbers: it holds none of the layer's
arithmetic (no normalisation, routing, skipping or expert math).  Both the
CPU oracle's tests and the GPU path's tests/bench take their inputs from here.

Every tensor gets its own generator, ``np.random.default_rng(SeedSequence(
[seed, cfg_id, layer, tensor_id]))``, so any tensor can be regenerated alone.
Tensors of the activation dtype are stored as their storage bits:
float32 arrays for ``"f32"`` and uint16 bf16 bit patterns for ``"bf16"``.
bf16 values are made by rounding the float32 draw to nearest-even.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# tensor ids for the per-tensor seed streams
X, GAMMA, W_ROUTER, ROUTER_BIAS, W_GATE, W_UP, W_DOWN, A_GSP, A_RCR, CALIB_X = range(10)


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Shape and distribution recipe of one MoE layer workload."""

    name: str
    cfg_id: int
    T: int  # tokens in the batch
    H: int  # hidden size
    E: int  # routed experts
    I: int  # expert intermediate size
    k: int  # experts per token (top-k)
    dtype: str  # "f32" or "bf16": activations and expert weights
    router_std: float = 0.02
    expert_std: float = 0.02
    table_sigma: float = 0.5  # lognormal(0, sigma) for the two per-expert tables
    zipf_s: float = 0.0  # >0: router bias b_e = -s*ln(r_e), r a seeded permutation of 1..E
    norm_topk: int = 1
    rms_eps: float = 1e-6
    skip_rates: tuple = (0.5,)

    def with_tokens(self, T: int) -> "LayerShape":
        return dataclasses.replace(self, T=int(T))


CONFIGS = {
    # tiny fp32 layer
    "tiny": LayerShape("tiny", 1, T=64, H=256, E=16, I=128, k=4, dtype="f32",
                       router_std=0.05, expert_std=0.02, table_sigma=0.5, skip_rates=(0.5,)),
    # Qwen3-30B-A3B-shaped layer (hidden 2048, 128 experts, top-8, inter 768), prefill T=1024
    "qwen3_30b_a3b": LayerShape("qwen3_30b_a3b", 2, T=1024, H=2048, E=128, I=768, k=8, dtype="bf16",
                                skip_rates=(0.0, 0.5, 0.6)),
    # same layer in decode: M tokens per step
    "qwen3_30b_a3b_decode": LayerShape("qwen3_30b_a3b_decode", 3, T=8, H=2048, E=128, I=768, k=8,
                                       dtype="bf16", skip_rates=(0.6,)),
    # larger layer (hidden 4096, inter 1408), T=4096, Zipf(1.1) router prior
    "glm45_air_shape": LayerShape("glm45_air_shape", 4, T=4096, H=4096, E=128, I=1408, k=8, dtype="bf16",
                                  table_sigma=0.7, zipf_s=1.1, skip_rates=(0.5,)),
    # one layer of the 48-layer stack (each layer has its own Zipf permutation)
    "stack48_layer": LayerShape("stack48_layer", 5, T=1024, H=2048, E=128, I=768, k=8, dtype="bf16",
                                zipf_s=1.1, skip_rates=(0.6,)),
}

DECODE_M = (1, 4, 8, 32, 64)
STACK_LAYERS = 48


def rng_for(seed: int, cfg_id: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(cfg_id), int(layer), int(tensor_id)]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) and return the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    out = np.empty(a.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        b = flat_u[s:s + step]
        flat_o[s:s + step] = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Decode uint16 bf16 bit patterns into float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_float(stored: np.ndarray) -> np.ndarray:
    """Exact float32 values of a stored activation-dtype tensor (f32 passthrough, bf16 bits decoded)."""
    if stored.dtype == np.uint16:
        return bf16_bits_to_f32(stored)
    return np.asarray(stored, dtype=np.float32)


def _normal(rng: np.random.Generator, shape, std: float, chunk: int = 1 << 25) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        out[s:s + m] = rng.standard_normal(m, dtype=np.float32)
        out[s:s + m] *= np.float32(std)
    return out.reshape(shape)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == "bf16" else np.ascontiguousarray(a, dtype=np.float32)


def make_tokens(shape: LayerShape, seed: int = 0, layer: int = 0, tensor_id: int = X, step: int = 0) -> np.ndarray:
    """Hidden states x ~ N(0,1) of shape [T, H] in the activation dtype (stored form).

    ``step`` selects a fresh draw (decode steps use step = 1, 2, ...)."""
    rng = np.random.default_rng(np.random.SeedSequence([int(seed), shape.cfg_id, int(layer), int(tensor_id), int(step)]))
    return _store(_normal(rng, (shape.T, shape.H), 1.0), shape.dtype)


def make_layer(shape: LayerShape, seed: int = 0, layer: int = 0, with_experts: bool = True) -> dict:
    """All parameters of one layer plus its input batch x, as numpy arrays.

    Layouts (row-major):
      x [T,H] (dtype), gamma [H] f32, w_router [E,H] f32, router_bias [E] f32 or None,
      w_gate [E,I,H], w_up [E,I,H], w_down [E,H,I] (dtype), a_gsp [E] f32, a_rcr [E] f32.
    """
    S = shape
    d = {"shape": S, "seed": seed, "layer": layer}
    d["x"] = make_tokens(S, seed, layer)
    d["gamma"] = rng_for(seed, S.cfg_id, layer, GAMMA).uniform(0.5, 1.5, S.H).astype(np.float32)
    d["w_router"] = _normal(rng_for(seed, S.cfg_id, layer, W_ROUTER), (S.E, S.H), S.router_std)
    if S.zipf_s > 0:
        r = rng_for(seed, S.cfg_id, layer, ROUTER_BIAS).permutation(S.E) + 1
        d["router_bias"] = np.array([-S.zipf_s * math.log(float(v)) for v in r], dtype=np.float32)
    else:
        d["router_bias"] = None
    if with_experts:
        d["w_gate"] = _store(_normal(rng_for(seed, S.cfg_id, layer, W_GATE), (S.E, S.I, S.H), S.expert_std), S.dtype)
        d["w_up"] = _store(_normal(rng_for(seed, S.cfg_id, layer, W_UP), (S.E, S.I, S.H), S.expert_std), S.dtype)
        d["w_down"] = _store(_normal(rng_for(seed, S.cfg_id, layer, W_DOWN), (S.E, S.H, S.I), S.expert_std), S.dtype)
    d["a_gsp"] = rng_for(seed, S.cfg_id, layer, A_GSP).lognormal(0.0, S.table_sigma, S.E).astype(np.float32)
    d["a_rcr"] = rng_for(seed, S.cfg_id, layer, A_RCR).lognormal(0.0, S.table_sigma, S.E).astype(np.float32)
    return d


def small_shape(T=40, H=128, E=8, I=64, k=3, dtype="f32", **kw) -> LayerShape:
    """An ad-hoc small layer for unit tests (cfg_id 100 keeps its streams apart)."""
    return LayerShape("small", kw.pop("cfg_id", 100), T=T, H=H, E=E, I=I, k=k, dtype=dtype, **kw)
