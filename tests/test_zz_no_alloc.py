"""moe_forward_static, the entry point that allocates nothing, against
moe_forward on the same inputs: every output bit for bit (both run the same
kernels; only where the slot activations, slot outputs and dispatch
workspace live differs).  Two calls in a row share the static buffer, the
second with a smaller batch, so stale rows of the first call must not leak
into the second."""
import numpy as np
import pytest
import torch

import workloads
import token_adaptive_expert_amd as ace
from workloads.device import make_layer_device, make_tokens_device

pytestmark = pytest.mark.gpu

OUTS = ("h", "logits", "topk_idx", "topk_gate", "keep", "offsets", "slot_pos", "y")


def _poison(b):
    for t in (b.h, b.logits, b.topk_idx, b.topk_gate, b.keep, b.offsets, b.sorted_token, b.sorted_gate, b.slot_pos,
              b.y):
        if t.is_floating_point():
            t.fill_(float("nan"))
        else:
            t.fill_(-7 if t.dtype != torch.uint8 else 7)


def _same(layer, x, tg, tr, path=ace.ACE_PATH_AUTO, residual=None):
    T = x.shape[0]
    ref, got = layer.buffers(T), layer.buffers(T)
    _poison(ref)
    _poison(got)
    layer.forward(x, tg, tr, ref, path, residual=residual)
    torch.cuda.synchronize()
    layer.forward_static(x, tg, tr, got, path, residual=residual)
    torch.cuda.synchronize()
    for name in OUTS:
        a, b = getattr(ref, name), getattr(got, name)
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name
    n = int(ref.offsets[-1].item())
    assert 0 < n <= T * layer.k
    for name in ("sorted_token", "sorted_gate"):
        a, b = getattr(ref, name)[:n], getattr(got, name)[:n]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name
    assert torch.isfinite(got.y.float()).all()
    return n


def test_forward_static_qwen3_shape_then_decode(dev):
    """Qwen3-30B-A3B-shaped bf16 layer in the bench configuration (packed
    weights and router): T = 1024 (grouped tiles, the largest batch the
    buffer holds), then T = 8 (the fused decode kernels) and T = 3 with a
    residual, each against moe_forward."""
    S = workloads.CONFIGS["qwen3_30b_a3b"]
    print(f"[no-alloc] {S}", flush=True)
    P = make_layer_device(S, dev, seed=0)
    layer = ace.AceMoeLayer(P["gamma"], P["w_router"], P["router_bias"], P["w_gate"], P["w_up"], P["w_down"],
                            P["a_gsp"], P["a_rcr"], S.k, S.norm_topk, "max", S.rms_eps).packed()
    tg, tr = 0.1, 0.1
    n = _same(layer, P["x"], tg, tr)
    assert 0.2 < 1.0 - n / (S.T * S.k) < 0.8
    x8 = make_tokens_device(S, dev, seed=0, step=3, T=8)
    _same(layer, x8, tg, tr)
    _same(layer, x8[:3].contiguous(), tg, tr, residual=x8[:3].contiguous())


def test_forward_static_tiny_fp32_both_tilings(dev):
    """The tiny f32 layer (T = 64, E = 16, top-4), grouped then split-K
    tiling, then a ragged 5-token batch."""
    S = workloads.CONFIGS["tiny"]
    P = make_layer_device(S, dev, seed=0)
    layer = ace.AceMoeLayer(P["gamma"], P["w_router"], None, P["w_gate"], P["w_up"], P["w_down"], P["a_gsp"],
                            P["a_rcr"], S.k, 1, "max", S.rms_eps)
    _same(layer, P["x"], 0.25, 0.25, ace.ACE_PATH_GROUPED)
    _same(layer, P["x"], 0.25, 0.25, ace.ACE_PATH_STREAM)
    _same(layer, P["x"][:5].contiguous(), 0.25, 0.25)
