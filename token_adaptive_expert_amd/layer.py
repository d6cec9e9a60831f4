"""Buffer-owning wrapper around the four C-ABI calls of one MoE layer forward.

All arithmetic runs in the HIP library; this file only allocates device
buffers (torch) and calls moe_route_skip -> moe_dispatch -> moe_expert_forward
-> moe_combine on one stream, with no host synchronisation in between.
"""
from __future__ import annotations

import copy
import dataclasses

import torch

from . import _lib


@dataclasses.dataclass
class LayerBuffers:
    """Outputs and scratch of one forward, sized for up to T tokens."""

    T: int
    h: torch.Tensor
    logits: torch.Tensor
    topk_idx: torch.Tensor
    topk_gate: torch.Tensor
    keep: torch.Tensor
    offsets: torch.Tensor
    sorted_token: torch.Tensor
    sorted_gate: torch.Tensor
    slot_pos: torch.Tensor
    act: torch.Tensor
    slot_out: torch.Tensor
    workspace: torch.Tensor
    y: torch.Tensor

    @staticmethod
    def allocate(T, H, E, I, k, dtype, device) -> "LayerBuffers":
        desc = _lib.make_desc(max(T, 1), H, E, I, k, dtype)
        ws = _lib.moe_workspace_bytes(desc)
        if ws == 0:
            raise _lib.AceMoeError(_lib.ACE_EINVAL, "moe_workspace_bytes", _lib.moe_last_error())
        slots = max(T * k, 1)
        z = dict(device=device)
        return LayerBuffers(
            T=T,
            h=torch.empty(T, H, dtype=dtype, **z),
            logits=torch.empty(T, E, dtype=torch.float32, **z),
            topk_idx=torch.empty(T, k, dtype=torch.int32, **z),
            topk_gate=torch.empty(T, k, dtype=torch.float32, **z),
            keep=torch.empty(T, k, dtype=torch.uint8, **z),
            offsets=torch.empty(E + 1, dtype=torch.int32, **z),
            sorted_token=torch.empty(slots, dtype=torch.int32, **z),
            sorted_gate=torch.empty(slots, dtype=torch.float32, **z),
            slot_pos=torch.empty(T, k, dtype=torch.int32, **z),
            act=torch.empty(slots, I, dtype=dtype, **z),
            slot_out=torch.empty(slots, H, dtype=dtype, **z),
            workspace=torch.empty(ws, dtype=torch.uint8, **z),
            y=torch.empty(T, H, dtype=dtype, **z),
        )


class AceMoeLayer:
    """One routed SwiGLU MoE layer with ACE slot skipping (device tensors).

    gamma [H] f32, w_router [E,H] f32, router_bias [E] f32 or None,
    w_gate/w_up [E,I,H] and w_down [E,H,I] in the activation dtype,
    a_gsp/a_rcr [E] f32 tables."""

    def __init__(self, gamma, w_router, router_bias, w_gate, w_up, w_down, a_gsp, a_rcr, k, norm_topk=1,
                 fusion="max", rms_eps=1e-6, weight_layout=_lib.ACE_LAYOUT_LINEAR,
                 router_layout=_lib.ACE_LAYOUT_LINEAR, H=None, expert_pool=0):
        self.gamma, self.w_router, self.router_bias = gamma, w_router, router_bias
        self.w_gate, self.w_up, self.w_down = w_gate, w_up, w_down
        self.a_gsp, self.a_rcr = a_gsp, a_rcr
        self.E, self.I, self.H = w_gate.shape
        self.k, self.norm_topk, self.fusion, self.rms_eps = int(k), int(norm_topk), fusion, float(rms_eps)
        self.dtype = w_gate.dtype
        self.weight_layout = int(weight_layout)
        self.router_layout = int(router_layout)
        self.expert_pool = int(expert_pool)  # 0: off; m: batch-level expert-pool cap in dispatch

    def desc(self, T: int):
        return _lib.make_desc(T, self.H, self.E, self.I, self.k, self.dtype, self.norm_topk, self.fusion, self.rms_eps,
                              self.weight_layout, self.router_layout, self.expert_pool)

    def packed(self, stream=None, router=True) -> "AceMoeLayer":
        """The same layer with its expert weights copied into the packed layout
        (moe_pack_weights; the tensors keep their shapes) and, for bf16
        layers when ``router`` is set, the router pre-split (moe_pack_router)."""
        d = self.desc(1)
        out = [self.w_gate, self.w_up, self.w_down]
        if self.weight_layout != _lib.ACE_LAYOUT_PACKED:
            out = []
            for which, w in ((0, self.w_gate), (0, self.w_up), (1, self.w_down)):
                p = torch.empty_like(w)
                _lib.moe_pack_weights(d, which, w, p, stream)
                out.append(p)
        w_router, rl = self.w_router, self.router_layout
        if router and self.dtype == torch.bfloat16 and rl != _lib.ACE_LAYOUT_PACKED:
            w_router = torch.empty(_lib.moe_router_packed_bytes(d), dtype=torch.uint8, device=self.w_router.device)
            _lib.moe_pack_router(d, self.w_router, w_router, stream)
            rl = _lib.ACE_LAYOUT_PACKED
        return AceMoeLayer(self.gamma, w_router, self.router_bias, out[0], out[1], out[2], self.a_gsp, self.a_rcr,
                           self.k, self.norm_topk, self.fusion, self.rms_eps, _lib.ACE_LAYOUT_PACKED, rl,
                           expert_pool=self.expert_pool)

    def with_pool(self, m: int) -> "AceMoeLayer":
        """The same layer (same tensors) with the batch-level expert-pool cap m
        (0: off) applied in dispatch."""
        out = copy.copy(self)
        out.expert_pool = int(m)
        return out

    def buffers(self, T: int) -> LayerBuffers:
        return LayerBuffers.allocate(T, self.H, self.E, self.I, self.k, self.dtype, self.w_gate.device)

    def route(self, x, tau_gsp, tau_rcr, b: LayerBuffers, logits_in=None, stream=None):
        T = x.shape[0]
        d = self.desc(T)
        _lib.moe_route_skip(d, x, self.gamma, self.w_router, self.router_bias, logits_in, b.logits, self.a_gsp,
                            self.a_rcr, tau_gsp, tau_rcr, b.h, b.topk_idx, b.topk_gate, b.keep, stream)

    def dispatch(self, T: int, b: LayerBuffers, stream=None):
        _lib.moe_dispatch(self.desc(T), b.topk_idx, b.topk_gate, b.keep, b.offsets, b.sorted_token, b.sorted_gate,
                          b.slot_pos, b.workspace, None, stream)

    def experts(self, T: int, b: LayerBuffers, path=_lib.ACE_PATH_AUTO, stream=None):
        _lib.moe_expert_forward(self.desc(T), path, b.h, self.w_gate, self.w_up, self.w_down, b.offsets,
                                b.sorted_token, b.sorted_gate, b.act, b.slot_out, b.workspace, None, stream)

    def combine(self, T: int, b: LayerBuffers, residual=None, stream=None):
        _lib.moe_combine(self.desc(T), b.slot_pos, b.slot_out, residual, b.y, stream)

    def forward(self, x, tau_gsp, tau_rcr, b: LayerBuffers | None = None, path=_lib.ACE_PATH_AUTO, logits_in=None,
                residual=None, stream=None) -> torch.Tensor:
        """The whole layer through moe_forward (one C call)."""
        T = x.shape[0]
        if b is None:
            b = self.buffers(T)
        if b.T < T:
            raise ValueError(f"buffers sized for {b.T} tokens, got {T}")
        _lib.moe_forward(self.desc(T), path, x, self.gamma, self.w_router, self.router_bias, logits_in, b.logits,
                         self.a_gsp, self.a_rcr, tau_gsp, tau_rcr, self.w_gate, self.w_up, self.w_down, residual, b.h,
                         b.topk_idx, b.topk_gate, b.keep, b.offsets, b.sorted_token, b.sorted_gate, b.slot_pos, b.act,
                         b.slot_out, b.y, b.workspace, None, stream)
        return b.y[:T]

    def forward_static(self, x, tau_gsp, tau_rcr, b: LayerBuffers, path=_lib.ACE_PATH_AUTO, logits_in=None,
                       residual=None, stream=None) -> torch.Tensor:
        """The whole layer through moe_forward_static: the library's static
        device scratch replaces b.act, b.slot_out and b.workspace (which are
        left untouched); every other buffer of b receives its output."""
        T = x.shape[0]
        if b.T < T:
            raise ValueError(f"buffers sized for {b.T} tokens, got {T}")
        _lib.moe_forward_static(self.desc(T), path, x, self.gamma, self.w_router, self.router_bias, logits_in,
                                b.logits, self.a_gsp, self.a_rcr, tau_gsp, tau_rcr, self.w_gate, self.w_up,
                                self.w_down, residual, b.h, b.topk_idx, b.topk_gate, b.keep, b.offsets,
                                b.sorted_token, b.sorted_gate, b.slot_pos, b.y, stream)
        return b.y[:T]

    def forward_steps(self, x, tau_gsp, tau_rcr, b: LayerBuffers | None = None, path=_lib.ACE_PATH_AUTO,
                      logits_in=None, residual=None, stream=None) -> torch.Tensor:
        """The same layer through the four step calls."""
        T = x.shape[0]
        if b is None:
            b = self.buffers(T)
        if b.T < T:
            raise ValueError(f"buffers sized for {b.T} tokens, got {T}")
        self.route(x, tau_gsp, tau_rcr, b, logits_in, stream)
        self.dispatch(T, b, stream)
        self.experts(T, b, path, stream)
        self.combine(T, b, residual, stream)
        return b.y[:T]


def build_tables(gamma, w_router, w_gate, w_up, w_down, eps=1e-6, workspace=None, stream=None):
    """A^GSP and A^RCR [E] f32 of one layer from its weights (moe_build_tables).
    Weights in the LINEAR layout on one device; ``workspace`` (uint8 tensor)
    defaults to the preferred size."""
    E, I, H = w_gate.shape
    d = _lib.make_desc(1, H, E, I, 1, w_gate.dtype)
    if workspace is None:
        n = _lib.moe_tables_workspace_bytes(d)
        if n == 0:
            raise _lib.AceMoeError(_lib.ACE_EINVAL, "moe_tables_workspace_bytes", _lib.moe_last_error())
        workspace = torch.empty(n, dtype=torch.uint8, device=w_gate.device)
    a_gsp = torch.empty(E, dtype=torch.float32, device=w_gate.device)
    a_rcr = torch.empty(E, dtype=torch.float32, device=w_gate.device)
    _lib.moe_build_tables(d, eps, gamma, w_router, w_gate, w_up, w_down, a_gsp, a_rcr, workspace, None, stream)
    return a_gsp, a_rcr
