"""A stack of ACE MoE layers with the residual x_{l+1} = x_l + y_l.

Every layer is an ``AceMoeLayer``; the residual add happens inside
moe_combine (its residual argument), so a stack step is the layers' four
C-ABI calls back to back on one stream with no host synchronisation.  This
module allocates buffers, keeps the per-layer thresholds and captures decode
steps in a HIP graph (torch.cuda.CUDAGraph): plumbing, no layer arithmetic.
"""
from __future__ import annotations

import torch

from . import _lib
from .layer import AceMoeLayer, LayerBuffers


class AceMoeStack:
    def __init__(self, layers: list[AceMoeLayer]):
        if not layers:
            raise ValueError("empty stack")
        self.layers = list(layers)
        self.tau: list[tuple[float, float]] = [(0.0, 0.0)] * len(self.layers)
        self.kept: list[int] = [0] * len(self.layers)  # kept slots per layer in the calibration pass

    def buffers(self, T: int) -> list[LayerBuffers]:
        """Two buffer sets used alternately: layer l reads the previous layer's y."""
        return [self.layers[0].buffers(T), self.layers[0].buffers(T)]

    def calibrate(self, x: torch.Tensor, rate: float, bufs=None) -> list[tuple[float, float]]:
        """Per-layer thresholds by on-device quantile mapping, layer by layer:
        layer l is calibrated on its own input (the residual stream after
        layers 0..l-1, themselves run with their calibrated thresholds)."""
        T = x.shape[0]
        bufs = self.buffers(T) if bufs is None else bufs
        dev = x.device
        tau_t = torch.zeros(2, dtype=torch.float32, device=dev)
        cur = x
        for l, lay in enumerate(self.layers):
            b = bufs[l % 2]
            d = lay.desc(T)
            lay.route(cur, 0.0, 0.0, b)
            ws = torch.empty(_lib.moe_calibrate_workspace_bytes(d), dtype=torch.uint8, device=dev)
            _lib.moe_calibrate_thresholds(d, b.topk_idx, b.topk_gate, lay.a_gsp, lay.a_rcr, rate, tau_t, None, ws)
            tg, tr = (float(v) for v in tau_t.cpu())
            self.tau[l] = (tg, tr)
            lay.forward(cur, tg, tr, b, residual=cur)
            self.kept[l] = int(b.offsets[lay.E].item())
            cur = b.y[:T]
        return list(self.tau)

    def forward(self, x: torch.Tensor, bufs=None, path=_lib.ACE_PATH_AUTO, stream=None) -> torch.Tensor:
        """x_L for input x_0 = x, each layer with its thresholds."""
        T = x.shape[0]
        bufs = self.buffers(T) if bufs is None else bufs
        cur = x
        for l, lay in enumerate(self.layers):
            b = bufs[l % 2]
            tg, tr = self.tau[l]
            lay.forward(cur, tg, tr, b, path, residual=cur, stream=stream)
            cur = b.y[:T]
        return cur

    def capture(self, M: int, path=_lib.ACE_PATH_AUTO):
        """A HIP graph of one stack step for M tokens.  Returns (graph, x_in,
        x_out): copy the step's tokens into x_in, replay, read x_out."""
        dev = self.layers[0].w_gate.device
        x_in = torch.zeros(M, self.layers[0].H, dtype=self.layers[0].dtype, device=dev)
        bufs = self.buffers(M)
        s = torch.cuda.Stream(device=dev)
        s.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(s):
            self.forward(x_in, bufs, path)  # warm-up outside the capture
        torch.cuda.current_stream(dev).wait_stream(s)
        torch.cuda.synchronize(dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            x_out = self.forward(x_in, bufs, path)
        g._ace_keep = (bufs,)  # the graph's buffers live as long as the graph
        return g, x_in, x_out
