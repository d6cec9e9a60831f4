#!/usr/bin/env python3
"""Benchmark of the ACE-skipped MoE layer forward on one MI355X.

A step is one pass of the whole layer (moe_route_skip -> moe_dispatch ->
moe_expert_forward -> moe_combine) over one batch.  The headline workload is
a Qwen3-30B-A3B-shaped layer (hidden 2048, 128 experts, top-8, expert
intermediate 768, bf16) at T = 1024 prefill tokens and 60% skip, thresholds
from on-device quantile mapping on the batch itself.  Inputs are seeded
synthetic data already resident in HBM; the expert weights rotate over
several copies so that no step finds the previous step's weights in cache.

Prints one JSON line.  Extra fields: decode µs/layer at M = 1..64 tokens,
prefill throughput at other skip rates, and the oracle timed on host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--skip", type=float, default=0.6)
    p.add_argument("--copies", type=int, default=8, help="weight copies rotated over the steps")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-tables", action="store_true", help="skip timing the offline table builder")
    p.add_argument("--no-stack", action="store_true", help="skip the 48-layer stack")
    p.add_argument("--decode-m", type=int, nargs="+", help="decode batch sizes to run (default: all)")
    p.add_argument("--only", choices=["decode", "glm", "t32k", "stack", "tables", "calib", "probes"],
                   help="run that leg alone and print its result (for profiling runs), not the contract line")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the GLM-4.5-Air-shaped layer, the T=32768 run and the dense GEMM ceiling")
    p.add_argument("--cpu-tokens", type=int, default=1024, help="tokens in the oracle's timed sample")
    p.add_argument("--path", type=int, default=0, help="0 auto, 1 grouped, 2 stream")
    p.add_argument("--layout", choices=["packed", "linear"], default="packed",
                   help="expert weight layout (packed once at setup, like the offline tables)")
    return p.parse_args()


class Bench:
    def __init__(self, args):
        import torch
        import workloads
        import token_adaptive_expert_amd as ace
        from workloads.torch_io import layer_to_torch

        self.torch, self.ace, self.workloads = torch, ace, workloads
        self.args = args
        self.dev = torch.device("cuda:0")
        self.S = workloads.CONFIGS["qwen3_30b_a3b"]
        t0 = time.time()
        self.L = workloads.make_layer(self.S, seed=0)
        P = layer_to_torch(self.L, self.dev)
        self.P = P
        # weight copies: copy 0 is the generated layer, the rest are device clones
        self.layers = []
        for c in range(max(1, args.copies)):
            if c == 0:
                Q = P
            else:
                Q = {n: (None if v is None else v.clone()) for n, v in P.items() if n != "x"}
            lay = ace.AceMoeLayer(Q["gamma"], Q["w_router"], Q["router_bias"], Q["w_gate"], Q["w_up"], Q["w_down"],
                                  Q["a_gsp"], Q["a_rcr"], self.S.k, self.S.norm_topk, "max", self.S.rms_eps)
            if args.layout == "packed":
                lay = lay.packed()
                if c > 0:
                    del Q["w_gate"], Q["w_up"], Q["w_down"]
            self.layers.append(lay)
        torch.cuda.synchronize()
        self.setup_s = time.time() - t0

    # ------------------------------------------------------------ helpers
    def calibrate(self, x, rate):
        """Thresholds for `rate` on batch x by on-device quantile mapping."""
        torch, ace = self.torch, self.ace
        lay = self.layers[0]
        T = x.shape[0]
        b = lay.buffers(T)
        lay.route(x, 0.0, 0.0, b)
        d = lay.desc(T)
        ws = torch.empty(ace.moe_calibrate_workspace_bytes(d), dtype=torch.uint8, device=self.dev)
        tau = torch.zeros(2, dtype=torch.float32, device=self.dev)
        ace.moe_calibrate_thresholds(d, b.topk_idx, b.topk_gate, lay.a_gsp, lay.a_rcr, rate, tau, None, ws)
        t = tau.cpu().numpy()
        return float(t[0]), float(t[1])

    def run_steps(self, x, tau, steps, warmup, path):
        """Whole-layer steps, weights rotating over the copies.  Returns
        (ms per step, buffers of the last step)."""
        torch = self.torch
        T = x.shape[0]
        bufs = self.layers[0].buffers(T)
        nl = len(self.layers)
        for i in range(warmup):
            self.layers[i % nl].forward(x, tau[0], tau[1], bufs, path)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            self.layers[(warmup + i) % nl].forward(x, tau[0], tau[1], bufs, path)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps, bufs

    def stage_ms(self, x, tau, stage, steps, path):
        """Mean duration of one expert kernel (gate/up or down) launched back to
        back on the current stream, HIP events around the whole run, weights
        rotating over the copies; routing and dispatch are done once before."""
        torch = self.torch
        T = x.shape[0]
        bufs = self.layers[0].buffers(T)
        self.layers[0].forward(x, tau[0], tau[1], bufs, path)
        nl = len(self.layers)
        for i in range(3):
            self.layers[i % nl].experts(T, bufs, path | stage)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            self.layers[(3 + i) % nl].experts(T, bufs, path | stage)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps

    def copy_ceiling(self, nbytes=2 << 30, reps=10):
        """Read+write bandwidth of a plain device-to-device copy (torch), as a
        measured ceiling beside the datasheet peak."""
        torch = self.torch
        a = torch.empty(nbytes // 2, dtype=torch.uint8, device=self.dev)
        b = torch.empty_like(a)
        b.copy_(a)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(reps):
            b.copy_(a)
        stop.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / reps
        del a, b
        return 2 * (nbytes // 2) / (ms * 1e-3) / 1e9

    def read_ceiling(self, nbytes=4 << 30, reps=10):
        """Streaming-read rate of moe_hbm_read_probe (one pass over a 4 GiB
        buffer with 16-byte loads on every compute unit), the best over a few
        grid sizes: a measured read ceiling beside the datasheet peak."""
        torch, ace = self.torch, self.ace
        buf = torch.ones(nbytes // 4, dtype=torch.int32, device=self.dev)
        ncu = torch.cuda.get_device_properties(self.dev).multi_processor_count
        best, by_grid = 0.0, {}
        for per_cu in (2, 4, 8, 16):
            wg = ncu * per_cu
            sink = torch.empty(wg, dtype=torch.int32, device=self.dev)
            ms = timed(torch, lambda i: ace.moe_hbm_read_probe(buf, sink, wg), reps, 2)
            gbs = nbytes / (ms * 1e-3) / 1e9
            by_grid[str(wg)] = round(gbs, 1)
            best = max(best, gbs)
        del buf
        return {"GBs": round(best, 1), "bytes": nbytes, "by_workgroups": by_grid,
                "kernel": "moe_hbm_read_probe (read only, 16-byte loads, 8 in flight per thread)"}

    def l2_load_rates(self, rounds=2048, reps=5):
        """Load rate from L2 per compute unit (moe_l2_load_probe on a 2 MiB
        buffer, 6 loads of 1 KB in flight per wave), alone and with 4 bf16
        MFMAs per loaded KB (the router's ratio), the blocks of a round
        consecutive or at the router planes' 64 KB / 512 KB spacing; 2 and 3
        workgroups of 4 waves per CU.  B/clk at the 2.4 GHz peak engine
        clock; MFMA busy = MFMA cycles (16 per 16x16x32 bf16 MFMA) over the
        SIMDs' cycles."""
        torch, ace = self.torch, self.ace
        buf = torch.randint(0, 255, (2 << 20,), dtype=torch.uint8, device=self.dev)
        ncu = torch.cuda.get_device_properties(self.dev).multi_processor_count
        out = []
        for mfma in (0, 4):
            for stride in (0, 1):
                for per_cu in (2, 3):
                    wg = ncu * per_cu
                    sink = torch.empty(wg * 4, dtype=torch.int32, device=self.dev)
                    it = max(1, rounds // per_cu)
                    ms = timed(torch, lambda i: ace.moe_l2_load_probe(buf, sink, wg, it, 6, mfma, stride), reps, 2)
                    cyc = ms * 1e-3 * 2.4e9
                    loads = wg * 4 * it * 6
                    out.append({"mfma_per_KB": mfma, "stride_mode": stride, "wg_per_cu": per_cu,
                                "B_per_clk_per_cu": round(loads * 1024 / ncu / cyc, 1),
                                "TBs": round(loads * 1024 / (ms * 1e-3) / 1e12, 1),
                                "mfma_busy": round(loads * mfma * 16 / (4 * ncu) / cyc, 3)})
        del buf
        return out

    def launch_floor(self, n=64, reps=20):
        """Time per kernel of a HIP graph of n back-to-back launches of a
        near-empty kernel (moe_hbm_read_probe on 16 bytes, one workgroup): the
        fixed cost every dependent launch of a layer pays."""
        torch, ace = self.torch, self.ace
        buf = torch.zeros(4, dtype=torch.int32, device=self.dev)
        sink = torch.empty(1, dtype=torch.int32, device=self.dev)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(n):
                ace.moe_hbm_read_probe(buf, sink, 1)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                ace.moe_hbm_read_probe(buf, sink, 1)
        ms = timed(torch, lambda i: g.replay(), reps, 3)
        return round(ms * 1e3 / n, 3)

    def counts(self, bufs):
        off = bufs.offsets.cpu().numpy().astype(np.int64)
        n_e = np.diff(off)
        return int(off[-1]), int((n_e > 0).sum())

    # ------------------------------------------------------------ legs
    def prefill(self, rate, kernel_timing=True):
        """Whole-layer steps timed alone; then each expert kernel timed alone."""
        x = self.P["x"]
        tau = self.calibrate(x, rate) if rate > 0 else (0.0, 0.0)
        ms, bufs = self.run_steps(x, tau, self.args.steps, self.args.warmup, self.args.path)
        gu = dn = None
        if kernel_timing:
            gu = self.stage_ms(x, tau, self.ace.ACE_STAGE_GATEUP, self.args.steps, self.args.path)
            dn = self.stage_ms(x, tau, self.ace.ACE_STAGE_DOWN, self.args.steps, self.args.path)
        n_kept, U = self.counts(bufs)
        return dict(tau=tau, ms=ms, gateup_ms=gu, down_ms=dn, n_kept=n_kept, U=U)

    def graph_ms(self, x, tau, layers, reps=50):
        """Mean ms of one replay of a HIP graph holding one forward of each
        layer in `layers` (the rotated copies) on batch x."""
        torch = self.torch
        bufs = [lay.buffers(x.shape[0]) for lay in layers]
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for lay, b in zip(layers, bufs):
                lay.forward(x, tau[0], tau[1], b)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for lay, b in zip(layers, bufs):
                lay.forward(x, tau[0], tau[1], b)
        ms = timed(torch, lambda i: g.replay(), reps, 3)
        return ms, bufs[-1]

    def decode(self, tau):
        """Decode steps of M fresh tokens, thresholds from the prefill
        calibration.  Primary: all rotated layers in one HIP graph (per-layer
        time = replay time / layers), as a decode loop runs; also eager
        back-to-back launches."""
        torch, workloads = self.torch, self.workloads
        from workloads.torch_io import to_torch
        out = {}
        S = self.S
        for M in (self.args.decode_m or workloads.DECODE_M):
            Sd = workloads.CONFIGS["qwen3_30b_a3b_decode"].with_tokens(M)
            x = to_torch(workloads.make_tokens(Sd, seed=0, step=1), self.dev)
            ms, bufs = self.run_steps(x, tau, max(self.args.steps, 50), self.args.warmup, 0)
            gms, _ = self.graph_ms(x, tau, self.layers)
            gms /= len(self.layers)
            iso = self.isolated_ms(x, tau)
            n_kept, U = self.counts(bufs)
            wbytes = U * 3 * S.H * S.I * 2
            out[M] = dict(us=gms * 1e3, eager_us=ms * 1e3, isolated_us=iso * 1e3, U=U, n_kept=n_kept,
                          retained_weight_MB=wbytes / 1e6, hbm_frac=(wbytes / (gms * 1e-3)) / (HBM_PEAK_GBS * 1e9))
        return out

    def isolated_ms(self, x, tau, reps=30):
        """Median ms of one layer forward launched alone: the device idle
        before it (synchronised), HIP events around the single call, weights
        rotating over the copies."""
        torch = self.torch
        bufs = self.layers[0].buffers(x.shape[0])
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t = []
        for i in range(reps + 3):
            lay = self.layers[i % len(self.layers)]
            torch.cuda.synchronize()
            start.record()
            lay.forward(x, tau[0], tau[1], bufs)
            stop.record()
            torch.cuda.synchronize()
            if i >= 3:
                t.append(start.elapsed_time(stop))
        return float(np.median(t))

    def decode_pool(self, tau, pools=(16, 32), Ms=(8, 32, 64)):
        """Decode with the batch-level expert-pool cap m (graph replays)."""
        workloads = self.workloads
        from workloads.torch_io import to_torch
        out = {}
        for m in pools:
            layers = [lay.with_pool(m) for lay in self.layers]
            row = {}
            for M in Ms:
                Sd = workloads.CONFIGS["qwen3_30b_a3b_decode"].with_tokens(M)
                x = to_torch(workloads.make_tokens(Sd, seed=0, step=1), self.dev)
                gms, b = self.graph_ms(x, tau, layers)
                n_kept, U = self.counts(b)
                row[str(M)] = {"us": round(gms * 1e3 / len(layers), 2), "U": U, "n_kept": n_kept}
            out[f"pool_{m}"] = row
        return out


def timed(torch, fn, steps, warmup):
    """Mean ms of fn(i) over `steps` calls after `warmup`, HIP events on the current stream."""
    for i in range(warmup):
        fn(i)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        fn(warmup + i)
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def layer_roof(S, T, U, n_kept, ms):
    """Algorithmic bytes and flops of one layer forward (executed slots and
    active experts only) and the fractions of the HBM and MFMA peaks."""
    b = U * 3 * S.H * S.I * 2 + S.E * S.H * 4 + T * S.H * 4 + 8 * S.E
    f = n_kept * 6 * S.H * S.I + 2 * T * S.H * S.E
    t = ms * 1e-3
    return {"alg_bytes": b, "alg_flops": f, "hbm_frac": round(b / t / (HBM_PEAK_GBS * 1e9), 4),
            "mfma_frac": round(f / t / (BF16_PEAK_TFLOPS * 1e12), 4),
            "roof_us": round(max(b / (HBM_PEAK_GBS * 1e9), f / (BF16_PEAK_TFLOPS * 1e12)) * 1e6, 1)}


def extra_prefill(B, name, S, T, rate, steps, warmup, P=None, layer=None, keep=None):
    """Whole-layer prefill of another workload (weights drawn on the device),
    thresholds by on-device quantile mapping on the batch itself, plus the
    gate/up kernel alone.  ``keep`` (a dict) receives the layer's linear
    device weights, its input and thresholds, for the oracle's timing leg."""
    torch, ace = B.torch, B.ace
    from workloads.device import make_layer_device, make_tokens_device
    if layer is None:
        P = make_layer_device(S, B.dev, seed=0)
        layer = ace.AceMoeLayer(P["gamma"], P["w_router"], P["router_bias"], P["w_gate"], P["w_up"],
                                P["w_down"], P["a_gsp"], P["a_rcr"], S.k, S.norm_topk, "max",
                                S.rms_eps).packed()
        if keep is None:
            del P["w_gate"], P["w_up"], P["w_down"]
    x = make_tokens_device(S, B.dev, seed=0, step=7, T=T) if T != S.T else P["x"]
    b = layer.buffers(T)
    layer.route(x, 0.0, 0.0, b)
    d = layer.desc(T)
    ws = torch.empty(ace.moe_calibrate_workspace_bytes(d), dtype=torch.uint8, device=B.dev)
    tau_t = torch.zeros(2, dtype=torch.float32, device=B.dev)
    ace.moe_calibrate_thresholds(d, b.topk_idx, b.topk_gate, layer.a_gsp, layer.a_rcr, rate, tau_t, None, ws)
    tg, tr = [float(v) for v in tau_t.cpu()]
    ms = timed(torch, lambda i: layer.forward(x, tg, tr, b), steps, warmup)
    gu = timed(torch, lambda i: layer.experts(T, b, ace.ACE_STAGE_GATEUP), steps, 2)
    dn = timed(torch, lambda i: layer.experts(T, b, ace.ACE_STAGE_DOWN), steps, 2)
    off = b.offsets.cpu().numpy().astype(np.int64)
    n_kept, U = int(off[-1]), int((np.diff(off) > 0).sum())
    gu_flops = n_kept * 4 * S.H * S.I
    gu_bytes = U * 2 * S.H * S.I * 2 + T * S.H * 2
    dn_bytes = U * S.H * S.I * 2
    out = {"workload": name, "T": T, "H": S.H, "E": S.E, "I": S.I, "k": S.k, "skip_target": rate,
           "skip_realized": round(1 - n_kept / (T * S.k), 5), "active_experts": U, "n_kept": n_kept,
           "max_rows_per_expert": int(np.diff(off).max()),
           "tokens_per_s": round(T / (ms * 1e-3), 1), "us_per_layer": round(ms * 1e3, 2),
           "gateup_us": round(gu * 1e3, 2), "gateup_tflops": round(gu_flops / (gu * 1e-3) / 1e12, 1),
           "gateup_mfma_frac": round(gu_flops / (gu * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4),
           "gateup_GBs": round(gu_bytes / (gu * 1e-3) / 1e9, 1),
           "gateup_hbm_frac": round(gu_bytes / (gu * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "down_us": round(dn * 1e3, 2), "down_GBs": round(dn_bytes / (dn * 1e-3) / 1e9, 1),
           "down_tflops": round(n_kept * 2 * S.H * S.I / (dn * 1e-3) / 1e12, 1)}
    out.update(layer_roof(S, T, U, n_kept, ms))
    if keep is not None:
        keep.update(P=P, x=x, tau=(tg, tr))
    return out


def dense_gemm_ceiling(B, M=32768, reps=10):
    """bf16 dense GEMM of the gate/up shape (K = H, N = 2I) through torch
    (hipBLASLt): a measured MFMA ceiling beside the datasheet peak."""
    torch, S = B.torch, B.S
    a = torch.randn(M, S.H, device=B.dev, dtype=torch.bfloat16)
    w = torch.randn(2 * S.I, S.H, device=B.dev, dtype=torch.bfloat16)
    wt = w.t().contiguous()
    ms = timed(torch, lambda i: torch.matmul(a, wt), reps, 3)
    return round(2 * M * S.H * 2 * S.I / (ms * 1e-3) / 1e12, 1)


def stack48(B, decode_steps=128, M=8, keep=None, keep_layers=(0, 23, 47), keep_tokens=32):
    """48 independent Qwen3-30B-A3B-shaped layers (each with its own Zipf(1.1)
    router prior; 58 GB of bf16 expert weights) with the residual stream:
    per-layer thresholds by on-device quantile mapping at 60% on the layers'
    own prefill inputs, then the 1024-token prefill and decode steps of 8
    fresh tokens, each step one HIP graph replay of all 48 layers.  After the
    timing, one untimed pass of each reads every layer's active experts U and
    kept slots n_kept back for the algorithmic bytes.  ``keep`` (a dict)
    receives, for the layers in keep_layers, their linear device weights,
    thresholds and the first keep_tokens rows of their prefill input x_l
    (the GPU's residual stream), for the oracle's timing leg."""
    torch, ace = B.torch, B.ace
    import workloads
    from workloads.device import make_layer_device, make_tokens_device
    S = workloads.CONFIGS["stack48_layer"]
    layers, x0, kept_P = [], None, {}
    for l in range(workloads.STACK_LAYERS):
        P = make_layer_device(S, B.dev, seed=0, layer=l, with_x=(l == 0))
        if l == 0:
            x0 = P["x"]
        layers.append(ace.AceMoeLayer(P["gamma"], P["w_router"], P["router_bias"], P["w_gate"], P["w_up"],
                                      P["w_down"], P["a_gsp"], P["a_rcr"], S.k, S.norm_topk, "max",
                                      S.rms_eps).packed())
        if keep is not None and l in keep_layers:
            kept_P[l] = P
        del P
    st = ace.AceMoeStack(layers)
    st.calibrate(x0, 0.6)
    bufs = st.buffers(S.T)
    pre_ms = timed(torch, lambda i: st.forward(x0, bufs), 5, 1)
    g, x_in, _ = st.capture(M)
    xs = make_tokens_device(S, B.dev, seed=0, step=1000, T=decode_steps * M).view(decode_steps, M, S.H)

    def step(i):
        x_in.copy_(xs[i % decode_steps])
        g.replay()

    dec_ms = timed(torch, step, decode_steps, 8)
    nl = len(layers)

    def per_layer(x, T):
        """One untimed pass layer by layer: (U, n_kept) of every layer, and
        the inputs x_l of the kept layers."""
        cur, U, nk, xl = x, [], [], {}
        for l, lay in enumerate(layers):
            if l in kept_P:
                xl[l] = cur[:keep_tokens].clone()
            b = bufs[l % 2] if T == S.T else dbufs[l % 2]
            lay.forward(cur, st.tau[l][0], st.tau[l][1], b, residual=cur)
            off = b.offsets[:lay.E + 1].cpu().numpy().astype(np.int64)
            nk.append(int(off[-1]))
            U.append(int((np.diff(off) > 0).sum()))
            cur = b.y[:T]
        return U, nk, xl

    dbufs = st.buffers(M)
    U_pre, nk_pre, xl = per_layer(x0, S.T)
    U_dec, nk_dec = [0] * nl, [0] * nl
    for i in range(4):   # decode steps 0..3: average U and n_kept
        u, n, _ = per_layer(xs[i], M)
        U_dec = [a + b for a, b in zip(U_dec, u)]
        nk_dec = [a + b for a, b in zip(nk_dec, n)]
    U_dec = [u / 4 for u in U_dec]
    nk_dec = [n / 4 for n in nk_dec]
    wl = 3 * S.H * S.I * 2
    fixed = S.E * S.H * 4 + 8 * S.E
    pre_bytes = sum(u * wl + fixed + S.T * S.H * 4 for u in U_pre)
    pre_flops = sum(n * 6 * S.H * S.I + 2 * S.T * S.H * S.E for n in nk_pre)
    dec_bytes = sum(u * wl + fixed + M * S.H * 4 for u in U_dec)
    skip = [1 - n / (S.T * S.k) for n in st.kept]
    out = {"workload": "48 qwen3_30b_a3b-shaped layers, Zipf(1.1) router priors, residual stream, 60% skip",
           "layers": nl, "weights_GB": round(nl * 3 * S.E * S.H * S.I * 2 / 1e9, 1),
           "prefill_tokens": S.T, "prefill_ms": round(pre_ms, 3),
           "prefill_tokens_per_s": round(S.T / (pre_ms * 1e-3), 1),
           "prefill_us_per_layer": round(pre_ms * 1e3 / nl, 2),
           "prefill_U_mean_min_max": [round(float(np.mean(U_pre)), 2), min(U_pre), max(U_pre)],
           "prefill_n_kept_total": int(sum(nk_pre)),
           "prefill_alg_bytes": int(pre_bytes), "prefill_alg_flops": int(pre_flops),
           "prefill_hbm_frac": round(pre_bytes / (pre_ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
           "prefill_mfma_frac": round(pre_flops / (pre_ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4),
           "decode_M": M, "decode_steps": decode_steps, "decode_ms_per_step": round(dec_ms, 4),
           "decode_us_per_layer": round(dec_ms * 1e3 / nl, 2),
           "decode_tokens_per_s": round(M / (dec_ms * 1e-3), 1),
           "decode_U_mean_per_layer": round(float(np.mean(U_dec)), 2),
           "decode_n_kept_mean_per_layer": round(float(np.mean(nk_dec)), 2),
           "decode_alg_bytes_per_step": int(dec_bytes),
           "decode_hbm_frac": round(dec_bytes / (dec_ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
           "decode_U_note": "U and n_kept averaged over decode steps 0-3 (one untimed eager pass each)",
           "calibration_skip_min_max": [round(min(skip), 5), round(max(skip), 5)]}
    if keep is not None:
        keep.update(S=S, layers={l: dict(P=kept_P[l], x=xl[l], tau=st.tau[l]) for l in kept_P})
    del st, layers, g, bufs, dbufs
    torch.cuda.empty_cache()
    return out


def calibration_leg(B, reps=5):
    """Time moe_calibrate_thresholds (per-layer thresholds by quantile mapping
    on the layer's own routed slots, 60% skip) at T = 1024 and 4096 on the
    generated layer; the skip count it yields is checked against the target."""
    torch, ace, S = B.torch, B.ace, B.S
    from workloads.device import make_tokens_device
    lay = B.layers[0]
    out = {}
    for T in (1024, 4096):
        x = B.P["x"] if T == S.T else make_tokens_device(S, B.dev, seed=0, step=11, T=T)
        b = lay.buffers(T)
        lay.route(x, 0.0, 0.0, b)
        d = lay.desc(T)
        ws = torch.empty(ace.moe_calibrate_workspace_bytes(d), dtype=torch.uint8, device=B.dev)
        tau = torch.zeros(2, dtype=torch.float32, device=B.dev)
        run = lambda i: ace.moe_calibrate_thresholds(d, b.topk_idx, b.topk_gate, lay.a_gsp, lay.a_rcr, 0.6, tau,
                                                     None, ws)
        ms = timed(torch, run, reps, 1)
        tg, tr = [float(v) for v in tau.cpu()]
        lay.route(x, tg, tr, b)
        skipped = int((b.keep == 0).sum().item())
        out[str(T)] = {"ms": round(ms, 4), "eligible_slots": T * (S.k - 1),
                       "skipped": skipped, "target": int(math.floor(0.6 * T * S.k + 0.5))}
    return out


def tables_build(B, reps=5):
    """Time moe_build_tables (A^GSP and A^RCR of the layer from its weights,
    done once per checkpoint) on the generated layer's linear weights.
    Gram MFMA work per expert: the 128x128 upper-triangular tiles of D, G_g and
    G_u, the last two with the gamma^2-scaled operand as three exact bf16
    planes (7 MFMA passes per tile); useful work counts each Gram once."""
    torch, ace, S, P = B.torch, B.ace, B.S, B.P
    d = ace.make_desc(1, S.H, S.E, S.I, 1, "bf16")
    ws = torch.empty(ace.moe_tables_workspace_bytes(d), dtype=torch.uint8, device=B.dev)
    args = (P["gamma"], P["w_router"], P["w_gate"], P["w_up"], P["w_down"])
    ace.build_tables(*args, workspace=ws)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g, r = ace.build_tables(*args, workspace=ws)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    nbk = S.I // 128
    tiles = nbk * (nbk + 1) // 2
    executed = S.E * tiles * 128 * 128 * S.H * 2 * 7
    useful = S.E * 3 * S.I * (S.I + 1) // 2 * S.H * 2
    weight_bytes = S.E * 3 * S.H * S.I * 2
    return {"ms": round(ms, 4), "experts": S.E,
            "mfma_tflop_executed": round(executed / 1e12, 4),
            "executed_tflops": round(executed / (ms * 1e-3) / 1e12, 1),
            "useful_tflops": round(useful / (ms * 1e-3) / 1e12, 1),
            "mfma_frac_whole_build": round(executed / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4),
            "weight_bytes": weight_bytes,
            "a_gsp_range": [round(float(g.min()), 4), round(float(g.max()), 4)],
            "a_rcr_range": [round(float(r.min()), 4), round(float(r.max()), 4)]}


def cpu_baseline(L, S, tau, ntok, min_seconds=10.0, max_passes=20):
    """The oracle, as it stands, over the first `ntok` tokens of the batch,
    repeated until at least `min_seconds` of host time (at most `max_passes`)."""
    import oracle
    cores = _blas_threads()
    x = L["x"][:ntok]
    t0 = time.time()
    passes = 0
    while passes < max_passes and (passes == 0 or time.time() - t0 < min_seconds):
        oracle.moe_layer(x, L["gamma"], L["w_router"], L["router_bias"], L["w_gate"], L["w_up"], L["w_down"],
                         L["a_gsp"], L["a_rcr"], tau[0], tau[1], S.k, bool(S.norm_topk), S.rms_eps, S.dtype)
        passes += 1
    dt = time.time() - t0
    return {"value": passes * ntok / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{passes} passes over the first {ntok} of the {S.T} prefill tokens of the same layer and "
                      f"thresholds, {dt:.1f} s of host time"}


class _DeviceExperts:
    """w[e] of a device tensor copied to host on demand (stored form), so the
    oracle copies only the experts its own routing selects."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, e):
        from workloads.torch_io import from_torch
        return from_torch(self.t[int(e)])


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return 1


def _oracle_pass(x, P, S, tau, host=None):
    """One call of the oracle's layer forward on the rows x (host, stored
    form), timed; weights from host arrays (``host``) or fetched from the
    device tensors of P expert by expert."""
    import oracle
    from workloads.torch_io import from_torch
    if host is None:
        host = {n: from_torch(P[n]) if P[n] is not None else None for n in
                ("gamma", "w_router", "router_bias", "a_gsp", "a_rcr")}
        host.update({n: _DeviceExperts(P[n]) for n in ("w_gate", "w_up", "w_down")})
    t0 = time.time()
    r = oracle.moe_layer(x, host["gamma"], host["w_router"], host["router_bias"], host["w_gate"], host["w_up"],
                         host["w_down"], host["a_gsp"], host["a_rcr"], tau[0], tau[1], S.k, bool(S.norm_topk),
                         S.rms_eps, S.dtype)
    return time.time() - t0, int(r["keep"].sum())


def cpu_by_config(B, head_tau, glm=None, stack=None, decode_M=8):
    """The oracle, as it stands, timed on the host cores for each other
    workload, on bounded samples: the tiny f32 layer (all 64 tokens, its
    thresholds by the oracle's own quantile mapping at 50%), one decode step
    of 8 tokens on the headline layer, the first 16 tokens of the
    GLM-4.5-Air-shaped layer, and the first 32 tokens of the inputs of
    layers 0, 23 and 47 of the 48-layer stack.  Each time includes the
    oracle's float64 copies of the experts it touches (its own per-call cache)."""
    import oracle
    import workloads
    from workloads.torch_io import from_torch
    out = {"cores": int(_blas_threads())}
    S1 = workloads.CONFIGS["tiny"]
    L1 = workloads.make_layer(S1)
    h = oracle.rmsnorm(L1["x"], L1["gamma"], S1.rms_eps, S1.dtype)
    lg = oracle.router_logits(h, L1["w_router"], None)
    idx = np.stack([oracle.topk_experts(lg[t], S1.k) for t in range(S1.T)])
    g = np.stack([oracle.topk_gates(lg[t], idx[t], True) for t in range(S1.T)])
    tg, tr, _, _ = oracle.quantile_thresholds(idx, g, L1["a_gsp"], L1["a_rcr"], 0.5)
    dt, nk = _oracle_pass(L1["x"], None, S1, (tg, tr), host=L1)
    out["tiny_f32_T64"] = {"tokens": S1.T, "seconds": round(dt, 3), "tokens_per_s": round(S1.T / dt, 1),
                           "n_kept": nk}
    Sd = workloads.CONFIGS["qwen3_30b_a3b_decode"].with_tokens(decode_M)
    xd = workloads.make_tokens(Sd, seed=0, step=1)
    dt, nk = _oracle_pass(xd, None, Sd, head_tau, host=B.L)
    out[f"decode_M{decode_M}"] = {"tokens": decode_M, "seconds_per_layer_step": round(dt, 3),
                                  "us_per_layer_step": round(dt * 1e6, 1), "n_kept": nk}
    if glm:
        Sg = workloads.CONFIGS["glm45_air_shape"]
        xg = from_torch(glm["x"][:16])
        dt, nk = _oracle_pass(xg, glm["P"], Sg, glm["tau"])
        out["glm45_air_shape_T4096"] = {"tokens": 16, "seconds": round(dt, 3), "tokens_per_s": round(16 / dt, 2),
                                        "n_kept": nk, "sample": "first 16 of the 4096 prefill tokens"}
    if stack:
        Ss = stack["S"]
        per = {}
        for l, rec in sorted(stack["layers"].items()):
            xl = from_torch(rec["x"])
            dt, nk = _oracle_pass(xl, rec["P"], Ss, rec["tau"])
            per[str(l)] = {"tokens": int(xl.shape[0]), "seconds": round(dt, 3),
                           "tokens_per_s": round(xl.shape[0] / dt, 1), "n_kept": nk}
        out["stack48_layers"] = per
    return out


def measured_traffic(kernel_key):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel_key)
    if not rec:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return rec["bytes_per_launch"] if h.hexdigest() == rec["sources_sha256"] else None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    B = Bench(args)
    S = B.S
    if args.only:
        import workloads
        if args.only in ("decode",):
            tau = B.calibrate(B.P["x"], args.skip)
            dec = B.decode(tau)
            out = {"decode_us_per_layer": {str(m): round(v["us"], 2) for m, v in dec.items()},
                   "decode_isolated_us_per_layer": {str(m): round(v["isolated_us"], 2) for m, v in dec.items()},
                   "U": {str(m): v["U"] for m, v in dec.items()}}
        elif args.only == "glm":
            out = extra_prefill(B, "glm45_air_shape MoE layer prefill (Zipf router prior)",
                                workloads.CONFIGS["glm45_air_shape"], 4096, 0.5, max(10, args.steps // 2), 3)
        elif args.only == "t32k":
            out = extra_prefill(B, "qwen3_30b_a3b layer at T=32768 (MFMA-bound supplement)", S, 32768, args.skip,
                                max(5, args.steps // 4), 2, P=B.P, layer=B.layers[0])
        elif args.only == "stack":
            out = stack48(B)
        elif args.only == "calib":
            out = calibration_leg(B)
        elif args.only == "probes":
            out = {"l2_load_probe": B.l2_load_rates(), "hbm_read_ceiling": B.read_ceiling()}
        else:
            out = tables_build(B)
        print(json.dumps({"only": args.only, "result": out}), flush=True)
        return
    head = B.prefill(args.skip)
    T = S.T
    value = T / (head["ms"] * 1e-3)
    # dominant kernel: grouped gate/up GEMM (+SiLU).  Algorithmic bytes per
    # launch: the active experts' gate and up weights and the token rows; the
    # act rows it writes are implementation traffic.  Down: the active
    # experts' down weights only (act read and bf16 slot rows written are
    # implementation traffic; y is written by the combine).
    gu_bytes = head["U"] * 2 * S.H * S.I * 2 + T * S.H * 2
    gu_impl = head["n_kept"] * S.I * 2
    gu_gbs = gu_bytes / (head["gateup_ms"] * 1e-3) / 1e9
    dn_bytes = head["U"] * S.H * S.I * 2
    dn_impl = head["n_kept"] * (S.I * 2 + S.H * 2)
    layer_bytes = head["U"] * 3 * S.H * S.I * 2 + S.E * S.H * 4 + T * S.H * 4 + 8 * S.E
    layer_flops = head["n_kept"] * 6 * S.H * S.I + 2 * T * S.H * S.E
    res = {
        "metric": "ACE-skipped MoE-layer tokens/s (T=1024 prefill) + decode µs/layer, % roofline",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3_30b_a3b MoE layer prefill: T=1024 H=2048 E=128 I=768 top-8, bf16, "
                               f"{int(args.skip * 100)}% skip, {args.copies} rotated weight copies",
                   "weight_layout": args.layout,
                   "T": T, "H": S.H, "E": S.E, "I": S.I, "k": S.k, "skip_target": args.skip,
                   "skip_realized": round(1 - head["n_kept"] / (T * S.k), 5), "active_experts": head["U"],
                   "tau": [head["tau"][0], head["tau"][1]]},
        "roofline": {"bound": "hbm", "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("expert_gemm_gateup_qwen3_30b_a3b_T1024_skip60"),
                     "kernel": "expert_gemm gate/up+SiLU (grouped)", "kernel_ms": round(head["gateup_ms"], 5),
                     "alg_bytes_per_launch": gu_bytes, "impl_bytes_per_launch": gu_impl,
                     "down_kernel_ms": round(head["down_ms"], 5),
                     "down_alg_bytes_per_launch": dn_bytes, "down_impl_bytes_per_launch": dn_impl,
                     "down_achieved": round(dn_bytes / (head["down_ms"] * 1e-3) / 1e9, 1),
                     "down_frac": round(dn_bytes / (head["down_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "layer_roofline": {"alg_bytes": layer_bytes, "alg_flops": layer_flops,
                           "hbm_frac": round(layer_bytes / (head["ms"] * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                           "mfma_frac": round(layer_flops / (head["ms"] * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4),
                           "us_per_layer": round(head["ms"] * 1e3, 2)},
    }
    res["hbm_copy_ceiling_GBs"] = round(B.copy_ceiling(), 1)
    res["hbm_read_ceiling"] = B.read_ceiling()
    res["graph_launch_floor_us"] = B.launch_floor()
    res["l2_load_probe"] = B.l2_load_rates()
    if not args.no_sweep:
        sweep = {}
        for r in (0.0, 0.5):
            o = B.prefill(r, kernel_timing=False)
            sweep[str(r)] = {"tokens_per_s": round(T / (o["ms"] * 1e-3), 1), "us_per_layer": round(o["ms"] * 1e3, 2),
                             "active_experts": o["U"], "n_kept": o["n_kept"]}
        sweep[str(args.skip)] = {"tokens_per_s": res["value"], "us_per_layer": res["layer_roofline"]["us_per_layer"],
                                 "active_experts": head["U"], "n_kept": head["n_kept"]}
        res["prefill_by_skip"] = sweep
    if not args.no_decode:
        dec = B.decode(head["tau"])
        res["decode_us_per_layer"] = {str(m): round(v["us"], 2) for m, v in dec.items()}
        res["decode_eager_us_per_layer"] = {str(m): round(v["eager_us"], 2) for m, v in dec.items()}
        res["decode_isolated_us_per_layer"] = {str(m): round(v["isolated_us"], 2) for m, v in dec.items()}
        res["decode_pool"] = B.decode_pool(head["tau"])
        res["decode_detail"] = {str(m): {k2: (round(v2, 4) if isinstance(v2, float) else v2) for k2, v2 in v.items()}
                                for m, v in dec.items()}
    glm_keep = {} if not args.no_cpu_baseline else None
    stack_keep = {} if not args.no_cpu_baseline else None
    if not args.no_extra:
        import workloads
        res["glm45_air_shape_prefill"] = extra_prefill(B, "glm45_air_shape MoE layer prefill (Zipf router prior)",
                                                       workloads.CONFIGS["glm45_air_shape"], 4096, 0.5,
                                                       max(10, args.steps // 2), 3, keep=glm_keep)
        res["mfma_bound_T32768"] = extra_prefill(B, "qwen3_30b_a3b layer at T=32768 (MFMA-bound supplement)", S,
                                                 32768, args.skip, 10, 2, P=B.P, layer=B.layers[0])
        res["dense_gemm_ceiling_tflops"] = dense_gemm_ceiling(B)
    if not args.no_stack:
        res["stack48"] = stack48(B, keep=stack_keep)
    if not args.no_tables:
        res["tables_build"] = tables_build(B)
        res["calibration"] = calibration_leg(B)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(B.L, S, head["tau"], args.cpu_tokens)
        res["cpu_baseline_by_config"] = cpu_by_config(B, head["tau"], glm_keep or None, stack_keep or None)
    # release device memory before the last line, so that the process ends
    # promptly once it has printed
    del B, glm_keep, stack_keep
    import gc
    gc.collect()
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
