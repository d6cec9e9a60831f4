"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads
from workloads.torch_io import from_torch, layer_to_torch
import token_adaptive_expert_amd as ace


def oracle_thresholds(L: dict, rate: float):
    """τ from the oracle's own routing of L's tokens (quantile mapping)."""
    S = L["shape"]
    if rate <= 0:
        return np.float32(0.0), np.float32(0.0)
    h = oracle.rmsnorm(L["x"], L["gamma"], S.rms_eps, S.dtype)
    lg = oracle.router_logits(h, L["w_router"], L["router_bias"])
    idx = np.stack([oracle.topk_experts(lg[t], S.k) for t in range(S.T)])
    g = np.stack([oracle.topk_gates(lg[t], idx[t], S.norm_topk) for t in range(S.T)])
    tg, tr, _, _ = oracle.quantile_thresholds(idx, g, L["a_gsp"], L["a_rcr"], rate)
    return tg, tr


class GpuLayer:
    """The HIP path on one layer.  ``P``: the layer's device tensors when they
    were drawn on the device (else copied from L); ``packed``: run with the
    packed expert weights and pre-split router, the configuration bench.py
    times."""

    def __init__(self, L: dict, device, fusion="max", norm_topk=None, P=None, packed=False, expert_pool=0):
        S = L["shape"]
        self.S = S
        self.P = layer_to_torch(L, device) if P is None else P
        P = self.P
        self.layer = ace.AceMoeLayer(P["gamma"], P["w_router"], P["router_bias"], P["w_gate"], P["w_up"],
                                     P["w_down"], P["a_gsp"], P["a_rcr"], S.k,
                                     S.norm_topk if norm_topk is None else norm_topk, fusion, S.rms_eps,
                                     expert_pool=expert_pool)
        if packed:
            self.layer = self.layer.packed()

    def run(self, tau_g, tau_r, path=ace.ACE_PATH_AUTO, logits_in=None, x=None, residual=None) -> dict:
        x = self.P["x"] if x is None else x
        T = x.shape[0]
        b = self.layer.buffers(T)
        # poison outputs so that unwritten entries show up
        for t in (b.act, b.slot_out, b.sorted_token, b.slot_pos, b.offsets, b.y):
            if t.is_floating_point():
                t.fill_(float("nan"))
            else:
                t.fill_(-7)
        li = None if logits_in is None else torch.from_numpy(np.ascontiguousarray(logits_in)).to(x.device)
        self.layer.forward(x, float(tau_g), float(tau_r), b, path, logits_in=li, residual=residual)
        torch.cuda.synchronize()
        out = {n: from_torch(getattr(b, n)) for n in ("h", "logits", "topk_idx", "topk_gate", "keep", "offsets",
                                                     "sorted_token", "sorted_gate", "slot_pos", "act", "slot_out",
                                                     "y")}
        out["keep"] = out["keep"].astype(bool)
        return out


def values(a: np.ndarray) -> np.ndarray:
    """Stored activation values as float64."""
    return oracle.as_f64(a)


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# The parity bar on layer outputs: relative L2 over the whole output, and a
# looser bound on every token's own row, so that one wrong row (a bad tile
# edge, a stale slot) cannot hide inside a large, otherwise correct output.
TOL = {"f32": 1e-5, "bf16": 1e-2}
TOKEN_TOL = {"f32": 1e-4, "bf16": 2e-2}


def check_y(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "y") -> float:
    """got, ref: [rows, H] values (float64).  Returns the worst row's error."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape and got.ndim == 2
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    g = rel_l2(got, ref)
    assert g <= TOL[dtype], f"{what}: rel-L2 {g:.3g} > {TOL[dtype]}"
    num = np.linalg.norm(got - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-300)
    per = num / den
    worst = int(np.argmax(per)) if per.size else -1
    if per.size:
        assert per[worst] <= TOKEN_TOL[dtype], f"{what}: row {worst} rel-L2 {per[worst]:.3g} > {TOKEN_TOL[dtype]}"
    return float(per[worst]) if per.size else 0.0


def check_routing_shared_logits(L: dict, g: dict, tau_g, tau_r, fusion="max", norm_topk=None):
    """The oracle's top-k, gates and skip mask on the GPU's own float32 logits
    must equal the GPU's bit for bit."""
    S = L["shape"]
    nt = S.norm_topk if norm_topk is None else norm_topk
    lg = g["logits"]
    T = lg.shape[0]
    idx = np.stack([oracle.topk_experts(lg[t], S.k) for t in range(T)]).reshape(T, S.k)
    gate = np.stack([oracle.topk_gates(lg[t], idx[t], nt) for t in range(T)]).reshape(T, S.k)
    keep = oracle.skip_mask(idx, gate, L["a_gsp"], L["a_rcr"], tau_g, tau_r, fusion)
    assert np.array_equal(g["topk_idx"], idx), "top-k indices differ"
    assert np.array_equal(g["topk_gate"].view(np.uint32), gate.view(np.uint32)), "gates differ"
    assert np.array_equal(g["keep"], keep), "skip masks differ"
    return idx, gate, keep


def check_dispatch(S, g: dict):
    off, tok, slot, pos = oracle.dispatch_order(g["topk_idx"], g["keep"], S.E)
    n = int(off[-1])
    assert np.array_equal(g["offsets"], off), "expert offsets differ"
    assert np.array_equal(g["sorted_token"][:n], tok), "sorted tokens differ"
    assert np.array_equal(g["slot_pos"], pos), "slot positions differ"
    expect_gate = g["topk_gate"][tok, slot] if n else np.zeros(0, np.float32)
    assert np.array_equal(g["sorted_gate"][:n].view(np.uint32), expect_gate.view(np.uint32))
    return off, tok, slot, pos


def heavy_tail_rows(g: dict, n_experts: int = 3, rows: int = 16) -> set:
    """Tokens of the last rows of the most loaded experts (the last, ragged
    m-tiles of their segments), from the GPU's own dispatch."""
    off = g["offsets"].astype(np.int64)
    n_e = np.diff(off)
    out = set()
    for e in np.argsort(-n_e, kind="stable")[:n_experts]:
        lo = max(int(off[e]), int(off[e + 1]) - rows)
        out.update(int(t) for t in g["sorted_token"][lo:int(off[e + 1])])
    return out
