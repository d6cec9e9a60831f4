"""Oracle for one MoE layer forward with ACE per-token slot skipping (test infrastructure).

Source: "ACE: Adaptive Calibration-Free Expert Skipping for MoE-based LLMs"
(picx.dev summary page).  Notation follows that page: x = x̄Γ is the RMSNorm
output, g_{t,i} the router gate of the i-th routed slot of token t,
A^GSP / A^RCR the per-expert tables, S^GSP ∩ S^RCR the skip set.

Readings where the page is silent (each also listed in the design notes):
  * the gate is a softmax over all experts' router logits, optionally
    renormalised over the k selected ones (``norm_topk``), computed in float64;
  * top-k order is (logit descending, expert index ascending), so the top-1
    slot is slot 0 and ties go to the lower index;
  * "falls below" is a strict ``<``; the two products g·A are single float32
    multiplies, compared in float32;
  * skipped slots are dropped, the remaining gates are not renormalised;
  * the RMSNorm output is stored in the activation dtype (bf16 models keep
    it in bf16), and the router reads that stored value;
  * experts use the nn.Linear layout: w_gate/w_up [E, I, H], w_down [E, H, I];
    the page's H×I matrix W^gate is w_gate[e] transposed.

Pins (tests/test_oracle_*.py): closed forms for RMSNorm, softmax, SiLU and
the scalar expert (tests/golden/scalar_expert.json), one-hot router rows,
crafted top-k ties, the page's invariants for the skip rule, hand-worked
skip masks for every fusion rule (tests/golden/skip_rule_example.json and,
for MEAN and SCORE with thresholds of unequal scale,
tests/golden/fusion_mean_score_example.json), MIN <= MEAN <= MAX ordering and
the gate-only nature of SCORE, the SwiGLU norm bound with SVD spectral norms,
a dense all-experts formulation at skip 0, and brute-force dispatch
invariants.
"""
from __future__ import annotations

import math

import numpy as np

from .pool import cap_expert_pool


def as_f64(a: np.ndarray) -> np.ndarray:
    """Values of a stored tensor as float64.  uint16 arrays hold bf16 bit patterns
    (bf16 is the upper half of an IEEE float32)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits, ties to even).

    Uses v = m·2^e with 0.5 <= |m| < 1: keep 8 bits of m.  Values here are far
    from bf16's overflow and subnormal ranges."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def store(v: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the activation dtype, returned as float64."""
    if dtype == "bf16":
        return round_to_bf16(v)
    if dtype == "f32":
        return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float, dtype: str) -> np.ndarray:
    """h = x̄Γ: each row divided by its root-mean-square, times the diagonal gain γ.

    Follows the input factorisation x = x̄Γ_l in the Theoretical Foundation
    section; the result is stored in the activation dtype."""
    xf = as_f64(x)
    h = np.empty_like(xf)
    g = np.asarray(gamma, dtype=np.float64)
    for t in range(xf.shape[0]):
        row = xf[t]
        rms = math.sqrt(float(np.mean(row * row)) + eps)
        h[t] = row / rms * g
    return store(h, dtype)


def router_logits(h: np.ndarray, w_router: np.ndarray, bias) -> np.ndarray:
    """Router logits h·W_rᵀ (+ b) in float64, returned rounded to float32.

    The page uses router gates g_{t,i} (Methodology, GSP score definition) but
    prints no router; this is the standard linear router of the MoE layer."""
    logits = as_f64(h) @ np.asarray(w_router, dtype=np.float64).T
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    return logits.astype(np.float32)


def topk_experts(logits_row: np.ndarray, k: int) -> np.ndarray:
    """The k routed experts of one token, in slot order: largest logit first,
    equal logits resolved to the lower expert index.  Slot 0 is the top-1 expert
    ("highest original router gate", Methodology section 3)."""
    l = np.asarray(logits_row, dtype=np.float32)
    order = np.argsort(-l, kind="stable")
    return order[:k].astype(np.int32)


def topk_gates(logits_row: np.ndarray, idx: np.ndarray, norm_topk: bool) -> np.ndarray:
    """Router gates g_{t,i} of the selected slots.

    Softmax of the float32 logits in float64 (shifted by the maximum logit);
    with ``norm_topk`` the gates are renormalised to sum to one over the k
    selected experts.  Sums run in ascending order (expert index, or slot
    index for the renormalisation).  Rounded to float32."""
    l = np.asarray(logits_row, dtype=np.float32).astype(np.float64)
    m = float(l.max())
    z = np.array([math.exp(float(v) - m) for v in l], dtype=np.float64)
    if norm_topk:
        s = 0.0
        for e in idx:
            s += float(z[e])
    else:
        s = 0.0
        for e in range(l.size):
            s += float(z[e])
    return np.array([z[e] / s for e in idx], dtype=np.float64).astype(np.float32)


def skip_mask(idx: np.ndarray, gate: np.ndarray, a_gsp: np.ndarray, a_rcr: np.ndarray,
              tau_gsp: float, tau_rcr: float, fusion: str = "max") -> np.ndarray:
    """keep[t, i] for all routed slots (Methodology sections 1-3).

    s^GSP = g·A^GSP(e_i) and s^RCR = g·A^RCR(e_i), each one float32 multiply.
    A view marks a slot low-contribution when its score is strictly below that
    view's threshold.  Conservative fusion (max of the two views' normalised
    scores) skips a slot only when both views mark it, i.e. the skip set is the
    intersection S^GSP ∩ S^RCR.  Slot 0, the top-1 expert, is always kept.

    ``fusion`` selects the single-view and alternative fusion rules that the
    page's ablations compare (Table 4: "gsp", "rcr"; Table 5: "min" is the
    union of the two skip sets, "mean" averages the two normalised scores
    s/τ and skips below one; "score" thresholds the bare gate against
    ``tau_gsp``)."""
    T, k = idx.shape
    keep = np.ones((T, k), dtype=bool)
    tg = np.float32(tau_gsp)
    tr = np.float32(tau_rcr)
    for t in range(T):
        for i in range(1, k):
            e = int(idx[t, i])
            g = np.float32(gate[t, i])
            sg = np.float32(g * np.float32(a_gsp[e]))
            sr = np.float32(g * np.float32(a_rcr[e]))
            low_g = bool(sg < tg)
            low_r = bool(sr < tr)
            if fusion == "max":
                skip = low_g and low_r
            elif fusion == "min":
                skip = low_g or low_r
            elif fusion == "gsp":
                skip = low_g
            elif fusion == "rcr":
                skip = low_r
            elif fusion == "mean":
                skip = (float(tg) > 0.0 and float(tr) > 0.0
                        and 0.5 * (float(sg) / float(tg) + float(sr) / float(tr)) < 1.0)
            elif fusion == "score":
                skip = bool(g < tg)
            else:
                raise ValueError(fusion)
            keep[t, i] = not skip
    return keep


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z·σ(z) = z / (1 + e^{-z})."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(h_row: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """f(x) = (SiLU(x̄ΓW^gate) ⊙ x̄ΓW^up) W^down for one token (Theoretical Foundation, eq. f).

    ``h_row`` is x̄Γ; wg, wu are [I, H] and wd is [H, I] (nn.Linear layout), so
    x̄ΓW^gate is wg @ h_row."""
    h = np.asarray(h_row, dtype=np.float64)
    a = wg @ h
    u = wu @ h
    return wd @ (silu(a) * u)


def dispatch_order(idx: np.ndarray, keep: np.ndarray, E: int):
    """Group the kept slots by expert.  Within an expert, slots follow token order.

    Returns (offsets [E+1], sorted_token [n_kept], sorted_slot [n_kept] (the
    routed slot index i), slot_pos [T, k] with -1 for skipped slots).  The page
    only names "expert dispatch"; this fixes a deterministic grouping."""
    T, k = idx.shape
    offsets = np.zeros(E + 1, dtype=np.int32)
    sorted_token, sorted_slot = [], []
    slot_pos = np.full((T, k), -1, dtype=np.int32)
    for e in range(E):
        offsets[e] = len(sorted_token)
        for t in range(T):
            for i in range(k):
                if keep[t, i] and int(idx[t, i]) == e:
                    slot_pos[t, i] = len(sorted_token)
                    sorted_token.append(t)
                    sorted_slot.append(i)
    offsets[E] = len(sorted_token)
    return offsets, np.array(sorted_token, dtype=np.int32), np.array(sorted_slot, dtype=np.int32), slot_pos


class _ExpertCache:
    """float64 copies of expert weights, made on first use."""

    def __init__(self, w_gate, w_up, w_down):
        self.w = (w_gate, w_up, w_down)
        self.cache = {}

    def __call__(self, e: int):
        if e not in self.cache:
            self.cache[e] = tuple(as_f64(w[e]) for w in self.w)
        return self.cache[e]


def moe_layer(x, gamma, w_router, router_bias, w_gate, w_up, w_down, a_gsp, a_rcr,
              tau_gsp: float, tau_rcr: float, k: int, norm_topk: bool = True, rms_eps: float = 1e-6,
              dtype: str = "f32", logits=None, tokens=None, fusion: str = "max", expert_pool: int = 0) -> dict:
    """Forward of one routed SwiGLU MoE layer with ACE slot skipping.

    y_t = Σ over kept slots i (ascending) of g_{t,i}·f_{e_i}(x_t); no residual.
    ``logits`` (float32 [T, E]) replaces the router's own logits when given, so
    that routing can be shared with another implementation.  ``tokens``
    restricts the expert computation to those token rows (y of other rows is
    left as NaN).  Returns h, logits, idx, gate, keep, y (float64) and the
    per-slot gated outputs ``slot_out[(t, i)]``.  ``expert_pool`` = m >= 1
    applies the batch-level expert-pool cap (``oracle.pool``) after the skip
    rule; the returned keep is the capped mask."""
    h = rmsnorm(x, gamma, rms_eps, dtype)
    T = h.shape[0]
    E = np.asarray(w_router).shape[0]
    if logits is None:
        logits = router_logits(h, w_router, router_bias)
    logits = np.asarray(logits, dtype=np.float32)
    idx = np.zeros((T, k), dtype=np.int32)
    gate = np.zeros((T, k), dtype=np.float32)
    for t in range(T):
        idx[t] = topk_experts(logits[t], k)
        gate[t] = topk_gates(logits[t], idx[t], norm_topk)
    keep = skip_mask(idx, gate, a_gsp, a_rcr, tau_gsp, tau_rcr, fusion)
    if expert_pool:
        keep = cap_expert_pool(idx, gate, keep, E, expert_pool)
    experts = _ExpertCache(w_gate, w_up, w_down)
    rows = range(T) if tokens is None else [int(t) for t in tokens]
    y = np.full((T, h.shape[1]), np.nan)
    slot_out = {}
    for t in rows:
        acc = np.zeros(h.shape[1], dtype=np.float64)
        for i in range(k):
            if not keep[t, i]:
                continue
            wg, wu, wd = experts(int(idx[t, i]))
            o = float(gate[t, i]) * swiglu_expert(h[t], wg, wu, wd)
            slot_out[(t, i)] = o
            acc += o
        y[t] = acc
    return {"h": h, "logits": logits, "idx": idx, "gate": gate, "keep": keep, "y": y, "slot_out": slot_out,
            "E": E}
