"""Oracle for ACE's offline per-expert tables A^GSP and A^RCR (test infrastructure).

Source: "ACE: Adaptive Calibration-Free Expert Skipping for MoE-based LLMs"
(picx.dev summary page), Methodology section 1 (Global Spectral Proxy: the two
factorisation paths a^up and a^gate, their geometric mean, layer-wise
normalisation) and section 2 (Router-Conditioned Refinement: centred router
weights, RMS-normalised directional prototype, amplification of the expert
along it), with the expert map f and x = x̄Γ of the Theoretical Foundation.

Page convention: row vectors; W^gate, W^up are H×I and W^down is I×H, so
W^gate = w_gate[e].T in the nn.Linear storage used here; Γ = diag(γ).

Readings where the page is silent (also listed in the design notes):
  * ε = 1e-6 in the layer-wise normalisations and in the prototype;
  * ρ_l (the prototype's scale) = 1, so q has unit RMS like x̄;
  * f is applied to q in the role of x̄, i.e. with Γ: f(q) uses qΓ;
  * A^RCR is normalised by the layer mean of ã^RCR exactly like A^GSP.

Pins (tests/test_oracle_tables.py): a hand-derived scalar expert, invariance
of A^GSP to a common scale of all W^down and of A^RCR to a shared translation
of the router rows (the page's stated property) and to a common scale,
‖ΓW^gate W^down‖_F against the trace identity with explicit Gram matrices,
the unit layer mean of both tables, and RCR closed forms with a gain γ ≠ 1
(a scalar expert with γ = 2 and a two-channel expert with γ = (2, 1/2)),
which fail if f(q) leaves Γ out, squares it or averages it.
"""
from __future__ import annotations

import math

import numpy as np

from .moe import as_f64, swiglu_expert


def gsp_raw(gamma, wg, wu, wd) -> float:
    """ã^GSP of one expert: sqrt(a^up · a^gate) with
    a^up = ‖ΓW^up‖_F·‖ΓW^gate W^down‖_F and a^gate = ‖ΓW^gate‖_F·‖ΓW^up W^down‖_F.
    wg, wu: [I, H]; wd: [H, I] (nn.Linear storage)."""
    G = np.diag(np.asarray(gamma, dtype=np.float64))
    Wg, Wu, Wd = wg.T, wu.T, wd.T          # H×I, H×I, I×H
    a_up = np.linalg.norm(G @ Wu) * np.linalg.norm(G @ Wg @ Wd)
    a_gate = np.linalg.norm(G @ Wg) * np.linalg.norm(G @ Wu @ Wd)
    return math.sqrt(a_up * a_gate)


def normalise(raw: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """A(e) = ã_e / (mean_j ã_j + ε): layer-wise normalisation."""
    raw = np.asarray(raw, dtype=np.float64)
    return raw / (raw.mean() + eps)


def gsp_table(gamma, w_gate, w_up, w_down, eps: float = 1e-6) -> np.ndarray:
    E = np.asarray(w_gate).shape[0]
    raw = np.array([gsp_raw(gamma, as_f64(w_gate[e]), as_f64(w_up[e]), as_f64(w_down[e])) for e in range(E)])
    return normalise(raw, eps)


def rcr_prototypes(w_router, eps: float = 1e-6, rho: float = 1.0) -> np.ndarray:
    """q_e = w̃_e / (RMS(w̃_e) + ε) · ρ with w̃_e = w_e − mean_j w_j (centred router rows)."""
    W = np.asarray(w_router, dtype=np.float64)
    Wc = W - W.mean(axis=0, keepdims=True)
    rms = np.sqrt(np.mean(Wc * Wc, axis=1, keepdims=True))
    return Wc / (rms + eps) * rho


def rcr_raw(q, gamma, wg, wu, wd, eps: float = 1e-6) -> float:
    """ã^RCR = ‖f(q)‖₂ / (‖q‖₂ + ε), f applied with q in the role of x̄."""
    f = swiglu_expert(np.asarray(q, dtype=np.float64) * np.asarray(gamma, dtype=np.float64), wg, wu, wd)
    return float(np.linalg.norm(f) / (np.linalg.norm(q) + eps))


def rcr_table(gamma, w_router, w_gate, w_up, w_down, eps: float = 1e-6, rho: float = 1.0) -> np.ndarray:
    E = np.asarray(w_gate).shape[0]
    Q = rcr_prototypes(w_router, eps, rho)
    raw = np.array([rcr_raw(Q[e], gamma, as_f64(w_gate[e]), as_f64(w_up[e]), as_f64(w_down[e]), eps)
                    for e in range(E)])
    return normalise(raw, eps)
