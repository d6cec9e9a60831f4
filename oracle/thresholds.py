"""Oracle for ACE's per-layer thresholds by quantile mapping (test infrastructure).

Source: "ACE: Adaptive Calibration-Free Expert Skipping for MoE-based LLMs"
(picx.dev summary page), Efficiency Results (Table 6: thresholds are built by
quantile mapping) and Methodology section 3 (max-fusion; a slot is skipped only
if both views mark it; the top-1 slot is kept).  The article page on ACE adds
that thresholds are matched to the workload (calibrated on its own tokens).

The page does not spell out quantile mapping.  Reading used here: the scores
of the eligible slots (every routed slot except the top-1) are ranked within
each view (ascending, ties by slot order t, then i).  Each slot's fused rank is
the larger of its two view ranks, which is max-fusion applied to the two
empirical quantiles.  A target skip rate ρ (over all T·k routed slots) asks for
n = floor(ρ·T·k + 1/2) skipped slots; the quantile level m is the largest with
#{fused rank < m} <= n, and each view's threshold τ_v is placed strictly
between its (m-1)-th and m-th smallest scores, so that "s_v < τ_v in both
views" selects exactly the slots whose fused rank is below m.

Pins (tests/test_oracle_thresholds.py): the skipped count lies in {n-1, n}
(adding one quantile step adds at most two slots), the selected set equals
the brute-force fused-rank set for every m on small inputs, ρ = 0 gives
τ = 0 and ρ = (k-1)/k skips every eligible slot.
"""
from __future__ import annotations

import math

import numpy as np


def slot_scores(idx: np.ndarray, gate: np.ndarray, a_table: np.ndarray) -> np.ndarray:
    """s[t, i] = g_{t,i}·A(e_{t,i}) as one float32 multiply (Methodology sections 1 and 2)."""
    T, k = idx.shape
    s = np.zeros((T, k), dtype=np.float32)
    for t in range(T):
        for i in range(k):
            s[t, i] = np.float32(np.float32(gate[t, i]) * np.float32(a_table[int(idx[t, i])]))
    return s


def _cut_between(lo: np.float32, hi: np.float32) -> np.float32:
    """A float32 threshold τ with lo < τ <= hi (midpoint, forced above lo)."""
    tau = np.float32((float(lo) + float(hi)) * 0.5)
    if not tau > lo:
        tau = np.nextafter(np.float32(lo), np.float32(np.inf))
    return np.float32(tau)


def quantile_thresholds(idx: np.ndarray, gate: np.ndarray, a_gsp: np.ndarray, a_rcr: np.ndarray,
                        skip_rate: float):
    """(τ^GSP, τ^RCR, m, n) for a target skip rate over the given routed slots."""
    T, k = idx.shape
    N = T * (k - 1)
    n = int(math.floor(skip_rate * T * k + 0.5))
    if n > N:
        raise ValueError("skip rate above (k-1)/k: the top-1 slot is never skipped")
    if n == 0 or N == 0:
        return np.float32(0.0), np.float32(0.0), 0, n
    sg = slot_scores(idx, gate, a_gsp)[:, 1:].reshape(-1)   # eligible slots in (t, i) order
    sr = slot_scores(idx, gate, a_rcr)[:, 1:].reshape(-1)
    order_g = np.argsort(sg, kind="stable")
    order_r = np.argsort(sr, kind="stable")
    rank_g = np.empty(N, dtype=np.int64)
    rank_r = np.empty(N, dtype=np.int64)
    rank_g[order_g] = np.arange(N)
    rank_r[order_r] = np.arange(N)
    fused = np.maximum(rank_g, rank_r)
    m = N if n >= N else int(np.sort(fused)[n])
    taus = []
    for s, order in ((sg, order_g), (sr, order_r)):
        srt = s[order]
        if m >= N:
            taus.append(np.nextafter(np.float32(srt[N - 1]), np.float32(np.inf)))
        else:
            taus.append(_cut_between(srt[m - 1], srt[m]))
    return np.float32(taus[0]), np.float32(taus[1]), m, n
