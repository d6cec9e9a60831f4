"""Pins of the quantile-mapping threshold oracle.

Source: "ACE: Adaptive Calibration-Free Expert Skipping for MoE-based LLMs"
(picx.dev summary page), Efficiency Results (Table 6, quantile mapping) and
Methodology section 3 (max-fusion, top-1 kept).
"""
import math

import numpy as np
import pytest

import oracle
import workloads


def _slots(seed, T=150, E=16, k=4, sigma=0.5):
    rng = np.random.default_rng(seed)
    l = rng.standard_normal((T, E)).astype(np.float32)
    idx = np.stack([oracle.topk_experts(l[t], k) for t in range(T)])
    g = np.stack([oracle.topk_gates(l[t], idx[t], True) for t in range(T)])
    return idx, g, rng.lognormal(0, sigma, E).astype(np.float32), rng.lognormal(0, sigma, E).astype(np.float32)


@pytest.mark.parametrize("rate", [0.0, 0.1, 0.3, 0.4, 0.5, 0.6, 0.7, 0.75])
def test_skipped_count_hits_target(rate):
    idx, g, a_g, a_r = _slots(1)
    T, k = idx.shape
    tg, tr, m, n = oracle.quantile_thresholds(idx, g, a_g, a_r, rate)
    keep = oracle.skip_mask(idx, g, a_g, a_r, tg, tr)
    skipped = int((~keep).sum())
    assert n == math.floor(rate * T * k + 0.5)
    assert skipped in (n - 1, n) if n > 0 else skipped == 0
    assert keep[:, 0].all()


def test_extremes():
    idx, g, a_g, a_r = _slots(2)
    tg, tr, m, n = oracle.quantile_thresholds(idx, g, a_g, a_r, 0.0)
    assert tg == 0.0 and tr == 0.0
    T, k = idx.shape
    tg, tr, m, n = oracle.quantile_thresholds(idx, g, a_g, a_r, (k - 1) / k)
    keep = oracle.skip_mask(idx, g, a_g, a_r, tg, tr)
    assert keep[:, 0].all() and not keep[:, 1:].any()
    with pytest.raises(ValueError):
        oracle.quantile_thresholds(idx, g, a_g, a_r, 0.9)


def test_selected_set_is_fused_rank_set_brute_force():
    """For each target, the slots skipped by the two thresholds are exactly the
    eligible slots whose larger view-rank is below m."""
    idx, g, a_g, a_r = _slots(3, T=30, E=8, k=3)
    T, k = idx.shape
    sg = np.array([[float(np.float32(g[t, i] * a_g[idx[t, i]])) for i in range(1, k)] for t in range(T)]).reshape(-1)
    sr = np.array([[float(np.float32(g[t, i] * a_r[idx[t, i]])) for i in range(1, k)] for t in range(T)]).reshape(-1)
    N = sg.size
    # brute-force ranks: number of slots that come before in (score, slot order)
    rg = np.array([sum(1 for j in range(N) if (sg[j], j) < (sg[s], s)) for s in range(N)])
    rr = np.array([sum(1 for j in range(N) if (sr[j], j) < (sr[s], s)) for s in range(N)])
    prev = None
    for n in range(0, N + 1):
        tg, tr, m, nn = oracle.quantile_thresholds(idx, g, a_g, a_r, n / (T * k))
        assert nn == n
        keep = oracle.skip_mask(idx, g, a_g, a_r, tg, tr)
        skipped = ~keep[:, 1:].reshape(-1)
        expect = np.maximum(rg, rr) < m
        assert np.array_equal(skipped, expect)
        # m is the largest level whose fused set fits the target
        assert expect.sum() <= n
        if n > 0:   # n = 0 short-cuts to τ = 0
            assert m == N or (np.maximum(rg, rr) < m + 1).sum() > n
        if prev is not None:
            assert np.all(skipped[prev])   # nested as the target grows
        prev = skipped


def test_tiny_workload_realizes_half():
    S = workloads.CONFIGS["tiny"]
    L = workloads.make_layer(S, with_experts=False)
    h = oracle.rmsnorm(L["x"], L["gamma"], S.rms_eps, "f32")
    lg = oracle.router_logits(h, L["w_router"], None)
    idx = np.stack([oracle.topk_experts(lg[t], S.k) for t in range(S.T)])
    g = np.stack([oracle.topk_gates(lg[t], idx[t], True) for t in range(S.T)])
    tg, tr, m, n = oracle.quantile_thresholds(idx, g, L["a_gsp"], L["a_rcr"], 0.5)
    keep = oracle.skip_mask(idx, g, L["a_gsp"], L["a_rcr"], tg, tr)
    assert n == S.T * S.k // 2 and int((~keep).sum()) in (n - 1, n)
