"""Pins of the CPU oracle against closed forms, the page's invariants and brute force.

Source of every rule: "ACE: Adaptive Calibration-Free Expert Skipping for
MoE-based LLMs" (picx.dev summary page): Theoretical Foundation (x = x̄Γ, eq. f,
the SwiGLU norm bound), Methodology sections 1-3 (s = g·A, max-fusion,
top-1 kept).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_unit_rms_without_gain():
    x = np.random.default_rng(1).standard_normal((5, 96)).astype(np.float32) * 3.0
    h = oracle.rmsnorm(x, np.ones(96), 0.0, "f32")
    rms = np.sqrt(np.mean(h * h, axis=1))
    assert np.allclose(rms, 1.0, rtol=1e-6)
    # direction preserved: h is a positive multiple of x
    cos = np.sum(h * x, axis=1) / np.linalg.norm(h, axis=1) / np.linalg.norm(x, axis=1)
    assert np.allclose(cos, 1.0, rtol=1e-6)


def test_rmsnorm_gain_is_diagonal():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 64)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, 64)
    h1 = oracle.rmsnorm(x, np.ones(64), 1e-6, "f32")
    hg = oracle.rmsnorm(x, g, 1e-6, "f32")
    assert np.allclose(hg, h1 * g, rtol=1e-6)


def test_rmsnorm_bf16_store_matches_independent_rounding():
    # the oracle's frexp/rint rounding against the input module's integer bit rounding
    v = np.random.default_rng(3).standard_normal(20000).astype(np.float32) * 7.0
    a = oracle.round_to_bf16(v.astype(np.float64))
    b = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(v)).astype(np.float64)
    assert np.array_equal(a, b)
    # ties to even: 1+2^-8 lies halfway between 1 and 1+2^-7
    assert oracle.round_to_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    assert oracle.round_to_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6


# ---------------------------------------------------------------- router
def test_router_one_hot_rows_select_columns():
    rng = np.random.default_rng(4)
    H, E = 12, 5
    W = rng.standard_normal((E, H)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    for j in (0, 7, 11):
        h = np.zeros((1, H))
        h[0, j] = 1.0
        assert np.array_equal(oracle.router_logits(h, W, b)[0], (W[:, j].astype(np.float64) + b).astype(np.float32))
    assert np.array_equal(oracle.router_logits(np.zeros((1, H)), W, None)[0], np.zeros(E, np.float32))


# ---------------------------------------------------------------- top-k
@pytest.mark.parametrize("logits,k,expect", [
    ([1.0, 3.0, 3.0, 2.0], 2, [1, 2]),
    ([1.0, 3.0, 3.0, 2.0], 1, [1]),
    ([0.0, 0.0, 0.0, 0.0], 3, [0, 1, 2]),
    ([-1.0, -5.0, -1.0, -0.5], 3, [3, 0, 2]),
    ([2.0, 1.0, 2.0, 1.0, 2.0], 4, [0, 2, 4, 1]),
])
def test_topk_crafted_ties(logits, k, expect):
    assert list(oracle.topk_experts(np.array(logits, np.float32), k)) == expect


def test_topk_brute_force_properties():
    rng = np.random.default_rng(5)
    for _ in range(200):
        E = int(rng.integers(2, 20))
        k = int(rng.integers(1, E + 1))
        l = rng.integers(-3, 4, E).astype(np.float32)  # many exact ties
        idx = list(oracle.topk_experts(l, k))
        assert len(set(idx)) == k
        # order: logit descending, equal logits by ascending index
        for a, b in zip(idx, idx[1:]):
            assert l[a] > l[b] or (l[a] == l[b] and a < b)
        # nothing unselected beats a selected one; at the cut, lower indices won
        rest = [e for e in range(E) if e not in idx]
        for e in rest:
            for s in idx:
                assert l[e] < l[s] or (l[e] == l[s] and e > s)


# ---------------------------------------------------------------- gates
def test_gates_closed_forms():
    E, k = 8, 3
    eq = np.zeros(E, np.float32)
    idx = oracle.topk_experts(eq, k)
    assert np.allclose(oracle.topk_gates(eq, idx, False), 1.0 / E, rtol=0, atol=1e-8)
    assert np.allclose(oracle.topk_gates(eq, idx, True), 1.0 / k, rtol=0, atol=1e-8)
    # two-way: logit gap d gives a gate ratio e^d
    l = np.array([1.5, -0.25], np.float32)
    g = oracle.topk_gates(l, np.array([0, 1]), True)
    assert abs(float(g[0]) / float(g[1]) - math.exp(1.75)) < 1e-6 * math.exp(1.75)
    assert abs(float(g[0]) - 1.0 / (1.0 + math.exp(-1.75))) < 1e-7


def test_gates_against_library_softmax_and_shift():
    rng = np.random.default_rng(6)
    for _ in range(20):
        E = int(rng.integers(2, 130))
        k = int(rng.integers(1, min(E, 16) + 1))
        l = (rng.standard_normal(E) * 2).astype(np.float32)
        idx = oracle.topk_experts(l, k)
        full = scipy.special.softmax(l.astype(np.float64))
        assert np.allclose(oracle.topk_gates(l, idx, False), full[idx].astype(np.float32), rtol=2e-7, atol=0)
        part = scipy.special.softmax(l[idx].astype(np.float64))
        gn = oracle.topk_gates(l, idx, True)
        assert np.allclose(gn, part.astype(np.float32), rtol=2e-7, atol=0)
        assert abs(float(np.sum(gn.astype(np.float64))) - 1.0) < 1e-6
    # huge logits must not overflow: the softmax is shifted by the maximum
    big = np.array([1e4, 1e4 - 1, -1e4], np.float32)
    g = oracle.topk_gates(big, np.array([0, 1]), True)
    assert np.all(np.isfinite(g)) and abs(float(g[0]) - 1 / (1 + math.exp(-1))) < 1e-7


# ---------------------------------------------------------------- SiLU and the expert
def test_silu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 30.0, -800.0, 800.0])
    s = oracle.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 1 / (1 + math.exp(-1))) < 1e-15
    assert abs(s[2] - (-1) / (1 + math.e)) < 1e-15
    assert abs(s[3] - 30.0) < 1e-10 and s[4] == 0.0 and s[5] == 800.0
    w = np.linspace(-20, 20, 401)
    assert np.all(np.abs(oracle.silu(w)) <= np.abs(w))  # the page's |SiLU(z)| <= |z|


def test_scalar_expert_golden():
    d = json.load(open(os.path.join(GOLDEN, "scalar_expert.json")))
    for c in d["cases"]:
        x = np.array([c["x"]], np.float64)
        h = oracle.rmsnorm(x, np.array(c["gamma"]), c["eps"], "f32")[0]
        assert np.allclose(h, c["h"], rtol=1e-7, atol=0), c["name"]
        f = oracle.swiglu_expert(np.array(c["h"]), np.array(c["w_gate"]), np.array(c["w_up"]), np.array(c["w_down"]))
        assert np.allclose(f, c["f"], rtol=1e-13, atol=1e-13), c["name"]


def test_swiglu_spectral_bound():
    """||f(x)|| <= ||x̄||²·||ΓW^gate||₂·||ΓW^up||₂·||W^down||₂ (Theoretical Foundation), SVD norms."""
    S = workloads.CONFIGS["tiny"]
    L = workloads.make_layer(S)
    xf = workloads.to_float(L["x"]).astype(np.float64)
    h = oracle.rmsnorm(L["x"], L["gamma"], S.rms_eps, "f32")
    xbar = h / L["gamma"].astype(np.float64)
    G = np.diag(L["gamma"].astype(np.float64))
    worst = 0.0
    for e in range(S.E):
        wg, wu, wd = (oracle.as_f64(L[n][e]) for n in ("w_gate", "w_up", "w_down"))
        s_g = np.linalg.svd(G @ wg.T, compute_uv=False)[0]   # page's H×I matrix ΓW^gate
        s_u = np.linalg.svd(G @ wu.T, compute_uv=False)[0]
        s_d = np.linalg.svd(wd.T, compute_uv=False)[0]       # page's I×H matrix W^down
        for t in range(S.T):
            f = oracle.swiglu_expert(h[t], wg, wu, wd)
            bound = float(xbar[t] @ xbar[t]) * s_g * s_u * s_d
            assert np.linalg.norm(f) <= bound * (1 + 1e-6)
            worst = max(worst, np.linalg.norm(f) / bound)
    assert worst > 0.0
    del xf


def test_layer_at_zero_threshold_is_plain_topk_moe():
    """τ = 0 keeps every slot: the layer is the ordinary top-k MoE, here in an
    independent dense form y = Σ_e M[:, e]·F_e with F_e over all tokens."""
    S = workloads.small_shape(T=24, H=32, E=6, I=16, k=3)
    L = workloads.make_layer(S)
    out = oracle.moe_layer(L["x"], L["gamma"], L["w_router"], None, L["w_gate"], L["w_up"], L["w_down"],
                           L["a_gsp"], L["a_rcr"], 0.0, 0.0, S.k, True, S.rms_eps, "f32")
    assert out["keep"].all()
    h = out["h"]
    M = np.zeros((S.T, S.E))
    for t in range(S.T):
        l = out["logits"][t].astype(np.float64)
        top = np.argsort(-l, kind="stable")[:S.k]
        w = np.exp(l[top] - l.max())
        M[t, top] = w / w.sum()
    y = np.zeros((S.T, S.H))
    for e in range(S.E):
        wg, wu, wd = (L[n][e].astype(np.float64) for n in ("w_gate", "w_up", "w_down"))
        A = h @ wg.T
        F = ((A / (1 + np.exp(-A))) * (h @ wu.T)) @ wd.T
        y += M[:, e:e + 1] * F
    assert np.allclose(out["y"], y, rtol=1e-6, atol=1e-9)


def test_layer_output_is_linear_in_gate_and_down():
    S = workloads.small_shape(T=6, H=16, E=4, I=8, k=2)
    L = workloads.make_layer(S)
    args = lambda wd: (L["x"], L["gamma"], L["w_router"], None, L["w_gate"], L["w_up"], wd, L["a_gsp"], L["a_rcr"],
                       0.0, 0.0, S.k, True, S.rms_eps, "f32")
    y1 = oracle.moe_layer(*args(L["w_down"]))["y"]
    y2 = oracle.moe_layer(*args(L["w_down"] * np.float32(2.0)))["y"]
    assert np.allclose(y2, 2 * y1, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- skip rule
def test_skip_rule_golden():
    d = json.load(open(os.path.join(GOLDEN, "skip_rule_example.json")))
    for tok in d["tokens"]:
        idx = np.array([tok["idx"]], np.int32)
        g = np.array([tok["gate"]], np.float32)
        for fusion in ("max", "min", "gsp", "rcr"):
            keep = oracle.skip_mask(idx, g, np.array(d["a_gsp"], np.float32), np.array(d["a_rcr"], np.float32),
                                    d["tau_gsp"], d["tau_rcr"], fusion)
            assert list(keep[0]) == tok["keep_" + fusion], fusion



def test_fusion_mean_and_score_golden():
    """Hand-worked MEAN and SCORE cases (Fusion Strategy Ablation, Table 5;
    the gate-only "Score" baseline of Table 1), with the thresholds of the
    two views 32x apart so that a mean of raw scores, a sum instead of a
    mean, or a max/min in place of the mean each decide some slot wrongly."""
    d = json.load(open(os.path.join(GOLDEN, "fusion_mean_score_example.json")))
    a_g, a_r = np.array(d["a_gsp"], np.float32), np.array(d["a_rcr"], np.float32)
    for tok in d["tokens"]:
        idx = np.array([tok["idx"]], np.int32)
        g = np.array([tok["gate"]], np.float32)
        for fusion in ("max", "min", "mean", "gsp", "rcr", "score"):
            tg = d["tau_score"] if fusion == "score" else d["tau_gsp"]
            keep = oracle.skip_mask(idx, g, a_g, a_r, tg, d["tau_rcr"], fusion)
            assert list(keep[0]) == tok["keep_" + fusion], fusion


def test_mean_rule_lies_between_min_and_max():
    """Averaging the two normalised scores: a slot MAX skips (both ratios
    below one) MEAN skips too, and a slot MEAN skips MIN skips too; MEAN is
    symmetric in the two views; a zero threshold makes MEAN skip nothing."""
    rng = np.random.default_rng(17)
    idx, g, a_g, a_r = _random_slots(rng)
    for tg, tr in ((0.1, 0.2), (0.05, 0.3), (0.2, 0.06), (0.02, 2.0)):
        k_max = oracle.skip_mask(idx, g, a_g, a_r, tg, tr, "max")
        k_mean = oracle.skip_mask(idx, g, a_g, a_r, tg, tr, "mean")
        k_min = oracle.skip_mask(idx, g, a_g, a_r, tg, tr, "min")
        assert np.all(k_mean <= k_max) and np.all(k_min <= k_mean)
        assert np.array_equal(k_mean, oracle.skip_mask(idx, g, a_r, a_g, tr, tg, "mean"))
        assert k_mean[:, 0].all()
        sg = (g * a_g[idx]).astype(np.float64)
        sr = (g * a_r[idx]).astype(np.float64)
        r = 0.5 * (sg / np.float32(tg) + sr / np.float32(tr))
        clear = np.abs(r - 1.0) > 1e-6
        clear[:, 0] = False
        assert np.array_equal(~k_mean[clear], (r < 1.0)[clear])
    assert oracle.skip_mask(idx, g, a_g, a_r, 0.0, 0.3, "mean").all()
    assert oracle.skip_mask(idx, g, a_g, a_r, 0.3, 0.0, "mean").all()


def test_score_rule_reads_the_gate_alone():
    """The "Score" baseline thresholds the router gate itself: changing either
    table, or the second threshold, changes nothing; the skipped slots are
    exactly the non-top-1 slots whose gate is below the threshold."""
    rng = np.random.default_rng(18)
    idx, g, a_g, a_r = _random_slots(rng)
    for tau in (0.05, 0.1, 0.2):
        base = oracle.skip_mask(idx, g, a_g, a_r, tau, 0.1, "score")
        expect = np.ones_like(base)
        expect[:, 1:] = ~(g[:, 1:] < np.float32(tau))
        assert np.array_equal(base, expect)
        assert 0 < (~base).sum() < base[:, 1:].size
        for ag2, ar2, tr2 in ((a_g * 100, a_r, 0.1), (a_g, a_r * 1e-3, 0.1), (a_r, a_g, 5.0)):
            assert np.array_equal(base, oracle.skip_mask(idx, g, ag2.astype(np.float32), ar2.astype(np.float32),
                                                         tau, tr2, "score"))


def _random_slots(rng, T=200, E=16, k=4):
    l = rng.standard_normal((T, E)).astype(np.float32)
    idx = np.stack([oracle.topk_experts(l[t], k) for t in range(T)])
    g = np.stack([oracle.topk_gates(l[t], idx[t], True) for t in range(T)])
    a_g = rng.lognormal(0, 0.5, E).astype(np.float32)
    a_r = rng.lognormal(0, 0.5, E).astype(np.float32)
    return idx, g, a_g, a_r


def test_skip_rule_invariants():
    rng = np.random.default_rng(7)
    idx, g, a_g, a_r = _random_slots(rng)
    inf = float("inf")
    assert oracle.skip_mask(idx, g, a_g, a_r, 0.0, 0.0).all()          # τ = 0 skips nothing
    assert oracle.skip_mask(idx, g, a_g, a_r, inf, 0.0).all()          # AND, not OR
    assert oracle.skip_mask(idx, g, a_g, a_r, 0.0, inf).all()
    only_top1 = oracle.skip_mask(idx, g, a_g, a_r, inf, inf)
    assert only_top1[:, 0].all() and not only_top1[:, 1:].any()        # top-1 always kept
    for tg, tr in ((0.1, 0.2), (0.05, 0.3), (0.2, 0.06)):
        keep = oracle.skip_mask(idx, g, a_g, a_r, tg, tr)
        assert keep[:, 0].all()
        sg = g.astype(np.float64) * a_g[idx]
        sr = g.astype(np.float64) * a_r[idx]
        fused = np.maximum(sg / tg, sr / tr)           # the page's max criterion on normalised scores
        clear = np.abs(fused - 1.0) > 1e-5
        clear[:, 0] = False
        assert np.array_equal(~keep[clear], (fused < 1.0)[clear])
        # intersection of the single-view skip sets
        kg = oracle.skip_mask(idx, g, a_g, a_r, tg, tr, "gsp")
        kr = oracle.skip_mask(idx, g, a_g, a_r, tg, tr, "rcr")
        assert np.array_equal(~keep, (~kg) & (~kr))
        assert np.array_equal(~oracle.skip_mask(idx, g, a_g, a_r, tg, tr, "min"), (~kg) | (~kr))


# ---------------------------------------------------------------- dispatch
def test_dispatch_invariants_brute_force():
    rng = np.random.default_rng(8)
    for _ in range(30):
        T, E = int(rng.integers(0, 50)), int(rng.integers(1, 12))
        k = int(rng.integers(1, E + 1))
        idx = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
        keep = rng.random((T, k)) < 0.6
        off, tok, slot, pos = oracle.dispatch_order(idx, keep, E)
        assert off[0] == 0 and off[E] == keep.sum() and np.all(np.diff(off) >= 0)
        for e in range(E):
            seg = tok[off[e]:off[e + 1]]
            assert np.all(np.diff(seg) > 0)      # tokens strictly ascending per expert
            assert len(seg) == int(((idx == e) & keep).sum())
        for p in range(len(tok)):
            t, i = tok[p], slot[p]
            assert keep[t, i] and pos[t, i] == p
        assert np.all(pos[~keep] == -1)


def test_skip_rule_is_strictly_below():
    """A score equal to its threshold does not "fall below" it: the slot is kept."""
    idx = np.array([[0, 1]], np.int32)
    g = np.array([[0.5, 0.5]], np.float32)
    a = np.array([1.0, 1.0], np.float32)
    assert oracle.skip_mask(idx, g, a, a, 0.5, 0.5).all()
    assert not oracle.skip_mask(idx, g, a, a, np.nextafter(np.float32(0.5), np.float32(1)), 0.75)[0, 1]
