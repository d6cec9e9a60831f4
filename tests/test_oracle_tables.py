"""Pins of the GSP / RCR table oracle.

Source: "ACE: Adaptive Calibration-Free Expert Skipping for MoE-based LLMs"
(picx.dev summary page), Methodology sections 1 (GSP) and 2 (RCR).
"""
import math

import numpy as np

import oracle
import workloads


def test_gsp_scalar_experts_closed_form():
    """H = I = 1: a^up = |γw_u|·|γw_g w_d| = a^gate, so ã = γ²|w_g w_u w_d|.
    Experts (3,5,7) and (1,1,1) with γ = 2 give ã = 420 and 4, A = ã / 212."""
    gamma = np.array([2.0])
    wg = np.array([[[3.0]], [[1.0]]])
    wu = np.array([[[5.0]], [[1.0]]])
    wd = np.array([[[7.0]], [[1.0]]])
    assert oracle.gsp_raw(gamma, wg[0], wu[0], wd[0]) == 420.0
    A = oracle.gsp_table(gamma, wg, wu, wd, eps=0.0)
    assert np.allclose(A, [420.0 / 212.0, 4.0 / 212.0], rtol=1e-15)


def test_gsp_two_paths_differ_and_use_the_right_factors():
    """H = I = 2 hand case.  Γ = diag(1, 2); W^gate = I₂ (H×I), W^up rows (1,1),(0,0),
    W^down = diag(3, 4).  ‖ΓW^up‖ = √2, ΓW^gate W^down = diag(3, 8) -> √73,
    ‖ΓW^gate‖ = √5, ΓW^up W^down = [[3,4],[0,0]] -> 5.  a^up = √146, a^gate = 5√5."""
    gamma = np.array([1.0, 2.0])
    Wg = np.eye(2)
    Wu = np.array([[1.0, 1.0], [0.0, 0.0]])
    Wd = np.diag([3.0, 4.0])
    raw = oracle.gsp_raw(gamma, Wg.T, Wu.T, Wd.T)   # storage is the transpose
    assert abs(raw - math.sqrt(math.sqrt(146.0) * 5.0 * math.sqrt(5.0))) < 1e-12


def _layer(seed=0):
    S = workloads.small_shape(T=4, H=64, E=6, I=32, k=2, cfg_id=120 + seed)
    return S, workloads.make_layer(S)


def test_gsp_frobenius_trace_identity():
    S, L = _layer()
    g = L["gamma"].astype(np.float64)
    for e in range(S.E):
        Wg, Wd = L["w_gate"][e].astype(np.float64).T, L["w_down"][e].astype(np.float64).T
        direct = np.linalg.norm(np.diag(g) @ Wg @ Wd) ** 2
        gram = np.sum((Wg.T @ np.diag(g * g) @ Wg) * (Wd @ Wd.T))
        assert abs(direct - gram) <= 1e-12 * direct


def test_gsp_invariant_to_common_down_scale_and_mean_one():
    S, L = _layer(1)
    A = oracle.gsp_table(L["gamma"], L["w_gate"], L["w_up"], L["w_down"], eps=0.0)
    A2 = oracle.gsp_table(L["gamma"], L["w_gate"], L["w_up"], L["w_down"] * np.float32(4.0), eps=0.0)
    assert np.allclose(A, A2, rtol=1e-12)
    assert abs(A.mean() - 1.0) < 1e-12
    # scaling one expert's down projection scales its raw score
    wd = L["w_down"].copy()
    wd[2] *= np.float32(2.0)
    raw0 = oracle.gsp_raw(L["gamma"], L["w_gate"][2], L["w_up"][2], L["w_down"][2])
    raw1 = oracle.gsp_raw(L["gamma"], L["w_gate"][2], L["w_up"][2], wd[2])
    assert abs(raw1 / raw0 - 2.0) < 1e-12


def test_rcr_prototypes_and_translation_invariance():
    S, L = _layer(2)
    W = L["w_router"].astype(np.float64)
    Q = oracle.rcr_prototypes(W, eps=0.0)
    assert np.allclose(np.sqrt(np.mean(Q * Q, axis=1)), 1.0)       # unit RMS (ρ = 1)
    Wc = W - W.mean(axis=0)
    cos = np.sum(Q * Wc, axis=1) / np.linalg.norm(Q, axis=1) / np.linalg.norm(Wc, axis=1)
    assert np.allclose(cos, 1.0)                                     # along the centred router row
    shift = np.random.default_rng(3).standard_normal(S.H)
    A = oracle.rcr_table(L["gamma"], W, L["w_gate"], L["w_up"], L["w_down"], eps=0.0)
    A_shift = oracle.rcr_table(L["gamma"], W + shift[None, :], L["w_gate"], L["w_up"], L["w_down"], eps=0.0)
    A_scale = oracle.rcr_table(L["gamma"], W * 3.0, L["w_gate"], L["w_up"], L["w_down"], eps=0.0)
    assert np.allclose(A, A_shift, rtol=1e-10) and np.allclose(A, A_scale, rtol=1e-10)
    assert abs(A.mean() - 1.0) < 1e-12


def test_rcr_scalar_expert_closed_form():
    """H = I = 1, two experts with router rows (1) and (-1): centred rows ±1,
    q = ±1.  γ = 1, expert 0 (w_g, w_u, w_d) = (ln 3, 2, 4): f(1) = 6·ln 3,
    ã₀ = 6 ln 3.  Expert 1 (ln 3, 2, 4) too: f(-1) = SiLU(-ln 3)·(-2)·4 =
    (-ln3/(1+3))·(-8) = 2 ln 3, ã₁ = 2 ln 3.  A = (1.5, 0.5)."""
    gamma = np.array([1.0])
    W = np.array([[1.0], [-1.0]])
    w = np.array([[[math.log(3.0)]], [[math.log(3.0)]]])
    u = np.array([[[2.0]], [[2.0]]])
    d = np.array([[[4.0]], [[4.0]]])
    A = oracle.rcr_table(gamma, W, w, u, d, eps=0.0)
    assert np.allclose(A, [1.5, 0.5], rtol=1e-14)


def test_rcr_scalar_experts_with_gain_closed_form():
    """The gain Γ enters f(q) (Methodology section 2 with x = x̄Γ of the
    Theoretical Foundation: q plays x̄).  H = I = 1, γ = 2, router rows (1) and
    (-1) -> q = ±1, so the expert sees qγ = ±2.  Both experts have
    (w_g, w_u, w_d) = (ln 3 / 2, 1, 1): expert 0 gets gate pre-activation
    ln 3 and up value 2, SiLU(ln 3)·2 = (3/4)·ln 3·2, so ã₀ = 1.5 ln 3;
    expert 1 gets -ln 3 and -2, SiLU(-ln 3)·(-2) = (-ln 3/4)·(-2), so
    ã₁ = 0.5 ln 3.  Without γ the two raw values would be SiLU(±ln 3 / 2)·(±1)
    and their ratio √3 instead of 3."""
    gamma = np.array([2.0])
    W = np.array([[1.0], [-1.0]])
    w = np.full((2, 1, 1), math.log(3.0) / 2.0)
    one = np.ones((2, 1, 1))
    Q = oracle.rcr_prototypes(W, eps=0.0)
    assert np.array_equal(Q, [[1.0], [-1.0]])
    assert abs(oracle.rcr_raw(Q[0], gamma, w[0], one[0], one[0], eps=0.0) - 1.5 * math.log(3.0)) < 1e-14
    assert abs(oracle.rcr_raw(Q[1], gamma, w[1], one[1], one[1], eps=0.0) - 0.5 * math.log(3.0)) < 1e-14
    assert np.allclose(oracle.rcr_table(gamma, W, w, one, one, eps=0.0), [1.5, 0.5], rtol=1e-14)


def test_rcr_gain_is_applied_per_channel():
    """H = 2, I = 1 hand case with an uneven gain γ = (2, 1/2) and q = (1, 1):
    qΓ = (2, 1/2).  w_g = (ln 3 / 4, ln 3) gives pre-activation ln 3/2 + ln 3/2
    = ln 3; w_u = (1, 2) gives up value 2 + 1 = 3; SiLU(ln 3)·3 = (9/4) ln 3.
    w_d = (3, 4)ᵀ: f = (9/4) ln 3·(3, 4), |f| = (45/4) ln 3, |q| = √2.
    A gain left out or squared changes the pre-activation to (5/4) ln 3, and
    one replaced by its mean to (25/16) ln 3."""
    gamma = np.array([2.0, 0.5])
    q = np.array([1.0, 1.0])
    wg = np.array([[math.log(3.0) / 4.0, math.log(3.0)]])
    wu = np.array([[1.0, 2.0]])
    wd = np.array([[3.0], [4.0]])
    expect = 45.0 / 4.0 * math.log(3.0) / math.sqrt(2.0)
    assert abs(oracle.rcr_raw(q, gamma, wg, wu, wd, eps=0.0) - expect) < 1e-13
