"""GPU parity of the offline table builder (moe_build_tables) against the
oracle's A^GSP and A^RCR ("ACE: Adaptive Calibration-Free Expert Skipping for
MoE-based LLMs", Methodology sections 1 and 2).

Tolerance.  The builder forms the Frobenius norms through I×I Gram matrices
whose MFMA products are exact (the γ²-scaled operand is split exactly into
bf16 planes; f32 weights use f32 MFMA) and accumulates each Gram entry over H
terms in float32, then sums entries in float64.  A float32 sum of H terms
errs by at most about H·2⁻²⁴ of the sum of |terms| (H = 2048: 1.2e-4) and
typically by √H·2⁻²⁴ (2.7e-6).  Each table entry is a square root of
products of such sums, divided by a mean of the same, which halves the
relative error of each factor.  RCR is a chain of float32 dot products of
length H and I.  The bar, 1e-4 relative per entry, is at the worst-case scale
of one factor and far above the typical one.  A dropped k-step, a wrong γ
power or a transposed operand moves entries by percent.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads.torch_io import layer_to_torch
import token_adaptive_expert_amd as ace

pytestmark = pytest.mark.gpu

RTOL = 1e-4


def spread_experts(L, seed=5):
    """Give the experts distinct scales (powers of two, exact in bf16) so the
    tables are far from uniform: scale w_gate[e], w_up[e], w_down[e] by
    2^a, 2^b, 2^c with small per-expert integers."""
    S = L["shape"]
    rng = np.random.default_rng(seed)
    E = S.E
    ex = rng.integers(-2, 3, size=(3, E))
    out = dict(L)
    for n, row in zip(("w_gate", "w_up", "w_down"), ex):
        v = workloads.to_float(L[n]) * (2.0 ** row)[:, None, None].astype(np.float32)
        out[n] = workloads._store(v.astype(np.float32), S.dtype)
    # shift some router rows so the prototypes differ in direction and scale
    wr = L["w_router"].copy()
    wr[: E // 2] *= np.float32(1.5)
    out["w_router"] = wr
    return out


def oracle_tables(L, eps=1e-6):
    args = (L["w_gate"], L["w_up"], L["w_down"])
    return (oracle.gsp_table(L["gamma"], *args, eps=eps),
            oracle.rcr_table(L["gamma"], L["w_router"], *args, eps=eps))


def gpu_tables(L, device, workspace_bytes=None):
    P = layer_to_torch(L, device)
    ws = None
    if workspace_bytes is not None:
        ws = torch.empty(workspace_bytes, dtype=torch.uint8, device=device)
    g, r = ace.build_tables(P["gamma"], P["w_router"], P["w_gate"], P["w_up"], P["w_down"], eps=1e-6, workspace=ws)
    torch.cuda.synchronize()
    return g.cpu().numpy(), r.cpu().numpy()


def check(L, device, **kw):
    ref_g, ref_r = oracle_tables(L)
    g, r = gpu_tables(L, device, **kw)
    assert np.all(np.isfinite(g)) and np.all(np.isfinite(r))
    eg = np.max(np.abs(g - ref_g) / ref_g)
    er = np.max(np.abs(r - ref_r) / ref_r)
    assert eg <= RTOL, f"A^GSP max rel err {eg:.3g}"
    assert er <= RTOL, f"A^RCR max rel err {er:.3g}"
    return g, r, ref_g, ref_r


@pytest.mark.parametrize("H,E,I", [(256, 16, 128), (128, 5, 256), (384, 3, 384)])
def test_tables_f32(dev, H, E, I):
    S = workloads.small_shape(T=1, H=H, E=E, I=I, k=2, dtype="f32", cfg_id=120)
    L = spread_experts(workloads.make_layer(S, seed=1))
    g, r, ref_g, ref_r = check(L, dev)
    # the spread gives tables far from uniform
    assert ref_g.max() / ref_g.min() > 4


@pytest.mark.parametrize("H,E,I", [(256, 12, 384), (512, 7, 128), (128, 20, 256)])
def test_tables_bf16(dev, H, E, I):
    S = workloads.small_shape(T=1, H=H, E=E, I=I, k=2, dtype="bf16", cfg_id=121)
    L = spread_experts(workloads.make_layer(S, seed=2))
    check(L, dev)


def test_tables_unscaled_layer(dev):
    """iid weights: A^GSP entries near 1; parity still per entry.  The layer
    mean of each table is m / (m + ε) for the raw mean m, slightly below 1
    when m is small (RCR's raw values are O(1e-2) here)."""
    S = workloads.small_shape(T=1, H=256, E=16, I=256, k=2, dtype="bf16", cfg_id=122)
    L = workloads.make_layer(S, seed=3)
    g, r, ref_g, ref_r = check(L, dev)
    assert np.all(np.abs(g - 1) < 0.05)
    assert abs(g.mean() - ref_g.mean()) < 1e-6 and abs(r.mean() - ref_r.mean()) < 1e-6
    assert 0.999 < r.mean() <= 1


def test_tables_full_width_subset(dev):
    """Qwen3-30B-A3B expert width (H=2048, I=768) on a subset of 6 experts:
    the oracle's dense products stay within seconds."""
    base = workloads.CONFIGS["qwen3_30b_a3b"]
    S = workloads.small_shape(T=1, H=base.H, E=6, I=base.I, k=2, dtype="bf16", cfg_id=123)
    L = spread_experts(workloads.make_layer(S, seed=4))
    check(L, dev)


def test_tables_batching_and_determinism(dev):
    """Smallest workspace (Gram batches of one expert) and the preferred one
    give bit-identical tables, and so do repeated calls."""
    S = workloads.small_shape(T=1, H=256, E=9, I=256, k=2, dtype="bf16", cfg_id=124)
    L = spread_experts(workloads.make_layer(S, seed=6))
    d = ace.make_desc(1, S.H, S.E, S.I, 2, "bf16")
    pref = ace.moe_tables_workspace_bytes(d)
    g1, r1 = gpu_tables(L, dev)
    g2, r2 = gpu_tables(L, dev)
    # one expert's transposed w_down: I*H*2 bytes; the rest is independent of the batch
    per = S.I * S.H * 2
    g3, r3 = gpu_tables(L, dev, workspace_bytes=pref - (S.E - 1) * per)
    for a, b in ((g1, g2), (r1, r2), (g1, g3), (r1, r3)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    ref_g, ref_r = oracle_tables(L)
    assert np.max(np.abs(g3 - ref_g) / ref_g) <= RTOL


def test_tables_feed_the_skip_rule(dev):
    """Tables built on the device drive moe_route_skip the same way as the
    oracle's tables: identical keep masks when both rules see the same gates
    (the oracle's skip rule fed with the device-built tables)."""
    S = workloads.small_shape(T=64, H=256, E=16, I=128, k=4, dtype="f32", cfg_id=125)
    L = spread_experts(workloads.make_layer(S, seed=7))
    g, r = gpu_tables(L, dev)
    from gpu_util import GpuLayer, check_routing_shared_logits
    L2 = dict(L, a_gsp=g, a_rcr=r)
    gl = GpuLayer(L2, dev)
    out = gl.run(0.05, 0.05)
    check_routing_shared_logits(L2, out, 0.05, 0.05)
