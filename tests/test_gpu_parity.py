"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer results (top-k indices, skip masks, dispatch order) must match bit for
bit when both sides read the same float32 logits; gates too (both take them
in float64 and round once).  Outputs must reach relative L2 <= 1e-5 (f32) and
<= 1e-2 (bf16) against the float64 oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import token_adaptive_expert_amd as ace
from gpu_util import (TOL, GpuLayer, check_dispatch, check_routing_shared_logits, check_y, heavy_tail_rows,
                      oracle_thresholds, rel_l2, values)

pytestmark = pytest.mark.gpu

PATHS = [ace.ACE_PATH_GROUPED, ace.ACE_PATH_STREAM]


def oracle_y(L, g, tau_g, tau_r, tokens=None, fusion="max", norm_topk=None):
    S = L["shape"]
    return oracle.moe_layer(L["x"], L["gamma"], L["w_router"], L["router_bias"], L["w_gate"], L["w_up"], L["w_down"],
                            L["a_gsp"], L["a_rcr"], tau_g, tau_r, S.k,
                            S.norm_topk if norm_topk is None else norm_topk, S.rms_eps, S.dtype,
                            logits=g["logits"], tokens=tokens, fusion=fusion)


def check_h_and_logits(L, g, logit_atol):
    S = L["shape"]
    h_ref = oracle.rmsnorm(L["x"], L["gamma"], S.rms_eps, S.dtype)
    h_gpu = values(g["h"])
    if S.dtype == "f32":
        assert np.max(np.abs(h_gpu - h_ref)) <= 1e-6 * max(1.0, np.max(np.abs(h_ref)))
    else:
        # at most one bf16 step apart, and rarely
        diff = np.abs(h_gpu - h_ref)
        assert np.all(diff <= np.abs(h_ref) * 2.0 ** -7 + 1e-30)
        assert np.mean(diff > 0) < 1e-3
    lg_ref = oracle.router_logits(h_ref, L["w_router"], L["router_bias"]).astype(np.float64)
    assert np.max(np.abs(g["logits"].astype(np.float64) - lg_ref)) <= logit_atol


def check_slot_outputs(L, g, ref, dtype):
    """Per-slot gate-scaled expert outputs (down GEMM rows) against the oracle,
    over all of them and row by row."""
    rows, refs = [], []
    for (t, i), o in ref["slot_out"].items():
        p = g["slot_pos"][t, i]
        rows.append(values(g["slot_out"][p]))
        refs.append(o)
    if rows:
        check_y(np.stack(rows), np.stack(refs), dtype, "slot_out")


# ---------------------------------------------------------------- tiny fp32 layer
@pytest.fixture(scope="module")
def tiny():
    S = workloads.CONFIGS["tiny"]
    L = workloads.make_layer(S)
    tg, tr = oracle_thresholds(L, 0.5)
    return L, tg, tr


@pytest.mark.parametrize("path", PATHS)
def test_tiny_fp32_layer(tiny, dev, path):
    L, tg, tr = tiny
    S = L["shape"]
    g = GpuLayer(L, dev).run(tg, tr, path)
    check_h_and_logits(L, g, logit_atol=1e-5)
    idx, gate, keep = check_routing_shared_logits(L, g, tg, tr)
    check_dispatch(S, g)
    n = math.floor(0.5 * S.T * S.k + 0.5)
    assert abs(int((~keep).sum()) - n) <= 2
    ref = oracle_y(L, g, tg, tr)
    check_y(values(g["y"]), ref["y"], "f32")
    check_slot_outputs(L, g, ref, "f32")


def test_oracle_logits_fed_to_gpu(tiny, dev):
    """Reverse direction: the oracle's logits through logits_in."""
    L, tg, tr = tiny
    S = L["shape"]
    h = oracle.rmsnorm(L["x"], L["gamma"], S.rms_eps, S.dtype)
    lg = oracle.router_logits(h, L["w_router"], None)
    g = GpuLayer(L, dev).run(tg, tr, logits_in=lg)
    assert np.array_equal(g["logits"], lg)
    idx = np.stack([oracle.topk_experts(lg[t], S.k) for t in range(S.T)])
    gate = np.stack([oracle.topk_gates(lg[t], idx[t], True) for t in range(S.T)])
    keep = oracle.skip_mask(idx, gate, L["a_gsp"], L["a_rcr"], tg, tr)
    assert np.array_equal(g["topk_idx"], idx)
    assert np.array_equal(g["topk_gate"], gate)
    assert np.array_equal(g["keep"], keep)


@pytest.mark.parametrize("fusion", ["max", "min", "mean", "gsp", "rcr", "score"])
def test_fusion_rules(tiny, dev, fusion):
    L, tg, tr = tiny
    tau_g = 0.12 if fusion == "score" else tg
    g = GpuLayer(L, dev, fusion=fusion).run(tau_g, tr)
    check_routing_shared_logits(L, g, tau_g, tr, fusion=fusion)
    check_dispatch(L["shape"], g)
    ref = oracle_y(L, g, tau_g, tr, fusion=fusion)
    check_y(values(g["y"]), ref["y"], "f32")


def test_threshold_extremes(tiny, dev):
    L, _, _ = tiny
    S = L["shape"]
    gl = GpuLayer(L, dev)
    g0 = gl.run(0.0, 0.0)
    assert g0["keep"].all() and g0["offsets"][-1] == S.T * S.k     # plain top-k MoE
    ref = oracle_y(L, g0, 0.0, 0.0)
    check_y(values(g0["y"]), ref["y"], "f32")
    gi = gl.run(float("inf"), float("inf"))
    assert gi["keep"][:, 0].all() and not gi["keep"][:, 1:].any()   # only the top-1 survives
    ref = oracle_y(L, gi, np.inf, np.inf)
    check_y(values(gi["y"]), ref["y"], "f32")
    # AND, not OR: one view alone never skips
    ga = gl.run(float("inf"), 0.0)
    assert ga["keep"].all()


def test_gates_without_topk_renormalisation(tiny, dev):
    L, tg, tr = tiny
    g = GpuLayer(L, dev, norm_topk=0).run(tg, tr)
    check_routing_shared_logits(L, g, tg, tr, norm_topk=0)
    ref = oracle_y(L, g, tg, tr, norm_topk=0)
    check_y(values(g["y"]), ref["y"], "f32")


def test_deterministic_and_residual(tiny, dev):
    L, tg, tr = tiny
    gl = GpuLayer(L, dev)
    a = gl.run(tg, tr)
    b = gl.run(tg, tr)
    for n in ("y", "slot_out", "sorted_token", "slot_pos"):
        m = a["offsets"][-1] if n in ("slot_out", "sorted_token") else None
        assert np.array_equal(a[n][:m].view(np.uint8), b[n][:m].view(np.uint8)), n
    c = gl.run(tg, tr, residual=gl.P["x"])
    expect = values(a["y"]) + values(L["x"])
    assert rel_l2(values(c["y"]), expect) <= 1e-6


# ---------------------------------------------------------------- bf16, ragged and edge shapes
def _bf16_case(T, H, E, I, k, rate, cfg_id, bias=None):
    S = workloads.small_shape(T=T, H=H, E=E, I=I, k=k, dtype="bf16", cfg_id=cfg_id)
    L = workloads.make_layer(S)
    if bias is not None:
        L["router_bias"] = bias
    tg, tr = oracle_thresholds(L, rate)
    return L, tg, tr


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", [
    dict(T=100, H=256, E=24, I=256, k=5, rate=0.5, cfg_id=101),
    dict(T=1, H=128, E=16, I=128, k=4, rate=0.0, cfg_id=102),
    dict(T=33, H=128, E=256, I=128, k=16, rate=0.6, cfg_id=103),
    dict(T=70, H=384, E=8, I=384, k=1, rate=0.0, cfg_id=104),
    dict(T=130, H=512, E=40, I=640, k=8, rate=0.7, cfg_id=105),
    # >= 256 routed slots per expert: the 128-row tiles with direct-to-LDS
    # staging (ragged last tile)
    dict(T=520, H=256, E=8, I=256, k=8, rate=0.5, cfg_id=107),
    # same load with H not a multiple of 256: that tier falls back to 64-row tiles
    dict(T=520, H=384, E=8, I=128, k=8, rate=0.3, cfg_id=108),
    # chunk counts that end inside the unrolled step sequences: gate/up 8, down 10
    # (both on the 128-row tiles), and gate/up 2
    dict(T=600, H=512, E=8, I=640, k=8, rate=0.4, cfg_id=109),
    dict(T=600, H=128, E=8, I=256, k=8, rate=0.4, cfg_id=110),
])
def test_bf16_shapes(dev, path, case):
    L, tg, tr = _bf16_case(**case)
    S = L["shape"]
    g = GpuLayer(L, dev).run(tg, tr, path)
    check_h_and_logits(L, g, logit_atol=2e-3)
    check_routing_shared_logits(L, g, tg, tr)
    check_dispatch(S, g)
    ref = oracle_y(L, g, tg, tr)
    check_y(values(g["y"]), ref["y"], "bf16")
    check_slot_outputs(L, g, ref, "bf16")


@pytest.mark.parametrize("path", PATHS)
def test_one_expert_takes_every_token(dev, path):
    """A strong router bias sends all 300 tokens to expert 3: its slot rows span
    several m-tiles of both tilings."""
    E = 16
    bias = np.zeros(E, np.float32)
    bias[3] = 20.0
    L, tg, tr = _bf16_case(T=300, H=256, E=E, I=256, k=4, rate=0.4, cfg_id=106, bias=bias)
    S = L["shape"]
    g = GpuLayer(L, dev).run(tg, tr, path)
    check_routing_shared_logits(L, g, tg, tr)
    off, _, _, _ = check_dispatch(S, g)
    assert off[4] - off[3] == S.T
    ref = oracle_y(L, g, tg, tr)
    check_y(values(g["y"]), ref["y"], "bf16")


@pytest.mark.parametrize("packed", [False, True])
def test_big_tier_light_and_full_tiles(dev, packed):
    """A skewed router at >= 256 routed slots per expert (the 128-row tier):
    experts with a handful of kept rows (the light path: only their row
    blocks, a deeper weight ring), experts of 33 to 128 rows and experts of
    several m-tiles (full tiles, ragged last tiles) in one launch.  Routing
    and dispatch bit for bit; y and every slot row within the bf16 bars."""
    E = 32
    r = np.random.default_rng(5).permutation(E) + 1
    bias = (-0.4 * np.log(r)).astype(np.float32)
    L, tg, tr = _bf16_case(T=1100, H=256, E=E, I=256, k=8, rate=0.5, cfg_id=111, bias=bias)
    S = L["shape"]
    g = GpuLayer(L, dev, packed=packed).run(tg, tr)
    check_routing_shared_logits(L, g, tg, tr)
    off, _, _, _ = check_dispatch(S, g)
    n_e = np.diff(off.astype(np.int64))
    assert np.sum((n_e >= 1) & (n_e <= 32)) >= 4 and np.sum(n_e > 256) >= 2, n_e
    ref = oracle_y(L, g, tg, tr)
    check_y(values(g["y"]), ref["y"], "bf16")
    check_slot_outputs(L, g, ref, "bf16")


@pytest.mark.parametrize("packed", [False, True])
def test_light_path_same_bits_as_full_tiles(dev, packed):
    """A token's act and slot rows for an expert do not depend on whether the
    expert's tile took the light path (at most 32 rows) or a full 128-row
    tile: the same MFMA chains in the same k order.  Crafted logits route
    tokens 0..19 to experts (0, 1) in both runs; expert 0 holds those 20 rows
    in run A and 200 rows in run B (a full first m-tile)."""
    E, k, T = 4, 2, 520  # T*k >= 256*E: the 128-row tier
    L, _, _ = _bf16_case(T=T, H=256, E=E, I=256, k=k, rate=0.0, cfg_id=112)
    rng = np.random.default_rng(3)

    def logits(n0):
        lg = rng.normal(0.0, 0.1, (T, E)).astype(np.float32)
        lg[:, 0] = -10.0                 # expert 0 only where forced below
        lg[:n0, 0] = 5.0
        lg[:n0, 1] = 4.0
        return lg

    base = logits(200)
    la, lb = base.copy(), base.copy()
    la[20:200] = logits(0)[20:200]       # run A: only tokens 0..19 reach expert 0
    gl = GpuLayer(L, dev, packed=packed)
    a = gl.run(0.0, 0.0, logits_in=la)
    b = gl.run(0.0, 0.0, logits_in=lb)
    assert np.diff(a["offsets"])[0] == 20 and np.diff(b["offsets"])[0] == 200
    for t in range(20):
        i = int(np.flatnonzero(a["topk_idx"][t] == 0)[0])
        assert b["topk_idx"][t, i] == 0
        pa, pb = a["slot_pos"][t, i], b["slot_pos"][t, i]
        for n in ("act", "slot_out"):
            assert np.array_equal(a[n][pa].view(np.uint16), b[n][pb].view(np.uint16)), (n, t)


# ---------------------------------------------------------------- seeded random shapes
def _random_case(i):
    rng = np.random.default_rng(9000 + i)
    dtype = "f32" if i % 4 == 0 else "bf16"
    E = int(rng.integers(2, 65))
    k = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.integers(1, max(2, 2048 // k)))
    H = 128 * int(rng.integers(1, 5))
    I = 128 * int(rng.integers(1, 5))
    S = workloads.small_shape(T=T, H=H, E=E, I=I, k=k, dtype=dtype, cfg_id=200 + i,
                              zipf_s=float(rng.choice([0.0, 1.1])), norm_topk=int(rng.integers(0, 2)))
    path = int(rng.choice(PATHS + [ace.ACE_PATH_AUTO]))
    fusion = str(rng.choice(["max", "max", "min", "mean", "gsp", "rcr", "score"]))
    rate = float(rng.choice([0.0, 0.3, 0.6]))
    packed = dtype == "bf16" and bool(rng.integers(0, 2))
    return S, path, fusion, rate, packed


@pytest.mark.parametrize("i", range(16))
def test_random_shapes(dev, i):
    """Seeded random layers (E 2..64, k 1..16, T up to 2047 slots, H and I from
    128 to 512, f32 and bf16, Zipf or flat routers, every fusion rule and
    tiling, both weight layouts) against the oracle: routing, gates, skip mask
    and dispatch bit for bit on shared logits, y and slot rows within the
    dtype's tolerance."""
    S, path, fusion, rate, packed = _random_case(i)
    print(f"[random case {i}] {S} path={path} fusion={fusion} rate={rate} packed={packed}", flush=True)
    L = workloads.make_layer(S)
    tg, tr = oracle_thresholds(L, min(rate, (S.k - 1) / S.k))
    g = GpuLayer(L, dev, fusion=fusion, packed=packed).run(tg, tr, path)
    check_routing_shared_logits(L, g, tg, tr, fusion=fusion)
    check_dispatch(S, g)
    ref = oracle_y(L, g, tg, tr, fusion=fusion)
    check_y(values(g["y"]), ref["y"], S.dtype)
    check_slot_outputs(L, g, ref, S.dtype)


@pytest.mark.parametrize("i", range(6))
def test_random_large_batches(dev, i):
    """Seeded random layers of 1000-4200 tokens (multi-workgroup dispatch, the
    32/64-token router, 64- and 128-row tiles): routing, gates, skip mask and
    dispatch bit for bit on shared logits; y on every token."""
    rng = np.random.default_rng(77000 + i)
    E = int(rng.choice([8, 16, 64, 128, 256]))
    k = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.integers(1000, 4200))
    H, I = 128 * int(rng.integers(1, 5)), 128 * int(rng.integers(1, 5))
    dtype = "bf16" if i % 5 else "f32"
    S = workloads.small_shape(T=T, H=H, E=E, I=I, k=k, dtype=dtype, cfg_id=600 + i,
                              zipf_s=float(rng.choice([0.0, 1.1])), norm_topk=int(rng.integers(0, 2)))
    path = int(rng.choice([0, 0, 1, 2]))
    fusion = str(rng.choice(["max", "max", "min", "mean"]))
    rate = float(rng.choice([0.0, 0.5, 0.6]))
    packed = dtype == "bf16" and bool(rng.integers(0, 2))
    print(f"[large random case {i}] {S} path={path} fusion={fusion} rate={rate} packed={packed}", flush=True)
    L = workloads.make_layer(S)
    tg, tr = oracle_thresholds(L, min(rate, (k - 1) / k))
    g = GpuLayer(L, dev, fusion=fusion, packed=packed).run(tg, tr, path)
    check_routing_shared_logits(L, g, tg, tr, fusion=fusion)
    check_dispatch(S, g)
    ref = oracle_y(L, g, tg, tr, fusion=fusion)
    check_y(values(g["y"]), ref["y"], dtype)


# ---------------------------------------------------------------- full Qwen3-30B-A3B-shaped layer
@pytest.fixture(scope="module")
def qwen():
    S = workloads.CONFIGS["qwen3_30b_a3b"]
    L = workloads.make_layer(S)
    tg, tr = oracle_thresholds(L, 0.6)
    return L, tg, tr


@pytest.mark.timeout(600)
def test_qwen3_prefill_full_size(qwen, dev):
    """The headline layer: y and every slot row against the oracle on all
    1024 tokens, globally and token by token."""
    L, tg, tr = qwen
    S = L["shape"]
    gl = GpuLayer(L, dev)
    g = gl.run(tg, tr)   # AUTO: the grouped tiling at T*k = 8192
    check_h_and_logits(L, g, logit_atol=2e-3)
    check_routing_shared_logits(L, g, tg, tr)
    check_dispatch(S, g)
    skipped = int((~g["keep"]).sum())
    assert abs(skipped / (S.T * S.k) - 0.6) < 0.01
    ref = oracle_y(L, g, tg, tr)
    check_y(values(g["y"]), ref["y"], "bf16")
    check_slot_outputs(L, g, ref, "bf16")
    # the other tiling gives the same layer output
    g2 = gl.run(tg, tr, path=ace.ACE_PATH_STREAM)
    assert rel_l2(values(g2["y"]), values(g["y"])) <= 1e-2
    # the configuration bench.py times (packed expert weights, pre-split
    # router): the same accumulation order, so bit-identical results
    gp = GpuLayer(L, dev, P=gl.P, packed=True).run(tg, tr)
    for name in ("h", "logits", "topk_idx", "topk_gate", "keep", "offsets", "sorted_token", "slot_pos", "y"):
        assert np.array_equal(gp[name], g[name]), name


@pytest.mark.timeout(600)
def test_qwen3_layer_T32768_sampled(qwen, dev):
    """The MFMA-bound size (T = 32768, 262144 routed slots) in the
    configuration bench.py times (packed weights, pre-split router): the
    64-token router, block-mode dispatch and 128-row tiles.  Top-k, gates,
    skip mask and dispatch bit-exact on every token (shared logits); logits
    and y on 1024+ tokens: the first and last 128, the last 32 rows of the
    four most loaded experts (their ragged last m-tiles) and random ones."""
    L, tg, tr = qwen
    S = L["shape"].with_tokens(32768)
    Lt = dict(L, x=workloads.make_tokens(S, seed=0, step=7), shape=S)
    g = GpuLayer(Lt, dev, packed=True).run(tg, tr)
    check_routing_shared_logits(Lt, g, tg, tr)
    check_dispatch(S, g)
    rng = np.random.default_rng(32768)
    rows = set([0, 1, 63, 64, 4095, 4096, 16383, 20000, 32766, 32767]) | heavy_tail_rows(g, 4, 32)
    rows |= set(range(128)) | set(range(S.T - 128, S.T))
    rest = np.setdiff1d(np.arange(S.T), np.array(sorted(rows)))
    rows |= set(rng.choice(rest, max(0, 1024 - len(rows)), replace=False).tolist())
    rows = sorted(rows)
    assert len(rows) >= 1024
    h_ref = oracle.rmsnorm(Lt["x"][rows], L["gamma"], S.rms_eps, S.dtype)
    lg_ref = oracle.router_logits(h_ref, L["w_router"], L["router_bias"]).astype(np.float64)
    assert np.max(np.abs(g["logits"][rows].astype(np.float64) - lg_ref)) <= 2e-3
    ref = oracle_y(Lt, g, tg, tr, tokens=rows)
    check_y(values(g["y"][rows]), ref["y"][rows], "bf16")


def test_router_variants_batch_invariant(qwen, dev):
    """A token's h and logits do not depend on the batch around it: the router
    variants picked by batch size (16 experts per workgroup for small batches,
    32, then 32 or 64 tokens per workgroup from T = 2048 and 4096) and the
    linear layout (weights split on the fly) must agree bit for bit on shared
    rows, and match the oracle on sampled rows."""
    from workloads.device import make_tokens_device
    L, tg, tr = qwen
    S = L["shape"]
    x = make_tokens_device(S, dev, seed=0, step=5, T=4100)
    gl = GpuLayer(L, dev, packed=True)
    full = gl.run(tg, tr, x=x)
    lin = GpuLayer(L, dev, P=gl.P).run(tg, tr, x=x)
    assert np.array_equal(full["h"], lin["h"])
    assert np.array_equal(full["logits"].view(np.uint32), lin["logits"].view(np.uint32))
    for T in (2050, 1024, 100, 3):
        part = gl.run(tg, tr, x=x[:T].contiguous())
        assert np.array_equal(part["h"], full["h"][:T]), T
        assert np.array_equal(part["logits"].view(np.uint32), full["logits"][:T].view(np.uint32)), T
    rows = [0, 15, 16, 63, 64, 2047, 2048, 4095, 4096, 4099]
    xh = x[rows].float().cpu().numpy()
    h_ref = oracle.rmsnorm(oracle.round_to_bf16(xh), L["gamma"], S.rms_eps, S.dtype)
    diff = np.abs(values(full["h"][rows]) - h_ref)
    assert np.all(diff <= np.abs(h_ref) * 2.0 ** -7 + 1e-30)
    lg_ref = oracle.router_logits(h_ref, L["w_router"], L["router_bias"]).astype(np.float64)
    assert np.max(np.abs(full["logits"][rows].astype(np.float64) - lg_ref)) <= 4e-3


def _route_only(x, gamma, packed, bias, E, dev):
    T, H = x.shape
    d = ace._lib.make_desc(T, H, E, 128, 8, torch.bfloat16, router_layout=ace._lib.ACE_LAYOUT_PACKED)
    z = dict(device=dev)
    logits = torch.empty(T, E, dtype=torch.float32, **z)
    h = torch.empty(T, H, dtype=torch.bfloat16, **z)
    ones = torch.ones(E, dtype=torch.float32, **z)
    ace._lib.moe_route_skip(d, x, gamma, packed, bias, None, logits, ones, ones, 0.0, 0.0, h,
                            torch.empty(T, 8, dtype=torch.int32, **z), torch.empty(T, 8, dtype=torch.float32, **z),
                            torch.empty(T, 8, dtype=torch.uint8, **z))
    torch.cuda.synchronize()
    return h.view(torch.int16).cpu().numpy(), logits.cpu().numpy()


@pytest.mark.parametrize("H,E,with_bias", [(2048, 128, True), (2048, 80, False), (4096, 128, False),
                                           (4096, 72, True)])
def test_router_two_kernel_batch_invariant(dev, H, E, with_bias):
    """From 4096 tokens at H = 2048 the RMSNorm and the router product run as
    two kernels (h first, then the logits from h; at H = 4096 the 64-token
    variant serves 4133 tokens); a token's h and logits must equal, bit for
    bit, those of the variants that smaller batches take (32 tokens per
    workgroup, 16 tokens, 16-expert sub-blocks), with a ragged last token
    block and, for E = 80 and 72, expert column blocks past E; sampled rows
    also against the oracle."""
    g = torch.Generator().manual_seed(H + E)
    T = 4096 + 37
    x = (torch.randn(T, H, generator=g) * 1.5).to(torch.bfloat16)
    gamma = torch.rand(H, generator=g) + 0.5
    w_r = torch.randn(E, H, generator=g) * 0.03
    bias = (torch.randn(E, generator=g) * 0.1) if with_bias else None
    xd, gd, wd = x.to(dev), gamma.to(dev), w_r.to(dev)
    bd = bias.to(dev) if bias is not None else None
    d1 = ace._lib.make_desc(1, H, E, 128, 8, torch.bfloat16)
    packed = torch.empty(ace._lib.moe_router_packed_bytes(d1), dtype=torch.uint8, device=dev)
    ace._lib.moe_pack_router(d1, wd, packed)
    h_full, lg_full = _route_only(xd, gd, packed, bd, E, dev)
    for Tp in (2050, 1000, 5):
        h_p, lg_p = _route_only(xd[:Tp].contiguous(), gd, packed, bd, E, dev)
        assert np.array_equal(h_p, h_full[:Tp]), Tp
        assert np.array_equal(lg_p.view(np.uint32), lg_full[:Tp].view(np.uint32)), Tp
    rows = [0, 63, 64, 1000, 4095, 4096, T - 1]
    xh = x[rows].float().numpy().astype(np.float64)
    h_ref = oracle.rmsnorm(xh, gamma.numpy().astype(np.float64), 1e-6, "bf16")
    h_gpu = torch.from_numpy(h_full[rows]).view(torch.bfloat16).float().numpy()
    assert np.all(np.abs(h_gpu - h_ref) <= np.abs(h_ref) * 2.0 ** -7 + 1e-30)
    b64 = bias.numpy().astype(np.float64) if bias is not None else None
    lg_ref = oracle.router_logits(h_ref, w_r.numpy().astype(np.float64), b64)
    assert np.max(np.abs(lg_full[rows].astype(np.float64) - lg_ref)) <= 4e-3


@pytest.mark.timeout(900)
def test_glm45_air_shape_full_size(dev):
    """GLM-4.5-Air-shaped layer (H=4096, E=128, I=1408, top-8, bf16, T=4096,
    Zipf(1.1) router prior, lognormal(0,0.7) tables, 50% skip), drawn on the
    device, run in the bench configuration; thresholds from the oracle's own
    quantile mapping; every token's routing, the dispatch and the layer
    output of every token checked (the Zipf-heavy experts hold ~2100 rows,
    so their m-tiles and ragged last tiles are all covered)."""
    from workloads.device import make_layer_device, to_host
    S = workloads.CONFIGS["glm45_air_shape"]
    P = make_layer_device(S, dev, seed=0)
    L = to_host(P)
    tg, tr = oracle_thresholds(L, 0.5)
    gl = GpuLayer(L, dev, P=P, packed=True)
    g = gl.run(tg, tr)
    check_h_and_logits(L, g, logit_atol=4e-3)
    check_routing_shared_logits(L, g, tg, tr)
    check_dispatch(S, g)
    skipped = int((~g["keep"]).sum())
    assert abs(skipped / (S.T * S.k) - 0.5) < 0.01
    ref = oracle_y(L, g, tg, tr)
    check_y(values(g["y"]), ref["y"], "bf16")
    # Zipf prior: some experts receive no kept slot and are never read
    n_e = np.diff(g["offsets"].astype(np.int64))
    assert (n_e == 0).sum() > 0


@pytest.mark.parametrize("M", workloads.DECODE_M)
def test_qwen3_decode_steps(qwen, dev, M):
    """Decode batches of M fresh tokens, thresholds transferred from the
    T=1024 calibration batch."""
    L, tg, tr = qwen
    S = workloads.CONFIGS["qwen3_30b_a3b_decode"].with_tokens(M)
    x = workloads.make_tokens(S, seed=0, step=1)
    Ld = dict(L)
    Ld["x"] = x
    Ld["shape"] = S
    gl = GpuLayer(Ld, dev)
    g = gl.run(tg, tr)
    check_routing_shared_logits(Ld, g, tg, tr)
    check_dispatch(S, g)
    ref = oracle_y(Ld, g, tg, tr)
    check_y(values(g["y"]), ref["y"], "bf16")
    for path in PATHS:
        gp = gl.run(tg, tr, path=path)
        check_y(values(gp["y"]), ref["y"], "bf16")


# ---------------------------------------------------------------- fused small-batch forward
def _fused_vs_steps(layer, x, tg, tr, residual):
    M = x.shape[0]
    b1, b2 = layer.buffers(M), layer.buffers(M)
    for b in (b1, b2):
        for t in (b.act, b.slot_out, b.sorted_token, b.sorted_gate, b.slot_pos, b.offsets, b.y, b.topk_idx):
            if t.is_floating_point():
                t.fill_(float("nan"))
            else:
                t.fill_(-7)
    layer.forward(x, tg, tr, b1, residual=residual)
    layer.forward_steps(x, tg, tr, b2, residual=residual)
    torch.cuda.synchronize()
    n = int(b1.offsets[-1].item())
    assert n == int(b2.offsets[-1].item())
    for name in ("h", "logits", "topk_idx", "topk_gate", "keep", "offsets", "slot_pos", "y"):
        a1, a2 = getattr(b1, name), getattr(b2, name)
        assert torch.equal(a1.view(torch.uint8), a2.view(torch.uint8)), name
    for name in ("sorted_token", "sorted_gate", "act", "slot_out"):
        a1, a2 = getattr(b1, name)[:n], getattr(b2, name)[:n]
        assert torch.equal(a1.view(torch.uint8), a2.view(torch.uint8)), name


@pytest.mark.parametrize("M", [1, 3, 8, 9, 17, 32])
@pytest.mark.parametrize("packed", [False, True])
def test_fused_forward_matches_steps(qwen, dev, M, packed):
    """moe_forward at decode sizes (top-k, gates, skip rule and dispatch inside
    the gate/up workgroups) equals the four step calls bit for bit."""
    L, tg, tr = qwen
    S = workloads.CONFIGS["qwen3_30b_a3b_decode"].with_tokens(M)
    Ld = dict(L, x=workloads.make_tokens(S, seed=0, step=3), shape=S)
    gl = GpuLayer(Ld, dev, packed=packed)
    _fused_vs_steps(gl.layer, gl.P["x"], float(tg), float(tr), gl.P["x"])


@pytest.mark.parametrize("fusion", ["max", "min", "mean", "score"])
@pytest.mark.parametrize("T", [1, 2, 6, 30])
def test_fused_forward_matches_steps_f32(tiny, dev, fusion, T):
    L, tg, tr = tiny
    gl = GpuLayer(L, dev, fusion=fusion)
    x = gl.P["x"][:T].contiguous()
    _fused_vs_steps(gl.layer, x, float(tg), float(tr), None)


def _adversarial_logits(T, E, rng):
    """Rows that stress the selection order: exact ties (a few distinct
    values, or all equal), signed zeros among negatives, -inf entries, huge
    magnitudes and neighbours one float32 ulp apart."""
    lg = rng.standard_normal((T, E)).astype(np.float32)
    for t in range(T):
        kind = t % 8
        if kind == 0:
            lg[t] = rng.choice(np.array([-1.0, 0.0, 1.0, 2.0], np.float32), E)
        elif kind == 1:
            lg[t] = np.float32(0.75)
        elif kind == 2:
            lg[t] = -np.abs(lg[t]) - 1.0
            z = rng.choice(E, size=min(E, 6), replace=False)
            lg[t, z] = np.where(np.arange(z.size) % 2 == 0, np.float32(0.0), np.float32(-0.0))
        elif kind == 3:
            lg[t, rng.choice(E, size=E // 2, replace=False)] = -np.inf
        elif kind == 4:
            lg[t] = (lg[t] * np.float32(1e30)).astype(np.float32)
        elif kind == 5:
            base = np.float32(1.5)
            steps = rng.integers(0, 3, E)
            lg[t] = np.array([np.nextafter(base, np.float32(2), dtype=np.float32) if s_ == 1 else
                              (np.nextafter(base, np.float32(1), dtype=np.float32) if s_ == 2 else base)
                              for s_ in steps], np.float32)
        elif kind == 6:
            n = E // 2
            lg[t, 0:2 * n:2] = lg[t, 1:2 * n:2]  # pairwise ties, the lower index first
    return lg


def test_stream_tiling_beyond_its_mtile_table(dev):
    """The split-K tiling forced on a batch with more m-tiles than its LDS
    m-tile table holds (256 experts x ~8 m-tiles): it falls back to the
    expert-major list; dispatch bit-exact, outputs within the bf16 bar."""
    S = workloads.small_shape(T=4000, H=128, E=256, I=128, k=8, dtype="bf16", cfg_id=880)
    L = workloads.make_layer(S)
    g = GpuLayer(L, dev).run(0.0, 0.0, path=ace.ACE_PATH_STREAM)
    off = check_dispatch(S, g)[0]
    assert int(np.sum((np.diff(off) + 15) // 16)) > 1024
    rows = [0, 1, 999, 2000, 3998, 3999]
    ref = oracle_y(L, g, 0.0, 0.0, tokens=rows)
    check_y(values(g["y"][rows]), ref["y"][rows], "bf16")


@pytest.mark.parametrize("E,k", [(16, 4), (64, 8), (65, 8), (128, 8), (128, 16), (150, 6), (192, 16), (256, 8), (256, 1)])
@pytest.mark.parametrize("norm_topk", [True, False])
def test_topk_adversarial_logits(dev, E, k, norm_topk):
    """Top-k indices, gates and the skip mask from crafted float32 logits
    (through logits_in) equal the oracle's bit for bit, for every per-lane
    layout of the selection (1 to 4 experts per lane)."""
    T = 48
    S = workloads.small_shape(T=T, H=128, E=E, I=128, k=k, dtype="f32", cfg_id=700 + E + k)
    L = workloads.make_layer(S)
    rng = np.random.default_rng(1000 * E + k)
    lg = _adversarial_logits(T, E, rng)
    tg = tr = 0.05
    g = GpuLayer(L, dev, norm_topk=int(norm_topk)).run(tg, tr, logits_in=lg)
    idx = np.stack([oracle.topk_experts(lg[t], k) for t in range(T)])
    gate = np.stack([oracle.topk_gates(lg[t], idx[t], norm_topk) for t in range(T)])
    keep = oracle.skip_mask(idx, gate, L["a_gsp"], L["a_rcr"], tg, tr)
    assert np.array_equal(g["topk_idx"], idx)
    assert np.array_equal(g["topk_gate"].view(np.uint32), gate.view(np.uint32))
    assert np.array_equal(g["keep"], keep)


@pytest.mark.parametrize("E,k,T", [(150, 6, 7), (256, 8, 8), (65, 3, 5), (65, 3, 2), (256, 8, 1)])
def test_fused_forward_matches_steps_wide_expert_sets(dev, E, k, T):
    """The fused decode path with 2 to 4 experts per lane in its top-k."""
    S = workloads.small_shape(T=T, H=256, E=E, I=128, k=k, dtype="bf16", cfg_id=760 + E)
    L = workloads.make_layer(S)
    tg, tr = oracle_thresholds(L, 0.5)
    gl = GpuLayer(L, dev, packed=True)
    _fused_vs_steps(gl.layer, gl.P["x"], float(tg), float(tr), None)


# ---------------------------------------------------------------- multi-workgroup dispatch
@pytest.mark.parametrize("T,k,E,keep_p,skew", [
    # recount mode (1024 < T*k <= 32768: one workgroup per 1024 slots)
    (513, 2, 7, 0.5, 0.0),       # 1026 slots: the second block holds two slots
    (1001, 3, 50, 0.6, 0.0),     # 3003 slots: the batch ends inside a four-slot quad
    (1367, 5, 96, 0.5, 1.1),     # 6835 slots, ragged last quad, Zipf-like prior
    (1100, 8, 200, 0.4, 1.1),    # 8800 slots, Zipf-like expert prior, many empty experts
    (3000, 6, 256, 0.9, 0.0),    # 18000 slots, E at its maximum
    (2049, 4, 64, 0.0, 0.0),     # only top-1 slots kept
    (4096, 8, 128, 1.0, 3.0),    # 32768 slots, all kept, a few experts take most slots
    # block mode (T*k > 32768: count, scan and row kernels)
    (16385, 2, 7, 0.5, 0.0),     # 32770 slots: the last 4096-slot block holds two
    (5000, 8, 128, 0.4, 1.1),    # 40000 slots, Zipf-like prior
    (40000, 1, 16, 1.0, 0.0),    # top-1 routing only
])
def test_dispatch_large_batches(dev, T, k, E, keep_p, skew):
    """Batches of more than 1024 slots spread over several workgroups (recount
    mode up to 32768 slots, then the per-block count, scan and row kernels):
    offsets, sorted tokens and gates and slot positions must equal
    oracle.dispatch_order bit for bit.  Rows hold k distinct experts drawn by
    Gumbel top-k from a power-law prior; the workspace starts as garbage."""
    rng = np.random.default_rng(T * 1000 + E)
    prior = -skew * np.log(np.arange(1, E + 1))
    idx = np.argsort(-(rng.gumbel(size=(T, E)) + prior), axis=1)[:, :k].astype(np.int32)
    gate = rng.random((T, k)).astype(np.float32)
    keep = rng.random((T, k)) < keep_p
    keep[:, 0] = True
    d = ace.make_desc(T, 128, E, 128, k, "bf16")
    nws = ace.moe_workspace_bytes(d)
    if T * k > 32768:
        assert nws >= 8 * E * ((T * k + 4095) // 4096)
    ws = torch.full((nws,), 0x7F, dtype=torch.uint8, device=dev)
    t_idx = torch.from_numpy(idx).to(dev)
    t_gate = torch.from_numpy(gate).to(dev)
    t_keep = torch.from_numpy(keep.astype(np.uint8)).to(dev)
    off = torch.full((E + 1,), -7, dtype=torch.int32, device=dev)
    tok = torch.full((T * k,), -7, dtype=torch.int32, device=dev)
    sg = torch.full((T * k,), -7.0, dtype=torch.float32, device=dev)
    pos = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    ace.moe_dispatch(d, t_idx, t_gate, t_keep, off, tok, sg, pos, ws)
    torch.cuda.synchronize()
    r_off, r_tok, r_slot, r_pos = oracle.dispatch_order(idx, keep, E)
    n = int(r_off[-1])
    assert np.array_equal(off.cpu().numpy(), r_off)
    assert np.array_equal(tok.cpu().numpy()[:n], r_tok)
    assert np.array_equal(pos.cpu().numpy(), r_pos)
    assert np.array_equal(sg.cpu().numpy()[:n].view(np.uint32), gate[r_tok, r_slot].view(np.uint32))


# ---------------------------------------------------------------- decode expert-pool cap
@pytest.mark.parametrize("M,pool", [(1, 1), (4, 2), (8, 4), (8, 16), (32, 8), (32, 40), (64, 16), (64, 300)])
def test_decode_expert_pool(qwen, dev, M, pool):
    """Batch-level expert-pool cap in moe_dispatch against oracle.cap_expert_pool:
    the GPU routes with the oracle's own logits (logits_in); which slots run,
    the dispatch order and y must match."""
    L, tg, tr = qwen
    S = workloads.CONFIGS["qwen3_30b_a3b_decode"].with_tokens(M)
    x = workloads.make_tokens(S, seed=0, step=2)
    Ld = dict(L, x=x, shape=S)
    h = oracle.rmsnorm(x, L["gamma"], S.rms_eps, S.dtype)
    lg = oracle.router_logits(h, L["w_router"], L["router_bias"])
    ref = oracle.moe_layer(x, L["gamma"], L["w_router"], L["router_bias"], L["w_gate"], L["w_up"], L["w_down"],
                           L["a_gsp"], L["a_rcr"], tg, tr, S.k, S.norm_topk, S.rms_eps, S.dtype, logits=lg,
                           expert_pool=pool)
    for packed in (False, True):
        gl = GpuLayer(Ld, dev, packed=packed, expert_pool=pool)
        g = gl.run(tg, tr, logits_in=lg)
        assert np.array_equal(g["topk_idx"], ref["idx"])
        assert np.array_equal(g["slot_pos"] >= 0, ref["keep"]), "capped keep differs"
        off, tok, slot, pos = oracle.dispatch_order(ref["idx"], ref["keep"], S.E)
        n = int(off[-1])
        assert np.array_equal(g["offsets"], off)
        assert np.array_equal(g["sorted_token"][:n], tok)
        assert np.array_equal(g["slot_pos"], pos)
        assert np.array_equal(g["sorted_gate"][:n].view(np.uint32), ref["gate"][tok, slot].view(np.uint32))
        check_y(values(g["y"]), ref["y"], "bf16")
        U = int((np.diff(off) > 0).sum())
        assert U <= max(pool, len(set(ref["idx"][:, 0].tolist())))


# ---------------------------------------------------------------- on-device quantile mapping
def _calibrate(gl, g, rate, dev):
    S = gl.S
    T = g["topk_idx"].shape[0]
    d = gl.layer.desc(T)
    ws = torch.empty(ace.moe_calibrate_workspace_bytes(d), dtype=torch.uint8, device=dev)
    tau = torch.full((2,), -1.0, dtype=torch.float32, device=dev)
    lvl = torch.full((2,), -1, dtype=torch.int32, device=dev)
    idx = torch.from_numpy(g["topk_idx"]).to(dev)
    gate = torch.from_numpy(g["topk_gate"]).to(dev)
    ace.moe_calibrate_thresholds(d, idx, gate, gl.P["a_gsp"], gl.P["a_rcr"], rate, tau, lvl, ws)
    torch.cuda.synchronize()
    return tau.cpu().numpy(), lvl.cpu().numpy()


@pytest.mark.parametrize("rate", [0.0, 0.1, 0.3, 0.5, 0.6, 0.75])
def test_calibration_matches_oracle(tiny, dev, rate):
    L, _, _ = tiny
    S = L["shape"]
    gl = GpuLayer(L, dev)
    g = gl.run(0.0, 0.0)
    tau, lvl = _calibrate(gl, g, rate, dev)
    tg, tr, m, n = oracle.quantile_thresholds(g["topk_idx"], g["topk_gate"], L["a_gsp"], L["a_rcr"], rate)
    assert tau[0] == tg and tau[1] == tr and lvl[1] == n and (n == 0 or lvl[0] == m)
    gk = gl.run(tau[0], tau[1])
    skipped = int((~gk["keep"]).sum())
    assert skipped in (n - 1, n) if n else skipped == 0


def test_calibration_with_tied_scores(tiny, dev):
    """Equal logits make every gate 1/k, so slots of one expert tie exactly;
    ties are ranked by slot order on both sides."""
    L, _, _ = tiny
    S = L["shape"]
    gl = GpuLayer(L, dev)
    g = gl.run(0.0, 0.0, logits_in=np.zeros((S.T, S.E), np.float32))
    for rate in (0.25, 0.5):
        tau, lvl = _calibrate(gl, g, rate, dev)
        tg, tr, m, n = oracle.quantile_thresholds(g["topk_idx"], g["topk_gate"], L["a_gsp"], L["a_rcr"], rate)
        assert tau[0] == tg and tau[1] == tr and lvl[0] == m


@pytest.mark.parametrize("rate", [0.5, 0.6])
def test_calibration_full_size(qwen, dev, rate):
    L, _, _ = qwen
    gl = GpuLayer(L, dev)
    g = gl.run(0.0, 0.0)
    tau, lvl = _calibrate(gl, g, rate, dev)
    tg, tr, m, n = oracle.quantile_thresholds(g["topk_idx"], g["topk_gate"], L["a_gsp"], L["a_rcr"], rate)
    assert tau[0] == tg and tau[1] == tr and lvl[0] == m and lvl[1] == n


# ---------------------------------------------------------------- packed weight layout
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("which", ["tiny", "bf16"])
def test_packed_layout_matches_linear_bitwise(tiny, dev, path, which):
    """The packed layout only moves weight bytes; the MFMA sequence is the
    same, so every output bit must match the linear layout."""
    if which == "tiny":
        L, tg, tr = tiny
    else:
        L, tg, tr = _bf16_case(T=77, H=384, E=12, I=640, k=3, rate=0.4, cfg_id=107)
    gl = GpuLayer(L, dev)
    a = gl.run(tg, tr, path)
    gl.layer = gl.layer.packed()
    torch.cuda.synchronize()
    b = gl.run(tg, tr, path)
    n = int(a["offsets"][-1])
    assert np.array_equal(a["logits"].view(np.uint32), b["logits"].view(np.uint32))   # pre-split router (bf16)
    for name in ("act", "slot_out"):
        assert np.array_equal(a[name][:n].view(np.uint8), b[name][:n].view(np.uint8)), name
    assert np.array_equal(a["y"].view(np.uint8), b["y"].view(np.uint8))
    # the packed copy is a permutation of the linear one
    w = gl.P["w_gate"].cpu()
    pw = gl.layer.w_gate.cpu()
    assert torch.equal(torch.sort(w.reshape(-1).view(torch.int16) if w.dtype == torch.bfloat16 else w.reshape(-1))[0],
                       torch.sort(pw.reshape(-1).view(torch.int16) if pw.dtype == torch.bfloat16 else pw.reshape(-1))[0])


def test_packed_layout_formula(dev):
    """Entries of the packed layout checked against its definition in the header."""
    E, H, I = 2, 128, 256
    d = ace.make_desc(1, H, E, I, 1, "f32")
    for which, (N, K) in ((0, (I, H)), (1, (H, I))):
        src = torch.arange(E * N * K, dtype=torch.float32, device=dev).reshape(E, N, K)
        dst = torch.empty_like(src)
        ace.moe_pack_weights(d, which, src, dst)
        torch.cuda.synchronize()
        V, KS = 4, 16
        flat = dst.reshape(-1).cpu().numpy()
        lin = src.cpu().numpy()
        Ng, Kj = N // 16, K // KS
        for (e, g, j, l, v) in [(0, 0, 0, 0, 0), (1, 3, 5, 37, 2), (1, Ng - 1, Kj - 1, 63, 3), (0, 2, 1, 16, 1)]:
            idx = (((e * Ng + g) * Kj + j) * 64 + l) * V + v
            assert flat[idx] == lin[e, 16 * g + l % 16, KS * j + V * (l // 16) + v]
        assert np.array_equal(np.sort(flat), np.sort(lin.reshape(-1)))


def test_packed_router_planes_sum_exactly(dev):
    """The three bf16 planes of moe_pack_router add up to the float32 router
    weights exactly, at the positions the header defines."""
    E, H = 20, 256
    w = (torch.randn(E, H, dtype=torch.float32, device=dev) * 0.02).contiguous()
    w[3, 5] = 1.0 + 2.0 ** -9 + 2.0 ** -20  # splits into 1, 2^-9 and 2^-20: all three planes
    d = ace.make_desc(1, H, E, 128, 2, "bf16")
    dst = torch.empty(ace.moe_router_packed_bytes(d), dtype=torch.uint8, device=dev)
    ace.moe_pack_router(d, w, dst)
    torch.cuda.synchronize()
    CB, nks = (E + 15) // 16, H // 32
    planes = dst.cpu().numpy().view(np.uint16).reshape(3, CB, nks, 64, 8)
    f = (planes.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wn = w.cpu().numpy()
    for e in range(CB * 16):
        for k in range(0, H, 7):
            c, j, q, v = e // 16, k // 32, (k % 32) // 8, k % 8
            l = q * 16 + e % 16
            tot = f[0, c, j, l, v] + f[1, c, j, l, v] + f[2, c, j, l, v]
            assert tot == (float(wn[e, k]) if e < E else 0.0), (e, k)
    # w[3, 5]: column block 0, k-step 0, lane 16*(5 // 8) + 3, element 5
    assert (f[0, 0, 0, 3, 5], f[1, 0, 0, 3, 5], f[2, 0, 0, 3, 5]) == (1.0, 2.0 ** -9, 2.0 ** -20)
