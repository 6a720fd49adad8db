"""GPU parity of the route stage (router GEMM, ordered top-k, gates)."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from tests.conftest import load_golden
from tests.gpu_util import (GATE_TOL, LOGIT_TOL, assert_close, certified_route_mismatch, dev,
                            host, lib, say, tdtype)
from workloads import CONFIGS, integer_router_case, make_inputs, small_layer_config

pytestmark = pytest.mark.gpu


def _topk(G, logits_np, k, gate):
    T, E = logits_np.shape
    desc = G.make_desc(T, 64, E, k, 64, "f32", gate, "swiglu")
    lg = dev(logits_np.astype(np.float32))
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    g = torch.empty((T, k), dtype=torch.float32, device="cuda")
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")
    G.topk_from_logits(desc, lg, idx, g, fl)
    torch.cuda.synchronize()
    return host(idx), host(g), int(host(fl)[0])


def test_topk_hand_derived_ties():
    G = lib()
    for c in load_golden("topk_ties.json")["cases"]:
        s = np.array([c["logits"]], np.float32)
        idx, _, fl = _topk(G, s, c["k"], "softmax")
        assert idx.tolist() == [c["idx"]], c
        assert bool(fl & G.FLAG_NONFINITE_LOGIT) == bool(c.get("nonfinite", False)), c


@pytest.mark.parametrize("E", [1, 2, 3, 4, 5, 8, 16, 31, 32, 64, 100, 128, 256, 512, 1024])
def test_topk_stage_exact_with_ties(E):
    """Scores rounded to one decimal (many exact ties, signed zeros): the GPU
    ordered ids must equal the oracle's on the same float32 scores."""
    G = lib()
    rng = np.random.default_rng(E)
    T = 333
    s = np.round(rng.standard_normal((T, E)) * 2, 1).astype(np.float32)
    s[rng.random((T, E)) < 0.05] = -0.0
    for k in sorted({1, min(E, 2), min(E, 8), min(E, 16)}):
        for gate in O.GATE_MODES:
            idx, g, fl = _topk(G, s, k, gate)
            ref, _ = O.topk_route(s, k)
            assert np.array_equal(idx, ref), (E, k, gate)
            assert_close(g, O.gate_weights(s.astype(np.float64), ref, gate), GATE_TOL,
                         f"gates E={E} k={k} {gate}")
            assert fl == 0


@pytest.mark.parametrize("E,k", [(4, 2), (8, 2), (128, 8), (256, 8), (64, 16)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_router_exact_on_integer_inputs(E, k, dtype):
    """Integer-valued h and W_r make every score an exact integer in any
    summation order: logits and the ordered routing must match exactly."""
    G = lib()
    T, d = 300, 128
    case = integer_router_case(T, d, E, seed=E + k)
    bias = np.zeros(E, np.float32)
    bias[::3] = 0.5
    desc = G.make_desc(T, d, E, k, 64, dtype, "softmax", "swiglu")
    dt = tdtype(dtype)
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    g = torch.empty((T, k), dtype=torch.float32, device="cuda")
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = G.alloc_workspace(desc)
    G.route(desc, dev(case["h"], dt), dev(case["w_router"], dt), dev(bias), lg, idx, g, fl, ws)
    torch.cuda.synchronize()
    ref = O.router_logits(case["h"], case["w_router"], bias)
    assert np.array_equal(host(lg).astype(np.float64), ref)
    ref_idx, _ = O.topk_route(ref, k)
    assert np.array_equal(host(idx), ref_idx)
    assert_close(host(g), O.gate_weights(ref, ref_idx, "softmax"), GATE_TOL, "gates")


@pytest.mark.parametrize("name", list(CONFIGS))
def test_router_layer_shapes(name):
    """Each layer's router at its real d and E (fewer tokens): scores within
    tolerance of float64, ordered ids exactly the oracle's top-k of the GPU
    scores, sets equal to the float64 routing except certified near ties."""
    G = lib()
    base = CONFIGS[name]
    cfg = small_layer_config(base, min(base.T, 1000))
    inp = make_inputs(cfg)
    say(f"route {name} T={cfg.T} d={cfg.d} E={cfg.E}")
    desc = G.make_desc(cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff, cfg.dtype, cfg.gate, cfg.act,
                       ep_size=cfg.ep_size, ep_rank=cfg.ep_rank)
    dt = tdtype(cfg.dtype)
    lg = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device="cuda")
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    g = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")
    bias = None if inp["bias"] is None else dev(inp["bias"])
    G.route(desc, dev(inp["h"], dt), dev(inp["w_router"], dt), bias, lg, idx, g, fl,
            G.alloc_workspace(desc))
    torch.cuda.synchronize()
    s64 = O.router_logits(inp["h"], inp["w_router"], inp["bias"])
    s32 = host(lg)
    assert_close(s32, s64, LOGIT_TOL, "logits")
    gi = host(idx)
    ref_on_gpu_scores, _ = O.topk_route(s32, cfg.k)
    assert np.array_equal(gi, ref_on_gpu_scores)
    near = certified_route_mismatch(gi, s32, s64, cfg.k)
    say(f"  certified near ties: {near}")
    assert len(near) <= max(2, cfg.T // 1000)
    # gates: both sides on the same float32 scores agree to the gate tolerance
    g = host(g).astype(np.float64)
    assert_close(g, O.gate_weights(s32.astype(np.float64), gi, cfg.gate), GATE_TOL,
                 "gates on the GPU scores")
    # against the float64 scores the gates move with the score error: for all
    # three forms |dg_j| <= g_j (|ds_j| + sum_i g_i |ds_i|) <= 2 max_e |ds_e| to
    # first order (softmax and normalised logistic have d log g_j / d s_i
    # bounded by delta_ij - g_i in size), so each token's bound is twice its
    # largest score error, plus the gate tolerance for the float32 arithmetic
    ds = np.abs(s32.astype(np.float64) - s64).max(axis=1, keepdims=True)
    gap = np.abs(g - O.gate_weights(s64, gi, cfg.gate))
    assert (gap <= 2 * ds + GATE_TOL).all(), float((gap - 2 * ds).max())
    assert int(host(fl)[0]) == 0


@pytest.mark.parametrize("E,k", [(8, 2), (16, 8), (256, 8), (512, 16)])
def test_sigmoid_gates_for_scores_far_below_zero(E, k):
    """Normalised logistic gates when the chosen scores lie far below zero,
    where the logistic itself underflows in float32 (below about -88): the
    gates are still finite and equal the float64 oracle's; also when a
    token's chosen scores straddle zero by hundreds."""
    G = lib()
    rng = np.random.default_rng(E * 7 + k)
    T = 200
    s = rng.uniform(-300.0, -100.0, (T, E)).astype(np.float32)
    s[T // 2:, 0] = rng.uniform(50.0, 400.0, T - T // 2).astype(np.float32)
    s[::7] = np.round(s[::7], 0)          # some exact ties among the far scores
    idx, g, fl = _topk(G, s, k, "sigmoid_topk_renorm")
    ref, _ = O.topk_route(s, k)
    assert np.array_equal(idx, ref)
    assert np.isfinite(g).all()
    assert_close(g, O.gate_weights(s.astype(np.float64), ref, "sigmoid_topk_renorm"), GATE_TOL,
                 f"far sigmoid gates E={E} k={k}")
    assert fl == 0
