"""Pins for the oracle's expert FFN, grouped FFN, combine and whole layer."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from tests import pins
from workloads import (CONFIGS, identity_scale_experts, make_inputs, marker_tokens,
                       small_layer_config)


def test_expert_scalar_closed_forms():
    pins.check_swiglu_scalar(O.expert_ffn)


def test_identity_scale_experts_are_exact():
    w1, w2 = identity_scale_experts(32, [1, 2, 4, 8])
    x = np.random.default_rng(0).standard_normal((10, 32))
    for e, c in enumerate([1, 2, 4, 8]):
        assert np.array_equal(O.expert_ffn(x, w1[e], w2[e], "relu"), c * x)


def test_single_expert_layer_reduces_to_library_swiglu_ffn():
    """E=1, k=1: every gate is 1 and the layer is a plain SwiGLU FFN, which
    torch's own silu and matmul evaluate independently."""
    rng = np.random.default_rng(1)
    T, d, dff = 9, 16, 24
    h = rng.standard_normal((T, d))
    w1 = rng.standard_normal((1, 2 * dff, d)) / 4
    w2 = rng.standard_normal((1, d, dff)) / 5
    wr = rng.standard_normal((d, 1))
    for gate in O.GATE_MODES:
        out = O.layer(h, wr, None, w1, w2, k=1, gate=gate, act="swiglu")
        ht = torch.from_numpy(h)
        g = torch.nn.functional.silu(ht @ torch.from_numpy(w1[0, :dff]).T)
        u = ht @ torch.from_numpy(w1[0, dff:]).T
        ref = ((g * u) @ torch.from_numpy(w2[0]).T).numpy()
        assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12), gate


def test_grouped_ffn_matches_row_by_row():
    rng = np.random.default_rng(2)
    E, d, dff = 5, 8, 6
    offsets = np.array([0, 3, 3, 7, 12, 13])
    x = rng.standard_normal((13, d))
    w1 = rng.standard_normal((E, 2 * dff, d))
    w2 = rng.standard_normal((E, d, dff))
    y = O.grouped_ffn(x, offsets, w1, w2, "swiglu")
    for e in range(E):
        for r in range(offsets[e], offsets[e + 1]):
            assert np.allclose(y[r], O.expert_ffn(x[r:r + 1], w1[e], w2[e], "swiglu")[0], atol=1e-12)


def _tiny(**over):
    cfg = CONFIGS["tiny_fp32"]
    inp = make_inputs(cfg)
    inp.update(over)
    return cfg, inp


def test_tiny_layer_equals_per_token_brute_force():
    cfg, inp = _tiny()
    out = O.layer(inp["h"], inp["w_router"], None, inp["w1"], inp["w2"], k=cfg.k,
                  gate=cfg.gate, act=cfg.act)
    bf = O.brute_force_tokens(inp["h"], inp["w_router"], None, inp["w1"], inp["w2"],
                              range(cfg.T), k=cfg.k, gate=cfg.gate, act=cfg.act)
    assert np.allclose(out["y"], bf, rtol=1e-12, atol=1e-12)
    assert out["flags"] == 0


def test_markers_through_identity_experts():
    """One-hot markers + experts f_e(h) = c_e h with distinct c_e: y_t must be
    (sum_j g_{t,j} c_{e_j}) h_t, so a wrong token or a gate attached to the
    wrong row changes the support or the magnitude."""
    cfg = CONFIGS["tiny_fp32"]
    scales = np.array([1.0, 2.0, 4.0, 8.0])
    w1, w2 = identity_scale_experts(cfg.d, scales)
    h = marker_tokens(cfg.T, cfg.d)
    wr = make_inputs(cfg)["w_router"]
    out = O.layer(h, wr, None, w1, w2, k=cfg.k, gate=cfg.gate, act="relu")
    coef = (out["gates"] * scales[out["idx"]]).sum(1)
    assert np.allclose(out["y"], coef[:, None] * h, rtol=1e-13, atol=0)
    assert (np.count_nonzero(out["y"], axis=1) == 1).all()


@pytest.mark.parametrize("cap", [0, 3, 20, 33])
def test_capacity_layer_equals_sequential_brute_force(cap):
    cfg, inp = _tiny()
    out = O.layer(inp["h"], inp["w_router"], None, inp["w1"], inp["w2"], k=cfg.k,
                  gate=cfg.gate, act=cfg.act, capacity=cap)
    bf = O.brute_force_tokens(inp["h"], inp["w_router"], None, inp["w1"], inp["w2"],
                              range(cfg.T), k=cfg.k, gate=cfg.gate, act=cfg.act, capacity=cap)
    assert np.allclose(out["y"], bf, rtol=1e-12, atol=1e-12)
    if cap == 0:
        assert not out["y"].any()


def test_expert_parallel_share_equals_brute_force_of_local_experts():
    base = CONFIGS["tiny_fp32"]
    cfg = small_layer_config(base, 40, E=8, ep_size=2, ep_rank=1)
    inp = make_inputs(cfg)            # local experts 4..7 only
    out = O.layer(inp["h"], inp["w_router"], None, inp["w1"], inp["w2"], k=2,
                  gate="sigmoid_topk_renorm", act="relu", ep_size=2, ep_rank=1)
    bf = O.brute_force_tokens(inp["h"], inp["w_router"], None, inp["w1"], inp["w2"],
                              range(40), k=2, gate="sigmoid_topk_renorm", act="relu",
                              ep_size=2, ep_rank=1)
    assert np.allclose(out["y"], bf, rtol=1e-12, atol=1e-12)
    # tokens with no local expert get nothing
    none_local = ~((out["idx"] >= 4).any(1))
    assert not out["y"][none_local].any()


def test_route_replay_uses_given_table():
    cfg, inp = _tiny()
    table = np.tile(np.array([[3, 1]], np.int32), (cfg.T, 1))
    out = O.layer(inp["h"], inp["w_router"], None, inp["w1"], inp["w2"], k=2,
                  gate=cfg.gate, act=cfg.act, route_idx=table)
    assert out["counts"].tolist() == [0, cfg.T, 0, cfg.T]
    bf = O.brute_force_tokens(inp["h"], inp["w_router"], None, inp["w1"], inp["w2"],
                              range(cfg.T), k=2, gate=cfg.gate, act=cfg.act, route_idx=table)
    assert np.allclose(out["y"], bf, rtol=1e-12, atol=1e-12)


def test_small_swiglu_layer_sampled_brute_force():
    cfg = small_layer_config(CONFIGS["finegrained_bf16"], 256, d=64, d_ff=32)
    inp = make_inputs(cfg)
    out = O.layer(inp["h"], inp["w_router"], inp["bias"], inp["w1"], inp["w2"], k=cfg.k,
                  gate=cfg.gate, act=cfg.act, capacity=O.capacity_from_factor(1.25, 256, 8, 128))
    toks = [0, 1, 17, 100, 255]
    bf = O.brute_force_tokens(inp["h"], inp["w_router"], inp["bias"], inp["w1"], inp["w2"], toks,
                              k=cfg.k, gate=cfg.gate, act=cfg.act,
                              capacity=O.capacity_from_factor(1.25, 256, 8, 128))
    assert np.allclose(out["y"][toks], bf, rtol=1e-12, atol=1e-12)
