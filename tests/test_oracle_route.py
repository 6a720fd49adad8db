"""Pins for the oracle's routing step: scores, ordered top-k, margin, gates."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests import pins
from workloads import integer_router_case


def test_topk_hand_derived_ties():
    pins.check_topk_golden(O.topk_route, O.NONFINITE_LOGIT)


def test_topk_matches_enumeration_on_integer_ties():
    pins.check_topk_brute(O.topk_route, seed=1)
    pins.check_topk_brute(O.topk_route, seed=2)


def test_topk_set_separates_chosen_from_rest():
    rng = np.random.default_rng(3)
    s = rng.integers(-3, 4, size=(300, 16)).astype(np.float64)
    idx, _ = O.topk_route(s, 5)
    for t in range(s.shape[0]):
        chosen = set(idx[t].tolist())
        worst = idx[t][-1]
        for b in range(16):
            if b not in chosen:
                assert pins._beats(s[t], worst, b)
        assert len(chosen) == 5


def test_topk_k_equals_e_is_full_order():
    s = np.array([[0.5, -1.0, 2.0]])
    idx, _ = O.topk_route(s, 3)
    assert idx.tolist() == [[2, 0, 1]]


def test_router_logits_exact_on_integer_inputs():
    case = integer_router_case(T=12, d=7, E=5, seed=0)
    h, w = case["h"], case["w_router"]
    s = O.router_logits(h, w)
    for t in range(12):
        for e in range(5):
            exact = sum(int(h[t, i]) * int(w[i, e]) for i in range(7))
            assert s[t, e] == exact
    b = np.array([0.5, -0.25, 0.0, 1.0, -2.0], np.float32)
    assert np.array_equal(O.router_logits(h, w, b), s + b.astype(np.float64))


def test_router_margin_values():
    s = np.array([[1.0, 3.0, 3.0, 2.0], [0.0, 5.0, 1.0, -1.0]])
    assert O.router_margin(s, 1).tolist() == [0.0, 4.0]
    assert O.router_margin(s, 2).tolist() == [1.0, 1.0]
    assert np.isinf(O.router_margin(s, 4)).all()


def test_gate_closed_forms():
    pins.check_gate_closed_forms(O.gate_weights)


@pytest.mark.parametrize("mode", O.GATE_MODES)
def test_gate_sums(mode):
    rng = np.random.default_rng(5)
    s = rng.standard_normal((50, 12)) * 3
    idx, _ = O.topk_route(s, 4)
    g = O.gate_weights(s, idx, mode)
    assert (g > 0).all()
    if mode == "softmax":
        assert (g.sum(1) < 1).all()
        assert np.allclose(O.gate_weights(s, np.argsort(-s, 1), mode).sum(1), 1.0, atol=1e-12)
        # gates follow the score order
        assert (np.diff(g, axis=1) <= 0).all()
    else:
        assert np.allclose(g.sum(1), 1.0, atol=1e-12)


def test_gates_equal_scores_are_uniform():
    s = np.zeros((1, 8))
    idx, _ = O.topk_route(s, 2)
    assert np.allclose(O.gate_weights(s, idx, "softmax"), 1 / 8)
    assert np.allclose(O.gate_weights(s, idx, "softmax_topk_renorm"), 1 / 2)
    assert np.allclose(O.gate_weights(s, idx, "sigmoid_topk_renorm"), 1 / 2)
