"""Planted mistakes in copies of oracle functions (CPU only): each pin must
reject the plausible bug it is meant to catch."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests import pins


def _topk_high_id_wins(logits, k):
    s = np.asarray(logits, np.float64)
    T, E = s.shape
    ids = np.broadcast_to(-np.arange(E), (T, E))
    order = np.lexsort((ids, -s), axis=1)
    return order[:, :k].astype(np.int32), 0 if np.isfinite(s).all() else O.NONFINITE_LOGIT


def _topk_ascending(logits, k):
    s = np.asarray(logits, np.float64)
    T, E = s.shape
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), s), axis=1)
    return order[:, :k].astype(np.int32), 0


def _ffn_swapped_gate_up(x, w1, w2, act):
    if act != "swiglu":
        return O.expert_ffn(x, w1, w2, act)
    dff = w2.shape[1]
    return O.expert_ffn(x, np.concatenate([w1[dff:], w1[:dff]]), w2, act)


def _ffn_sigmoid_not_silu(x, w1, w2, act):
    if act != "swiglu":
        return O.expert_ffn(x, w1, w2, act)
    dff = w2.shape[1]
    g = np.asarray(x, np.float64) @ np.asarray(w1[:dff], np.float64).T
    u = np.asarray(x, np.float64) @ np.asarray(w1[dff:], np.float64).T
    return (1 / (1 + np.exp(-g)) * u) @ np.asarray(w2, np.float64).T


def _gates_always_renorm(logits, idx, mode):
    if mode == "softmax":
        mode = "softmax_topk_renorm"
    return O.gate_weights(logits, idx, mode)


def _plan_first_choice_priority(idx, E, capacity=-1, max_rows=None, ep_size=1, ep_rank=0):
    """Fills capacity with all first choices before any second choice."""
    idx = np.asarray(idx)
    T, k = idx.shape
    p = O.dispatch_plan(idx, E, -1, max_rows)
    if capacity < 0:
        return p
    dest = np.full((T, k), -1, np.int64)
    accepted = np.zeros(E, np.int64)
    kept = np.minimum(p["counts"], capacity)
    offsets = np.concatenate([[0], np.cumsum(kept)])
    for j in range(k):
        for t in range(T):
            e = idx[t, j]
            if accepted[e] < capacity:
                dest[t, j] = offsets[e] + accepted[e]
                accepted[e] += 1
    out = dict(p)
    out.update(dest=dest, kept=kept, offsets=offsets)
    return out


def _plan_inclusive_offsets(idx, E, capacity=-1, max_rows=None, ep_size=1, ep_rank=0):
    p = O.dispatch_plan(idx, E, capacity, max_rows, ep_size, ep_rank)
    out = dict(p)
    out["offsets"] = np.concatenate([np.cumsum(p["kept"]), [p["kept"].sum()]])
    return out


def _combine_pre_permutation_index(y_perm, idx, gates, dest, lo=0, hi=None):
    """Scatters returned rows by the pre-permutation token index."""
    T, k = np.asarray(idx).shape
    y = np.zeros((T, y_perm.shape[1]))
    for t in range(T):
        for j in range(k):
            if dest[t, j] >= 0:
                y[t] += gates[t, j] * y_perm[min(t * k + j, y_perm.shape[0] - 1)]
    return y


@pytest.mark.parametrize("bad", [_topk_high_id_wins, _topk_ascending])
def test_topk_pins_reject(bad):
    with pytest.raises(AssertionError):
        pins.check_topk_golden(bad, O.NONFINITE_LOGIT)
        pins.check_topk_brute(bad)


@pytest.mark.parametrize("bad", [_ffn_swapped_gate_up, _ffn_sigmoid_not_silu])
def test_ffn_pins_reject(bad):
    with pytest.raises(AssertionError):
        pins.check_swiglu_scalar(bad)


def test_gate_pins_reject_unwanted_renormalisation():
    with pytest.raises(AssertionError):
        pins.check_gate_closed_forms(_gates_always_renorm)


@pytest.mark.parametrize("bad", [_plan_first_choice_priority, _plan_inclusive_offsets])
def test_plan_pins_reject(bad):
    with pytest.raises(AssertionError):
        pins.check_capacity_tables(bad)


def test_combine_pin_rejects_pre_permutation_scatter():
    with pytest.raises(AssertionError):
        pins.check_wrong_token_fixture(O.dispatch_plan, O.permute, _combine_pre_permutation_index)
