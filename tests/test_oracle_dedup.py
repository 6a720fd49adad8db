"""Pins for the oracle's deduplicated expert-parallel packing (dedup_pack):
a hand-derived table, two special cases that reduce to independently pinned
results, invariants on random routing, and a planted ordering mistake."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.conftest import load_golden


def test_hand_derived_table_and_capacity_case():
    g = load_golden("dedup_pack.json")
    idx = np.array(g["idx"])
    plan = O.dispatch_plan(idx, g["E"])
    r = O.dedup_pack(idx, plan["dest"], g["E"], g["ep_size"])
    assert r["pair_dest"].tolist() == g["pair_dest"]
    assert r["pair_token"].tolist() == g["pair_token"]
    assert r["pair_splits"].tolist() == g["pair_splits"]
    assert r["pair_displs"].tolist() == g["pair_displs"]
    assert int(r["pair_splits"].sum()) == g["send_rows"] < g["assignments"]
    c = g["capacity_case"]
    plan = O.dispatch_plan(idx, g["E"], capacity=c["capacity"])
    r = O.dedup_pack(idx, plan["dest"], g["E"], g["ep_size"])
    assert r["pair_dest"].tolist() == c["pair_dest"]
    assert r["pair_token"].tolist() == c["pair_token"]
    assert r["pair_splits"].tolist() == c["pair_splits"]


def _routes(rng, T, E, k):
    return np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])


def test_one_expert_per_rank_reduces_to_the_plan():
    """With one expert per rank every pair is one assignment and pairs sort
    as (expert, token): the dedup rows are the plan's rows."""
    rng = np.random.default_rng(3)
    idx = _routes(rng, 97, 8, 3)
    plan = O.dispatch_plan(idx, 8)
    r = O.dedup_pack(idx, plan["dest"], 8, 8)
    assert np.array_equal(r["pair_dest"], plan["dest"])
    assert np.array_equal(r["pair_token"], plan["src_token"])
    assert np.array_equal(r["pair_splits"], plan["counts"])


def test_one_rank_sends_each_token_once():
    rng = np.random.default_rng(4)
    idx = _routes(rng, 50, 16, 4)
    idx[7] = -1                      # a token with no valid slot sends nothing
    plan = O.dispatch_plan(idx, 16)
    r = O.dedup_pack(idx, plan["dest"], 16, 1)
    sent = sorted(set(np.nonzero((plan["dest"] >= 0).any(1))[0].tolist()))
    assert r["pair_token"].tolist() == sent
    for t in range(50):
        want = sent.index(t) if t in sent else -1
        assert all(v == (want if plan["dest"][t, j] >= 0 else -1)
                   for j, v in enumerate(r["pair_dest"][t]))


@pytest.mark.parametrize("seed,cap", [(5, -1), (6, 3), (7, 0)])
def test_invariants_on_skewed_routing(seed, cap):
    rng = np.random.default_rng(seed)
    T, E, k, ep = 300, 32, 6, 4
    w = np.arange(1, E + 1, dtype=np.float64) ** -1.1
    idx = np.stack([rng.choice(E, size=k, replace=False, p=w / w.sum()) for _ in range(T)])
    plan = O.dispatch_plan(idx, E, capacity=cap, ep_size=ep)
    r = O.dedup_pack(idx, plan["dest"], E, ep)
    el = E // ep
    sent = plan["dest"] >= 0
    pairs = {(int(idx[t, j]) // el, t) for t, j in zip(*np.nonzero(sent))}
    assert int(r["pair_splits"].sum()) == len(pairs) == len(r["pair_token"])
    assert int(sent.sum()) >= len(pairs)
    for t, j in zip(*np.nonzero(sent)):
        p = r["pair_dest"][t, j]
        assert r["pair_token"][p] == t
        rank = int(idx[t, j]) // el
        assert r["pair_displs"][rank] <= p < r["pair_displs"][rank] + r["pair_splits"][rank]
    assert (r["pair_dest"][~sent] == -1).all()
    for rank in range(ep):
        seg = r["pair_token"][r["pair_displs"][rank]:r["pair_displs"][rank] + r["pair_splits"][rank]]
        assert (np.diff(seg) > 0).all()          # tokens ascending within a rank


def test_token_major_order_is_rejected():
    """A plausible mistake -- numbering pairs token-major -- fails the table."""
    g = load_golden("dedup_pack.json")
    idx = np.array(g["idx"])
    el = g["E"] // g["ep_size"]
    pairs = sorted({(t, int(idx[t, j]) // el) for t in range(len(idx)) for j in range(2)})
    wrong = [[pairs.index((t, int(idx[t, j]) // el)) for j in range(2)] for t in range(len(idx))]
    assert wrong != g["pair_dest"]
