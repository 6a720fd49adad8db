"""Pins for the oracle's grouping step: counts, capacity, offsets, dest,
inverse permutation, expert-parallel splits."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests import pins
from tests.conftest import load_golden


def test_capacity_hand_built_tables():
    pins.check_capacity_tables(O.dispatch_plan)


def test_wrong_token_fixture():
    pins.check_wrong_token_fixture(O.dispatch_plan, O.permute, O.unpermute_combine)


@pytest.mark.parametrize("m", [0, 1])
def test_worked_maps_counts_remote_and_payload(m):
    f = load_golden("p1_worked_maps.json")
    mp = f["maps"][m]
    route = np.array(mp["route"])[:, None]
    origin = np.array(f["origin_rank"])
    R = f["ranks"]
    dest_counts = np.zeros(R, np.int64)
    remote = local = 0
    remote_tokens = []
    for r in range(R):
        mine = np.nonzero(origin == r)[0]
        p = O.dispatch_plan(route[mine], E=R * f["experts_per_rank"], ep_size=R, ep_rank=r)
        dest_counts += p["send_splits"]
        local += int(p["send_splits"][r])
        remote += int(p["send_splits"].sum() - p["send_splits"][r])
        for row in range(p["src_token"].shape[0]):
            t = mine[p["src_token"][row]]
            seg = int(np.searchsorted(p["send_displs"], row, side="right") - 1)
            if seg != r:
                remote_tokens.append(f["tokens"][t])
    assert dest_counts.tolist() == mp["destination_counts"]
    assert remote == mp["remote_vectors"] and local == mp["local_assignments"]
    assert sorted(remote_tokens) == mp["remote_tokens"]
    # a d=1024 bf16 row is exactly the pages' 2 KiB vector
    assert 1024 * 2 == f["bytes_per_vector"]
    assert remote * f["bytes_per_vector"] == mp["remote_payload_bytes"]


def test_capacity_formula_values():
    # cf * T * k / E at the two capacity-mode layers, worked by hand:
    # 1.0 * 4096 * 2 / 8 = 1024 and 1.25 * 16384 * 8 / 128 = 1280.
    assert O.capacity_from_factor(1.0, 4096, 2, 8) == 1024
    assert O.capacity_from_factor(1.25, 16384, 8, 128) == 1280
    assert O.capacity_from_factor(1.0, 10, 1, 3) == 3      # 3.33 -> floor
    assert O.capacity_from_factor(None, 4096, 2, 8) == -1


def _check_invariants(idx, E, cap, p):
    T, k = idx.shape
    flat = idx.reshape(-1)
    dest = p["dest"].reshape(-1)
    assert p["counts"].sum() == T * k
    assert (p["kept"] == (p["counts"] if cap < 0 else np.minimum(p["counts"], cap))).all()
    assert (np.diff(p["offsets"]) == p["kept"]).all() and p["offsets"][0] == 0
    kept_rows = dest[dest >= 0]
    n = int(p["offsets"][-1])
    assert sorted(kept_rows.tolist()) == list(range(n))           # injective onto [0, n)
    a = np.nonzero(dest >= 0)[0]
    assert (p["src_token"][dest[a]] == a // k).all()               # inverse permutation
    assert (p["src_slot"][dest[a]] == a % k).all()
    for e in range(E):
        members = np.nonzero(flat == e)[0]
        rows = dest[members]
        kept_members = members[rows >= 0]
        # kept = the first kept[e] members in (token, slot) order, rows ascending
        assert kept_members.tolist() == members[: p["kept"][e]].tolist()
        r = rows[rows >= 0]
        assert r.tolist() == list(range(p["offsets"][e], p["offsets"][e + 1]))


@pytest.mark.parametrize("cap", [-1, 0, 5, 40])
@pytest.mark.parametrize("E,k", [(4, 1), (8, 2), (16, 4)])
def test_plan_invariants_random(E, k, cap):
    rng = np.random.default_rng(E * 100 + k + cap)
    T = 97
    # skewed ids so some experts overflow and some are empty
    w = np.arange(1, E + 1, dtype=np.float64) ** -1.5
    w /= w.sum()
    idx = np.stack([rng.choice(E, size=k, replace=False, p=w) for _ in range(T)]).astype(np.int32)
    p = O.dispatch_plan(idx, E, cap)
    _check_invariants(idx, E, cap, p)
    assert bool(p["flags"] & O.DROPPED) == bool((p["kept"] < p["counts"]).any())


def test_ep_splits_cover_all_rows():
    rng = np.random.default_rng(9)
    idx = rng.integers(0, 16, size=(200, 2)).astype(np.int32)
    for cap in (-1, 20):
        p = O.dispatch_plan(idx, 16, cap, ep_size=4, ep_rank=1)
        assert p["send_splits"].sum() == p["offsets"][-1]
        assert p["send_displs"].tolist() == [0] + np.cumsum(p["send_splits"])[:-1].tolist()
        for r in range(4):
            assert p["send_splits"][r] == p["kept"][4 * r:4 * r + 4].sum()


def test_row_overflow_keeps_prefix():
    idx = np.zeros((10, 1), np.int32)
    p = O.dispatch_plan(idx, 2, -1, max_rows=4)
    assert p["dest"][:, 0].tolist() == [0, 1, 2, 3] + [-2] * 6
    assert p["flags"] & O.ROW_OVERFLOW
    assert p["src_token"].tolist() == [0, 1, 2, 3]


def test_permute_copies_rows_exactly():
    rng = np.random.default_rng(4)
    h = rng.standard_normal((30, 8)).astype(np.float32)
    idx = rng.integers(0, 5, size=(30, 3)).astype(np.int32)
    p = O.dispatch_plan(idx, 5, 4)
    x = O.permute(h, p["dest"], int(p["offsets"][-1]))
    for row in range(x.shape[0]):
        assert np.array_equal(x[row], h[p["src_token"][row]])
