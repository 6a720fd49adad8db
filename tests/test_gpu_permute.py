"""GPU parity of the permute stage on replayed route tables: counts, capacity
drops, offsets, dest, inverse map, expert-parallel splits and flags must
equal the oracle bit for bit, and x_perm rows must be exact copies."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from tests.conftest import load_golden
from tests.gpu_util import check_plan, dev, host, lib, say, tdtype

pytestmark = pytest.mark.gpu


def _permute(G, idx_np, E, *, d=64, dtype="bf16", capacity=-1, max_rows=None, ep_size=1,
             ep_rank=0, h=None, seed=0):
    idx_np = np.asarray(idx_np, np.int32)
    if idx_np.ndim == 1:
        idx_np = idx_np[:, None]
    T, k = idx_np.shape
    desc = G.make_desc(T, d, E, k, 64, dtype, "softmax", "swiglu", ep_size=ep_size,
                       ep_rank=ep_rank, capacity=capacity, max_rows=max_rows)
    if h is None:
        h = np.random.default_rng(seed).standard_normal((T, d)).astype(np.float32)
        if dtype == "bf16":
            h = host(dev(h, torch.bfloat16))
    bufs = G.alloc_buffers(desc)
    ws = G.alloc_workspace(desc)
    G.permute(desc, dev(h, tdtype(dtype)), dev(idx_np), bufs.x_perm, bufs.counts, bufs.offsets,
              bufs.dest, bufs.src_token, bufs.src_slot, bufs.send_splits, bufs.send_displs,
              bufs.flags, ws)
    torch.cuda.synchronize()
    return desc, bufs, h


def _check_rows(bufs, h, ref):
    x = host(bufs.x_perm)
    n = ref["src_token"].shape[0]
    assert np.array_equal(x[:n], h[ref["src_token"]]), "x_perm rows"


def test_capacity_tables():
    G = lib()
    for c in load_golden("capacity_tables.json")["cases"]:
        route = np.array(c["route"], np.int32)
        desc, bufs, h = _permute(G, route, c["E"], capacity=c["capacity"], max_rows=c["max_rows"])
        for key in ("counts", "offsets", "dest"):
            assert host(getattr(bufs, key)).tolist() == c[key], (c["name"], key)
        n = len(c["src_token"])
        assert host(bufs.src_token)[:n].tolist() == c["src_token"], c["name"]
        assert host(bufs.src_slot)[:n].tolist() == c["src_slot"], c["name"]
        assert int(host(bufs.flags)[0]) == c["flags"], c["name"]
        ref = check_plan(G, desc, route, bufs, c["E"], c["capacity"], c["max_rows"])
        _check_rows(bufs, h, ref)


def test_wrong_token_fixture():
    G = lib()
    f = load_golden("wrong_token_abc.json")
    desc, bufs, h = _permute(G, np.array(f["route"]), f["E"])
    for key in ("counts", "offsets", "dest"):
        assert host(getattr(bufs, key)).tolist() == f[key], key
    assert host(bufs.src_token).tolist() == f["src_token"]
    assert np.array_equal(host(bufs.x_perm), h[f["src_token"]])


@pytest.mark.parametrize("m", [0, 1])
def test_worked_maps_splits_and_payload(m):
    """Each origin rank packs its tokens into per-destination segments; with
    d=1024 bf16 rows (2 KiB) the remote payload is the pages' figure."""
    G = lib()
    f = load_golden("p1_worked_maps.json")
    mp = f["maps"][m]
    route = np.array(mp["route"], np.int32)[:, None]
    origin = np.array(f["origin_rank"])
    R = f["ranks"]
    dest_counts = np.zeros(R, np.int64)
    remote = local = 0
    for r in range(R):
        mine = np.nonzero(origin == r)[0]
        desc, bufs, _ = _permute(G, route[mine], R, d=1024, ep_size=R, ep_rank=r)
        splits = host(bufs.send_splits)
        dest_counts += splits
        local += int(splits[r])
        remote += int(splits.sum() - splits[r])
        row_bytes = bufs.x_perm.shape[1] * bufs.x_perm.element_size()
    assert dest_counts.tolist() == mp["destination_counts"]
    assert (remote, local) == (mp["remote_vectors"], mp["local_assignments"])
    assert remote * row_bytes == mp["remote_payload_bytes"]


def _skewed_routes(rng, T, E, k, dup=False):
    w = np.arange(1, E + 1, dtype=np.float64) ** -1.2
    w /= w.sum()
    if dup:
        return rng.choice(E, size=(T, k), p=w).astype(np.int32)
    return np.stack([rng.choice(E, size=k, replace=False, p=w) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 127, 128, 129, 1000])
@pytest.mark.parametrize("E,k", [(4, 1), (8, 2), (128, 8), (256, 8), (1024, 16)])
def test_random_replay_bit_exact(T, E, k):
    G = lib()
    rng = np.random.default_rng(T * 7 + E)
    idx = _skewed_routes(rng, T, E, k)
    cap_opts = [-1, 0, max(1, T * k // E // 2), T * k]
    for cap in cap_opts:
        desc, bufs, h = _permute(G, idx, E, capacity=cap, seed=T)
        ref = check_plan(G, desc, idx, bufs, E, cap, T * k)
        _check_rows(bufs, h, ref)


def test_duplicate_ids_in_a_row_and_ep_share():
    G = lib()
    rng = np.random.default_rng(11)
    idx = _skewed_routes(rng, 500, 16, 4, dup=True)
    for cap in (-1, 30):
        desc, bufs, h = _permute(G, idx, 16, capacity=cap, ep_size=4, ep_rank=2)
        ref = check_plan(G, desc, idx, bufs, 16, cap, 2000, 4, 2)
        _check_rows(bufs, h, ref)


def test_fp32_rows_and_odd_width():
    G = lib()
    rng = np.random.default_rng(5)
    idx = _skewed_routes(rng, 77, 8, 2)
    for d in (32, 30, 1):
        desc, bufs, h = _permute(G, idx, 8, d=d, dtype="f32")
        ref = check_plan(G, desc, idx, bufs, 8, -1, 154)
        _check_rows(bufs, h, ref)


def test_empty_batch():
    G = lib()
    desc, bufs, _ = _permute(G, np.zeros((0, 2), np.int32), 8)
    assert host(bufs.counts).tolist() == [0] * 8
    assert host(bufs.offsets).tolist() == [0] * 9
    assert host(bufs.send_splits).tolist() == [0]
    assert int(host(bufs.flags)[0]) == 0


def test_bad_ids_and_row_overflow_flags():
    G = lib()
    idx = np.array([[0, 9], [1, -3], [1, 0], [0, 1]], np.int32)
    desc, bufs, _ = _permute(G, idx, 4, max_rows=3)
    check_plan(G, desc, idx, bufs, 4, -1, 3)
    fl = int(host(bufs.flags)[0])
    assert fl & G.FLAG_BAD_EXPERT_ID and fl & G.FLAG_ROW_OVERFLOW
    d = host(bufs.dest)
    assert d[0, 1] == -1 and d[1, 1] == -1 and (d == -2).sum() == 3


def test_all_tokens_to_one_expert_large():
    G = lib()
    T, E, k = 20000, 64, 2
    idx = np.stack([np.zeros(T, np.int32), np.arange(T, dtype=np.int32) % 63 + 1], 1)
    for cap in (-1, 5000):
        desc, bufs, h = _permute(G, idx, E, capacity=cap, d=128)
        ref = check_plan(G, desc, idx, bufs, E, cap, T * k)
        _check_rows(bufs, h, ref)
        say(f"one-hot expert cap={cap} counts[0]={host(bufs.counts)[0]}")


@pytest.mark.parametrize("cap", [-1, 30])
def test_large_plan_takes_the_separate_scan_path(cap):
    """157 tiles x 1024 experts exceeds the plan size the rank kernel scans by
    itself, so the standalone scan kernel runs; results must not change."""
    G = lib()
    T, E, k = 20000, 1024, 2
    rng = np.random.default_rng(21)
    idx = _skewed_routes(rng, T, E, k)
    desc, bufs, h = _permute(G, idx, E, capacity=cap, d=64)
    ref = check_plan(G, desc, idx, bufs, E, cap, T * k)
    _check_rows(bufs, h, ref)


@pytest.mark.parametrize("T,E,k", [(8192, 8, 2), (8193, 8, 2), (16000, 16, 2), (4096, 1024, 4),
                                   (2048, 256, 8), (2049, 256, 8)])
def test_plan_paths_around_the_size_switches(T, E, k):
    """Plans with at most 4096 tile x expert counts are scanned inside the
    rank launch, larger ones by a separate scan launch; cases around that
    switch and at the layer sizes (2^14 assignments), with and without
    capacity, must match the oracle."""
    G = lib()
    rng = np.random.default_rng(T + E)
    idx = _skewed_routes(rng, T, E, k)
    for cap in (-1, max(1, T * k // E - 3)):
        desc, bufs, h = _permute(G, idx, E, capacity=cap, d=64)
        ref = check_plan(G, desc, idx, bufs, E, cap, T * k)
        _check_rows(bufs, h, ref)
