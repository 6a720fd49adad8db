"""GPU parity of the grouped expert FFN and of unpermute + combine."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from tests.gpu_util import TOL, assert_close, dev, host, lib, say, tdtype

pytestmark = pytest.mark.gpu


def _rand(rng, shape, scale, dtype):
    a = (rng.standard_normal(shape) * scale).astype(np.float32)
    if dtype == "bf16":
        a = host(dev(a, torch.bfloat16))
    return a


def _ffn_case(G, sizes, d, dff, act, dtype, ep_size=1, ep_rank=0, max_rows=None, seed=0):
    rng = np.random.default_rng(seed)
    E = len(sizes) * ep_size
    el = len(sizes)
    counts = np.zeros(E, np.int64)
    counts[ep_rank * el:(ep_rank + 1) * el] = sizes
    # rows of non-local experts sit before/after the local segment too
    if ep_size > 1:
        counts[:ep_rank * el] = 3
        counts[(ep_rank + 1) * el:] = 2
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1]) if max_rows is None else max_rows
    x = _rand(rng, (rows, d), 1.0, dtype)
    w1r = 2 * dff if act == "swiglu" else dff
    w1 = _rand(rng, (el, w1r, d), d ** -0.5, dtype)
    w2 = _rand(rng, (el, d, dff), dff ** -0.5, dtype)
    desc = G.make_desc(max(1, rows), d, E, 1, dff, dtype, "softmax", act, ep_size=ep_size,
                       ep_rank=ep_rank, max_rows=rows)
    dt = tdtype(dtype)
    y = torch.full((rows, d), 7.0, dtype=dt, device="cuda")
    G.grouped_ffn(desc, dev(x, dt), dev(offsets), dev(w1, dt), dev(w2, dt), y,
                  G.alloc_workspace(desc))
    torch.cuda.synchronize()
    ref = O.grouped_ffn(x, offsets, w1, w2, act, ep_rank * el, (ep_rank + 1) * el, rows)
    lo = min(int(offsets[ep_rank * el]), rows)
    hi = min(int(offsets[(ep_rank + 1) * el]), rows)
    got = host(y)
    err = assert_close(got[lo:hi], ref[lo:hi], TOL[dtype], f"y_perm {act} {dtype} {sizes}")
    # rows outside the local groups are not touched
    assert (got[:lo] == 7.0).all() and (got[hi:] == 7.0).all()
    return err


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("act", ["swiglu", "relu"])
def test_ragged_groups_with_empty_experts(dtype, act):
    G = lib()
    err = _ffn_case(G, [0, 1, 129, 300, 64, 0, 255], 128, 192, act, dtype)
    say(f"ffn {dtype} {act} max err {err}")


def test_many_tiles_per_expert_and_wide_shapes():
    G = lib()
    _ffn_case(G, [700, 5, 1030], 512, 384, "swiglu", "bf16", seed=3)
    _ffn_case(G, [260, 0, 0, 3], 1024, 2816, "swiglu", "bf16", seed=4)


def test_expert_parallel_local_segment_only():
    G = lib()
    _ffn_case(G, [40, 0, 130, 17], 256, 128, "swiglu", "bf16", ep_size=3, ep_rank=1, seed=5)
    _ffn_case(G, [40, 0, 130, 17], 32, 64, "relu", "f32", ep_size=3, ep_rank=2, seed=6)


def test_rows_clamped_to_max_rows():
    G = lib()
    # offsets say 300 rows but only 200 are allocated: the tail is not computed
    _ffn_case(G, [100, 200], 128, 128, "swiglu", "bf16", max_rows=200, seed=7)


def test_short_tiles_and_leftover_launch_keep_the_bits():
    """Ten experts of 7 row tiles each, 8 of them ending in a tile of at most
    half its rows. With 4 column tiles per row tile (d_ff = 512) the first GEMM
    has 280 tiles: one whole round of a 256-workgroup grid plus 24 leftover
    tiles, which go to the second launch; the tile table puts 6 short row
    tiles last for that (two groups of row tiles), and short tiles run on half
    of the waves. Outputs must match the oracle, and each expert's rows must
    carry the same bits as when that expert runs alone (another table)."""
    G = lib()
    sizes = [6 * 256 + r for r in (16, 100, 128, 129, 200, 16, 24, 64, 84, 4)]
    _ffn_case(G, sizes, 256, 512, "swiglu", "bf16", seed=11)
    rng = np.random.default_rng(11)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(offsets[-1])
    d, dff, el = 256, 512, len(sizes)
    x = dev(_rand(rng, (rows, d), 1.0, "bf16"), torch.bfloat16)
    w1 = dev(_rand(rng, (el, 2 * dff, d), d ** -0.5, "bf16"), torch.bfloat16)
    w2 = dev(_rand(rng, (el, d, dff), dff ** -0.5, "bf16"), torch.bfloat16)
    desc = G.make_desc(rows, d, el, 1, dff, "bf16", "softmax", "swiglu", max_rows=rows)
    y = torch.zeros((rows, d), dtype=torch.bfloat16, device="cuda")
    G.grouped_ffn(desc, x, dev(offsets), w1, w2, y, G.alloc_workspace(desc))
    for e in range(el):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        de = G.make_desc(hi - lo, d, 1, 1, dff, "bf16", "softmax", "swiglu", max_rows=hi - lo)
        ye = torch.zeros((hi - lo, d), dtype=torch.bfloat16, device="cuda")
        G.grouped_ffn(de, x[lo:hi].contiguous(), dev(np.array([0, hi - lo], np.int32)),
                      w1[e:e + 1].contiguous(), w2[e:e + 1].contiguous(), ye,
                      G.alloc_workspace(de))
        torch.cuda.synchronize()
        assert torch.equal(ye, y[lo:hi]), f"expert {e} differs when run alone"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("E,k,ep", [(8, 2, (1, 0)), (128, 8, (1, 0)), (256, 8, (8, 3)), (4, 1, (2, 1))])
def test_unpermute_combine(dtype, E, k, ep):
    G = lib()
    rng = np.random.default_rng(E + k)
    T, d = 333, 256
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    plan = O.dispatch_plan(idx, E, capacity=max(1, T * k // E - 2), ep_size=ep[0], ep_rank=ep[1])
    rows = int(plan["offsets"][-1])
    yp = _rand(rng, (rows, d), 1.0, dtype)
    gate = rng.random((T, k)).astype(np.float32)
    desc = G.make_desc(T, d, E, k, 64, dtype, "softmax", "swiglu", ep_size=ep[0], ep_rank=ep[1],
                       max_rows=rows)
    dt = tdtype(dtype)
    y = torch.empty((T, d), dtype=dt, device="cuda")
    G.unpermute_combine(desc, dev(yp, dt), dev(idx), dev(gate), dev(plan["dest"].astype(np.int32)), y)
    torch.cuda.synchronize()
    el = E // ep[0]
    ref = O.unpermute_combine(yp, idx, gate, plan["dest"], ep[1] * el, (ep[1] + 1) * el)
    assert_close(host(y), ref, TOL[dtype] if dtype == "bf16" else 1e-6, "combine")


def test_grouped_ffn_reports_rows_past_max_rows():
    """A replayed offsets table whose local groups end past max_rows: the
    rows that fit are computed, the rest are not, and ROW_OVERFLOW is set in
    the flags word; a table that fits leaves the word clear, and groups of
    other ranks past max_rows do not count."""
    G = lib()
    rng = np.random.default_rng(21)
    d, dff = 128, 128
    w1 = dev(_rand(rng, (2, 2 * dff, d), d ** -0.5, "bf16"), torch.bfloat16)
    w2 = dev(_rand(rng, (2, d, dff), dff ** -0.5, "bf16"), torch.bfloat16)
    x = dev(_rand(rng, (300, d), 1.0, "bf16"), torch.bfloat16)
    for offsets, R, ep, rank, want in (([0, 100, 300], 200, 1, 0, True),
                                       ([0, 100, 300], 300, 1, 0, False),
                                       ([0, 100, 150, 250, 300], 160, 2, 0, False),
                                       ([0, 100, 150, 250, 300], 260, 2, 1, True)):
        E = len(offsets) - 1
        desc = G.make_desc(R, d, E, 1, dff, "bf16", "softmax", "swiglu", ep_size=ep,
                           ep_rank=rank, max_rows=R)
        fl = torch.zeros(1, dtype=torch.int32, device="cuda")
        y = torch.zeros((R, d), dtype=torch.bfloat16, device="cuda")
        G.grouped_ffn(desc, x[:R].contiguous(), dev(np.array(offsets, np.int32)), w1, w2, y,
                      G.alloc_workspace(desc), flags=fl)
        torch.cuda.synchronize()
        assert bool(int(host(fl)[0]) & G.FLAG_ROW_OVERFLOW) == want, (offsets, R, ep, rank)
