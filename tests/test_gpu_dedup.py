"""GPU parity of the deduplicated expert-parallel packing (moe_pack_dedup):
pair rows, pair map, per-rank splits and the receive map must equal the
oracle's dedup_pack bit for bit; the send buffer must hold exact token rows;
and the local experts run on the deduplicated rows through the gathered
GEMM must reproduce the plain path's y_perm bits."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from tests.gpu_util import dev, host, lib, run_layer, say, tdtype, upload_layer
from workloads import CONFIGS, make_inputs, small_layer_config

pytestmark = pytest.mark.gpu


def _pack(G, desc, h, idx, bufs, ws):
    dt = G.torch_dtype(desc)
    P = G.max_pairs(desc)
    out = dict(
        send_buf=torch.full((P, desc.d), float("nan"), dtype=dt, device="cuda"),
        pair_dest=torch.full((desc.T, desc.k), -7, dtype=torch.int32, device="cuda"),
        pair_token=torch.full((P,), -7, dtype=torch.int32, device="cuda"),
        pair_splits=torch.full((desc.ep_size,), -7, dtype=torch.int64, device="cuda"),
        pair_displs=torch.full((desc.ep_size,), -7, dtype=torch.int64, device="cuda"),
        recv_rows=torch.full((desc.max_rows,), -7, dtype=torch.int32, device="cuda"))
    G.pack_dedup(desc, h, idx, bufs.dest, bufs.src_token, bufs.src_slot, bufs.offsets,
                 out["send_buf"], out["pair_dest"], out["pair_token"], out["pair_splits"],
                 out["pair_displs"], out["recv_rows"], ws)
    torch.cuda.synchronize()
    return out


def _check_pack(desc, h, idx_np, bufs, out):
    """Everything moe_pack_dedup writes, against the oracle and the plan."""
    dest = host(bufs.dest).astype(np.int64)
    ref = O.dedup_pack(idx_np, dest, desc.E, desc.ep_size)
    n = int(ref["pair_splits"].sum())
    assert np.array_equal(host(out["pair_dest"]), ref["pair_dest"]), "pair_dest"
    assert np.array_equal(host(out["pair_token"])[:n], ref["pair_token"]), "pair_token"
    assert (host(out["pair_token"])[n:] == -7).all(), "pair_token past the pairs"
    assert host(out["pair_splits"]).tolist() == ref["pair_splits"].tolist(), "pair_splits"
    assert host(out["pair_displs"]).tolist() == ref["pair_displs"].tolist(), "pair_displs"
    tok = out["pair_token"][:n].long()
    assert torch.equal(out["send_buf"][:n], h[tok]), "send rows are exact token rows"
    # receive map over the local experts' rows: the pair row of that row's slot
    el = desc.E // desc.ep_size
    offs = host(bufs.offsets)
    lo = min(int(offs[desc.ep_rank * el]), desc.max_rows)
    hi = min(int(offs[(desc.ep_rank + 1) * el]), desc.max_rows)
    st, ss = host(bufs.src_token)[lo:hi], host(bufs.src_slot)[lo:hi]
    want = ref["pair_dest"][st, ss] if hi > lo else np.zeros(0, np.int64)
    got = host(out["recv_rows"])
    assert np.array_equal(got[lo:hi], want), "recv_rows"
    assert (got[:lo] == -7).all() and (got[hi:] == -7).all(), "recv_rows outside the local rows"
    r0, r1 = ref["pair_displs"][desc.ep_rank], ref["pair_displs"][desc.ep_rank] + \
        ref["pair_splits"][desc.ep_rank]
    assert ((want >= r0) & (want < r1)).all(), "local rows come from this rank's segment"
    return ref, lo, hi


# (layer, tokens, ep_size, ep_rank)
LAYER_CASES = [("tiny_fp32", 64, 2, 1), ("small_bf16", 1024, 1, 0), ("small_bf16", 1024, 4, 1),
               ("finegrained_bf16", 1024, 8, 3), ("finegrained_bf16", 1024, 128, 5),
               ("ep_share_bf16", 512, 8, 0), ("mixtral_bf16", 256, 2, 1)]


@pytest.mark.parametrize("name,T,ep,rank", LAYER_CASES)
def test_layer_pack_and_ffn_on_deduplicated_rows(name, T, ep, rank):
    G = lib()
    base = CONFIGS[name]
    cfg = small_layer_config(base, T, ep_size=ep, ep_rank=rank)
    inp = make_inputs(cfg)
    for cf in base.capacity_factors:
        cap = O.capacity_from_factor(cf, cfg.T, cfg.k, cfg.E)
        say(f"dedup {name} T={T} ep={ep}/{rank} cf={cf}")
        desc, dv = upload_layer(G, cfg, inp, capacity=cap)
        y, b, ws = run_layer(G, desc, dv)
        out = _pack(G, desc, dv["h"], b.topk_idx, b, ws)
        ref, lo, hi = _check_pack(desc, dv["h"], host(b.topk_idx), b, out)
        sent = int((host(b.dest) >= 0).sum())
        say(f"  {sent} sent slots -> {int(ref['pair_splits'].sum())} pair rows")
        y2 = torch.zeros_like(b.y_perm)
        G.grouped_ffn_gather(desc, out["send_buf"], out["recv_rows"], b.offsets, dv["w1"],
                             dv["w2"], y2, ws)
        torch.cuda.synchronize()
        assert torch.equal(y2[lo:hi], b.y_perm[lo:hi]), "FFN on deduplicated rows"


def _replay(G, idx_np, E, *, d=64, dtype="bf16", capacity=-1, max_rows=None, ep_size=1,
            ep_rank=0, seed=0):
    idx_np = np.asarray(idx_np, np.int32)
    T, k = idx_np.shape
    desc = G.make_desc(T, d, E, k, 64, dtype, "softmax", "swiglu", ep_size=ep_size,
                       ep_rank=ep_rank, capacity=capacity, max_rows=max_rows)
    h = dev(np.random.default_rng(seed).standard_normal((T, d)).astype(np.float32),
            tdtype(dtype))
    bufs = G.alloc_buffers(desc, x_perm=False)
    ws = G.alloc_workspace(desc)
    idx = dev(idx_np)
    bufs.flags.zero_()
    G.permute(desc, h, idx, None, bufs.counts, bufs.offsets, bufs.dest, bufs.src_token,
              bufs.src_slot, bufs.send_splits, bufs.send_displs, bufs.flags, ws)
    torch.cuda.synchronize()
    out = _pack(G, desc, h, idx, bufs, ws)
    return _check_pack(desc, h, idx_np, bufs, out)


def _routes(rng, T, E, k, dup=False):
    w = np.arange(1, E + 1, dtype=np.float64) ** -1.2
    w /= w.sum()
    if dup:
        return rng.choice(E, size=(T, k), p=w).astype(np.int32)
    return np.stack([rng.choice(E, size=k, replace=False, p=w) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T", [1, 127, 128, 129, 1000])
@pytest.mark.parametrize("E,k,ep", [(8, 2, 4), (128, 8, 8), (256, 8, 32), (64, 16, 64)])
def test_replayed_routes_bit_exact(T, E, k, ep):
    G = lib()
    rng = np.random.default_rng(T * 13 + E)
    idx = _routes(rng, T, E, k)
    for cap in (-1, 0, max(1, T * k // E // 2)):
        _replay(G, idx, E, capacity=cap, ep_size=ep, ep_rank=ep // 2, seed=T)


def test_hand_derived_table_on_the_gpu():
    """The hand-derived four-token table: 8 slots become 6 send rows."""
    G = lib()
    idx = np.array([[0, 1], [1, 2], [3, 2], [0, 3]], np.int32)
    ref, _, _ = _replay(G, idx, 4, ep_size=2, ep_rank=1)
    assert ref["pair_token"].tolist() == [0, 1, 3, 1, 2, 3]
    ref, _, _ = _replay(G, idx, 4, capacity=1, ep_size=2, ep_rank=0)
    assert ref["pair_token"].tolist() == [0, 1, 2]


def test_duplicates_bad_ids_overflow_and_fp32():
    """Repeated experts in a token's row, invalid ids, rows clamped by
    max_rows (dest = -2 slots are not sent) and unaligned fp32 rows."""
    G = lib()
    rng = np.random.default_rng(17)
    idx = _routes(rng, 500, 16, 4, dup=True)
    idx[3, 1], idx[10, 0] = -1, 99
    _replay(G, idx, 16, ep_size=4, ep_rank=2)
    _replay(G, idx, 16, ep_size=4, ep_rank=3, max_rows=900)
    _replay(G, idx, 16, capacity=20, ep_size=2, ep_rank=0, d=30, dtype="f32")


def test_empty_batch_and_single_rank():
    G = lib()
    ref, lo, hi = _replay(G, np.zeros((0, 2), np.int32), 8, ep_size=4, ep_rank=1)
    assert ref["pair_splits"].tolist() == [0] * 4 and lo == hi == 0
    rng = np.random.default_rng(2)
    ref, _, _ = _replay(G, _routes(rng, 300, 8, 2), 8)
    assert ref["pair_token"].tolist() == list(range(300))   # one row per token


def test_many_pairs_take_the_separate_scan_path():
    """79 token tiles x 64 ranks exceeds the plan size the rank kernel scans
    by itself, so the pair plan runs the standalone scan; bits must hold."""
    G = lib()
    rng = np.random.default_rng(23)
    idx = _routes(rng, 10000, 128, 4)
    _replay(G, idx, 128, ep_size=64, ep_rank=63)
