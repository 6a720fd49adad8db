"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
library through its binding, and compare with the CPU oracle."""
import sys

import numpy as np
import torch

from oracle import moe_oracle as O

TOL = {"bf16": 2e-2, "f32": 1e-4}
GATE_TOL = 1e-5
LOGIT_TOL = 1e-4


def lib():
    import grouped_expert_ffn_amd as G  # the HIP library; raises if it is not built
    return G


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tdtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def dev(a, dt=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    return t.to(dt) if dt is not None else t


def host(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def assert_close(got, ref, tol, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if got.size == 0:
        return 0.0, 0.0
    err = np.abs(got - ref)
    bad = err > tol * (1.0 + np.abs(ref))
    rel = err / np.maximum(np.abs(ref), 1e-30)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tol {tol}; "
                           f"max abs {err.max():.3e}, max rel {rel.max():.3e}")
    return float(err.max()), float(rel[np.abs(ref) > 1e-3].max() if (np.abs(ref) > 1e-3).any() else 0)


def certified_route_mismatch(idx_gpu, logits_gpu, logits64, k):
    """Tokens whose expert SET differs between the GPU routing and the fp64
    routing. Each must be a certified near tie: for every expert a chosen
    only by one side and b chosen only by the other, the fp64 gap |s_a - s_b|
    is within the GPU's own score errors |ds_a| + |ds_b|. Returns the list of
    (token, margin) and asserts every mismatch is certified."""
    ref_idx, _ = O.topk_route(logits64, k)
    out = []
    d = np.abs(np.asarray(logits_gpu, np.float64) - logits64)
    for t in range(idx_gpu.shape[0]):
        a_set, b_set = set(idx_gpu[t].tolist()), set(ref_idx[t].tolist())
        if a_set == b_set:
            continue
        for a in a_set - b_set:
            for b in b_set - a_set:
                gap = abs(logits64[t, a] - logits64[t, b])
                assert gap <= d[t, a] + d[t, b] + 1e-12, (t, a, b, gap, d[t, a], d[t, b])
        out.append((t, float(O.router_margin(logits64[t:t + 1], k)[0])))
    return out


def check_plan(G, desc, idx_np, bufs, E, capacity, max_rows, ep_size=1, ep_rank=0):
    """Every integer output of the permute stage must equal the oracle's plan
    computed from the same (GPU or replayed) routing, bit for bit."""
    ref = O.dispatch_plan(idx_np, E, capacity, max_rows, ep_size, ep_rank)
    assert host(bufs.counts).tolist() == ref["counts"].tolist(), "counts"
    assert host(bufs.offsets).tolist() == ref["offsets"].tolist(), "offsets"
    assert np.array_equal(host(bufs.dest), ref["dest"]), "dest"
    n = ref["src_token"].shape[0]
    assert np.array_equal(host(bufs.src_token)[:n], ref["src_token"]), "src_token"
    assert np.array_equal(host(bufs.src_slot)[:n], ref["src_slot"]), "src_slot"
    assert host(bufs.send_splits).tolist() == ref["send_splits"].tolist(), "send_splits"
    assert host(bufs.send_displs).tolist() == ref["send_displs"].tolist(), "send_displs"
    mask = O.BAD_EXPERT_ID | O.DROPPED | O.ROW_OVERFLOW
    assert (int(host(bufs.flags)[0]) & mask) == (ref["flags"] & mask), "flags"
    return ref


def upload_layer(G, cfg, inp, capacity=-1, max_rows=None, T=None, h=None):
    """Device copies of one layer's inputs and a descriptor."""
    T = cfg.T if T is None else T
    dt = tdtype(cfg.dtype)
    desc = G.make_desc(T, cfg.d, cfg.E, cfg.k, cfg.d_ff, cfg.dtype, cfg.gate, cfg.act,
                       ep_size=cfg.ep_size, ep_rank=cfg.ep_rank, capacity=capacity,
                       max_rows=max_rows)
    dv = dict(
        h=dev(inp["h"][:T] if h is None else h, dt),
        w_router=dev(inp["w_router"], dt),
        bias=None if inp.get("bias") is None else dev(inp["bias"], torch.float32),
        w1=dev(inp["w1"], dt), w2=dev(inp["w2"], dt))
    return desc, dv


def run_layer(G, desc, dv, bufs=None, ws=None, y=None):
    if bufs is None:
        bufs = G.alloc_buffers(desc)
    if ws is None:
        ws = G.alloc_workspace(desc)
    if y is None:
        y = torch.empty((desc.T, desc.d), dtype=G.torch_dtype(desc), device="cuda")
    bufs.flags.zero_()
    G.layer_forward(desc, dv["h"], dv["w_router"], dv["bias"], dv["w1"], dv["w2"], y, bufs, ws)
    torch.cuda.synchronize()
    return y, bufs, ws


def sample_tokens(T, n, seed, always=()):
    """n distinct random tokens plus the given ones, sorted."""
    rng = np.random.default_rng(seed)
    pick = rng.choice(T, size=min(n, T), replace=False).tolist() if T else []
    return sorted(set(pick) | {t for t in always if 0 <= t < T})


def edge_rows(offsets, e_lo, e_hi, max_rows, bm=256, short_all=128, per_edge=8, seed=0):
    """Grouped rows at the edges of each local expert's 256-row M-tiles: the
    first rows of its first tile, and the rows of its last tile (all of them
    when that tile holds at most `short_all` rows, which is what makes it a
    short tile, the kind the GEMMs run on half their waves and move into the
    leftover launch; else `per_edge` from each end and a few inside)."""
    rng = np.random.default_rng(seed)
    offs = np.asarray(offsets, np.int64)
    out = []
    for e in range(e_lo, e_hi):
        r0, r1 = min(int(offs[e]), max_rows), min(int(offs[e + 1]), max_rows)
        if r1 <= r0:
            continue
        rows = set(range(r0, r0 + per_edge))
        mt = (r1 - r0 + bm - 1) // bm
        t0 = r0 + (mt - 1) * bm
        if r1 - t0 <= short_all:
            rows.update(range(t0, r1))
        else:
            rows.update(range(t0, t0 + per_edge))
            rows.update(range(r1 - per_edge, r1))
            rows.update(rng.integers(t0, r1, per_edge).tolist())
        # only this expert's own rows: [r0, r1), all below max_rows
        out.extend(r for r in rows if r0 <= r < r1)
    return sorted(set(out))


def check_tokens_vs_oracle(cfg, inp, y, idx_gpu, toks, capacity=-1, what="y", T=None):
    """y[toks] against the per-token oracle y_t = sum over kept e of
    g_{t,e} f_e(h_t), evaluated on the GPU's routing (route replay) with the
    oracle's own float64 scores for the gates."""
    T = cfg.T if T is None else T
    toks = list(toks)
    if not toks:
        return (0.0, 0.0)
    want = O.brute_force_tokens(inp["h"][:T], inp["w_router"], inp.get("bias"), inp["w1"],
                                inp["w2"], toks, k=cfg.k, gate=cfg.gate, act=cfg.act,
                                capacity=capacity, ep_size=cfg.ep_size, ep_rank=cfg.ep_rank,
                                route_idx=idx_gpu)
    got = host(y[torch.as_tensor(toks, device="cuda")])
    return assert_close(got, want, TOL[cfg.dtype], what)


def check_rows_vs_oracle(cfg, inp, y_rows, rows, src_token, offsets, what="y_perm rows"):
    """Expert outputs of grouped rows against the oracle's f_e on the token
    each row holds (the local expert owning row r is the one whose range
    offsets[e]..offsets[e+1] contains r)."""
    rows = np.asarray(rows, np.int64)
    if rows.size == 0:
        return (0.0, 0.0)
    offs = np.asarray(offsets, np.int64)
    e_of = np.searchsorted(offs, rows, side="right") - 1
    lo = cfg.ep_rank * (cfg.E // cfg.ep_size)
    want = np.zeros((rows.size, cfg.d))
    for e in np.unique(e_of):
        m = e_of == e
        want[m] = O.expert_ffn(inp["h"][np.asarray(src_token)[rows[m]]], inp["w1"][e - lo],
                               inp["w2"][e - lo], cfg.act)
    return assert_close(np.asarray(y_rows, np.float64), want, TOL[cfg.dtype], what)
