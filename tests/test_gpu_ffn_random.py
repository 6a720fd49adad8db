"""Seeded random layouts of the grouped expert FFN (bf16): ragged groups with
empty experts, one-row experts and short last tiles, several widths. Small
layouts leave most tiles past the last whole round of the persistent grid,
so they run in the second (leftover) launch, cut into pieces; which short
tiles go there depends on the layout. Every case is checked against the
oracle, and each expert's rows must carry the same bits as when that expert
runs alone (a different tile table, grid and leftover split: the K order of
every output is the same whatever the decomposition)."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from tests.gpu_util import TOL, assert_close, dev, host, lib, say

pytestmark = pytest.mark.gpu


def _layout(rng):
    el = int(rng.integers(1, 24))
    kind = rng.integers(0, 4, el)
    sizes = np.where(kind == 0, 0,                                   # empty
             np.where(kind == 1, rng.integers(1, 129, el),           # one short tile
             np.where(kind == 2, 256 * rng.integers(1, 6, el) + rng.integers(1, 65, el),
                      rng.integers(1, 1300, el))))                   # anything
    d = 64 * int(rng.integers(1, 9))
    dff = 64 * int(rng.integers(1, 9))
    act = "swiglu" if rng.random() < 0.7 else "relu"
    # spare rows beyond the groups: a larger grid (sized from max_rows), so
    # more of the tiles fall in the leftover launch
    slack = int(rng.choice([0, 2048, 16384]))
    return [int(v) for v in sizes], d, dff, act, slack


def _run(G, x, offsets, w1, w2, rows, d, dff, el, act, slack=0):
    R = rows + slack
    xs = torch.zeros((R, d), dtype=torch.bfloat16, device="cuda")
    xs[:rows] = x
    desc = G.make_desc(max(1, R), d, el, 1, dff, "bf16", "softmax", act, max_rows=R)
    y = torch.zeros((R, d), dtype=torch.bfloat16, device="cuda")
    G.grouped_ffn(desc, xs, dev(offsets), w1, w2, y, G.alloc_workspace(desc))
    return y[:rows]


@pytest.mark.parametrize("seed", range(16))
def test_random_layout_matches_oracle_and_per_expert_bits(seed):
    G = lib()
    rng = np.random.default_rng(5000 + seed)
    sizes, d, dff, act, slack = _layout(rng)
    el = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(offsets[-1])
    say(f"seed {seed}: {el} experts, rows {rows} (+{slack} spare), d {d}, d_ff {dff}, {act}, "
        f"sizes {sizes}")
    if rows == 0:
        return
    w1r = 2 * dff if act == "swiglu" else dff
    xb = dev((rng.standard_normal((rows, d))).astype(np.float32), torch.bfloat16)
    w1b = dev((rng.standard_normal((el, w1r, d)) * d ** -0.5).astype(np.float32), torch.bfloat16)
    w2b = dev((rng.standard_normal((el, d, dff)) * dff ** -0.5).astype(np.float32), torch.bfloat16)
    y = _run(G, xb, offsets, w1b, w2b, rows, d, dff, el, act, slack)
    torch.cuda.synchronize()
    ref = O.grouped_ffn(host(xb), offsets, host(w1b), host(w2b), act, 0, el, rows)
    assert_close(host(y), ref, TOL["bf16"], f"random layout seed {seed}")
    for e in range(el):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        ye = _run(G, xb[lo:hi].contiguous(), np.array([0, hi - lo], np.int32),
                  w1b[e:e + 1].contiguous(), w2b[e:e + 1].contiguous(), hi - lo, d, dff, 1, act)
        torch.cuda.synchronize()
        assert torch.equal(ye, y[lo:hi]), f"seed {seed}: expert {e} differs when run alone"


@pytest.mark.parametrize("seed", range(4))
def test_leftover_pieces_with_streamed_weights(seed):
    """Twelve experts at d = 1024, d_ff = 4096 hold 302 MB of weights, more
    than the 256 MiB last-level cache, so the leftover launch loads its weight
    slices non-temporal; random ragged groups with short last tiles put tiles
    there. Outputs against the oracle, and each expert's bits against that
    expert run alone (whose weights fit the cache: the other load policy)."""
    G = lib()
    rng = np.random.default_rng(7000 + seed)
    el, d, dff, act = 12, 1024, 4096, "swiglu"
    # full row tiles per expert; the row-tile count M is nudged to 1..4 mod 8,
    # so the SwiGLU GEMM's 32 column tiles per row tile leave 32..128 tiles
    # after its last whole round of 256 workgroups: the leftover launch
    q = rng.integers(0, 3, el)
    i = 0
    while (el + int(q.sum())) % 8 not in (1, 2, 3, 4):
        q[i % el] += 1
        i += 1
    sizes = [int(v) for v in 256 * q + rng.integers(1, 129, el)]
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(offsets[-1])
    say(f"streamed-weights seed {seed}: rows {rows}, sizes {sizes}")
    xb = dev((rng.standard_normal((rows, d))).astype(np.float32), torch.bfloat16)
    w1b = dev((rng.standard_normal((el, 2 * dff, d)) * d ** -0.5).astype(np.float32), torch.bfloat16)
    w2b = dev((rng.standard_normal((el, d, dff)) * dff ** -0.5).astype(np.float32), torch.bfloat16)
    y = _run(G, xb, offsets, w1b, w2b, rows, d, dff, el, act)
    torch.cuda.synchronize()
    ref = O.grouped_ffn(host(xb), offsets, host(w1b), host(w2b), act, 0, el, rows)
    assert_close(host(y), ref, TOL["bf16"], f"streamed weights seed {seed}")
    for e in range(el):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        ye = _run(G, xb[lo:hi].contiguous(), np.array([0, hi - lo], np.int32),
                  w1b[e:e + 1].contiguous(), w2b[e:e + 1].contiguous(), hi - lo, d, dff, 1, act)
        torch.cuda.synchronize()
        assert torch.equal(ye, y[lo:hi]), f"seed {seed}: expert {e} differs when run alone"


@pytest.mark.parametrize("d,dff,act", [(128, 4224, "swiglu"), (256, 1024, "relu")])
def test_remainder_rows_riding_on_full_tiles(d, dff, act):
    """Groups of k full 256-row tiles plus s rows: when ceil(s / 16) <= k the
    s rows ride on the expert's full tiles (16 per tile and column tile)
    instead of forming a short tile; otherwise the short tile stays. Exact
    multiples of 16, partial last blocks, one block per tile in every column
    (k = ceil(s / 16)), a one-row remainder and non-riding groups sit side by
    side. With spare rows the grid is 256 workgroups, and the 33 column tiles
    of the first GEMM (d_ff = 4224) take the column tile past one round's
    share, where the riders move to other tiles. Outputs against the oracle,
    and each expert's bits against that expert run alone."""
    G = lib()
    rng = np.random.default_rng(7100 + d)
    sizes = [256 * 2 + 16, 256 * 3 + 48, 256 * 5 + 64, 256 * 8 + 128, 256 + 5, 256 + 100, 60, 0,
             256 * 4, 256 * 8 + 1, 256 * 3 + 47]
    el = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(offsets[-1])
    say(f"riders: {el} experts, rows {rows}, d {d}, d_ff {dff}, {act}, sizes {sizes}")
    w1r = 2 * dff if act == "swiglu" else dff
    xb = dev((rng.standard_normal((rows, d))).astype(np.float32), torch.bfloat16)
    w1b = dev((rng.standard_normal((el, w1r, d)) * d ** -0.5).astype(np.float32), torch.bfloat16)
    w2b = dev((rng.standard_normal((el, d, dff)) * dff ** -0.5).astype(np.float32), torch.bfloat16)
    y = _run(G, xb, offsets, w1b, w2b, rows, d, dff, el, act, 16384)
    torch.cuda.synchronize()
    ref = O.grouped_ffn(host(xb), offsets, host(w1b), host(w2b), act, 0, el, rows)
    assert_close(host(y), ref, TOL["bf16"], f"riders d {d}")
    for e in range(el):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        ye = _run(G, xb[lo:hi].contiguous(), np.array([0, hi - lo], np.int32),
                  w1b[e:e + 1].contiguous(), w2b[e:e + 1].contiguous(), hi - lo, d, dff, 1, act)
        torch.cuda.synchronize()
        assert torch.equal(ye, y[lo:hi]), f"riders d {d}: expert {e} differs when run alone"


@pytest.mark.parametrize("seed", range(8))
def test_random_remainders_match_oracle_and_per_expert_bits(seed):
    """Groups of 0-9 full tiles plus 0-255 rows: remainders above half a tile
    (a partial tile of their own), short remainders that ride on their
    expert's full tiles, and short ones whose expert has too few full tiles,
    at random widths and grid sizes. Against the oracle, and each expert's
    bits against that expert run alone."""
    G = lib()
    rng = np.random.default_rng(90000 + seed)
    el = int(rng.integers(1, 20))
    sizes = [int(v) for v in 256 * rng.integers(0, 10, el) + rng.integers(0, 256, el)]
    d = 64 * int(rng.integers(1, 5))
    dff = 64 * int(rng.integers(1, 40))
    act = "swiglu" if rng.random() < 0.6 else "relu"
    slack = int(rng.choice([0, 4096, 16384]))
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(offsets[-1])
    say(f"remainders seed {seed}: {el} experts, rows {rows} (+{slack} spare), d {d}, "
        f"d_ff {dff}, {act}, sizes {sizes}")
    if rows == 0:
        return
    w1r = 2 * dff if act == "swiglu" else dff
    xb = dev(rng.standard_normal((rows, d)).astype(np.float32), torch.bfloat16)
    w1b = dev((rng.standard_normal((el, w1r, d)) * d ** -0.5).astype(np.float32), torch.bfloat16)
    w2b = dev((rng.standard_normal((el, d, dff)) * dff ** -0.5).astype(np.float32), torch.bfloat16)
    y = _run(G, xb, offsets, w1b, w2b, rows, d, dff, el, act, slack)
    torch.cuda.synchronize()
    ref = O.grouped_ffn(host(xb), offsets, host(w1b), host(w2b), act, 0, el, rows)
    assert_close(host(y), ref, TOL["bf16"], f"remainders seed {seed}")
    for e in range(el):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        ye = _run(G, xb[lo:hi].contiguous(), np.array([0, hi - lo], np.int32),
                  w1b[e:e + 1].contiguous(), w2b[e:e + 1].contiguous(), hi - lo, d, dff, 1, act)
        torch.cuda.synchronize()
        assert torch.equal(ye, y[lo:hi]), f"remainders seed {seed}: expert {e} differs alone"


@pytest.mark.parametrize("seed", range(6))
def test_random_remainders_gathered_rows_give_the_same_bits(seed):
    """The gathered first GEMM (token rows read from h through src_token) on
    random remainder layouts, riding and leftover tiles included: bitwise
    equal to the copying path on the rows copied into expert order."""
    G = lib()
    rng = np.random.default_rng(91000 + seed)
    el = int(rng.integers(1, 16))
    sizes = [int(v) for v in 256 * rng.integers(0, 8, el) + rng.integers(0, 256, el)]
    d = 64 * int(rng.integers(1, 4))
    dff = 64 * int(rng.integers(1, 24))
    act = "swiglu" if rng.random() < 0.6 else "relu"
    slack = int(rng.choice([0, 4096, 16384]))
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(offsets[-1])
    say(f"gathered remainders seed {seed}: {el} experts, rows {rows} (+{slack}), d {d}, "
        f"d_ff {dff}, {act}, sizes {sizes}")
    if rows == 0:
        return
    R = rows + slack
    w1r = 2 * dff if act == "swiglu" else dff
    h = dev(rng.standard_normal((R, d)).astype(np.float32), torch.bfloat16)
    src = np.zeros(R, np.int32)
    src[:rows] = rng.permutation(R)[:rows]
    w1b = dev((rng.standard_normal((el, w1r, d)) * d ** -0.5).astype(np.float32), torch.bfloat16)
    w2b = dev((rng.standard_normal((el, d, dff)) * dff ** -0.5).astype(np.float32), torch.bfloat16)
    desc = G.make_desc(R, d, el, 1, dff, "bf16", "softmax", act, max_rows=R)
    ws = G.alloc_workspace(desc)
    off = dev(offsets)
    src_d = dev(src)
    y_g = torch.zeros((R, d), dtype=torch.bfloat16, device="cuda")
    G.grouped_ffn_gather(desc, h, src_d, off, w1b, w2b, y_g, ws)
    x_perm = h[src_d.long()].contiguous()
    y_c = torch.zeros((R, d), dtype=torch.bfloat16, device="cuda")
    G.grouped_ffn(desc, x_perm, off, w1b, w2b, y_c, ws)
    torch.cuda.synchronize()
    assert torch.equal(y_g[:rows], y_c[:rows]), f"gathered remainders seed {seed}: bits differ"


# wide layers with many ragged experts: several rounds of the persistent grid,
# riders, short tiles and leftover launches; seed 91011 draws 682 MiB of
# weights, past the 256 MiB last-level cache, so its leftover pieces load
# their weights non-temporal
@pytest.mark.parametrize("seed", [91000, 91001, 91002, 91003, 91011])
def test_wide_random_layouts_sampled_rows_and_per_expert_bits(seed):
    G = lib()
    rng = np.random.default_rng(seed)
    el = int(rng.integers(1, 40))
    full = rng.integers(0, 12, el)
    rem = rng.integers(0, 256, el)
    sizes = [int(v) for v in 256 * full + rem]
    d = 256 * int(rng.integers(1, 9))
    dff = 256 * int(rng.integers(1, 17))
    act = "swiglu" if rng.random() < 0.7 else "relu"
    slack = int(rng.choice([0, 1000]))
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(offsets[-1])
    w1r = 2 * dff if act == "swiglu" else dff
    say(f"seed {seed}: {el} experts, rows {rows} (+{slack} spare), d {d}, d_ff {dff}, {act}, "
        f"weights {el * (w1r + dff) * d * 2 / 2 ** 20:.0f} MiB")
    if rows == 0:
        return
    xb = dev(rng.standard_normal((rows, d)).astype(np.float32), torch.bfloat16)
    w1b = dev((rng.standard_normal((el, w1r, d)) * d ** -0.5).astype(np.float32), torch.bfloat16)
    w2b = dev((rng.standard_normal((el, d, dff)) * dff ** -0.5).astype(np.float32), torch.bfloat16)
    y = _run(G, xb, offsets, w1b, w2b, rows, d, dff, el, act, slack)
    torch.cuda.synchronize()
    # the first and last row of every 256-row tile, each expert's last rows, random rows
    pick = set(rng.choice(rows, size=min(rows, 128), replace=False).tolist())
    for e in range(el):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for r in range(lo, hi, 256):
            pick.update({r, min(r + 255, hi - 1)})
        if hi > lo:
            pick.update(range(max(lo, hi - 3), hi))
    pick = np.array(sorted(pick), np.int64)
    xs, w1s, w2s = host(xb), host(w1b), host(w2b)
    e_of = np.searchsorted(offsets.astype(np.int64), pick, side="right") - 1
    want = np.zeros((pick.size, d))
    for e in np.unique(e_of):
        m = e_of == e
        want[m] = O.expert_ffn(xs[pick[m]], w1s[e], w2s[e], act)
    assert_close(host(y[torch.as_tensor(pick, device="cuda")]), want, TOL["bf16"],
                 f"seed {seed}: sampled rows")
    for e in range(el):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        ye = _run(G, xb[lo:hi].contiguous(), np.array([0, hi - lo], np.int32),
                  w1b[e:e + 1].contiguous(), w2b[e:e + 1].contiguous(), hi - lo, d, dff, 1, act)
        torch.cuda.synchronize()
        assert torch.equal(ye, y[lo:hi]), f"seed {seed}: expert {e} differs when run alone"
