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
