"""Checks that pin the CPU oracle to values fixed by the pages or by
mathematics (hand-derived fixtures, closed forms, brute force). Each check
takes the oracle function it examines as an argument, so the same check can
also be run against a deliberately broken copy (tests/test_oracle_mutations.py)
to show that it would catch that mistake."""
import itertools

import numpy as np

from tests.conftest import load_golden


def _beats(s, a, b):
    return s[a] > s[b] or (s[a] == s[b] and a < b)


def brute_force_ordered_topk(s, k):
    """The unique ordered k-sequence in which every member beats every expert
    not placed before it (finite scores only), found by enumeration."""
    E = len(s)
    found = []
    for seq in itertools.permutations(range(E), k):
        ok = True
        for i, a in enumerate(seq):
            for b in range(E):
                if b in seq[: i + 1]:
                    continue
                if not _beats(s, a, b):
                    ok = False
                    break
            if not ok:
                break
        if ok:
            found.append(list(seq))
    assert len(found) == 1, found
    return found[0]


def check_topk_golden(topk_fn, nonfinite_flag):
    for c in load_golden("topk_ties.json")["cases"]:
        s = np.array([c["logits"]], np.float64)
        idx, flags = topk_fn(s, c["k"])
        assert idx.tolist() == [c["idx"]], (c, idx)
        assert bool(flags & nonfinite_flag) == bool(c.get("nonfinite", False)), c


def check_topk_brute(topk_fn, seed=0):
    rng = np.random.default_rng(seed)
    for E in (2, 4, 6, 8):
        s = rng.integers(-2, 3, size=(40, E)).astype(np.float64)
        for k in range(1, min(E, 4) + 1):
            idx, _ = topk_fn(s, k)
            for t in range(s.shape[0]):
                assert idx[t].tolist() == brute_force_ordered_topk(s[t], k), (E, k, t)


def check_gate_closed_forms(gate_fn):
    g = load_golden("closed_forms.json")["gates"]
    s = np.array([g["logits"]])
    idx = np.array([g["idx"]])
    for mode in ("softmax", "softmax_topk_renorm", "sigmoid_topk_renorm"):
        got = gate_fn(s, idx, mode)[0]
        assert np.allclose(got, g[mode], rtol=0, atol=1e-12), (mode, got)


def check_swiglu_scalar(ffn_fn):
    for c in load_golden("closed_forms.json")["swiglu_scalar"]:
        x = np.array([[c["x"]]])
        w1 = np.array([[c["wg"]], [c["wu"]]])
        w2 = np.array([[c["w2"]]])
        got = ffn_fn(x, w1, w2, "swiglu")[0, 0]
        assert abs(got - c["y"]) < 1e-12, (c, got)
    for c in load_golden("closed_forms.json")["relu_scalar"]:
        got = ffn_fn(np.array([[c["x"]]]), np.array([[c["w1"]]]), np.array([[c["w2"]]]), "relu")[0, 0]
        assert abs(got - c["y"]) < 1e-12, (c, got)


def check_capacity_tables(plan_fn):
    for c in load_golden("capacity_tables.json")["cases"]:
        p = plan_fn(np.array(c["route"]), c["E"], c["capacity"], c["max_rows"])
        for key in ("counts", "kept", "offsets", "dest", "src_token", "src_slot"):
            assert np.asarray(p[key]).tolist() == c[key], (c["name"], key, p[key])
        assert p["flags"] == c["flags"], (c["name"], p["flags"])


def check_wrong_token_fixture(plan_fn, permute_fn, combine_fn):
    """Markers through permute -> identity expert -> combine: every token must
    get back exactly its own marker (unpermute page, A/B/C scenario)."""
    f = load_golden("wrong_token_abc.json")
    route = np.array(f["route"])
    p = plan_fn(route, f["E"], -1, None)
    for key in ("counts", "offsets", "dest", "src_token", "src_slot"):
        assert np.asarray(p[key]).tolist() == f[key], key
    h = np.array([[1.0, 0, 0], [0, 1.0, 0], [0, 0, 1.0]])
    x = permute_fn(h, p["dest"], int(p["offsets"][-1]))
    y = combine_fn(x, route, np.ones(route.shape), p["dest"], 0, f["E"])
    assert np.array_equal(y, h), y
