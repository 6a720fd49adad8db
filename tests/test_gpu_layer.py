"""GPU parity of the fused layer call (route -> permute -> grouped FFN ->
unpermute/combine) against the oracle, plus the properties the pages ask
for: identity/marker experts, determinism, batch invariance, graph capture."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from tests.gpu_util import (LOGIT_TOL, TOL, assert_close, certified_route_mismatch, check_plan,
                            check_rows_vs_oracle, check_tokens_vs_oracle, dev, edge_rows, host,
                            lib, run_layer, sample_tokens, say, upload_layer)
from workloads import (CONFIGS, identity_scale_experts, make_inputs, marker_tokens,
                       small_layer_config)

pytestmark = pytest.mark.gpu


def _check_layer(G, cfg, inp, desc, y, bufs, capacity, sample=None):
    """Stage-exact routing and plan, then outputs against the oracle run on
    the GPU's own routing (route replay) with float64 scores for the gates."""
    T, k, E = desc.T, cfg.k, cfg.E
    h = inp["h"][:T]
    s32 = host(bufs.logits)
    s64 = O.router_logits(h, inp["w_router"], inp["bias"])
    assert_close(s32, s64, LOGIT_TOL, "logits")
    gi = host(bufs.topk_idx)
    ref_idx, _ = O.topk_route(s32, k)
    assert np.array_equal(gi, ref_idx), "ordered top-k of the GPU scores"
    near = certified_route_mismatch(gi, s32, s64, k)
    ref = check_plan(G, desc, gi, bufs, E, capacity, desc.max_rows, cfg.ep_size, cfg.ep_rank)
    n = ref["src_token"].shape[0]
    rows = np.arange(n) if sample is None else np.unique(np.linspace(0, max(n - 1, 0), min(n, 512)).astype(int))
    if n:
        assert np.array_equal(host(bufs.x_perm[torch.as_tensor(rows, device="cuda")]),
                              h[ref["src_token"][rows]]), "x_perm rows"
    toks = range(T) if sample is None else sample
    toks = list(toks)
    want = O.brute_force_tokens(h, inp["w_router"], inp["bias"], inp["w1"], inp["w2"], toks,
                                k=k, gate=cfg.gate, act=cfg.act, capacity=capacity,
                                ep_size=cfg.ep_size, ep_rank=cfg.ep_rank, route_idx=gi)
    got = host(y[torch.as_tensor(toks, device="cuda")]) if toks else np.zeros((0, cfg.d))
    err = assert_close(got, want, TOL[cfg.dtype], f"y {cfg.name}")
    say(f"  {cfg.name} T={T} cap={capacity}: max abs/rel err {err}, near ties {len(near)}, "
        f"flags {int(host(bufs.flags)[0])}")
    return ref, near


def test_tiny_layer_full_parity():
    G = lib()
    cfg = CONFIGS["tiny_fp32"]
    inp = make_inputs(cfg)
    desc, dv = upload_layer(G, cfg, inp)
    y, bufs, _ = run_layer(G, desc, dv)
    _, near = _check_layer(G, cfg, inp, desc, y, bufs, -1)
    assert not near
    full = O.layer(inp["h"], inp["w_router"], None, inp["w1"], inp["w2"], k=cfg.k,
                   gate=cfg.gate, act=cfg.act)
    assert_close(host(y), full["y"], TOL["f32"], "y vs oracle layer")


@pytest.mark.parametrize("cap", [0, 3, 20, 31])
def test_tiny_layer_capacity(cap):
    G = lib()
    cfg = CONFIGS["tiny_fp32"]
    inp = make_inputs(cfg)
    desc, dv = upload_layer(G, cfg, inp, capacity=cap)
    y, bufs, _ = run_layer(G, desc, dv)
    _check_layer(G, cfg, inp, desc, y, bufs, cap)
    if cap == 0:
        assert not host(y).any()


def test_identity_experts_and_marker_tokens():
    """f_e(h) = c_e h with c = 1, 2, 4, 8 and one-hot markers: every output
    row is its own marker scaled by sum_j g_j c_(e_j); a row from the wrong
    token changes the support, a gate on the wrong row the magnitude."""
    G = lib()
    cfg = CONFIGS["tiny_fp32"]
    inp = make_inputs(cfg)
    scales = np.array([1.0, 2.0, 4.0, 8.0])
    inp["w1"], inp["w2"] = identity_scale_experts(cfg.d, scales)
    inp["h"] = marker_tokens(cfg.T, cfg.d)
    desc, dv = upload_layer(G, cfg, inp)
    y, bufs, _ = run_layer(G, desc, dv)
    gi = host(bufs.topk_idx)
    s64 = O.router_logits(inp["h"], inp["w_router"])
    coef = (O.gate_weights(s64, gi, cfg.gate) * scales[gi]).sum(1)
    got = host(y)
    assert_close(got, coef[:, None] * inp["h"], TOL["f32"], "markers")
    assert np.array_equal(got != 0, inp["h"] != 0)


# layer shapes at reduced T, full d / d_ff / E / k, every capacity mode
SMALL_T = {"tiny_fp32": 64, "small_bf16": 1024, "mixtral_bf16": 256,
           "finegrained_bf16": 1024, "ep_share_bf16": 512}


@pytest.mark.parametrize("name", list(CONFIGS))
def test_layer_shapes_reduced_tokens(name):
    G = lib()
    base = CONFIGS[name]
    cfg = small_layer_config(base, SMALL_T[name])
    inp = make_inputs(cfg)
    for cf in base.capacity_factors:
        cap = O.capacity_from_factor(cf, cfg.T, cfg.k, cfg.E)
        assert G.capacity_from_factor(cf, cfg.T, cfg.k, cfg.E) == cap
        say(f"layer {name} T={cfg.T} cf={cf}")
        desc, dv = upload_layer(G, cfg, inp, capacity=cap)
        y, bufs, _ = run_layer(G, desc, dv)
        _check_layer(G, cfg, inp, desc, y, bufs, cap)


@pytest.mark.slow
@pytest.mark.parametrize("name", list(CONFIGS))
def test_layer_full_size_sampled(name):
    """The layer at its full size, in the launch configuration the benchmark
    times: routing and plan are checked on every token, x_perm on sampled
    rows, and the oracle checks a stratified sample: y on 64 random tokens
    plus every token whose row sits at an edge of an expert's row tiles (all
    rows of each expert's last tile when it is short: the tiles the expert
    GEMMs run on half their waves and move into their leftover launch, whose
    weight loads are non-temporal when the experts' weights exceed the
    last-level cache), and the expert outputs y_perm of those rows."""
    G = lib()
    cfg = CONFIGS[name]
    say(f"full {name}: drawing inputs")
    inp = make_inputs(cfg)
    el = cfg.E // cfg.ep_size
    for cf in cfg.capacity_factors:
        cap = O.capacity_from_factor(cf, cfg.T, cfg.k, cfg.E)
        say(f"full {name} cf={cf}: running")
        desc, dv = upload_layer(G, cfg, inp, capacity=cap)
        y, bufs, _ = run_layer(G, desc, dv)
        ref, near = _check_layer(G, cfg, inp, desc, y, bufs, cap,
                                 sample=sample_tokens(cfg.T, 64, 99, (0, cfg.T - 1)))
        assert len(near) <= max(2, cfg.T // 2000)
        counts = ref["counts"]
        say(f"  histogram (first 16 experts) {counts[:16].tolist()}, empty experts "
            f"{int((counts == 0).sum())}, dropped {int((ref['dest'] == -1).sum())}, "
            f"splits {ref['send_splits'].tolist()}")
        rows = edge_rows(ref["offsets"], cfg.ep_rank * el, (cfg.ep_rank + 1) * el,
                         desc.max_rows, short_all=128 if el <= 8 else 0,
                         per_edge=4 if el > 8 else 8, seed=7)
        src = ref["src_token"]
        err = check_rows_vs_oracle(cfg, inp, host(bufs.y_perm[torch.as_tensor(rows, device="cuda")]),
                                   rows, src, ref["offsets"], f"y_perm edge rows {name}")
        toks = sorted(set(int(src[r]) for r in rows))
        err2 = check_tokens_vs_oracle(cfg, inp, y, host(bufs.topk_idx), toks, cap,
                                      f"y edge tokens {name}")
        say(f"  edge rows {len(rows)} (tokens {len(toks)}): y_perm err {err}, y err {err2}")
        del dv, y, bufs
        torch.cuda.empty_cache()


def test_optional_outputs_left_null():
    """The fused call with every optional buffer NULL (the workspace holds
    the routing and plan) gives y bitwise equal to the call with every
    buffer given, in both dispatch modes, and within tolerance of the oracle."""
    G = lib()
    for name, T in (("finegrained_bf16", 1024), ("tiny_fp32", 64), ("ep_share_bf16", 256)):
        base = CONFIGS[name]
        cfg = small_layer_config(base, T)
        inp = make_inputs(cfg)
        cap = O.capacity_from_factor(base.capacity_factors[-1], cfg.T, cfg.k, cfg.E)
        say(f"optional outputs NULL: {name} T={T} cap={cap}")
        desc, dv = upload_layer(G, cfg, inp, capacity=cap)
        y_full, b_full, ws = run_layer(G, desc, dv)
        for gather in (False, True):
            b = G.alloc_buffers(desc, x_perm=not gather, outputs=False)
            y = torch.full_like(y_full, float("nan"))
            G.layer_forward(desc, dv["h"], dv["w_router"], dv["bias"], dv["w1"], dv["w2"], y,
                            b, ws)
            torch.cuda.synchronize()
            assert torch.equal(y, y_full), (name, gather)
        check_tokens_vs_oracle(cfg, inp, y, host(b_full.topk_idx), range(T), cap,
                               f"y {name} optional outputs NULL")


def test_run_twice_bitwise_identical():
    G = lib()
    cfg = small_layer_config(CONFIGS["finegrained_bf16"], 2048)
    inp = make_inputs(cfg)
    cap = O.capacity_from_factor(1.25, cfg.T, cfg.k, cfg.E)
    desc, dv = upload_layer(G, cfg, inp, capacity=cap)
    y1, b1, ws = run_layer(G, desc, dv)
    y1 = y1.clone()
    snap = {f: getattr(b1, f).clone() for f in ("logits", "topk_idx", "topk_gate", "dest", "y_perm")}
    y2, b2, _ = run_layer(G, desc, dv, bufs=b1, ws=ws)
    assert torch.equal(y1, y2)
    for f, v in snap.items():
        assert torch.equal(v, getattr(b2, f)), f


def test_dropless_batch_invariance():
    """A token alone-in-a-smaller-batch and in the full batch gets the same
    scores, route and output bits (dropless; capacity couples the batch)."""
    G = lib()
    cfg = small_layer_config(CONFIGS["small_bf16"], 2048)
    inp = make_inputs(cfg)
    desc, dv = upload_layer(G, cfg, inp)
    y_full, b_full, _ = run_layer(G, desc, dv)
    sub = np.arange(300, 300 + 777)
    desc_s, dv_s = upload_layer(G, cfg, inp, T=len(sub), h=inp["h"][sub])
    y_sub, b_sub, _ = run_layer(G, desc_s, dv_s)
    ts = torch.as_tensor(sub, device="cuda")
    assert torch.equal(b_full.logits[ts], b_sub.logits)
    assert torch.equal(b_full.topk_idx[ts], b_sub.topk_idx)
    assert torch.equal(y_full[ts], y_sub)


def test_graph_capture_replays_match_eager():
    """The fused call holds no host sync or device-to-host copy, so it can be
    captured; replays with eager work in between must match the eager run."""
    G = lib()
    cfg = small_layer_config(CONFIGS["finegrained_bf16"], 1024)
    inp = make_inputs(cfg)
    desc, dv = upload_layer(G, cfg, inp)
    y_eager, bufs, ws = run_layer(G, desc, dv)
    y_eager = y_eager.clone()
    y = torch.empty_like(y_eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        G.layer_forward(desc, dv["h"], dv["w_router"], dv["bias"], dv["w1"], dv["w2"], y, bufs, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        G.layer_forward(desc, dv["h"], dv["w_router"], dv["bias"], dv["w1"], dv["w2"], y, bufs, ws)
    for i in range(3):
        y.zero_()
        bufs.x_perm.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {i}"
