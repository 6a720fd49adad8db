"""GPU parity of the fused dispatch: the first expert GEMM reading token rows
straight from h through src_token (moe_grouped_ffn_gather, and the fused
call with x_perm NULL) must give bit-identical results to the path that
copies the rows into x_perm first, and the oracle parity that path has."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from tests.gpu_util import (TOL, assert_close, check_rows_vs_oracle, check_tokens_vs_oracle, host,
                            lib, run_layer, sample_tokens, say, upload_layer)
from workloads import CONFIGS, make_inputs, small_layer_config

pytestmark = pytest.mark.gpu

SMALL_T = {"tiny_fp32": 64, "small_bf16": 1024, "mixtral_bf16": 256,
           "finegrained_bf16": 1024, "ep_share_bf16": 512}


def _both(G, desc, dv):
    """The fused call with and without x_perm on the same inputs."""
    y_a, b_a, _ = run_layer(G, desc, dv)
    b_g = G.alloc_buffers(desc, x_perm=False)
    y_g, b_g, _ = run_layer(G, desc, dv, bufs=b_g)
    return (y_a, b_a), (y_g, b_g)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_fused_call_without_x_perm_is_bit_identical(name):
    G = lib()
    base = CONFIGS[name]
    cfg = small_layer_config(base, SMALL_T[name])
    inp = make_inputs(cfg)
    for cf in base.capacity_factors:
        cap = O.capacity_from_factor(cf, cfg.T, cfg.k, cfg.E)
        say(f"gather {name} T={cfg.T} cf={cf}")
        desc, dv = upload_layer(G, cfg, inp, capacity=cap)
        (y_a, b_a), (y_g, b_g) = _both(G, desc, dv)
        for f in ("logits", "topk_idx", "topk_gate", "counts", "offsets", "dest",
                  "send_splits", "send_displs", "flags"):
            assert torch.equal(getattr(b_a, f), getattr(b_g, f)), f
        n = min(int(host(b_a.offsets)[-1]), desc.max_rows)
        assert torch.equal(b_a.src_token[:n], b_g.src_token[:n])
        assert torch.equal(y_a, y_g), "y differs between gathered and copied rows"
        el = cfg.E // cfg.ep_size
        lo, hi = host(b_a.offsets)[[cfg.ep_rank * el, (cfg.ep_rank + 1) * el]]
        hi = min(int(hi), desc.max_rows)
        assert torch.equal(b_a.y_perm[lo:hi], b_g.y_perm[lo:hi]), "local y_perm rows"
        # and the gathered path's output against the oracle
        toks = sample_tokens(cfg.T, 96, cfg.T, (0, cfg.T - 1))
        err = check_tokens_vs_oracle(cfg, inp, y_g, host(b_g.topk_idx), toks, cap,
                                     f"gathered y {name}")
        say(f"  oracle on {len(toks)} tokens: max abs/rel err {err}")


def test_gather_stage_call_matches_grouped_ffn_and_oracle():
    """moe_permute without x_perm makes the same plan; moe_grouped_ffn_gather
    on it gives the rows moe_grouped_ffn gives on x_perm, and both match the
    oracle's expert FFN on those rows."""
    G = lib()
    cfg = small_layer_config(CONFIGS["finegrained_bf16"], 777)
    inp = make_inputs(cfg)
    desc, dv = upload_layer(G, cfg, inp)
    y, b, ws = run_layer(G, desc, dv)
    plan = {f: getattr(b, f).clone() for f in ("counts", "offsets", "dest", "src_token",
                                                 "src_slot", "send_splits", "send_displs")}
    b2 = G.alloc_buffers(desc, x_perm=False)
    b2.flags.zero_()
    G.permute(desc, dv["h"], b.topk_idx, None, b2.counts, b2.offsets, b2.dest, b2.src_token,
              b2.src_slot, b2.send_splits, b2.send_displs, b2.flags, ws)
    n = int(host(b.offsets)[-1])
    for f, v in plan.items():
        got = getattr(b2, f)
        if f in ("src_token", "src_slot"):
            got, v = got[:n], v[:n]
        assert torch.equal(got, v), f
    G.grouped_ffn_gather(desc, dv["h"], b2.src_token, b2.offsets, dv["w1"], dv["w2"],
                         b2.y_perm, ws)
    torch.cuda.synchronize()
    assert torch.equal(b2.y_perm[:n], b.y_perm[:n])
    rows = np.unique(np.linspace(0, n - 1, 64).astype(int))
    src = host(b.src_token)[rows]
    offs = host(b.offsets)
    experts = np.searchsorted(offs, rows, side="right") - 1
    for r, t, e in zip(rows, src, experts):
        ref = O.expert_ffn(inp["h"][t][None, :], inp["w1"][e], inp["w2"][e], cfg.act)[0]
        assert_close(host(b2.y_perm[r])[None, :], ref[None, :], TOL["bf16"], f"row {r}")


def test_gather_with_rows_clamped_to_max_rows():
    """More assignments than rows: the gathered GEMM stops at max_rows like
    the copying one, and the fused calls agree bit for bit."""
    G = lib()
    cfg = small_layer_config(CONFIGS["small_bf16"], 600)
    inp = make_inputs(cfg)
    desc, dv = upload_layer(G, cfg, inp, max_rows=900)
    (y_a, b_a), (y_g, b_g) = _both(G, desc, dv)
    assert int(host(b_a.flags)[0]) & G.FLAG_ROW_OVERFLOW
    assert torch.equal(y_a, y_g)
    assert torch.equal(b_a.y_perm[:900], b_g.y_perm[:900])


@pytest.mark.slow
def test_fused_call_without_x_perm_full_mixtral_layer():
    """The Mixtral-shaped layer at full size: gathered and copied rows give
    the same output bits."""
    G = lib()
    cfg = CONFIGS["mixtral_bf16"]
    inp = make_inputs(cfg)
    desc, dv = upload_layer(G, cfg, inp)
    (y_a, _), (y_g, b_g) = _both(G, desc, dv)
    assert torch.equal(y_a, y_g)
    toks = sample_tokens(cfg.T, 48, 17, (0, cfg.T - 1))
    check_tokens_vs_oracle(cfg, inp, y_g, host(b_g.topk_idx), toks, -1, "gathered y, Mixtral")


@pytest.mark.parametrize("name,T", [("small_bf16", 1024), ("finegrained_bf16", 1024),
                                    ("ep_share_bf16", 512), ("tiny_fp32", 64)])
def test_ablation_baselines_give_the_grouped_bits(name, T):
    """The benchmark's baselines (one grouped call per expert; the padded
    [E_loc, C, d] layout) run the same kernels on the same rows, so they
    must reproduce the grouped call's output bits."""
    import bench
    G = lib()
    cfg = small_layer_config(CONFIGS[name], T)
    inp = make_inputs(cfg)
    desc, dv = upload_layer(G, cfg, inp)
    y, b, _ = run_layer(G, desc, dv)
    info, y_grp, y_pe, y_pad = bench.ablation_baselines(G, desc, b.x_perm, b.offsets,
                                                        dv["w1"], dv["w2"], reps=1)
    say(f"ablation {name}: {info}")
    el = cfg.E // cfg.ep_size
    lo, hi = host(b.offsets)[[cfg.ep_rank * el, (cfg.ep_rank + 1) * el]]
    assert torch.equal(y_grp[lo:hi], b.y_perm[lo:hi])
    assert torch.equal(y_pe[lo:hi], y_grp[lo:hi])
    assert torch.equal(y_pad[lo:hi], y_grp[lo:hi])
    assert info["real_rows"] == int(hi - lo)
    # each baseline's rows against the oracle's f_e of the token they hold
    rows = np.unique(np.linspace(lo, hi - 1, 64).astype(int)) if hi > lo else np.zeros(0, int)
    offs, src = host(b.offsets), host(b.src_token)
    ri = torch.as_tensor(rows, device="cuda")
    for tag, yy in (("per expert", y_pe), ("padded", y_pad)):
        err = check_rows_vs_oracle(cfg, inp, host(yy[ri]), rows, src, offs,
                                   f"ablation {tag} {name}")
        say(f"  {tag}: oracle err on {len(rows)} rows {err}")
