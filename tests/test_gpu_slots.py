"""GPU parity of the slot-ordered FFN output (moe_grouped_ffn_slots) and its
combine (moe_combine_slots): every computed slot row must hold the bits of
y_perm[dest] from the plain path, rows of other slots stay untouched, the
combined output must equal moe_unpermute_combine's bit for bit, and both
are checked against the oracle: slot rows against f_e of their token, the
combined output against the per-token oracle (or the oracle layer when rows
are clamped), each slot's expert output weighted by its own token's gate."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from tests.gpu_util import (TOL, assert_close, check_rows_vs_oracle, check_tokens_vs_oracle, host,
                            lib, run_layer, sample_tokens, say, upload_layer)
from workloads import CONFIGS, make_inputs, small_layer_config

pytestmark = pytest.mark.gpu


def _slots_path(G, desc, dv, b, ws):
    dt = G.torch_dtype(desc)
    y_slots = torch.full((desc.T * desc.k, desc.d), float("nan"), dtype=dt, device="cuda")
    G.grouped_ffn_slots(desc, dv["h"], b.src_token, b.src_slot, b.offsets, dv["w1"], dv["w2"],
                        y_slots, ws)
    y2 = torch.full((desc.T, desc.d), float("nan"), dtype=dt, device="cuda")
    G.combine_slots(desc, y_slots, b.topk_idx, b.topk_gate, b.dest, y2)
    torch.cuda.synchronize()
    return y_slots, y2


def _check(desc, b, y, y_slots, y2, el):
    dest = host(b.dest).astype(np.int64)
    idx = host(b.topk_idx).astype(np.int64)
    local = (idx // el) == desc.ep_rank
    used = (dest >= 0) & local
    t, j = np.nonzero(used)
    slots = torch.from_numpy(t * desc.k + j).cuda()
    rows = torch.from_numpy(dest[t, j]).cuda()
    assert torch.equal(y_slots[slots], b.y_perm[rows]), "slot rows differ from y_perm[dest]"
    t2, j2 = np.nonzero(~used)
    if len(t2):
        untouched = y_slots[torch.from_numpy(t2 * desc.k + j2).cuda()]
        assert torch.isnan(untouched.float()).all(), "rows of unused slots were written"
    assert torch.equal(y2, y), "combine from slots differs from the plain combine"
    return int(used.sum())


def _oracle(cfg, inp, b, y2, y_slots, cap, seed=0, n_tok=96, n_slots=64):
    """y2 on sampled tokens against the per-token oracle; sampled slot rows
    of y_slots against f_e of their token."""
    T, k = cfg.T, cfg.k
    gi = host(b.topk_idx)
    toks = sample_tokens(T, n_tok, seed, (0, T - 1))
    e1 = check_tokens_vs_oracle(cfg, inp, y2, gi, toks, cap, f"y from slots {cfg.name}")
    el = cfg.E // cfg.ep_size
    dest = host(b.dest).astype(np.int64)
    used = (dest >= 0) & ((gi // el) == cfg.ep_rank)
    t, j = np.nonzero(used)
    if len(t) > n_slots:
        pick = np.random.default_rng(seed).choice(len(t), n_slots, replace=False)
        t, j = t[pick], j[pick]
    e2 = check_rows_vs_oracle(cfg, inp, host(y_slots[torch.from_numpy(t * k + j).cuda()]),
                              dest[t, j], host(b.src_token), host(b.offsets),
                              f"slot rows {cfg.name}")
    say(f"  oracle: y err {e1}, slot rows err {e2} ({len(toks)} tokens, {len(t)} slots)")


# (layer, tokens, ep_size, ep_rank)
CASES = [("tiny_fp32", 64, 1, 0), ("small_bf16", 1024, 1, 0), ("small_bf16", 1024, 4, 1),
         ("mixtral_bf16", 256, 1, 0), ("finegrained_bf16", 1024, 1, 0),
         ("ep_share_bf16", 512, 8, 0)]


@pytest.mark.parametrize("name,T,ep,rank", CASES)
def test_slot_rows_and_combine_bit_identical(name, T, ep, rank):
    G = lib()
    base = CONFIGS[name]
    cfg = small_layer_config(base, T, ep_size=ep, ep_rank=rank)
    inp = make_inputs(cfg)
    for cf in base.capacity_factors:
        cap = O.capacity_from_factor(cf, cfg.T, cfg.k, cfg.E)
        say(f"slots {name} T={T} ep={ep}/{rank} cf={cf}")
        desc, dv = upload_layer(G, cfg, inp, capacity=cap)
        y, b, ws = run_layer(G, desc, dv)
        y_slots, y2 = _slots_path(G, desc, dv, b, ws)
        n = _check(desc, b, y, y_slots, y2, cfg.E // cfg.ep_size)
        say(f"  {n} slot rows checked")
        _oracle(cfg, inp, b, y2, y_slots, cap, seed=T + ep)


def test_slots_with_rows_clamped_to_max_rows():
    G = lib()
    cfg = small_layer_config(CONFIGS["small_bf16"], 600)
    inp = make_inputs(cfg)
    desc, dv = upload_layer(G, cfg, inp, max_rows=900)
    y, b, ws = run_layer(G, desc, dv)
    assert int(host(b.flags)[0]) & G.FLAG_ROW_OVERFLOW
    y_slots, y2 = _slots_path(G, desc, dv, b, ws)
    _check(desc, b, y, y_slots, y2, cfg.E)
    # slots past max_rows are not computed: the oracle layer with the same
    # row limit, on the GPU's routing
    ref = O.layer(inp["h"], inp["w_router"], inp["bias"], inp["w1"], inp["w2"], k=cfg.k,
                  gate=cfg.gate, act=cfg.act, max_rows=900, route_idx=host(b.topk_idx))
    assert_close(host(y2), ref["y"], TOL[cfg.dtype], "y from slots, rows clamped")


@pytest.mark.slow
def test_slots_full_mixtral_layer():
    G = lib()
    cfg = CONFIGS["mixtral_bf16"]
    inp = make_inputs(cfg)
    desc, dv = upload_layer(G, cfg, inp)
    y, b, ws = run_layer(G, desc, dv)
    y_slots, y2 = _slots_path(G, desc, dv, b, ws)
    _check(desc, b, y, y_slots, y2, cfg.E)
    _oracle(cfg, inp, b, y2, y_slots, -1, seed=3, n_tok=64, n_slots=64)
