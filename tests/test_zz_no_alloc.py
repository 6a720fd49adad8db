"""The no-workspace permute (moe_permute_no_workspace) against moe_permute
with a caller workspace, through the C ABI: two calls in a row on one GPU,
the second with fewer tokens, must both give moe_permute's plan and rows bit
for bit (the second call reuses the fixed scratch the first one left), and
the plan must equal the oracle's."""
import numpy as np
import pytest
import torch

from tests.gpu_util import check_plan, dev, host, lib, say
from workloads import CONFIGS, make_inputs, small_layer_config

pytestmark = pytest.mark.gpu


def _bufs(G, desc):
    b = G.alloc_buffers(desc)
    b.flags.zero_()
    return b


def _compare(G, desc, h, idx, cap):
    ref = _bufs(G, desc)
    G.permute(desc, h, idx, ref.x_perm, ref.counts, ref.offsets, ref.dest, ref.src_token,
              ref.src_slot, ref.send_splits, ref.send_displs, ref.flags, G.alloc_workspace(desc))
    got = _bufs(G, desc)
    G.permute_no_workspace(desc, h, idx, got.x_perm, got.counts, got.offsets, got.dest,
                           got.src_token, got.src_slot, got.send_splits, got.send_displs,
                           got.flags)
    torch.cuda.synchronize()
    for f in ("counts", "offsets", "dest", "send_splits", "send_displs", "flags"):
        assert torch.equal(getattr(got, f), getattr(ref, f)), f
    n = min(int(host(ref.offsets)[-1]), desc.max_rows)
    for f in ("src_token", "src_slot", "x_perm"):
        assert torch.equal(getattr(got, f)[:n], getattr(ref, f)[:n]), f
    check_plan(G, desc, host(idx), got, desc.E, cap, desc.max_rows, desc.ep_size, desc.ep_rank)
    return n


@pytest.mark.parametrize("name,T1,T2", [("finegrained_bf16", 4096, 1000),
                                        ("small_bf16", 2048, 129),
                                        ("ep_share_bf16", 1024, 64)])
def test_permute_no_workspace_matches_permute_twice(name, T1, T2):
    G = lib()
    base = CONFIGS[name]
    for T in (T1, T2):
        cfg = small_layer_config(base, T)
        inp = make_inputs(cfg)
        cap = -1 if base.capacity_factors[-1] is None else int(
            base.capacity_factors[-1] * T * cfg.k // cfg.E)
        desc = G.make_desc(T, cfg.d, cfg.E, cfg.k, cfg.d_ff, cfg.dtype, cfg.gate, cfg.act,
                           ep_size=cfg.ep_size, ep_rank=cfg.ep_rank, capacity=cap)
        rng = np.random.default_rng(T)
        # skewed ids: low experts hot, so several tile histograms are lopsided
        idx = np.stack([rng.choice(cfg.E, size=cfg.k, replace=False,
                                   p=np.arange(cfg.E, 0, -1) / (cfg.E * (cfg.E + 1) / 2))
                        for _ in range(T)]).astype(np.int32)
        n = _compare(G, desc, dev(inp["h"], torch.bfloat16), dev(idx), cap)
        say(f"no-workspace permute {name} T={T} cap={cap}: {n} rows equal")


def test_permute_no_workspace_rejects_beyond_its_scratch():
    G = lib()
    desc = G.make_desc(131073, 64, 1024, 2, 64, "bf16", "softmax", "swiglu")
    with pytest.raises(G.MoeError) as e:
        G._check(G._lib.moe_permute_no_workspace(
            __import__("ctypes").byref(desc), *([__import__("ctypes").c_void_p(1 << 20)] * 11),
            None), "moe_permute_no_workspace")
    assert e.value.status == 8
