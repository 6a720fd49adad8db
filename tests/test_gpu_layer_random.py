"""GPU parity of the whole layer on seeded random configurations: token
count, widths, expert count, k, activation, gate form, dtype, capacity,
expert-parallel share and router bias all drawn per case. Each case checks the
copying path against the oracle (routing and plan bit-exact, y within
tolerance of the per-token oracle on the GPU's routing), the gathered and
slot-ordered paths bitwise against it, and the deduplicated expert-parallel
packing against the oracle, with the local experts run from its pair rows
bitwise equal to the plain path's rows."""
import numpy as np
import pytest
import torch

from tests.gpu_util import host, lib, run_layer, say, upload_layer
from tests.test_gpu_dedup import _check_pack, _pack
from tests.test_gpu_layer import _check_layer
from workloads import LayerConfig, make_inputs

pytestmark = pytest.mark.gpu


def random_layer(seed):
    """One configuration and its capacity factor (None: dropless)."""
    rng = np.random.default_rng(seed)
    E = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16, 32, 64]))
    k = int(rng.integers(1, min(E, 8) + 1))
    ep = int(rng.choice([e for e in (1, 2, 4, 8) if E % e == 0]))
    fp32 = rng.random() < 0.15
    cfg = LayerConfig(
        f"random{seed}", 200 + seed % 50, T=int(rng.integers(1, 1500)),
        d=(int(rng.integers(1, 7)) * 16 if fp32 else 64 * int(rng.integers(1, 7))),
        E=E, k=k,
        d_ff=(int(rng.integers(1, 9)) * 16 if fp32 else 64 * int(rng.integers(1, 25))),
        act=str(rng.choice(["swiglu", "relu"])),
        gate=str(rng.choice(["softmax", "softmax_topk_renorm", "sigmoid_topk_renorm"])),
        dtype="f32" if fp32 else "bf16", ep_size=ep, ep_rank=int(rng.integers(0, ep)),
        zipf_bias=(1.2, 1.2) if rng.random() < 0.3 else None)
    cf = rng.choice([None, None, 0.5, 1.0, 1.25])
    return cfg, (None if cf is None else float(cf))


@pytest.mark.parametrize("seed", range(70000, 70048))
def test_random_layer_against_oracle_and_fused_paths(seed):
    G = lib()
    cfg, cf = random_layer(seed)
    capacity = G.capacity_from_factor(-1.0 if cf is None else cf, cfg.T, cfg.k, cfg.E)
    say(f"seed {seed}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} d_ff={cfg.d_ff} {cfg.act} "
        f"{cfg.gate} {cfg.dtype} ep={cfg.ep_size}/{cfg.ep_rank} capacity={capacity} "
        f"zipf={cfg.zipf_bias is not None}")
    inp = make_inputs(cfg)
    desc, dv = upload_layer(G, cfg, inp, capacity=capacity)
    y, bufs, ws = run_layer(G, desc, dv)
    _check_layer(G, cfg, inp, desc, y, bufs, capacity)
    if cfg.dtype != "bf16":
        return
    # fused dispatch: the first expert GEMM reads the rows from h
    y2, _, _ = run_layer(G, desc, dv, bufs=G.alloc_buffers(desc, x_perm=False), ws=ws)
    assert torch.equal(y2, y), "gathered path"
    # slot-ordered output and its combine
    ys = torch.zeros((cfg.T * cfg.k, cfg.d), dtype=y.dtype, device="cuda")
    G.grouped_ffn_slots(desc, dv["h"], bufs.src_token, bufs.src_slot, bufs.offsets, dv["w1"],
                        dv["w2"], ys, ws)
    y3 = torch.empty_like(y)
    G.combine_slots(desc, ys, bufs.topk_idx, bufs.topk_gate, bufs.dest, y3)
    torch.cuda.synchronize()
    assert torch.equal(y3, y), "slot path"
    # one send row per (destination rank, token) pair, and the experts run from those rows
    out = _pack(G, desc, dv["h"], bufs.topk_idx, bufs, ws)
    _, lo, hi = _check_pack(desc, dv["h"], host(bufs.topk_idx), bufs, out)
    y4 = torch.zeros_like(bufs.y_perm)
    G.grouped_ffn_gather(desc, out["send_buf"], out["recv_rows"], bufs.offsets, dv["w1"],
                         dv["w2"], y4, ws)
    torch.cuda.synchronize()
    assert torch.equal(y4[lo:hi], bufs.y_perm[lo:hi]), "experts run from the pair rows"
