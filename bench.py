"""Benchmark of the MoE token-dispatch layer on one MI355X.

One step = one pass of the whole layer over one batch resident in HBM:
route (router GEMM + top-k + gates) -> permute (plan + row copy) -> grouped
expert FFN (two grouped GEMMs) -> unpermute + combine. The step is issued as
the four stage calls in order (the same kernels, in the same order, as the
fused call), with HIP events on the launch stream between stages so each
stage's duration comes from the timed region itself.

Prints one JSON line: routed tokens/s (tokens of the batch per second of
layer time), a roofline entry for the dominant kernel (the grouped FFN's
two MFMA GEMMs), per-stage figures, and the CPU oracle timed on a bounded
sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--skip-cpu-baseline]
                    [--cold-steps N]

After the timed steps, N more steps run one by one, each after a 512 MiB
write that evicts the 256 MiB last-level cache (MALL); their event-timed
median is reported as "cold_mall" beside (not in) the main figure.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FP32_PEAK_TFLOPS = 157.3


def ffn_flops(n_rows, d, dff, act):
    return (6 if act == "swiglu" else 4) * n_rows * d * dff


FFN_SOURCES = ("common.h", "gemm_core.h", "ffn.hip")


def kernel_source_sha(names=FFN_SOURCES):
    """Hash of the named kernel sources (default: those of the grouped FFN)."""
    h = hashlib.sha256()
    for name in names:
        h.update(open(os.path.join(ROOT, "grouped_expert_ffn_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def library_sha():
    """Hash of every HIP source of the library and its public header."""
    csrc = os.path.join(ROOT, "grouped_expert_ffn_amd", "csrc")
    h = hashlib.sha256(open(os.path.join(ROOT, "include", "moe_dispatch.h"), "rb").read())
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """Per-launch HBM bytes of the grouped FFN from the committed rocprofv3
    counter summary, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"pmc_grouped_ffn_{workload}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"^source_sha:\s*(\w+)", text, re.M)
    m_b = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_sha or not m_b or m_sha.group(1) != kernel_source_sha():
        return None
    return float(m_b.group(1))


def cpu_baseline(cfg, inp, capacity, sample_tokens, min_seconds):
    """The oracle, untouched, on the first `sample_tokens` tokens of the same
    workload (all expert weights), timed on the host cores; the sample is
    run repeatedly until at least `min_seconds` of CPU work has been timed."""
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    Ts = min(sample_tokens, cfg.T)
    cap = capacity if capacity < 0 else O.capacity_from_factor(
        capacity / (cfg.T * cfg.k / cfg.E), Ts, cfg.k, cfg.E)
    runs, total = 0, 0.0
    while total < min_seconds:
        t0 = time.perf_counter()
        O.layer(inp["h"][:Ts], inp["w_router"], inp["bias"], inp["w1"], inp["w2"], k=cfg.k,
                gate=cfg.gate, act=cfg.act, capacity=cap, ep_size=cfg.ep_size,
                ep_rank=cfg.ep_rank)
        total += time.perf_counter() - t0
        runs += 1
    return {"value": Ts * runs / total, "unit": "routed tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"first {Ts} of {cfg.T} tokens of {cfg.name}, all expert weights, "
                      f"float64 numpy oracle, {runs} run(s) in {total:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_bf16")
    ap.add_argument("--cf", type=float, default=None, help="capacity factor (default dropless)")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0)
    ap.add_argument("--gather", action="store_true",
                    help="fused dispatch: permute makes only the plan and the first expert GEMM "
                         "reads token rows from h through src_token")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="extra steps, each after a 512 MiB write that evicts the 256 MiB MALL, "
                         "timed one by one with events (reported beside the main figure)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the "
              "expert-parallel exchange across GPUs is not part of it", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration_mib:
        # a plain copy of known size: reads N bytes, writes N bytes per launch
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "launches": 3}), flush=True)
        return
    import grouped_expert_ffn_amd as G
    from workloads import CONFIGS, make_inputs

    cfg = CONFIGS[args.workload]
    inp = make_inputs(cfg)
    capacity = G.capacity_from_factor(args.cf, cfg.T, cfg.k, cfg.E)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dev = lambda a, t=None: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(t or dt)  # noqa
    desc = G.make_desc(cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff, cfg.dtype, cfg.gate, cfg.act,
                       ep_size=cfg.ep_size, ep_rank=cfg.ep_rank, capacity=capacity)
    h, wr = dev(inp["h"]), dev(inp["w_router"])
    bias = None if inp["bias"] is None else dev(inp["bias"], torch.float32)
    w1, w2 = dev(inp["w1"]), dev(inp["w2"])
    gather = args.gather
    b = G.alloc_buffers(desc, x_perm=not gather)
    ws = G.alloc_workspace(desc)
    y = torch.empty((cfg.T, cfg.d), dtype=dt, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        G.route(desc, h, wr, bias, b.logits, b.topk_idx, b.topk_gate, b.flags, ws)
        if ev is not None:
            ev[1].record(stream)
        G.permute(desc, h, b.topk_idx, b.x_perm, b.counts, b.offsets, b.dest, b.src_token,
                  b.src_slot, b.send_splits, b.send_displs, b.flags, ws)
        if ev is not None:
            ev[2].record(stream)
        if gather:
            G.grouped_ffn_gather(desc, h, b.src_token, b.offsets, w1, w2, b.y_perm, ws)
        else:
            G.grouped_ffn(desc, b.x_perm, b.offsets, w1, w2, b.y_perm, ws)
        if ev is not None:
            ev[3].record(stream)
        G.unpermute_combine(desc, b.y_perm, b.topk_idx, b.topk_gate, b.dest, y)
        if ev is not None:
            ev[4].record(stream)

    b.flags.zero_()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    stage = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in evs])  # ms

    # the same step with a cold last-level cache: a 512 MiB write before each
    # step evicts the 256 MiB MALL (outside the events that time the step)
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
               for _ in range(args.cold_steps)]
        for i in range(args.cold_steps):
            flush.fill_(i & 0xff)
            step(cev[i])
        torch.cuda.synchronize()
        cst = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in cev])
        cold = {"steps": args.cold_steps, "ms_per_step": float(np.median(cst.sum(axis=1))),
                "route_ms": float(np.median(cst[:, 0])), "permute_ms": float(np.median(cst[:, 1])),
                "grouped_ffn_ms": float(np.median(cst[:, 2])),
                "combine_ms": float(np.median(cst[:, 3]))}
        cold["tokens_per_s"] = cfg.T / (cold["ms_per_step"] / 1e3)
        del flush
    st_ms = np.median(stage, axis=0)
    flags = int(b.flags.item())
    offs = b.offsets.cpu().numpy().astype(np.int64)
    el = cfg.E // cfg.ep_size
    lo, hi = cfg.ep_rank * el, (cfg.ep_rank + 1) * el
    n_kept = int(offs[-1])
    n_local = int(offs[hi] - offs[lo])
    eb = 2 if cfg.dtype == "bf16" else 4
    Tk = cfg.T * cfg.k
    # algorithmic bytes: permute reads each token row once and writes each kept
    # assignment's row, plus 12 B of ids/rows per assignment; combine reads the
    # local kept rows and writes one row per token, plus 12 B per assignment
    permute_bytes = (0 if gather else cfg.T * cfg.d * eb + n_kept * cfg.d * eb) + 12 * Tk
    combine_bytes = n_local * cfg.d * eb + cfg.T * cfg.d * eb + 12 * Tk
    flops = ffn_flops(n_local, cfg.d, cfg.d_ff, cfg.act)
    ffn_s = st_ms[2] / 1e3
    peak = BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else FP32_PEAK_TFLOPS
    achieved = flops / ffn_s / 1e12
    traffic = measured_traffic(cfg.name)
    ms_per_step = wall / args.steps * 1e3
    out = {
        "metric": "routed tokens/sec per MoE layer (route+permute+FFN+combine)",
        "value": cfg.T * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) weights)",
        "config": {"workload": f"{cfg.name}: {cfg.description}", "T": cfg.T, "d": cfg.d,
                   "E": cfg.E, "k": cfg.k, "d_ff": cfg.d_ff, "act": cfg.act, "gate": cfg.gate,
                   "experts_local": el, "capacity": capacity, "parallelism": "1 GPU",
                   "dispatch": "rows gathered by the first expert GEMM" if gather
                   else "rows copied into expert order"},
        "roofline": {"kernel": "grouped expert FFN (tile map + SwiGLU GEMM + down GEMM)",
                     "bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "flops_per_launch": flops, "launch_ms": st_ms[2]},
        "stages": {
            "route_ms": st_ms[0], "permute_ms": st_ms[1], "grouped_ffn_ms": st_ms[2],
            "combine_ms": st_ms[3],
            "permute_GBs": permute_bytes / (st_ms[1] / 1e3) / 1e9,
            "combine_GBs": combine_bytes / (st_ms[3] / 1e3) / 1e9,
            "permute_plus_combine_hbm_frac":
                (permute_bytes + combine_bytes) / ((st_ms[1] + st_ms[3]) / 1e3) / 1e9 / HBM_PEAK_GBS,
            "rows_kept": n_kept, "rows_local": n_local, "flags": flags,
        },
        "cold_mall": cold,
        "env": {"device": torch.cuda.get_device_name(), "torch": torch.__version__,
                "hip": torch.version.hip, "library_sha": library_sha()},
    }
    if not args.skip_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, capacity, args.cpu_sample_tokens,
                                          args.cpu_min_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
