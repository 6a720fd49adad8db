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
                    [--warm-steps N] [--clock-steps N] [--gather] [--slots] [--ablation]
                    [--dedup]

Each timed step runs right after a 512 MiB write that evicts the 256 MiB
last-level cache (MALL), outside the step's events, so no step finds its
inputs or weights left in the MALL by the one before; `value` is the batch's
tokens over the summed event time of the K steps. After them, N steps back
to back without the eviction are reported as "warm_mall", and the GFX clock
is sampled while a further set of steps runs ("gpu_clock").

Peaks: HBM 8 TB/s and dense bf16 MFMA 2.5 PFLOP/s, MI355X's published
figures (2.5 PFLOP/s is 256 CUs x 4096 bf16 FLOP per clock at 2.4 GHz,
2.5166 PFLOP/s before rounding, so fractions against the unrounded product
read 0.7% lower).
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


def measured_clock(workload):
    """Time-weighted shader clock (GHz) of the expert GEMM kernels from the
    committed rocprofv3 counter summary (GRBM_GUI_ACTIVE per dispatch), if it
    was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"mfma_grouped_ffn_{workload}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"^source_sha:\s*(\w+)", text, re.M)
    m_c = re.search(r"^gemm_clock_ghz:\s*([0-9.]+)", text, re.M)
    if not m_sha or not m_c or m_sha.group(1) != kernel_source_sha():
        return None
    return float(m_c.group(1))


def host_description():
    """CPU model and the BLAS numpy links, for the CPU baseline's record."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()
                if i.get("user_api") == "blas"]
        blas = ", ".join(libs) or None
    except Exception:  # pragma: no cover
        pass
    return model, blas


def core_counts():
    """Physical cores, logical CPUs, and the CPUs this process may run on
    (a container or lease can hold fewer than the machine has)."""
    phys = None
    try:
        import psutil
        phys = psutil.cpu_count(logical=False)
    except Exception:  # pragma: no cover
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        avail = None
    return {"physical_cores": phys, "logical_cpus": os.cpu_count(),
            "cpus_available_to_process": avail}


def git_sha():
    """The commit of the working tree, or, in a copy without .git, the one the
    library was built from (recorded by the build)."""
    import subprocess
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                           text=True, timeout=30)
        if r.returncode == 0 and r.stdout.strip():
            return {"git_sha": r.stdout.strip(), "source": "working tree"}
    except (OSError, subprocess.SubprocessError):
        pass
    path = os.path.join(ROOT, "grouped_expert_ffn_amd", "_build", "build_info.json")
    try:
        info = json.load(open(path))
        return {"git_sha": info.get("git_sha"), "git_dirty_at_build": info.get("git_dirty"),
                "source": "recorded when the library was built"}
    except (OSError, ValueError):
        return {"git_sha": None, "source": "unavailable"}


def env_record(torch):
    rocm = None
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    rec = {"device": torch.cuda.get_device_name(), "torch": torch.__version__,
           "hip": torch.version.hip, "rocm": rocm, "library_sha": library_sha()}
    rec.update(git_sha())
    return rec


def gpu_clock_during(run, n_steps):
    """GFX clock samples (MHz, amdsmi) taken while `run(n_steps)` layer steps
    execute back to back: the steps are enqueued first, then the clock is
    read until an event after them has completed."""
    if n_steps <= 0:
        return None
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        handle = handles[0]
        # the device torch runs on, matched by PCI bus (amdsmi lists every GPU
        # of the machine, whatever the process may see)
        props = torch.cuda.get_device_properties(torch.cuda.current_device())
        bus = getattr(props, "pci_bus_id", None)
        if bus is not None and len(handles) > 1:
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)      # "dddd:bb:dd.f"
                if int(bdf.split(":")[1], 16) == int(bus):
                    handle = h
                    break
        acc = []

        def read():
            # the SMU's metrics table (refreshed about every millisecond where
            # the host allows it) has the current GFX clock of every XCD; its
            # activity accumulator shows whether the table was refreshed
            m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
            acc.append(m.get("gfx_activity_acc"))
            per_xcd = [v for v in (m.get("current_gfxclks") or [])
                       if isinstance(v, (int, float)) and 0 < v < 65535]
            cur = m.get("current_gfxclk")
            avg = m.get("average_gfxclk_frequency")
            val = float(np.mean(per_xcd)) if per_xcd else (
                float(cur) if isinstance(cur, (int, float)) and 0 < cur < 65535 else None)
            return val, (float(avg) if isinstance(avg, (int, float)) and 0 < avg < 65535
                         else None)
        max_clk = amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX).get("max_clk")
        read()
    except Exception as e:  # pragma: no cover - depends on the host's driver access
        return {"error": f"{type(e).__name__}: {e}"}
    torch.cuda.synchronize()
    run(n_steps)
    done = torch.cuda.Event()
    done.record(torch.cuda.current_stream())
    samples, avgs = [], []
    t0 = time.perf_counter()
    while not done.query():
        cur, avg = read()
        if cur is not None:
            samples.append(cur)
        if avg is not None:
            avgs.append(avg)
        time.sleep(0.001)
    span = time.perf_counter() - t0
    torch.cuda.synchronize()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:  # pragma: no cover
        pass
    if not samples and not avgs:
        return {"error": "no clock sample while the steps ran"}
    refreshed = len(set(a for a in acc if a is not None)) > 1
    rec = {"samples": len(samples), "steps": n_steps, "span_s": span, "max_clk_mhz": max_clk,
           "metrics_refreshed": refreshed,
           "source": "amdsmi GPU metrics (current GFX clock averaged over the XCDs, and the "
                     "SMU's own running average), sampled while the steps ran"
                     + ("" if refreshed else "; the table did not change while the steps ran, "
                        "so these values do not describe them")}
    if samples:
        rec.update(gfx_mhz_median=float(np.median(samples)), gfx_mhz_min=min(samples),
                   gfx_mhz_max=max(samples))
    if avgs:
        rec.update(avg_gfx_mhz_median=float(np.median(avgs)))
    return rec


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
    model, blas = host_description()
    rec = {"value": Ts * runs / total, "unit": "routed tokens/s", "cores": int(cores),
           "cores_are": "BLAS threads the oracle's matrix products ran on (its other steps "
                        "are single-threaded numpy)",
           "kind": "oracle", "cpu_model": model, "blas": blas}
    rec.update(core_counts())
    return dict(rec, **{
            "sample": f"first {Ts} of {cfg.T} tokens of {cfg.name}, all expert weights, "
                      f"float64 numpy oracle, {runs} run(s) in {total:.1f} s"})


def ablation_baselines(G, desc, x_perm, offsets, w1, w2, reps=5):
    """The grouped expert FFN beside two ways of running the same experts
    that it replaces ("Dropless MoE Is a Runtime Problem as Much as a Model
    Design", grouped GEMM paragraph: no launch per expert, no padding to a
    common capacity), all with this library's kernels on the same plan:

      per_expert: one grouped-FFN call per local expert on its own rows;
      padded:     every local expert padded to C = the largest group, as one
                  grouped call over uniform groups ([E_loc, C, d] layout).

    Each real row goes through the same tile decomposition and K order, so
    all three give the same bits. Returns the timings (median of `reps`,
    HIP events on the current stream) and the three y_perm copies."""
    import torch
    dt = x_perm.dtype
    el = desc.E // desc.ep_size
    lo = desc.ep_rank * el
    offs = offsets.cpu().numpy().astype(np.int64)
    rows0 = min(int(offs[lo]), desc.max_rows)
    n = [max(0, min(int(offs[lo + e + 1]), desc.max_rows) - min(int(offs[lo + e]), desc.max_rows))
         for e in range(el)]
    first = [min(int(offs[lo + e]), desc.max_rows) for e in range(el)]
    d = desc.d
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    # grouped: the library's call
    ws = G.alloc_workspace(desc)
    y_grp = torch.zeros((desc.max_rows, d), dtype=dt, device="cuda")
    t_grp = timed(lambda: G.grouped_ffn(desc, x_perm, offsets, w1, w2, y_grp, ws))

    # per expert: E_loc calls, each a one-expert layer over that expert's rows
    y_pe = torch.zeros_like(y_grp)
    calls = []
    n_max = max(n + [1])
    d1 = G.make_desc(n_max, d, 1, 1, desc.d_ff, "bf16" if desc.dtype == 1 else "f32",
                     "softmax", "swiglu" if desc.act == 1 else "relu", max_rows=n_max)
    ws1 = G.alloc_workspace(d1)
    for e in range(el):
        if n[e] == 0:
            continue
        de = G.make_desc(n[e], d, 1, 1, desc.d_ff, "bf16" if desc.dtype == 1 else "f32",
                         "softmax", "swiglu" if desc.act == 1 else "relu", max_rows=n[e])
        oe = torch.tensor([0, n[e]], dtype=torch.int32, device="cuda")
        calls.append((de, x_perm[first[e]:first[e] + n[e]], oe, w1[e:e + 1], w2[e:e + 1],
                      y_pe[first[e]:first[e] + n[e]]))

    def per_expert():
        for de, xe, oe, a, b, ye in calls:
            G.grouped_ffn(de, xe, oe, a, b, ye, ws1)
    t_pe = timed(per_expert)

    # padded: [E_loc, C, d] with C the largest group, zero rows past each group
    C = max(n + [1])
    x_pad = torch.zeros((el * C, d), dtype=dt, device="cuda")
    for e in range(el):
        x_pad[e * C:e * C + n[e]] = x_perm[first[e]:first[e] + n[e]]
    dp = G.make_desc(el * C, d, el, 1, desc.d_ff, "bf16" if desc.dtype == 1 else "f32",
                     "softmax", "swiglu" if desc.act == 1 else "relu", max_rows=el * C)
    op = torch.arange(0, (el + 1) * C, C, dtype=torch.int32, device="cuda")
    y_pad = torch.empty((el * C, d), dtype=dt, device="cuda")
    wsp = G.alloc_workspace(dp)
    t_pad = timed(lambda: G.grouped_ffn(dp, x_pad, op, w1, w2, y_pad, wsp))
    y_pad_rows = torch.zeros_like(y_grp)
    for e in range(el):
        y_pad_rows[first[e]:first[e] + n[e]] = y_pad[e * C:e * C + n[e]]
    real = sum(n)
    info = {"grouped_ms": t_grp, "per_expert_ms": t_pe, "per_expert_calls": len(calls),
            "padded_ms": t_pad, "padded_rows": el * C, "real_rows": real,
            "padding_frac": 1.0 - real / max(1, el * C), "largest_group": C,
            "first_local_row": rows0}
    return info, y_grp, y_pe, y_pad_rows


def dedup_bench(G, desc, h, b, w1, w2, ws, reps=10):
    """Expert-parallel packing with one send row per (destination rank,
    token) pair, timed on the step's own plan beside the plan-only permute,
    and the local experts run from the deduplicated rows; their output rows
    are compared bit for bit with the step's y_perm."""
    import torch
    P, dt = G.max_pairs(desc), G.torch_dtype(desc)
    i32 = dict(dtype=torch.int32, device="cuda")
    send = torch.empty((P, desc.d), dtype=dt, device="cuda")
    pair_dest = torch.empty((desc.T, desc.k), **i32)
    pair_token = torch.empty((P,), **i32)
    splits = torch.empty((desc.ep_size,), dtype=torch.int64, device="cuda")
    displs = torch.empty_like(splits)
    recv = torch.empty((desc.max_rows,), **i32)
    y2 = torch.empty_like(b.y_perm)
    stream = torch.cuda.current_stream()
    c = [torch.empty_like(b.counts), torch.empty_like(b.offsets), torch.empty_like(b.dest),
         torch.empty_like(b.src_token), torch.empty_like(b.src_slot),
         torch.empty_like(b.send_splits), torch.empty_like(b.send_displs),
         torch.zeros_like(b.flags)]

    def plan_only():
        G.permute(desc, h, b.topk_idx, None, *c, ws)

    def pack():
        G.pack_dedup(desc, h, b.topk_idx, b.dest, b.src_token, b.src_slot, b.offsets, send,
                     pair_dest, pair_token, splits, displs, recv, ws)

    def ffn():
        G.grouped_ffn_gather(desc, send, recv, b.offsets, w1, w2, y2, ws)

    def timed(fn):
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))

    info = {"plan_only_permute_ms": timed(plan_only), "pack_dedup_ms": timed(pack)}
    info["grouped_ffn_from_pairs_ms"] = timed(ffn)
    offs = b.offsets.cpu().numpy().astype(np.int64)
    el = desc.E // desc.ep_size
    lo = min(int(offs[desc.ep_rank * el]), desc.max_rows)
    hi = min(int(offs[(desc.ep_rank + 1) * el]), desc.max_rows)
    n_pairs = int(splits.sum().item())
    n_slots = int((b.dest >= 0).sum().item())
    n_tok = int(torch.unique(pair_token[:n_pairs]).numel())
    eb = 2 if desc.dtype == G.DTYPE_BF16 else 4
    row = desc.d * eb
    Tk = desc.T * desc.k
    # reads each sent token's row once and writes each pair row; ids: idx and
    # dest read by three kernels, pid / first_row / pair_dest written (4 B each)
    pack_bytes = (n_tok + n_pairs) * row + 36 * Tk + 12 * n_pairs
    info.update({
        "send_rows_one_per_slot": n_slots, "send_rows_one_per_pair": n_pairs,
        "payload_bytes_one_per_slot": n_slots * row, "payload_bytes_one_per_pair": n_pairs * row,
        "payload_reduction": 1.0 - n_pairs / max(n_slots, 1),
        "pair_splits": splits.cpu().tolist(),
        "pack_GBs": pack_bytes / (info["pack_dedup_ms"] / 1e3) / 1e9,
        "ffn_rows_bitwise_equal": bool(torch.equal(y2[lo:hi], b.y_perm[lo:hi]))})
    return info


def router_margin_report(cfg, logits, h, wr, bias):
    """Router margin (the gap between each token's k-th and (k+1)-th score,
    "How Does Mixture-of-Experts Routing Affect LLM Repeatability?", router-
    margin passage) of the step's float32 scores, and what the float32
    rounding did to the routing: the scores recomputed in float64 from the
    same bf16 or float32 operands (a plain torch product, outside the step),
    the largest score error, the tokens whose top-k set differs between the
    two, and the tokens whose float64 margin is within twice that error (the
    near ties a differently rounded router could order otherwise). Reporting
    only: no part of the step."""
    import torch
    k, E = cfg.k, cfg.E
    if k >= E:
        return None
    vals, _ = torch.topk(logits, k + 1, dim=1)
    margin = (vals[:, k - 1] - vals[:, k]).double()
    exact = h.double() @ wr.double()
    if bias is not None:
        exact = exact + bias.double()[None, :]
    err = float((logits.double() - exact).abs().max())
    v64, i64 = torch.topk(exact, k + 1, dim=1)
    _, i32 = torch.topk(logits, k, dim=1)
    set32 = torch.sort(i32, dim=1).values
    set64 = torch.sort(i64[:, :k], dim=1).values
    flips = int((set32 != set64).any(dim=1).sum())
    m64 = v64[:, k - 1] - v64[:, k]
    q = torch.quantile(margin.float().cpu(), torch.tensor([0.01, 0.5])).tolist()
    return {"kth_minus_next_min": float(margin.min()), "kth_minus_next_p01": q[0],
            "kth_minus_next_median": q[1], "score_err_max_vs_f64": err,
            "topk_set_differs_from_f64": flips,
            "near_ties_f64_margin_within_2err": int((m64 <= 2 * err).sum())}


def routing_report(cfg, b, capacity, eb, h=None, wr=None, bias=None):
    """The step's routing population: assignments per expert, rows kept and
    dropped per expert (capacity mode), the router margin, and for an
    expert-parallel share the rows, payload bytes and message count of each
    destination's segment."""
    counts = b.counts.cpu().numpy().astype(np.int64)
    kept = counts if capacity < 0 else np.minimum(counts, capacity)
    rep = {"counts_per_expert": counts.tolist(), "kept_per_expert": kept.tolist(),
           "dropped_per_expert": (counts - kept).tolist(), "dropped": int((counts - kept).sum()),
           "empty_experts": int((counts == 0).sum())}
    if h is not None:
        rep["router_margin"] = router_margin_report(cfg, b.logits, h, wr, bias)
    if cfg.ep_size > 1:
        splits = b.send_splits.cpu().numpy().astype(np.int64)
        remote = [r for r in range(cfg.ep_size) if r != cfg.ep_rank]
        rep["send_rows_per_rank"] = splits.tolist()
        rep["payload_bytes_per_remote_rank"] = [int(splits[r]) * cfg.d * eb for r in remote]
        rep["messages"] = int(sum(1 for r in remote if splits[r] > 0))
    return rep


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
    ap.add_argument("--slots", action="store_true",
                    help="fused dispatch and slot-ordered output: permute makes only the plan, "
                         "the first expert GEMM gathers token rows from h, the second writes "
                         "each row to its (token, slot) row, and combine reads those")
    ap.add_argument("--ablation", action="store_true",
                    help="also time the grouped FFN beside a launch per expert and the padded "
                         "capacity layout, with the same kernels on the same plan")
    ap.add_argument("--dedup", action="store_true",
                    help="also time expert-parallel packing with one send row per "
                         "(rank, token) pair and the local experts run from those rows")
    ap.add_argument("--warm-steps", type=int, default=20,
                    help="extra steps back to back without evicting the MALL, timed by the "
                         "wall clock (reported beside the main figure)")
    ap.add_argument("--clock-steps", type=int, default=40,
                    help="extra steps run back to back while the GFX clock is sampled")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (for counter calibration)")
    args = ap.parse_args()
    if args.dedup and args.slots:
        ap.error("--dedup compares with the step's y_perm, which --slots does not write")
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
    slots = args.slots
    gather = args.gather or slots
    b = G.alloc_buffers(desc, x_perm=not gather)
    y_slots = (torch.empty((cfg.T * cfg.k, cfg.d), dtype=dt, device="cuda") if slots else None)
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
        if slots:
            G.grouped_ffn_slots(desc, h, b.src_token, b.src_slot, b.offsets, w1, w2, y_slots, ws,
                                flags=b.flags)
        elif gather:
            G.grouped_ffn_gather(desc, h, b.src_token, b.offsets, w1, w2, b.y_perm, ws,
                                 flags=b.flags)
        else:
            G.grouped_ffn(desc, b.x_perm, b.offsets, w1, w2, b.y_perm, ws, flags=b.flags)
        if ev is not None:
            ev[3].record(stream)
        if slots:
            G.combine_slots(desc, y_slots, b.topk_idx, b.topk_gate, b.dest, y)
        else:
            G.unpermute_combine(desc, b.y_perm, b.topk_idx, b.topk_gate, b.dest, y)
        if ev is not None:
            ev[4].record(stream)

    # Timed region: K steps, each right after a 512 MiB write that evicts the
    # 256 MiB last-level cache (MALL), so every step starts with its inputs in
    # HBM and none in the MALL. The write sits outside the step's events;
    # the step time is the sum of the four stage intervals.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    b.flags.zero_()
    for i in range(args.warmup):
        flush.fill_(i & 0xff)
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush.fill_(i & 0xff)
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in evs])  # ms
    step_ms = stage.sum(axis=1)

    # the same steps back to back without the write (what stays in the MALL
    # from one step to the next is reused), timed by the wall clock
    warm = None
    if args.warm_steps > 0:
        wev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
               for _ in range(args.warm_steps)]
        torch.cuda.synchronize()
        tw = time.perf_counter()
        for i in range(args.warm_steps):
            step(wev[i])
        torch.cuda.synchronize()
        tw = time.perf_counter() - tw
        wst = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in wev])
        warm = {"steps": args.warm_steps, "ms_per_step_wall": tw / args.warm_steps * 1e3,
                "tokens_per_s_wall": cfg.T * args.warm_steps / tw,
                "ms_per_step": float(wst.sum(axis=1).mean()),
                "grouped_ffn_ms": float(np.median(wst[:, 2]))}
    clock = gpu_clock_during(lambda n: [step() for _ in range(n)], args.clock_steps)
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
    ms_per_step = float(step_ms.mean())
    out = {
        "metric": "routed tokens/sec per MoE layer (route+permute+FFN+combine)",
        "value": cfg.T * args.steps / (step_ms.sum() / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) weights)",
        "config": {"workload": f"{cfg.name}: {cfg.description}", "T": cfg.T, "d": cfg.d,
                   "E": cfg.E, "k": cfg.k, "d_ff": cfg.d_ff, "act": cfg.act, "gate": cfg.gate,
                   "experts_local": el, "capacity": capacity, "parallelism": "1 GPU",
                   "dispatch": ("rows gathered by the first expert GEMM, output written in "
                                "(token, slot) order" if slots else
                                "rows gathered by the first expert GEMM" if gather
                                else "rows copied into expert order")},
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
        "routing": routing_report(cfg, b, capacity, eb, h, wr, bias),
        "timing": {"mall": "evicted before every timed step (512 MiB write outside the "
                           "step's events)",
                   "value_from": "sum of the timed steps' event durations",
                   "step_ms_median": float(np.median(step_ms)),
                   "step_ms_min": float(step_ms.min()), "step_ms_max": float(step_ms.max()),
                   "wall_s_incl_evictions": wall},
        "warm_mall": warm,
        "gpu_clock": dict(clock or {}, gemm_clock_ghz_counters=measured_clock(cfg.name),
                          gemm_clock_source="GRBM_GUI_ACTIVE / 8 XCDs / duration of the expert "
                          "GEMM dispatches, time-weighted, from the committed rocprofv3 summary "
                          "of this workload on the same kernel sources (null otherwise)"),
        "env": env_record(torch),
    }
    if args.ablation:
        b_x = b.x_perm
        if gather:   # the baselines run on expert-ordered rows
            b_x = torch.empty((desc.max_rows, cfg.d), dtype=dt, device="cuda")
            G.permute(desc, h, b.topk_idx, b_x, b.counts, b.offsets, b.dest, b.src_token,
                      b.src_slot, b.send_splits, b.send_displs, b.flags, ws)
        info, y_grp, y_pe, y_pad = ablation_baselines(G, desc, b_x, b.offsets, w1, w2)
        flops_useful = ffn_flops(n_local, cfg.d, cfg.d_ff, cfg.act)
        for key in ("grouped", "per_expert", "padded"):
            info[key + "_useful_TFLOPs"] = flops_useful / (info[key + "_ms"] / 1e3) / 1e12
        info["bitwise_equal"] = bool(torch.equal(y_grp, y_pe) and torch.equal(y_grp, y_pad))
        out["ablation"] = info
    if args.dedup:
        out["dedup"] = dedup_bench(G, desc, h, b, w1, w2, ws)
    if not args.skip_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, capacity, args.cpu_sample_tokens,
                                          args.cpu_min_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
