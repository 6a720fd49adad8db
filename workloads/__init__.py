"""Seeded synthetic inputs for the MoE token-dispatch layer.

This module only *draws inputs*: token rows, router weights, an optional
router bias and expert weights, plus a few hand-structured input families
(integer-valued router cases, identity/scale experts, one-hot marker tokens).
It holds none of the layer's arithmetic: no routing, gating, grouping,
capacity or FFN evaluation. Both the CPU oracle and the GPU path read their
inputs from here, and nothing here reads from either of them.

Workload shapes (five layers):

  tiny_fp32          T=64     d=32   E=4   k=2 d_ff=64    ReLU   softmax gates          fp32
  small_bf16         T=4096   d=1024 E=8   k=2 d_ff=2816  SwiGLU softmax gates          bf16
  mixtral_bf16       T=8192   d=4096 E=8   k=2 d_ff=14336 SwiGLU softmax renormalised   bf16
  finegrained_bf16   T=16384  d=2048 E=128 k=8 d_ff=768   SwiGLU softmax + Zipf bias    bf16
  ep_share_bf16      T=32768  d=7168 E=256 k=8 d_ff=2048  SwiGLU sigmoid renormalised   bf16
                     (32 of the 256 experts local: expert-parallel rank 0 of 8)

Distributions: h ~ N(0,1); every weight ~ N(0, 1/fan_in) with fan_in the
input width of that matrix (d for the router and the first expert matrix,
d_ff for the second). For bf16 layers every value is rounded to the nearest
bf16 (ties to even) at draw time, so the float32 arrays returned here hold
exactly the bf16 values the GPU receives.

Seeding: each array is drawn from ``np.random.default_rng([base, part])``
with ``base = 1000*layer_id + slot`` (slot: h=0, router=1, w1=2, w2=3) and
``part`` a fixed chunk index (expert id for expert weights, a fixed row-block
index for h). Chunks are fixed, so the values do not depend on how many
threads draw them.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "LayerConfig", "CONFIGS", "get_config", "make_inputs", "round_to_bf16",
    "zipf_router_bias", "identity_scale_experts", "marker_tokens",
    "integer_router_case", "small_layer_config",
]

_H_ROWS_PER_CHUNK = 2048


@dataclass(frozen=True)
class LayerConfig:
    name: str
    layer_id: int          # seed base selector
    T: int                 # tokens
    d: int                 # hidden width
    E: int                 # experts (global)
    k: int                 # experts per token
    d_ff: int              # expert inner width
    act: str               # "relu" | "swiglu"
    gate: str              # "softmax" | "softmax_topk_renorm" | "sigmoid_topk_renorm"
    dtype: str             # "f32" | "bf16"
    ep_size: int = 1
    ep_rank: int = 0
    capacity_factors: tuple = (None,)   # None = dropless
    zipf_bias: Optional[tuple] = None   # (alpha, scale) for a Zipf-rank router bias
    description: str = ""

    @property
    def E_local(self) -> int:
        return self.E // self.ep_size

    @property
    def local_experts(self) -> range:
        return range(self.ep_rank * self.E_local, (self.ep_rank + 1) * self.E_local)

    @property
    def w1_rows(self) -> int:
        return 2 * self.d_ff if self.act == "swiglu" else self.d_ff


CONFIGS = {
    "tiny_fp32": LayerConfig(
        "tiny_fp32", 1, T=64, d=32, E=4, k=2, d_ff=64, act="relu",
        gate="softmax", dtype="f32",
        description="tiny dropless fp32 layer, ReLU experts d->64->d"),
    "small_bf16": LayerConfig(
        "small_bf16", 2, T=4096, d=1024, E=8, k=2, d_ff=2816, act="swiglu",
        gate="softmax", dtype="bf16", capacity_factors=(None, 1.0),
        description="small bf16 layer, dropless and capacity factor 1.0"),
    "mixtral_bf16": LayerConfig(
        "mixtral_bf16", 3, T=8192, d=4096, E=8, k=2, d_ff=14336, act="swiglu",
        gate="softmax_topk_renorm", dtype="bf16",
        description="Mixtral-shaped bf16 layer, top-2 renormalised gates, dropless"),
    "finegrained_bf16": LayerConfig(
        "finegrained_bf16", 4, T=16384, d=2048, E=128, k=8, d_ff=768, act="swiglu",
        gate="softmax", dtype="bf16", capacity_factors=(None, 1.25),
        zipf_bias=(1.2, 1.2),
        description="fine-grained skewed routing (Zipf router bias), dropless and cf=1.25"),
    "ep_share_bf16": LayerConfig(
        "ep_share_bf16", 5, T=32768, d=7168, E=256, k=8, d_ff=2048, act="swiglu",
        gate="sigmoid_topk_renorm", dtype="bf16", ep_size=8, ep_rank=0,
        description="one GPU's share of an expert-parallel layer: 32 of 256 experts local"),
}


def get_config(name: str) -> LayerConfig:
    return CONFIGS[name]


def small_layer_config(base: LayerConfig, T: int, name: Optional[str] = None, **over) -> LayerConfig:
    """A copy of ``base`` with fewer tokens (and optional overrides), for
    parity cases sized so the CPU oracle finishes in seconds."""
    fields = dict(base.__dict__)
    fields.update(name=name or f"{base.name}_T{T}", T=T)
    fields.update(over)
    return LayerConfig(**fields)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values in place to the nearest bfloat16 (ties to even);
    the result stays float32 and holds exactly representable bf16 values."""
    assert a.dtype == np.float32
    u = a.view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return a


def _normal_block(seed, shape, scale, bf16):
    rng = np.random.default_rng(seed)
    out = np.empty(shape, np.float32)
    rng.standard_normal(dtype=np.float32, out=out)
    if scale != 1.0:
        out *= np.float32(scale)
    if bf16:
        round_to_bf16(out)
    return out


def _threads():
    try:
        import os
        n = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        n = 8
    return max(1, min(16, n))


def zipf_router_bias(E: int, alpha: float, scale: float) -> np.ndarray:
    """Per-expert router bias ``scale * ln(w_{e+1})`` where ``w_r`` is the
    Zipf(alpha) probability of rank r among E ranks; expert e has rank e+1,
    so low expert ids are hot. Returned as float32 (the value both sides use)."""
    r = np.arange(1, E + 1, dtype=np.float64)
    w = r ** (-alpha)
    w /= w.sum()
    return (scale * np.log(w)).astype(np.float32)


def make_inputs(cfg: LayerConfig, *, experts: str = "local", with_h: bool = True,
                threads: Optional[int] = None) -> dict:
    """Draw one layer's inputs.

    Returns float32 numpy arrays (bf16-valued for bf16 layers):
      h         [T, d]
      w_router  [d, E]            (s_t = h_t W_r)
      bias      [E] or None
      w1        [E_sel, w1_rows, d]   gate rows then up rows for SwiGLU
      w2        [E_sel, d, d_ff]
      expert_ids  the global ids of the experts drawn (local ones by default,
                  or ``experts="all"``)
    """
    bf16 = cfg.dtype == "bf16"
    base = 1000 * cfg.layer_id
    nthreads = threads or _threads()
    ids = list(cfg.local_experts) if experts == "local" else list(range(cfg.E))
    out: dict = {"config": cfg, "expert_ids": np.asarray(ids, np.int64)}

    jobs = []
    if with_h:
        h = np.empty((cfg.T, cfg.d), np.float32)
        nchunks = (cfg.T + _H_ROWS_PER_CHUNK - 1) // _H_ROWS_PER_CHUNK

        def hjob(c):
            r0 = c * _H_ROWS_PER_CHUNK
            r1 = min(cfg.T, r0 + _H_ROWS_PER_CHUNK)
            h[r0:r1] = _normal_block([base + 0, c], (r1 - r0, cfg.d), 1.0, bf16)
        jobs += [(hjob, c) for c in range(nchunks)]
        out["h"] = h

    w1 = np.empty((len(ids), cfg.w1_rows, cfg.d), np.float32)
    w2 = np.empty((len(ids), cfg.d, cfg.d_ff), np.float32)

    def w1job(i):
        w1[i] = _normal_block([base + 2, ids[i]], (cfg.w1_rows, cfg.d), 1.0 / math.sqrt(cfg.d), bf16)

    def w2job(i):
        w2[i] = _normal_block([base + 3, ids[i]], (cfg.d, cfg.d_ff), 1.0 / math.sqrt(cfg.d_ff), bf16)
    jobs += [(w1job, i) for i in range(len(ids))] + [(w2job, i) for i in range(len(ids))]

    with ThreadPoolExecutor(nthreads) as ex:
        for f in [ex.submit(fn, a) for fn, a in jobs]:
            f.result()

    out["w_router"] = _normal_block([base + 1, 0], (cfg.d, cfg.E), 1.0 / math.sqrt(cfg.d), bf16)
    out["bias"] = zipf_router_bias(cfg.E, *cfg.zipf_bias) if cfg.zipf_bias else None
    out["w1"] = w1
    out["w2"] = w2
    return out


# ---------------------------------------------------------------------------
# Hand-structured input families
# ---------------------------------------------------------------------------

def identity_scale_experts(d: int, scales) -> tuple:
    """ReLU experts with d_ff = 2d whose map is ``x -> c_e * x`` exactly:
    W1_e = [I; -I] and W2_e = c_e [I, -I], because relu(x) - relu(-x) = x.
    Returns (w1 [E, 2d, d], w2 [E, d, 2d]) as float32."""
    eye = np.eye(d, dtype=np.float32)
    w1 = np.stack([np.concatenate([eye, -eye], 0) for _ in scales])
    w2 = np.stack([np.float32(c) * np.concatenate([eye, -eye], 1) for c in scales])
    return w1, w2


def marker_tokens(T: int, d: int) -> np.ndarray:
    """One-hot marker rows ``h_t = (1 + t // d) * e_(t mod d)``: every token
    differs from every other in its support or its magnitude."""
    h = np.zeros((T, d), np.float32)
    t = np.arange(T)
    h[t, t % d] = (1 + t // d).astype(np.float32)
    return h


def integer_router_case(T: int, d: int, E: int, seed: int) -> dict:
    """Router inputs whose logits are small integers in any summation order:
    h in {-2..2}, W_r in {-1,0,1}. Ties between experts are frequent."""
    rng = np.random.default_rng([777, seed])
    h = rng.integers(-2, 3, size=(T, d)).astype(np.float32)
    w = rng.integers(-1, 2, size=(d, E)).astype(np.float32)
    return {"h": h, "w_router": w}
