"""CPU oracle for the MoE token-dispatch layer (route -> group -> expert FFN -> combine).

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module. The product path (the
HIP library and its Python binding) never calls it and shares no code,
constant or helper with it.

Everything is plain numpy in float64. Each function follows one passage of
the pages (cited by page title and passage):

* "How Does Mixture-of-Experts Routing Affect LLM Repeatability?" (wpnews.pro),
  the simplified token-choice layer: scores s_t = h_t W_r, chosen set
  E_t = TopK(s_t, k), output y_t = sum over e in E_t of g_{t,e} f_e(h_t);
  the router-margin passage m_t = s_(k) - s_(k+1); the capacity passage
  (drops resolved in request/token order).
* "MoE Token Dispatch: Why an All-Reduce Result Does Not Describe the
  Exchange" (Leviathan Systems), section "Follow one documented dispatch and
  return path": counts and communication splits from the routing map, tokens
  and probabilities rearranged per expert, outputs restored to their origin.
* "How does dropless MoE dispatch differ from capacity factor token
  dropping?" (zenaique), section "Why per-expert buffers exist in
  expert-parallel training": the per-expert cap, overflow assignments dropped;
  a dropped assignment skips the FFN and keeps only the residual.
* "Dropless MoE Is a Runtime Problem as Much as a Model Design"
  (solar-565): dropless grouping into variable-length expert batches,
  overflow detection on device-side metadata.

Readings where the pages are silent (each listed in the design notes):
ties in the top-k go to the lower expert id; ranking is on the logits;
softmax gates are not renormalised unless the layer says so; capacity is
floor(cf * T * k / E); drops follow ascending (token, slot) order; gates of
dropped slots are not renormalised; the SwiGLU first matrix holds the gate
rows, then the up rows.

Parity unpinned: none of the functions below is without a pin; the exact
float values of the bf16 GPU path are compared within tolerance only.
"""
from __future__ import annotations

import math

import numpy as np

# Device flag bits of the layer's overflow/diagnostic word (this module's own
# definition; the GPU library defines its own and the tests compare values).
ROW_OVERFLOW = 1
BAD_EXPERT_ID = 2
NONFINITE_LOGIT = 4
DROPPED = 8

GATE_MODES = ("softmax", "softmax_topk_renorm", "sigmoid_topk_renorm")
ACTS = ("relu", "swiglu")


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Route
# ---------------------------------------------------------------------------

def router_logits(h, w_router, bias=None):
    """Router scores s_t = h_t W_r (+ bias), one row per token, in float64.

    Repeatability page, token-choice layer formula. ``w_router`` is [d, E] as
    the product h_t W_r implies; the optional per-expert bias is part of the
    score used both for selection and for the gates."""
    s = _f64(h) @ _f64(w_router)
    if bias is not None:
        s = s + _f64(bias)[None, :]
    return s


def topk_route(logits, k):
    """E_t = TopK(s_t, k) for every token, as an ordered list.

    Repeatability page, token-choice formula and its demand for stable score
    ordering with deterministic tie handling. Reading: order by score
    descending, equal scores by expert id ascending; -0 and +0 are equal; a
    NaN score ranks below every number (and raises the non-finite flag).
    Returns (idx [T,k] int32, flags)."""
    s = _f64(logits)
    T, E = s.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    flags = 0 if np.isfinite(s).all() else NONFINITE_LOGIT
    ids = np.broadcast_to(np.arange(E), (T, E))
    # lexsort: last key is primary. NaN sorts last, which ranks it lowest.
    order = np.lexsort((ids, -s), axis=1)
    return order[:, :k].astype(np.int32), flags


def router_margin(logits, k):
    """m_t = s_(k) - s_(k+1), the gap between the k-th and (k+1)-th largest
    scores (repeatability page, router-margin passage). +inf when k == E."""
    s = np.sort(_f64(logits), axis=1)[:, ::-1]
    if k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


def gate_weights(logits, idx, mode):
    """Gate weights g_{t,e} of the chosen experts, in the order of ``idx``.

    The repeatability page names g_{t,e} without fixing its form; the layer
    configurations fix three forms:
      softmax              softmax over all E scores, taken at the chosen ids
      softmax_topk_renorm  softmax over the k chosen scores only
      sigmoid_topk_renorm  logistic of each chosen score, divided by their sum
    """
    s = _f64(logits)
    idx = np.asarray(idx)
    if mode == "softmax":
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        p = e / e.sum(axis=1, keepdims=True)
        return np.take_along_axis(p, idx, axis=1)
    sel = np.take_along_axis(s, idx, axis=1)
    if mode == "softmax_topk_renorm":
        e = np.exp(sel - sel.max(axis=1, keepdims=True))
        return e / e.sum(axis=1, keepdims=True)
    if mode == "sigmoid_topk_renorm":
        with np.errstate(over="ignore"):
            sig = 1.0 / (1.0 + np.exp(-sel))
        return sig / sig.sum(axis=1, keepdims=True)
    raise ValueError(mode)


def route(h, w_router, bias, k, gate_mode):
    """Scores, ordered top-k ids and gates for a batch of tokens."""
    s = router_logits(h, w_router, bias)
    idx, flags = topk_route(s, k)
    return s, idx, gate_weights(s, idx, gate_mode), flags


# ---------------------------------------------------------------------------
# Group (permute plan)
# ---------------------------------------------------------------------------

def capacity_from_factor(cf, T, k, E):
    """Per-expert capacity, floor(cf * T * k / E), or -1 (dropless) for cf None.

    Capacity page: the cap is a factor times the tokens per expert; the
    routed-assignment count T*k stands for "total tokens" so that the cap
    scales with k (the reading the layer configurations use)."""
    if cf is None:
        return -1
    return int(math.floor(cf * T * k / E))


def dispatch_plan(idx, E, capacity=-1, max_rows=None, ep_size=1, ep_rank=0):
    """Group the (token, slot) assignments by expert.

    Dispatch page, "Follow one documented dispatch and return path": per-expert
    counts and communication splits come from the routing map, and tokens are
    rearranged into per-expert groups. Capacity page: an expert keeps at most
    ``capacity`` assignments and the overflow is dropped; the repeatability
    page has capacity resolved in request order, read here as ascending
    (token, slot) order.

    Returns a dict:
      counts[E]      assignments per expert before capacity
      kept[E]        min(counts, capacity)
      offsets[E+1]   exclusive scan of kept: expert e owns rows offsets[e]..offsets[e+1]
      dest[T,k]      row of each assignment; -1 dropped by capacity;
                     -2 when its row would be >= max_rows (row overflow)
      src_token[n], src_slot[n]   inverse map for rows 0..n-1, n = min(offsets[E], max_rows)
      send_splits[ep_size], send_displs[ep_size]  rows per expert-parallel rank
      flags
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    flags = 0
    valid = (flat >= 0) & (flat < E)
    if not valid.all():
        flags |= BAD_EXPERT_ID
    counts = np.zeros(E, np.int64)
    for e in range(E):
        counts[e] = int(np.count_nonzero(flat == e))
    kept = counts.copy() if capacity < 0 else np.minimum(counts, capacity)
    if (kept < counts).any():
        flags |= DROPPED
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(kept)
    if max_rows is None:
        max_rows = int(offsets[E])

    dest = np.full(T * k, -1, np.int64)
    for e in range(E):
        members = np.nonzero(flat == e)[0]          # ascending (token, slot) order
        keep = members[: kept[e]]
        dest[keep] = offsets[e] + np.arange(kept[e])
    over = dest >= max_rows
    if over.any():
        flags |= ROW_OVERFLOW
        dest[over] = -2

    n = int(min(offsets[E], max_rows))
    src_token = np.full(n, -1, np.int64)
    src_slot = np.full(n, -1, np.int64)
    a = np.nonzero(dest >= 0)[0]
    src_token[dest[a]] = a // k
    src_slot[dest[a]] = a % k

    if E % ep_size:
        raise ValueError("E must be a multiple of ep_size")
    el = E // ep_size
    send_displs = np.array([offsets[r * el] for r in range(ep_size)], np.int64)
    send_splits = np.array([offsets[(r + 1) * el] - offsets[r * el] for r in range(ep_size)], np.int64)
    return dict(counts=counts, kept=kept, offsets=offsets, dest=dest.reshape(T, k),
                src_token=src_token, src_slot=src_slot, send_splits=send_splits,
                send_displs=send_displs, flags=flags, capacity=capacity,
                max_rows=max_rows, ep_size=ep_size, ep_rank=ep_rank)


def permute(h, dest, rows=None):
    """x_perm[dest[t,j]] = h[t] for every materialised assignment (an exact copy)."""
    h = np.asarray(h)
    dest = np.asarray(dest)
    T, k = dest.shape
    if rows is None:
        rows = int(dest.max()) + 1 if (dest >= 0).any() else 0
    x = np.zeros((rows, h.shape[1]), h.dtype)
    t, j = np.nonzero(dest >= 0)
    x[dest[t, j]] = h[t]
    return x


def dedup_pack(idx, dest, E, ep_size):
    """Expert-parallel send packing with token deduplication.

    "Dropless MoE Is a Runtime Problem as Much as a Model Design",
    expert-parallelism paragraph: when top-k routing sends one token to
    several experts on the same destination, the token needs to cross the
    network only once. Here every (destination rank, token) pair with at
    least one sent slot gets one send row; a slot is sent when the plan
    materialised it (dest >= 0), and its rank is its expert's owner,
    expert // (E / ep_size). Pair rows are ordered by rank, then token, so
    each rank's rows form one contiguous segment.

    Returns a dict:
      pair_dest[T,k]   send row of each slot's (rank, token) pair; -1 unsent
      pair_token[P]    token of each pair row
      pair_splits[ep], pair_displs[ep]   rows and first row of each rank
    """
    idx = np.asarray(idx, np.int64)
    dest = np.asarray(dest, np.int64)
    T, k = idx.shape
    if E % ep_size:
        raise ValueError("E must be a multiple of ep_size")
    el = E // ep_size
    sent = dest >= 0
    pairs = sorted({(int(idx[t, j]) // el, t) for t in range(T) for j in range(k) if sent[t, j]})
    row = {p: i for i, p in enumerate(pairs)}
    pair_dest = np.full((T, k), -1, np.int64)
    for t in range(T):
        for j in range(k):
            if sent[t, j]:
                pair_dest[t, j] = row[(int(idx[t, j]) // el, t)]
    pair_token = np.array([t for _, t in pairs], np.int64)
    ranks = np.array([r for r, _ in pairs], np.int64)
    pair_splits = np.array([int(np.count_nonzero(ranks == r)) for r in range(ep_size)], np.int64)
    pair_displs = np.concatenate([[0], np.cumsum(pair_splits)[:-1]]).astype(np.int64)
    return dict(pair_dest=pair_dest, pair_token=pair_token, pair_splits=pair_splits,
                pair_displs=pair_displs)


# ---------------------------------------------------------------------------
# Experts
# ---------------------------------------------------------------------------

def silu(a):
    """silu(a) = a * logistic(a) = a / (1 + exp(-a))."""
    a = _f64(a)
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def expert_ffn(x, w1, w2, act):
    """One expert f_e on a batch of rows, in float64.

    The repeatability page has each expert apply its own feed-forward map
    f_e; its form comes from the layer configurations:
      relu:    relu(x W1^T) W2^T          w1 [d_ff, d], w2 [d, d_ff]
      swiglu:  (silu(x Wg^T) * (x Wu^T)) W2^T, with w1 = [Wg; Wu] of shape [2 d_ff, d]
    """
    x = _f64(x)
    w1 = _f64(w1)
    w2 = _f64(w2)
    if act == "relu":
        return np.maximum(x @ w1.T, 0.0) @ w2.T
    if act == "swiglu":
        dff = w2.shape[1]
        gate = x @ w1[:dff].T
        up = x @ w1[dff:].T
        return (silu(gate) * up) @ w2.T
    raise ValueError(act)


def grouped_ffn(x_perm, offsets, w1, w2, act, expert_lo=0, expert_hi=None, max_rows=None):
    """Run every local expert on its contiguous group of rows.

    Dropless page: the experts' variable-length batches are one grouped
    computation over ragged groups; here that is simply one ``expert_ffn``
    per group. ``w1``/``w2`` hold the local experts expert_lo..expert_hi-1.
    Rows outside the local groups stay zero."""
    offsets = np.asarray(offsets)
    if expert_hi is None:
        expert_hi = len(offsets) - 1
    rows = x_perm.shape[0]
    lim = rows if max_rows is None else min(rows, max_rows)
    y = np.zeros((rows, w2.shape[1]), np.float64)
    for i, e in enumerate(range(expert_lo, expert_hi)):
        r0, r1 = int(offsets[e]), min(int(offsets[e + 1]), lim)
        if r1 > r0:
            y[r0:r1] = expert_ffn(x_perm[r0:r1], w1[i], w2[i], act)
    return y


# ---------------------------------------------------------------------------
# Unpermute + combine
# ---------------------------------------------------------------------------

def unpermute_combine(y_perm, idx, gates, dest, expert_lo=0, expert_hi=None):
    """y_t = sum_j g_{t,j} * y_perm[dest[t,j]], over the materialised
    assignments whose expert is local, restoring every output to its token.

    Dispatch page: postprocessing restores order and shape; the unpermute page
    ("moe-unpermute-wrong-token"): each returned row must land on its own
    token, with the probability of that same token. Capacity page: a dropped
    assignment contributes nothing (the residual is added by the caller)."""
    idx = np.asarray(idx)
    dest = np.asarray(dest)
    g = _f64(gates)
    T, k = idx.shape
    if expert_hi is None:
        expert_hi = int(idx.max()) + 1 if idx.size else 0
    y = np.zeros((T, y_perm.shape[1]), np.float64)
    for j in range(k):
        use = (dest[:, j] >= 0) & (idx[:, j] >= expert_lo) & (idx[:, j] < expert_hi)
        t = np.nonzero(use)[0]
        y[t] += g[t, j, None] * _f64(y_perm[dest[t, j]])
    return y


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------

def layer(h, w_router, bias, w1, w2, *, k, gate, act, capacity=-1, max_rows=None,
          ep_size=1, ep_rank=0, route_idx=None):
    """The full layer on the expert-sorted path. ``route_idx`` replays a
    stored route table instead of selecting (repeatability page, route
    replay). Returns every intermediate."""
    s = router_logits(h, w_router, bias)
    E = s.shape[1]
    if route_idx is None:
        idx, rflags = topk_route(s, k)
    else:
        idx, rflags = np.asarray(route_idx, np.int32), (0 if np.isfinite(s).all() else NONFINITE_LOGIT)
    g = gate_weights(s, np.clip(idx, 0, E - 1), gate)
    plan = dispatch_plan(idx, E, capacity, max_rows, ep_size, ep_rank)
    el = E // ep_size
    lo, hi = ep_rank * el, (ep_rank + 1) * el
    rows = plan["max_rows"] if max_rows is not None else int(plan["offsets"][E])
    x_perm = permute(h, plan["dest"], rows)
    y_perm = grouped_ffn(x_perm, plan["offsets"], w1, w2, act, lo, hi, plan["max_rows"])
    y = unpermute_combine(y_perm, idx, g, plan["dest"], lo, hi)
    out = dict(plan)
    out.update(logits=s, idx=idx, gates=g, x_perm=x_perm, y_perm=y_perm, y=y,
               flags=plan["flags"] | rflags)
    return out


def brute_force_tokens(h, w_router, bias, w1, w2, tokens, *, k, gate, act,
                       capacity=-1, ep_size=1, ep_rank=0, route_idx=None):
    """y_t computed literally per token, with no permutation:
    y_t = sum over kept e in E_t of g_{t,e} f_e(h_t).

    Capacity is decided by walking the tokens in order and counting how many
    earlier assignments each expert has already accepted, so this needs all
    tokens up to max(tokens) when capacity is finite. Only local experts
    contribute. Returns [len(tokens), d] float64."""
    h = np.asarray(h)
    E = np.asarray(w_router).shape[1]
    el = E // ep_size
    lo = ep_rank * el
    tokens = list(tokens)
    last = max(tokens) if tokens else -1
    need = list(range(0, last + 1)) if capacity >= 0 else tokens
    # scores of the tokens that take part (one row each; rows are independent)
    s_all = router_logits(h[need], w_router, bias) if need else np.zeros((0, E))
    row_of = {t: i for i, t in enumerate(need)}
    accepted = np.zeros(E, np.int64)
    kept_of = {}
    for t in need:
        s = s_all[row_of[t]:row_of[t] + 1]
        if route_idx is None:
            ranked = sorted(range(E), key=lambda e: (-s[0, e], e))
            sel = ranked[:k]
        else:
            sel = [int(v) for v in route_idx[t]]
        g = gate_weights(s, np.asarray([sel]), gate)[0]
        keep = []
        for j, e in enumerate(sel):
            if capacity >= 0:
                if accepted[e] < capacity:
                    accepted[e] += 1
                    keep.append((j, e))
            else:
                keep.append((j, e))
        kept_of[t] = (keep, g)
    # y_t = sum of g_{t,e} f_e(h_t) over the kept local experts; each expert
    # is evaluated once on the stack of sampled tokens that need it
    uses = {}
    for i, t in enumerate(tokens):
        keep, g = kept_of[t]
        for j, e in keep:
            if lo <= e < lo + el:
                uses.setdefault(e, []).append((i, t, g[j]))
    out = np.zeros((len(tokens), h.shape[1]), np.float64)
    for e, lst in uses.items():
        f = expert_ffn(h[[t for _, t, _ in lst]], w1[e - lo], w2[e - lo], act)
        for r, (i, _, gj) in enumerate(lst):
            out[i] += gj * f[r]
    return out
