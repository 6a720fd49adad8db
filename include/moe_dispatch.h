/*
 * moe_dispatch.h -- C ABI of the MI355X (gfx950) MoE token-dispatch layer.
 *
 * The layer computes, for every token t (the simplified token-choice layer of
 * "How Does Mixture-of-Experts Routing Affect LLM Repeatability?"):
 *
 *     s_t = h_t W_r (+ b),   E_t = TopK(s_t, k),   y_t = sum_{e in E_t} g_{t,e} f_e(h_t)
 *
 * along the staged path of "MoE Token Dispatch: Why an All-Reduce Result Does
 * Not Describe the Exchange", section "Follow one documented dispatch and
 * return path": route -> per-expert counts and splits -> rows rearranged into
 * per-expert groups -> experts -> outputs restored to their tokens.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument except `desc` and `ws_bytes`-style sizes is a
 *    DEVICE pointer owned by the caller; the library allocates nothing, keeps
 *    no state between calls (beyond a per-device cache of the CU count,
 *    safe to fill from several threads) and never frees caller memory.
 *  - All work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *    the default stream). No entry point synchronises, copies device->host or
 *    reads device data on the host, so every call can be captured in a graph.
 *  - Row-major layouts. `dtype` (MOE_DTYPE_F32 or MOE_DTYPE_BF16) is the
 *    element type of h, w_router, w1, w2, x_perm, y_perm and y. Logits and
 *    gates are always float32; ids, counts, offsets, dest and the inverse map
 *    are int32; expert-parallel splits are int64 (row units).
 *  - Host-detectable argument errors return a non-zero moe_status_t before
 *    anything is enqueued. Data-dependent conditions are OR-ed into the
 *    caller-zeroed device word `flags` (MOE_FLAG_*); the caller reads it when
 *    it chooses to (the periodic overflow check of "Dropless MoE Is a Runtime
 *    Problem as Much as a Model Design", device-side metadata paragraph).
 *  - A launch failure returns MOE_ERR_HIP; the HIP error is left for the
 *    caller's next HIP call to report.
 *  - `ws`/`ws_bytes`: caller-allocated device scratch of at least
 *    moe_workspace_size() bytes, 256-byte aligned. Calls that share a
 *    workspace must be ordered on one stream.
 */
#ifndef MOE_DISPATCH_H
#define MOE_DISPATCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,       /* inconsistent or unsupported sizes */
  MOE_ERR_ALIGN = 3,       /* a bf16 buffer is not 16-byte aligned */
  MOE_ERR_DTYPE = 4,       /* unknown dtype */
  MOE_ERR_UNSUPPORTED = 5, /* unknown gate or activation mode */
  MOE_ERR_WORKSPACE = 6,   /* workspace missing, misaligned or too small */
  MOE_ERR_HIP = 7,         /* a kernel launch failed */
  MOE_ERR_SCRATCH = 8      /* beyond the fixed scratch of moe_permute_no_workspace */
} moe_status_t;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype_t;

/* Gate forms g_{t,e} of the chosen experts (the pages name g_{t,e}; the three
 * forms are the ones the supported layers use). */
typedef enum {
  MOE_GATE_SOFTMAX = 0,             /* softmax over all E scores, not renormalised */
  MOE_GATE_SOFTMAX_TOPK_RENORM = 1, /* softmax over the k chosen scores */
  MOE_GATE_SIGMOID_TOPK_RENORM = 2  /* logistic(s) of the chosen, divided by their sum */
} moe_gate_t;

/* Expert map f_e. RELU: relu(x W1^T) W2^T with w1 [E_loc, d_ff, d].
 * SWIGLU: (silu(x Wg^T) * (x Wu^T)) W2^T with w1 [E_loc, 2*d_ff, d] holding
 * the gate rows Wg first, then the up rows Wu. w2 is [E_loc, d, d_ff]. */
typedef enum { MOE_ACT_RELU = 0, MOE_ACT_SWIGLU = 1 } moe_act_t;

/* Bits of the device flags word. */
#define MOE_FLAG_ROW_OVERFLOW 1u    /* kept rows exceed max_rows; those rows get dest = -2 */
#define MOE_FLAG_BAD_EXPERT_ID 2u   /* a (replayed) expert id outside [0, E); dest = -1 */
#define MOE_FLAG_NONFINITE_LOGIT 4u /* a router score is NaN or +-Inf */
#define MOE_FLAG_DROPPED 8u         /* capacity dropped at least one assignment (informational) */

typedef struct moe_layer_desc {
  int64_t T;        /* tokens, >= 0, with T * k < 2^31 */
  int32_t d;        /* hidden width (bf16: multiple of 64) */
  int32_t E;        /* experts, global count, 1..1024 */
  int32_t k;        /* experts per token, 1..min(E, 16) */
  int32_t d_ff;     /* expert inner width (bf16: multiple of 64, and
                       (2 * d_ff + 256) * d * 2 bytes below 4 GiB) */
  int32_t dtype;    /* moe_dtype_t */
  int32_t gate;     /* moe_gate_t */
  int32_t act;      /* moe_act_t */
  int32_t ep_size;  /* expert-parallel ranks, >= 1, divides E */
  int32_t ep_rank;  /* this GPU's rank; its local experts are
                       [ep_rank*E/ep_size, (ep_rank+1)*E/ep_size) */
  int32_t reserved; /* must be 0 */
  int64_t capacity; /* per-expert cap; < 0 means dropless */
  int64_t max_rows; /* rows allocated in x_perm / y_perm (T*k never overflows), < 2^31 */
} moe_layer_desc_t;

/* Per-expert capacity floor(cf * T * k / E) for a capacity factor cf > 0, or
 * -1 (dropless) for cf <= 0. Capacity page ("How does dropless MoE dispatch
 * differ from capacity factor token dropping?", section "Why per-expert
 * buffers exist in expert-parallel training"), with the routed-assignment
 * count T*k standing for the total tokens. Host-only, no device work. */
int64_t moe_capacity_from_factor(double cf, int64_t T, int32_t k, int32_t E);

/* Bytes of device workspace any entry point needs for `desc` (the fused call
 * needs the most; the stage calls need no more). Host-only. */
moe_status_t moe_workspace_size(const moe_layer_desc_t* desc, size_t* bytes);

/* Route: logits[T,E] = h[T,d] . w_router[d,E] (+ router_bias[E]), then the
 * ordered top-k ids (score descending, equal scores to the lower expert id,
 * -0 == +0, NaN below every number) and their gates.
 * Repeatability page: token-choice formula and the demand for stable score
 * ordering with deterministic tie handling.
 *   h          [T,d] dtype          w_router  [d,E] dtype
 *   router_bias [E] float32 or NULL  logits   [T,E] float32 (written)
 *   topk_idx   [T,k] int32 (written) topk_gate [T,k] float32 (written)
 *   flags      [1] uint32, OR-ed with MOE_FLAG_NONFINITE_LOGIT
 * Each token's scores are summed in an order that does not depend on T or
 * on the other tokens, so a token routes the same alone or in any batch. */
moe_status_t moe_route(const moe_layer_desc_t* desc, const void* h, const void* w_router,
                       const float* router_bias, float* logits, int32_t* topk_idx,
                       float* topk_gate, uint32_t* flags, void* ws, size_t ws_bytes,
                       void* stream);

/* Top-k and gates only, from caller logits [T,E] float32 (same rules as
 * moe_route): the selection E_t = TopK(s_t, k) and the gates g_{t,e} of the
 * repeatability page's token-choice formula, applied to scores the caller
 * already holds (for instance scores replayed from a stored run, the page's
 * route-replay passage). No workspace.
 *   topk_idx [T,k] int32, topk_gate [T,k] float32 (written)
 *   flags    [1] uint32, OR-ed with MOE_FLAG_NONFINITE_LOGIT */
moe_status_t moe_topk_from_logits(const moe_layer_desc_t* desc, const float* logits,
                                  int32_t* topk_idx, float* topk_gate, uint32_t* flags,
                                  void* stream);

/* Permute: group the (token, slot) assignments of topk_idx [T,k] by expert
 * and copy the token rows into x_perm [max_rows,d]. x_perm may be NULL: then
 * only the plan below is made and no row is copied (the rows can be read in
 * place by moe_grouped_ffn_gather).
 * Dispatch page ("Follow one documented dispatch and return path"): counts
 * and communication splits from the routing map, tokens rearranged per
 * expert. Capacity page and the repeatability page's capacity passage: at
 * most `capacity` assignments per expert are kept, overflow is dropped in
 * ascending (token, slot) order.
 *   counts   [E]   assignments per expert before capacity
 *   offsets  [E+1] exclusive scan of min(counts, capacity): expert e owns
 *                  rows offsets[e]..offsets[e+1]-1, members in (token, slot) order
 *   dest     [T,k] row of each assignment; -1 dropped (capacity or bad id);
 *                  -2 row >= max_rows (MOE_FLAG_ROW_OVERFLOW)
 *   src_token, src_slot [max_rows] inverse map, written for rows
 *                  0..min(offsets[E], max_rows)-1; later rows untouched
 *   send_splits, send_displs [ep_size] rows and first row of each
 *                  expert-parallel rank's contiguous segment (send buffers)
 *   flags    OR-ed with BAD_EXPERT_ID, DROPPED, ROW_OVERFLOW
 * Every output is bit-exact and independent of launch timing. */
moe_status_t moe_permute(const moe_layer_desc_t* desc, const void* h, const int32_t* topk_idx,
                         void* x_perm, int32_t* counts, int32_t* offsets, int32_t* dest,
                         int32_t* src_token, int32_t* src_slot, int64_t* send_splits,
                         int64_t* send_displs, uint32_t* flags, void* ws, size_t ws_bytes,
                         void* stream);

/* moe_permute for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments and results as moe_permute, without the workspace.
 * The plan's per-tile expert histograms go to a fixed 4 MiB device array
 * inside the library instead, one per GPU, allocated when the library is
 * loaded and held until the process ends; the call itself allocates
 * nothing. Limit: ceil(T / 128) * E <= 2^20 (for example T <= 131072 tokens
 * at E = 1024), else MOE_ERR_SCRATCH before anything is enqueued. Every
 * call on one GPU shares that array: calls that overlap on a GPU (other
 * streams, other threads) race and must be ordered by the caller. Nothing
 * in the array needs clearing between calls (each call writes every entry it
 * reads). The first call on a device, with that device current, looks up the
 * array's device address (a HIP runtime query, no allocation). */
moe_status_t moe_permute_no_workspace(const moe_layer_desc_t* desc, const void* h,
                                      const int32_t* topk_idx, void* x_perm, int32_t* counts,
                                      int32_t* offsets, int32_t* dest, int32_t* src_token,
                                      int32_t* src_slot, int64_t* send_splits,
                                      int64_t* send_displs, uint32_t* flags, void* stream);

/* Grouped expert FFN: for every local expert e, rows offsets[e]..offsets[e+1]-1
 * (clamped to max_rows) of x_perm go through f_e into the same rows of y_perm
 * [max_rows,d]; other rows of y_perm are untouched. One launch per GEMM over
 * all ragged groups ("Dropless MoE Is a Runtime Problem as Much as a Model
 * Design", grouped GEMM paragraph). bf16 runs on MFMA with float32
 * accumulation; the SwiGLU product is formed in float32 and stored as bf16.
 *   w1 [E_loc, d_ff or 2*d_ff, d], w2 [E_loc, d, d_ff] (local experts only)
 *   flags [1] uint32 or NULL: OR-ed with MOE_FLAG_ROW_OVERFLOW when the local
 *         groups end past max_rows (offsets[e_hi] > max_rows, e_hi the first
 *         expert after the local ones), i.e. when rows were not computed; the
 *         same device-side overflow check as moe_permute (dropless page,
 *         device-side metadata paragraph) for offsets a caller replays */
moe_status_t moe_grouped_ffn(const moe_layer_desc_t* desc, const void* x_perm,
                             const int32_t* offsets, const void* w1, const void* w2,
                             void* y_perm, uint32_t* flags, void* ws, size_t ws_bytes,
                             void* stream);

/* The same grouped expert FFN with dispatch fused into the first GEMM: row r
 * of an expert's group is read straight from h [T,d] at token src_token[r]
 * (the inverse map moe_permute writes), so the rows are never copied into
 * x_perm. h may also be a deduplicated send buffer from moe_pack_dedup,
 * with its recv_rows in place of src_token.
 * "Dropless MoE Is a Runtime Problem as Much as a Model Design",
 * expert-parallelism paragraph: fusing dispatch into the expert computation
 * removes an intermediate write and its read. Results are bit-identical to
 * moe_grouped_ffn on x_perm. bf16 needs T*min(k,ep_size)*d*2 bytes below
 * 4 GiB (MOE_ERR_SHAPE otherwise). flags as for moe_grouped_ffn. */
moe_status_t moe_grouped_ffn_gather(const moe_layer_desc_t* desc, const void* h,
                                    const int32_t* src_token, const int32_t* offsets,
                                    const void* w1, const void* w2, void* y_perm,
                                    uint32_t* flags, void* ws, size_t ws_bytes, void* stream);

/* Both ends of the grouped expert FFN fused with the data movement around
 * it: the first GEMM reads token rows from h through src_token (as
 * moe_grouped_ffn_gather), and the second GEMM's epilogue writes grouped row
 * r to row src_token[r] * k + src_slot[r] of y_slots [T*k, d], the row of its
 * (token, slot) pair, so that moe_combine_slots reads each token's k rows
 * contiguously. Same page and paragraph as moe_grouped_ffn_gather (fusing
 * dispatch and combine into the expert computation). The rows written hold
 * the same bits as y_perm[dest] of moe_grouped_ffn; rows of slots not
 * computed here (dropped, remote or past max_rows) are left untouched.
 * Needs the bf16 size limit of moe_grouped_ffn_gather (MOE_ERR_SHAPE
 * otherwise). flags as for moe_grouped_ffn. */
moe_status_t moe_grouped_ffn_slots(const moe_layer_desc_t* desc, const void* h,
                                   const int32_t* src_token, const int32_t* src_slot,
                                   const int32_t* offsets, const void* w1, const void* w2,
                                   void* y_slots, uint32_t* flags, void* ws, size_t ws_bytes,
                                   void* stream);

/* Expert-parallel packing with token deduplication: one send row per
 * (destination rank, token) pair instead of one per (token, slot).
 * "Dropless MoE Is a Runtime Problem as Much as a Model Design",
 * expert-parallelism paragraph: a token routed to several experts on one
 * destination needs to cross the network once. Inputs are the routing and
 * the plan of moe_permute (x_perm may have been NULL there): a slot is sent
 * when dest >= 0, to rank topk_idx / (E / ep_size).
 *   send_buf    [T*min(k,ep_size), d] pair rows, ordered by rank then token;
 *               rows past the pair count are untouched
 *   pair_dest   [T,k] send row of each slot's pair, -1 for unsent slots
 *   pair_token  [T*min(k,ep_size)] token of each pair row
 *   pair_splits, pair_displs [ep_size] rows and first row of each rank
 *   recv_rows   [max_rows] for this rank's grouped rows offsets[e_lo]..
 *               min(offsets[e_hi], max_rows)-1: the send row holding that
 *               row's token, so moe_grouped_ffn_gather(desc, send_buf,
 *               recv_rows, ...) runs the local experts on the deduplicated rows
 * Bit-exact and independent of launch timing. Needs the workspace of desc. */
moe_status_t moe_pack_dedup(const moe_layer_desc_t* desc, const void* h, const int32_t* topk_idx,
                            const int32_t* dest, const int32_t* src_token,
                            const int32_t* src_slot, const int32_t* offsets, void* send_buf,
                            int32_t* pair_dest, int32_t* pair_token, int64_t* pair_splits,
                            int64_t* pair_displs, int32_t* recv_rows, void* ws,
                            size_t ws_bytes, void* stream);

/* Unpermute + combine: y[t] = sum_j topk_gate[t,j] * y_perm[dest[t,j]] over
 * slots with dest >= 0 whose expert is local, summed in float32 in slot
 * order, rounded once to dtype. Tokens with no such slot get zeros (the
 * residual is the caller's). Unpermute page ("moe-unpermute-wrong-token"):
 * each row returns to its own token with that token's probability. */
moe_status_t moe_unpermute_combine(const moe_layer_desc_t* desc, const void* y_perm,
                                   const int32_t* topk_idx, const float* topk_gate,
                                   const int32_t* dest, void* y, void* stream);

/* The same combine on slot rows: y[t] = sum_j topk_gate[t,j] *
 * y_slots[t*k + j] over the slots moe_unpermute_combine would use (dest >= 0,
 * expert local), in the same float32 order, so y is bit-identical to
 * moe_unpermute_combine on y_perm. y_slots [T*k, d] as written by
 * moe_grouped_ffn_slots; dest [T,k] from the plan. */
moe_status_t moe_combine_slots(const moe_layer_desc_t* desc, const void* y_slots,
                               const int32_t* topk_idx, const float* topk_gate,
                               const int32_t* dest, void* y, void* stream);

/* Buffers of the fused call, device pointers with the shapes given above.
 * Only y_perm is required. Every other field may be NULL: the call then
 * keeps that intermediate in its workspace (moe_workspace_size includes
 * room for all of them) and the caller does not receive it. A NULL x_perm
 * also changes the path: the permute step makes only the plan and the
 * first expert GEMM reads the rows from h (as moe_grouped_ffn_gather), so
 * no expert-parallel send buffer is produced. A NULL flags word means no
 * overflow report. */
typedef struct moe_layer_buffers {
  float* logits;        /* [T,E] */
  int32_t* topk_idx;    /* [T,k] */
  float* topk_gate;     /* [T,k] */
  int32_t* counts;      /* [E] */
  int32_t* offsets;     /* [E+1] */
  int32_t* dest;        /* [T,k] */
  int32_t* src_token;   /* [max_rows] */
  int32_t* src_slot;    /* [max_rows] */
  int64_t* send_splits; /* [ep_size] */
  int64_t* send_displs; /* [ep_size] */
  void* x_perm;         /* [max_rows,d] dtype */
  void* y_perm;         /* [max_rows,d] dtype */
  uint32_t* flags;      /* [1], caller-zeroed */
} moe_layer_buffers_t;

/* The whole layer in one call: y_t = sum over e in TopK(h_t W_r, k) of
 * g_{t,e} f_e(h_t) (the repeatability page's token-choice formula), run as
 * the staged path of the dispatch page ("Follow one documented dispatch and
 * return path"): route, permute, grouped FFN, unpermute + combine, enqueued
 * back to back on `stream` with no host synchronisation. Equivalent to the
 * four stage calls in order (with buffers->x_perm NULL: moe_permute without
 * x_perm, then moe_grouped_ffn_gather).
 *   h [T,d], w_router [d,E], router_bias [E] float32 or NULL, w1, w2 as for
 *   moe_grouped_ffn, y [T,d] (written; excludes the residual)
 *   buffers: required (non-NULL), with the optional fields described above
 * Errors: as the stage calls; MOE_ERR_NULL when buffers, buffers->y_perm or
 * a required input is NULL. */
moe_status_t moe_layer_forward(const moe_layer_desc_t* desc, const void* h, const void* w_router,
                               const float* router_bias, const void* w1, const void* w2, void* y,
                               const moe_layer_buffers_t* buffers, void* ws, size_t ws_bytes,
                               void* stream);

/* Static text for a status code. */
const char* moe_status_str(moe_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DISPATCH_H */
