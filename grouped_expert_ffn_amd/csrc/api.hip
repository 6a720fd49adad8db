// C ABI entry points: argument validation on the host, then kernel launches
// enqueued on the caller's stream. Nothing here synchronises, copies device
// data to the host or allocates memory.
#include <algorithm>
#include <atomic>

#include "common.h"

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace moe {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static size_t elt_bytes(int dtype) { return dtype == MOE_DTYPE_BF16 ? 2 : 4; }

// rows of a deduplicated send buffer: one per (destination rank, token) pair
static int64_t max_pairs(const moe_layer_desc_t& d) {
  return d.T * (int64_t)std::min(d.k, d.ep_size);
}
static size_t dedup_scratch_ints(const moe_layer_desc_t& d);

// The fused call's scratch copies of its optional outputs, in LayerScratch
// order, each 256-byte aligned. Returns the bytes; with `ws` non-null also
// carves the pointers from ws + offset.
static size_t layer_scratch(const moe_layer_desc_t& d, char* base, LayerScratch* out) {
  const size_t TE = (size_t)d.T * d.E, Tk = (size_t)d.T * d.k, R = (size_t)d.max_rows;
  const size_t sizes[] = {TE * 4, Tk * 4, Tk * 4, (size_t)d.E * 4, ((size_t)d.E + 1) * 4,
                          Tk * 4, R * 4, R * 4, (size_t)d.ep_size * 8, (size_t)d.ep_size * 8,
                          4};
  void* p[11];
  size_t off = 0;
  for (int i = 0; i < 11; ++i) {
    p[i] = base ? base + off : nullptr;
    off += align256(sizes[i]);
  }
  if (out) {
    out->logits = (float*)p[0];
    out->topk_idx = (int32_t*)p[1];
    out->topk_gate = (float*)p[2];
    out->counts = (int32_t*)p[3];
    out->offsets = (int32_t*)p[4];
    out->dest = (int32_t*)p[5];
    out->src_token = (int32_t*)p[6];
    out->src_slot = (int32_t*)p[7];
    out->send_splits = (int64_t*)p[8];
    out->send_displs = (int64_t*)p[9];
    out->flags = (uint32_t*)p[10];
  }
  return off;
}
static size_t layer_scratch_bytes(const moe_layer_desc_t& d) {
  return layer_scratch(d, nullptr, nullptr);
}

Workspace workspace_layout(const moe_layer_desc_t& d) {
  Workspace w{};
  size_t off = 0;
  w.wrt = off;
  if (d.dtype == MOE_DTYPE_BF16) off += align256((size_t)router_n_pad(d.E) * d.d * 2);
  w.tile_hist = off;
  const int64_t n_tiles = (d.T + kTokTile - 1) / kTokTile;
  off += align256((size_t)n_tiles * d.E * 4);
  w.gemm_tiles = off;
  off += align256((size_t)(2 * gemm_max_mtiles(d) + 1) * sizeof(int4));
  w.act = off;
  off += align256((size_t)d.max_rows * d.d_ff * elt_bytes(d.dtype));
  w.dedup = off;
  off += align256(dedup_scratch_ints(d) * 4);
  w.layer = off;
  off += layer_scratch_bytes(d);
  w.total = off;
  return w;
}

// int32 entries of the deduplicated packing's scratch: pid and first_row
// [T,k], pair_slot [max pairs], counts [E], offsets [E+1], flags [1]
static size_t dedup_scratch_ints(const moe_layer_desc_t& d) {
  const size_t tk = (size_t)d.T * d.k;
  return 2 * tk + (size_t)max_pairs(d) + 2 * (size_t)d.E + 2;
}

static DedupScratch dedup_scratch(const moe_layer_desc_t& d, char* ws) {
  const Workspace w = workspace_layout(d);
  int32_t* p = reinterpret_cast<int32_t*>(ws + w.dedup);
  const size_t tk = (size_t)d.T * d.k;
  DedupScratch s;
  s.tile_hist = reinterpret_cast<int32_t*>(ws + w.tile_hist);
  s.pid = p;
  s.first_row = p + tk;
  s.pair_slot = p + 2 * tk;
  s.counts = s.pair_slot + max_pairs(d);
  s.offsets = s.counts + d.E;
  s.flags = reinterpret_cast<uint32_t*>(s.offsets + d.E + 1);
  return s;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static moe_status_t check_desc(const moe_layer_desc_t* d) {
  if (!d) return MOE_ERR_NULL;
  if (d->dtype != MOE_DTYPE_F32 && d->dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  if (d->gate < MOE_GATE_SOFTMAX || d->gate > MOE_GATE_SIGMOID_TOPK_RENORM)
    return MOE_ERR_UNSUPPORTED;
  if (d->act != MOE_ACT_RELU && d->act != MOE_ACT_SWIGLU) return MOE_ERR_UNSUPPORTED;
  if (d->reserved != 0) return MOE_ERR_SHAPE;
  if (d->T < 0 || d->d < 1 || d->d_ff < 1) return MOE_ERR_SHAPE;
  if (d->E < 1 || d->E > kMaxE) return MOE_ERR_SHAPE;
  if (d->k < 1 || d->k > kMaxK || d->k > d->E) return MOE_ERR_SHAPE;
  if (d->ep_size < 1 || d->E % d->ep_size != 0) return MOE_ERR_SHAPE;
  if (d->ep_rank < 0 || d->ep_rank >= d->ep_size) return MOE_ERR_SHAPE;
  if (d->max_rows < 0 || d->max_rows >= (int64_t)1 << 31) return MOE_ERR_SHAPE;
  if (d->T * (int64_t)d->k >= (int64_t)1 << 31) return MOE_ERR_SHAPE;
  if (d->dtype == MOE_DTYPE_BF16) {
    if (d->d % 64 != 0 || d->d_ff % 64 != 0) return MOE_ERR_SHAPE;
    // the expert GEMMs address one tile's operands with 32-bit byte offsets:
    // gate and up weight rows of one expert, and 512 rows of either width
    const int64_t lim = (int64_t)1 << 32;
    if ((2 * (int64_t)d->d_ff + 256) * d->d * 2 >= lim) return MOE_ERR_SHAPE;
    if ((int64_t)512 * std::max(d->d, d->d_ff) * 2 >= lim) return MOE_ERR_SHAPE;
  }
  return MOE_OK;
}

static moe_status_t check_ws(const moe_layer_desc_t* d, void* ws, size_t ws_bytes) {
  const size_t need = workspace_layout(*d).total;
  if (need == 0) return MOE_OK;
  if (!ws || ((uintptr_t)ws & 255u) != 0 || ws_bytes < need) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

struct Buf {
  const void* p;
  int64_t n;     // elements; a zero-size buffer may be NULL
  bool data;     // element type is `dtype` (needs 16-byte alignment for bf16)
};

static moe_status_t check_bufs(const moe_layer_desc_t* d, std::initializer_list<Buf> bs) {
  for (const Buf& b : bs) {
    if (b.n == 0) continue;
    if (!b.p) return MOE_ERR_NULL;
    if (((uintptr_t)b.p & 3u) != 0) return MOE_ERR_ALIGN;
    if (b.data && d->dtype == MOE_DTYPE_BF16 && !aligned16(b.p)) return MOE_ERR_ALIGN;
  }
  return MOE_OK;
}

#define MOE_TRY(x)                     \
  do {                                 \
    moe_status_t st__ = (x);           \
    if (st__ != MOE_OK) return st__;   \
  } while (0)

#define HIP_TRY(x)                                \
  do {                                            \
    if ((x) != hipSuccess) return MOE_ERR_HIP;    \
  } while (0)

static moe_status_t do_route(const moe_layer_desc_t& d, const void* h, const void* w_router,
                             const float* bias, float* logits, int32_t* idx, float* gate,
                             uint32_t* flags, char* ws, hipStream_t s) {
  if (d.dtype == MOE_DTYPE_BF16) {
    const Workspace w = workspace_layout(d);
    bf16* wt = reinterpret_cast<bf16*>(ws + w.wrt);
    const int E_pad = router_n_pad(d.E);
    HIP_TRY(launch_transpose_router_bf16((const bf16*)w_router, wt, d.d, d.E, E_pad, s));
    HIP_TRY(launch_router_bf16((const bf16*)h, wt, bias, logits, d.T, d.d, d.E, E_pad, s));
  } else {
    HIP_TRY(launch_router_f32((const float*)h, (const float*)w_router, bias, logits, d.T, d.d,
                              d.E, s));
  }
  HIP_TRY(launch_topk(logits, idx, gate, flags, d.T, d.E, d.k, d.gate, s));
  return MOE_OK;
}

static moe_status_t do_permute(const moe_layer_desc_t& d, const void* h, const int32_t* idx,
                               void* x_perm, int32_t* counts, int32_t* offsets, int32_t* dest,
                               int32_t* src_token, int32_t* src_slot, int64_t* splits,
                               int64_t* displs, uint32_t* flags, char* ws, hipStream_t s) {
  const Workspace w = workspace_layout(d);
  int32_t* tile_hist = reinterpret_cast<int32_t*>(ws + w.tile_hist);
  HIP_TRY(launch_dispatch_plan(idx, tile_hist, counts, offsets, dest, src_token, src_slot, splits,
                               displs, flags, d.T, d.E, d.k, d.capacity, d.max_rows, d.ep_size,
                               s));
  // without x_perm only the plan is made (the rows are gathered later)
  if (x_perm)
    HIP_TRY(launch_permute_rows(h, dest, x_perm, d.T, d.k, (int)(d.d * elt_bytes(d.dtype)), s));
  return MOE_OK;
}

// rows == null: x holds the expert-ordered rows (x_perm); otherwise x is h and
// row i of the grouped operand is h[rows[i]]
// o_tok != null: grouped row r is written to row o_tok[r] * k + o_slot[r]
// flags (may be null): OR-ed with ROW_OVERFLOW when local rows lie past max_rows
static moe_status_t do_ffn(const moe_layer_desc_t& d, const void* x, const int32_t* rows,
                           const int32_t* offsets, const void* w1, const void* w2, void* y_perm,
                           uint32_t* flags, char* ws, hipStream_t s,
                           const int32_t* o_tok = nullptr, const int32_t* o_slot = nullptr) {
  const Workspace w = workspace_layout(d);
  HIP_TRY(launch_grouped_ffn(d, x, rows, offsets, w1, w2, y_perm, ws + w.act,
                             reinterpret_cast<int4*>(ws + w.gemm_tiles), flags, s, o_tok,
                             o_slot));
  return MOE_OK;
}

// gathered bf16 rows are addressed with 32-bit byte offsets from h
// (h: token rows [T,d], or a deduplicated send buffer of up to max_pairs rows)
static moe_status_t check_gather(const moe_layer_desc_t& d) {
  if (d.dtype == MOE_DTYPE_BF16 && max_pairs(d) * d.d * 2 >= ((int64_t)1 << 32))
    return MOE_ERR_SHAPE;
  return MOE_OK;
}

static moe_status_t do_combine(const moe_layer_desc_t& d, const void* y_perm, const int32_t* idx,
                               const float* gate, const int32_t* dest, void* y, hipStream_t s,
                               bool slots = false) {
  const int el = d.E / d.ep_size;
  HIP_TRY(launch_combine(y_perm, idx, gate, dest, y, d.T, d.k, d.d, d.dtype, d.ep_rank * el,
                         (d.ep_rank + 1) * el, s, slots));
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

MOE_EXPORT int64_t moe_capacity_from_factor(double cf, int64_t T, int32_t k, int32_t E) {
  if (!(cf > 0.0) || E <= 0) return -1;
  // floor(cf * T * k / E), evaluated in double like the definition reads
  double c = cf * (double)T * (double)k / (double)E;
  return (int64_t)c;
}

MOE_EXPORT moe_status_t moe_workspace_size(const moe_layer_desc_t* desc, size_t* bytes) {
  MOE_TRY(check_desc(desc));
  if (!bytes) return MOE_ERR_NULL;
  *bytes = workspace_layout(*desc).total;
  return MOE_OK;
}

MOE_EXPORT moe_status_t moe_route(const moe_layer_desc_t* desc, const void* h,
                                  const void* w_router, const float* router_bias, float* logits,
                                  int32_t* topk_idx, float* topk_gate, uint32_t* flags, void* ws,
                                  size_t ws_bytes, void* stream) {
  MOE_TRY(check_desc(desc));
  const moe_layer_desc_t& d = *desc;
  const int64_t TE = d.T * d.E, Tk = d.T * d.k;
  MOE_TRY(check_bufs(desc, {{h, d.T * d.d, true}, {w_router, (int64_t)d.d * d.E, true},
                            {logits, TE, false}, {topk_idx, Tk, false}, {topk_gate, Tk, false},
                            {flags, 1, false}}));
  if (router_bias && ((uintptr_t)router_bias & 3u)) return MOE_ERR_ALIGN;
  MOE_TRY(check_ws(desc, ws, ws_bytes));
  return do_route(*desc, h, w_router, router_bias, logits, topk_idx, topk_gate, flags,
                  (char*)ws, (hipStream_t)stream);
}

MOE_EXPORT moe_status_t moe_topk_from_logits(const moe_layer_desc_t* desc, const float* logits,
                                             int32_t* topk_idx, float* topk_gate,
                                             uint32_t* flags, void* stream) {
  MOE_TRY(check_desc(desc));
  const int64_t TE = desc->T * desc->E, Tk = desc->T * desc->k;
  MOE_TRY(check_bufs(desc, {{logits, TE, false}, {topk_idx, Tk, false}, {topk_gate, Tk, false},
                            {flags, 1, false}}));
  HIP_TRY(launch_topk(logits, topk_idx, topk_gate, flags, desc->T, desc->E, desc->k, desc->gate,
                      (hipStream_t)stream));
  return MOE_OK;
}

MOE_EXPORT moe_status_t moe_permute(const moe_layer_desc_t* desc, const void* h,
                                    const int32_t* topk_idx, void* x_perm, int32_t* counts,
                                    int32_t* offsets, int32_t* dest, int32_t* src_token,
                                    int32_t* src_slot, int64_t* send_splits,
                                    int64_t* send_displs, uint32_t* flags, void* ws,
                                    size_t ws_bytes, void* stream) {
  MOE_TRY(check_desc(desc));
  const moe_layer_desc_t& d = *desc;
  const int64_t Tk = d.T * d.k, R = d.max_rows;
  MOE_TRY(check_bufs(desc, {{h, d.T * d.d, true}, {x_perm, x_perm ? R * d.d : 0, true},
                            {topk_idx, Tk, false},
                            {counts, d.E, false}, {offsets, d.E + 1, false}, {dest, Tk, false},
                            {src_token, R, false}, {src_slot, R, false}, {flags, 1, false},
                            {send_splits, d.ep_size, false}, {send_displs, d.ep_size, false}}));
  MOE_TRY(check_ws(desc, ws, ws_bytes));
  return do_permute(*desc, h, topk_idx, x_perm, counts, offsets, dest, src_token, src_slot,
                    send_splits, send_displs, flags, (char*)ws, (hipStream_t)stream);
}

MOE_EXPORT moe_status_t moe_grouped_ffn(const moe_layer_desc_t* desc, const void* x_perm,
                                        const int32_t* offsets, const void* w1, const void* w2,
                                        void* y_perm, uint32_t* flags, void* ws, size_t ws_bytes,
                                        void* stream) {
  MOE_TRY(check_desc(desc));
  const moe_layer_desc_t& d = *desc;
  const int64_t R = d.max_rows, el = d.E / d.ep_size;
  const int64_t w1n = el * (d.act == MOE_ACT_SWIGLU ? 2 : 1) * d.d_ff * d.d, w2n = el * d.d * d.d_ff;
  MOE_TRY(check_bufs(desc, {{x_perm, R * d.d, true}, {y_perm, R * d.d, true}, {w1, w1n, true},
                            {w2, w2n, true}, {offsets, d.E + 1, false}}));
  if (flags && ((uintptr_t)flags & 3u)) return MOE_ERR_ALIGN;
  MOE_TRY(check_ws(desc, ws, ws_bytes));
  return do_ffn(*desc, x_perm, nullptr, offsets, w1, w2, y_perm, flags, (char*)ws,
                (hipStream_t)stream);
}

MOE_EXPORT moe_status_t moe_grouped_ffn_gather(const moe_layer_desc_t* desc, const void* h,
                                               const int32_t* src_token, const int32_t* offsets,
                                               const void* w1, const void* w2, void* y_perm,
                                               uint32_t* flags, void* ws, size_t ws_bytes,
                                               void* stream) {
  MOE_TRY(check_desc(desc));
  const moe_layer_desc_t& d = *desc;
  MOE_TRY(check_gather(d));
  const int64_t R = d.max_rows, el = d.E / d.ep_size;
  const int64_t w1n = el * (d.act == MOE_ACT_SWIGLU ? 2 : 1) * d.d_ff * d.d, w2n = el * d.d * d.d_ff;
  MOE_TRY(check_bufs(desc, {{h, d.T * d.d, true}, {src_token, R, false},
                            {y_perm, R * d.d, true}, {w1, w1n, true}, {w2, w2n, true},
                            {offsets, d.E + 1, false}}));
  if (flags && ((uintptr_t)flags & 3u)) return MOE_ERR_ALIGN;
  MOE_TRY(check_ws(desc, ws, ws_bytes));
  return do_ffn(d, h, src_token, offsets, w1, w2, y_perm, flags, (char*)ws, (hipStream_t)stream);
}

MOE_EXPORT moe_status_t moe_grouped_ffn_slots(const moe_layer_desc_t* desc, const void* h,
                                              const int32_t* src_token, const int32_t* src_slot,
                                              const int32_t* offsets, const void* w1,
                                              const void* w2, void* y_slots, uint32_t* flags,
                                              void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_desc(desc));
  const moe_layer_desc_t& d = *desc;
  MOE_TRY(check_gather(d));
  const int64_t R = d.max_rows, el = d.E / d.ep_size;
  const int64_t w1n = el * (d.act == MOE_ACT_SWIGLU ? 2 : 1) * d.d_ff * d.d, w2n = el * d.d * d.d_ff;
  MOE_TRY(check_bufs(desc, {{h, d.T * d.d, true}, {src_token, R, false}, {src_slot, R, false},
                            {y_slots, d.T * d.k * d.d, true}, {w1, w1n, true}, {w2, w2n, true},
                            {offsets, d.E + 1, false}}));
  if (flags && ((uintptr_t)flags & 3u)) return MOE_ERR_ALIGN;
  MOE_TRY(check_ws(desc, ws, ws_bytes));
  return do_ffn(d, h, src_token, offsets, w1, w2, y_slots, flags, (char*)ws,
                (hipStream_t)stream, src_token, src_slot);
}

MOE_EXPORT moe_status_t moe_combine_slots(const moe_layer_desc_t* desc, const void* y_slots,
                                          const int32_t* topk_idx, const float* topk_gate,
                                          const int32_t* dest, void* y, void* stream) {
  MOE_TRY(check_desc(desc));
  const moe_layer_desc_t& d = *desc;
  const int64_t Tk = d.T * d.k;
  MOE_TRY(check_bufs(desc, {{y_slots, Tk * d.d, true}, {topk_idx, Tk, false},
                            {topk_gate, Tk, false}, {dest, Tk, false}, {y, d.T * d.d, true}}));
  return do_combine(d, y_slots, topk_idx, topk_gate, dest, y, (hipStream_t)stream, true);
}

MOE_EXPORT moe_status_t moe_pack_dedup(const moe_layer_desc_t* desc, const void* h,
                                       const int32_t* topk_idx, const int32_t* dest,
                                       const int32_t* src_token, const int32_t* src_slot,
                                       const int32_t* offsets, void* send_buf,
                                       int32_t* pair_dest, int32_t* pair_token,
                                       int64_t* pair_splits, int64_t* pair_displs,
                                       int32_t* recv_rows, void* ws, size_t ws_bytes,
                                       void* stream) {
  MOE_TRY(check_desc(desc));
  const moe_layer_desc_t& d = *desc;
  const int64_t Tk = d.T * d.k, R = d.max_rows, P = max_pairs(d);
  MOE_TRY(check_bufs(desc, {{h, d.T * d.d, true}, {topk_idx, Tk, false}, {dest, Tk, false},
                            {src_token, R, false}, {src_slot, R, false},
                            {offsets, d.E + 1, false}, {send_buf, P * d.d, true},
                            {pair_dest, Tk, false}, {pair_token, P, false},
                            {pair_splits, d.ep_size, false}, {pair_displs, d.ep_size, false},
                            {recv_rows, R, false}}));
  MOE_TRY(check_ws(desc, ws, ws_bytes));
  HIP_TRY(launch_pack_dedup(h, topk_idx, dest, src_token, src_slot, offsets, send_buf, pair_dest,
                            pair_token, pair_splits, pair_displs, recv_rows,
                            dedup_scratch(d, (char*)ws), d.T, d.E, d.k, d.ep_size, d.ep_rank,
                            d.max_rows, (int)(d.d * elt_bytes(d.dtype)), (hipStream_t)stream));
  return MOE_OK;
}

MOE_EXPORT moe_status_t moe_unpermute_combine(const moe_layer_desc_t* desc, const void* y_perm,
                                              const int32_t* topk_idx, const float* topk_gate,
                                              const int32_t* dest, void* y, void* stream) {
  MOE_TRY(check_desc(desc));
  const moe_layer_desc_t& d = *desc;
  const int64_t Tk = d.T * d.k;
  MOE_TRY(check_bufs(desc, {{y_perm, d.max_rows * d.d, true}, {y, d.T * d.d, true},
                            {topk_idx, Tk, false}, {topk_gate, Tk, false}, {dest, Tk, false}}));
  return do_combine(*desc, y_perm, topk_idx, topk_gate, dest, y, (hipStream_t)stream);
}

MOE_EXPORT moe_status_t moe_layer_forward(const moe_layer_desc_t* desc, const void* h,
                                          const void* w_router, const float* router_bias,
                                          const void* w1, const void* w2, void* y,
                                          const moe_layer_buffers_t* b, void* ws,
                                          size_t ws_bytes, void* stream) {
  MOE_TRY(check_desc(desc));
  if (!b) return MOE_ERR_NULL;
  const moe_layer_desc_t& d = *desc;
  const int64_t TE = d.T * d.E, Tk = d.T * d.k, R = d.max_rows, el = d.E / d.ep_size;
  const int64_t w1n = el * (d.act == MOE_ACT_SWIGLU ? 2 : 1) * d.d_ff * d.d;
  const int64_t w2n = el * d.d * d.d_ff;
  // required: inputs, y and y_perm; every other buffer may be NULL (a
  // workspace copy stands in for it)
  MOE_TRY(check_bufs(desc, {{h, d.T * d.d, true}, {w_router, (int64_t)d.d * d.E, true},
                            {w1, w1n, true}, {w2, w2n, true}, {y, d.T * d.d, true},
                            {b->y_perm, R * d.d, true}}));
  auto opt = [&](const void* p, int64_t n, bool data) -> moe_status_t {
    return p ? check_bufs(desc, {{p, n, data}}) : MOE_OK;
  };
  MOE_TRY(opt(b->x_perm, R * d.d, true));
  MOE_TRY(opt(b->logits, TE, false));
  MOE_TRY(opt(b->topk_idx, Tk, false));
  MOE_TRY(opt(b->topk_gate, Tk, false));
  MOE_TRY(opt(b->counts, d.E, false));
  MOE_TRY(opt(b->offsets, d.E + 1, false));
  MOE_TRY(opt(b->dest, Tk, false));
  MOE_TRY(opt(b->src_token, R, false));
  MOE_TRY(opt(b->src_slot, R, false));
  MOE_TRY(opt(b->send_splits, d.ep_size, false));
  MOE_TRY(opt(b->send_displs, d.ep_size, false));
  MOE_TRY(opt(b->flags, 1, false));
  if (router_bias && ((uintptr_t)router_bias & 3u)) return MOE_ERR_ALIGN;
  if (!b->x_perm) MOE_TRY(check_gather(d));
  MOE_TRY(check_ws(desc, ws, ws_bytes));
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  LayerScratch o;
  layer_scratch(d, w + workspace_layout(d).layer, &o);
  float* logits = b->logits ? b->logits : o.logits;
  int32_t* idx = b->topk_idx ? b->topk_idx : o.topk_idx;
  float* gate = b->topk_gate ? b->topk_gate : o.topk_gate;
  int32_t* counts = b->counts ? b->counts : o.counts;
  int32_t* offsets = b->offsets ? b->offsets : o.offsets;
  int32_t* dest = b->dest ? b->dest : o.dest;
  int32_t* src_token = b->src_token ? b->src_token : o.src_token;
  int32_t* src_slot = b->src_slot ? b->src_slot : o.src_slot;
  int64_t* splits = b->send_splits ? b->send_splits : o.send_splits;
  int64_t* displs = b->send_displs ? b->send_displs : o.send_displs;
  uint32_t* flags = b->flags ? b->flags : o.flags;
  MOE_TRY(do_route(d, h, w_router, router_bias, logits, idx, gate, flags, w, s));
  MOE_TRY(do_permute(d, h, idx, b->x_perm, counts, offsets, dest, src_token, src_slot, splits,
                     displs, flags, w, s));
  // without x_perm the first expert GEMM gathers its rows from h
  if (b->x_perm)
    MOE_TRY(do_ffn(d, b->x_perm, nullptr, offsets, w1, w2, b->y_perm, flags, w, s));
  else
    MOE_TRY(do_ffn(d, h, src_token, offsets, w1, w2, b->y_perm, flags, w, s));
  return do_combine(d, b->y_perm, idx, gate, dest, y, s);
}

// ---------------------------------------------------------------------------
// moe_permute without a workspace, for callers that cannot allocate. Its only
// scratch, the per-tile expert histograms of the plan, lives in this fixed
// device array (one copy per GPU, held until the process ends). Host code
// reaches it only through the device address hipGetSymbolAddress returns,
// looked up once per device on the first call with that device current.
constexpr int64_t kNoWsHistInts = int64_t(1) << 20;   // 4 MiB of int32 counts
static __device__ __align__(256) int32_t scratch[kNoWsHistInts];

static std::atomic<int32_t*> g_scratch_ptr[64];

static moe_status_t no_ws_scratch(int32_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  int32_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return MOE_ERR_HIP;
    p = static_cast<int32_t*>(q);
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MOE_OK;
}

MOE_EXPORT moe_status_t moe_permute_no_workspace(
    const moe_layer_desc_t* desc, const void* h, const int32_t* topk_idx, void* x_perm,
    int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src_token, int32_t* src_slot,
    int64_t* send_splits, int64_t* send_displs, uint32_t* flags, void* stream) {
  MOE_TRY(check_desc(desc));
  const moe_layer_desc_t& d = *desc;
  const int64_t Tk = d.T * d.k, R = d.max_rows;
  MOE_TRY(check_bufs(desc, {{h, d.T * d.d, true}, {x_perm, x_perm ? R * d.d : 0, true},
                            {topk_idx, Tk, false},
                            {counts, d.E, false}, {offsets, d.E + 1, false}, {dest, Tk, false},
                            {src_token, R, false}, {src_slot, R, false}, {flags, 1, false},
                            {send_splits, d.ep_size, false}, {send_displs, d.ep_size, false}}));
  const int64_t n_tiles = (d.T + kTokTile - 1) / kTokTile;
  if (n_tiles * d.E > kNoWsHistInts) return MOE_ERR_SCRATCH;
  int32_t* tile_hist = nullptr;
  MOE_TRY(no_ws_scratch(&tile_hist));
  hipStream_t s = (hipStream_t)stream;
  // every histogram entry the plan reads is written first in the same call,
  // so nothing left from an earlier call needs clearing
  HIP_TRY(launch_dispatch_plan(topk_idx, tile_hist, counts, offsets, dest, src_token, src_slot,
                               send_splits, send_displs, flags, d.T, d.E, d.k, d.capacity,
                               d.max_rows, d.ep_size, s));
  if (x_perm)
    HIP_TRY(launch_permute_rows(h, dest, x_perm, d.T, d.k, (int)(d.d * elt_bytes(d.dtype)), s));
  return MOE_OK;
}

MOE_EXPORT const char* moe_status_str(moe_status_t st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "inconsistent or unsupported sizes";
    case MOE_ERR_ALIGN: return "a buffer is misaligned (bf16 buffers need 16 bytes)";
    case MOE_ERR_DTYPE: return "unknown dtype";
    case MOE_ERR_UNSUPPORTED: return "unknown gate or activation mode";
    case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "a HIP kernel launch failed";
    case MOE_ERR_SCRATCH:
      return "the problem exceeds the fixed device scratch of the no-workspace entry point";
  }
  return "unknown status";
}
