// Internal declarations shared by the HIP translation units of the MoE
// dispatch library (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_dispatch.h"

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kTokTile = 128;   // tokens per dispatch tile (histogram / rank kernels)
constexpr int kMaxE = 1024;
constexpr int kMaxK = 16;

// Workspace layout, shared by moe_workspace_size and the entry points.
struct Workspace {
  size_t wrt;        // router weight transposed to [E_pad, d] bf16 (bf16 route only)
  size_t tile_hist;  // [n_tiles, E] int32 per-tile expert counts, then their prefixes
  size_t gemm_tiles; // [2, max_mtiles] int4 tile tables of the two expert GEMMs,
                     // then their common length
  size_t act;        // [max_rows, d_ff] dtype: SwiGLU/ReLU activations
  size_t dedup;      // deduplicated packing: pid, first_row [T,k]; pair_slot [pairs];
                     // counts [E], offsets [E+1], flags [1] (int32)
  size_t layer;      // the fused call's own copies of the outputs its caller may
                     // leave NULL (see LayerScratch)
  size_t total;
};

// Outputs of the fused layer call that its caller may pass as NULL, carved
// from the workspace: each field is the caller's buffer or this scratch copy.
struct LayerScratch {
  float* logits;        // [T,E]
  int32_t* topk_idx;    // [T,k]
  float* topk_gate;     // [T,k]
  int32_t* counts;      // [E]
  int32_t* offsets;     // [E+1]
  int32_t* dest;        // [T,k]
  int32_t* src_token;   // [max_rows]
  int32_t* src_slot;    // [max_rows]
  int64_t* send_splits; // [ep_size]
  int64_t* send_displs; // [ep_size]
  uint32_t* flags;      // [1] (never read by the library, so never cleared)
};

// Scratch of the deduplicated packing, carved from the workspace.
struct DedupScratch {
  int32_t* tile_hist;
  int32_t* pid;        // [T,k] rank of a token's first slot to that rank, else -1
  int32_t* first_row;  // [T,k] pair row planned for those first slots
  int32_t* pair_slot;  // [pairs] slot of each pair's first slot (plan by-product)
  int32_t* counts;     // [ep_size] pairs per rank (plan by-product)
  int32_t* offsets;    // [ep_size + 1]
  uint32_t* flags;     // [1] the plan's flags on the pair table (not reported)
};

Workspace workspace_layout(const moe_layer_desc_t& d);
int router_n_pad(int E);
int64_t gemm_max_mtiles(const moe_layer_desc_t& d);

// ---- launchers (return hipSuccess or the launch error) ----
hipError_t launch_transpose_router_bf16(const bf16* w, bf16* wt, int d, int E, int E_pad,
                                        hipStream_t s);
hipError_t launch_router_bf16(const bf16* h, const bf16* wt, const float* bias, float* logits,
                              int64_t T, int d, int E, int E_pad, hipStream_t s);
hipError_t launch_router_f32(const float* h, const float* w, const float* bias, float* logits,
                             int64_t T, int d, int E, hipStream_t s);
hipError_t launch_topk(const float* logits, int32_t* idx, float* gate, uint32_t* flags,
                       int64_t T, int E, int k, int gate_mode, hipStream_t s);

hipError_t launch_dispatch_plan(const int32_t* idx, int32_t* tile_hist, int32_t* counts,
                                int32_t* offsets, int32_t* dest, int32_t* src_token,
                                int32_t* src_slot, int64_t* send_splits, int64_t* send_displs,
                                uint32_t* flags, int64_t T, int E, int k, int64_t capacity,
                                int64_t max_rows, int ep_size, hipStream_t s);
hipError_t launch_permute_rows(const void* h, const int32_t* dest, void* x_perm, int64_t T,
                               int k, int row_bytes, hipStream_t s);
hipError_t launch_pack_dedup(const void* h, const int32_t* idx, const int32_t* dest,
                             const int32_t* src_token, const int32_t* src_slot,
                             const int32_t* offsets, void* send_buf, int32_t* pair_dest,
                             int32_t* pair_token, int64_t* pair_splits, int64_t* pair_displs,
                             int32_t* recv_rows, const DedupScratch& w, int64_t T, int E, int k,
                             int ep_size, int ep_rank, int64_t max_rows, int row_bytes,
                             hipStream_t s);
// slots: y_perm holds slot rows [T*k, d] (row t*k + j for slot j of token t)
// instead of expert-ordered rows addressed through dest
hipError_t launch_combine(const void* y_perm, const int32_t* idx, const float* gate,
                          const int32_t* dest, void* y, int64_t T, int k, int d, int dtype,
                          int e_lo, int e_hi, hipStream_t s, bool slots = false);

hipError_t launch_grouped_ffn(const moe_layer_desc_t& desc, const void* x_perm,
                              const int32_t* rows, const int32_t* offsets, const void* w1,
                              const void* w2, void* y_perm, void* act, int4* tiles,
                              uint32_t* flags, hipStream_t s, const int32_t* o_tok = nullptr,
                              const int32_t* o_slot = nullptr);

}  // namespace moe
