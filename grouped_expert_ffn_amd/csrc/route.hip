// Route: router scores s_t = h_t W_r (+ b), ordered top-k and gate weights.
//
// "How Does Mixture-of-Experts Routing Affect LLM Repeatability?", the
// token-choice layer formula and its demand for stable score ordering with
// deterministic tie handling: ids are ordered by score descending, equal
// scores go to the lower expert id, -0 equals +0 and a NaN ranks below every
// number (NaN or +-Inf raise MOE_FLAG_NONFINITE_LOGIT).
#include <atomic>
#include <type_traits>

#include "gemm_core.h"

namespace moe {

int router_n_pad(int E) {
  if (E <= 16) return 16;
  if (E <= 32) return 32;
  if (E <= 64) return 64;
  if (E <= 128) return 128;
  return (E + 255) / 256 * 256;
}

// ---------------------------------------------------------------------------
// W_r [d, E] -> W_r^T [E_pad, d] (rows E..E_pad-1 zero), so both router
// operands are K-contiguous for the MFMA tile.
__global__ __launch_bounds__(256) void transpose_router_kernel(const bf16* __restrict__ w,
                                                               bf16* __restrict__ wt, int d,
                                                               int E, int E_pad) {
  __shared__ bf16 tile[32][33];
  const int k0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int r = ty; r < 32; r += 8) {
    int k = k0 + r, e = e0 + tx;
    tile[r][tx] = (k < d && e < E) ? w[(int64_t)k * E + e] : (bf16)0.0f;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    int e = e0 + r, k = k0 + tx;
    if (e < E_pad && k < d) wt[(int64_t)e * d + k] = tile[tx][r];
  }
}

hipError_t launch_transpose_router_bf16(const bf16* w, bf16* wt, int d, int E, int E_pad,
                                        hipStream_t s) {
  dim3 grid((d + 31) / 32, (E_pad + 31) / 32);
  hipLaunchKernelGGL(transpose_router_kernel, grid, dim3(256), 0, s, w, wt, d, E, E_pad);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16 router on MFMA: logits[T, E] = h[T, d] . W_r^T[E_pad, d]^T + bias.
// Every token's dot products run over K in an order fixed by E and d alone
// (never by T or by the token's neighbours), so a token's scores do not
// depend on its batch.
//
// E <= 32: one workgroup per 16 tokens; its eight waves take interleaved
// 32-wide K steps, reading token and weight fragments straight from global
// memory into 16x16x32 MFMAs, and the eight partial sums are added in wave
// order through LDS. The token rows stream once with many loads in flight.
constexpr int kSkinnyWaves = 8;

template <int NB>
__global__ __launch_bounds__(64 * kSkinnyWaves) void router_skinny_kernel(
    const bf16* __restrict__ h, const bf16* __restrict__ wt, const float* __restrict__ bias,
    float* __restrict__ logits, int64_t T, int d, int E) {
  __shared__ f32x4 red[kSkinnyWaves][NB][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  int64_t tr = t0 + lr;
  tr = tr < T ? tr : T - 1;
  const bf16* hp = h + tr * d + lq * 8;
  const bf16* wp = wt + (int64_t)lr * d + lq * 8;
  f32x4 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nks = d / 32;
  // this wave's K steps are wave, wave + 8, ...; the loads of U of them are
  // issued before their MFMAs, so U token-row loads per wave are in flight
  // (the token rows stream once: non-temporal, leaving W_r^T in the cache)
  constexpr int U = 8;
  for (int ks0 = wave; ks0 < nks; ks0 += U * kSkinnyWaves) {
    bf16x8 hv[U], wv[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = ks0 + u * kSkinnyWaves;
      hv[u] = bf16x8{};
      if (ks < nks) hv[u] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(hp + ks * 32));
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        // rows E..E_pad-1 of W_r^T are zero: their lanes skip the load
        wv[u][b] = bf16x8{};
        if (ks < nks && b * 16 + lr < E)
          wv[u][b] = *reinterpret_cast<const bf16x8*>(wp + (int64_t)b * 16 * d + ks * 32);
      }
    }
    // MFMAs in ascending K, as one chain per output
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ks0 + u * kSkinnyWaves >= nks) break;
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[u][b], hv[u], acc[b], 0, 0, 0);
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) red[wave][b][lane] = acc[b];
  __syncthreads();
  if (wave == 0) {
    const int64_t t = t0 + lr;
    if (t < T) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        f32x4 sum = red[0][b][lane];
#pragma unroll
        for (int w = 1; w < kSkinnyWaves; ++w) sum += red[w][b][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = b * 16 + lq * 4 + i;   // lane holds experts 4*lq+i of token lr
          if (e < E) logits[t * E + e] = sum[i] + (bias ? bias[e] : 0.0f);
        }
      }
    }
  }
}

// E >= 64: the direct-load MFMA tile with a float epilogue (bias added there).
// A router tile has few MFMAs per K slice (BN = E_pad columns at most), so
// three slice buffers keep two slices in flight.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void router_tile_kernel(
    const bf16* __restrict__ h, const bf16* __restrict__ wt, const float* __restrict__ bias,
    float* __restrict__ logits, int64_t T, int d, int E, int E_pad, int n_m, int n_n) {
  using TG = TileGemmDL<BM, BN, WM, WN, EPI_ROUTER_F32, 64, 16, false, 3>;
  __shared__ __attribute__((aligned(1024))) bf16 lds[TG::LDS_ELEMS];
  const int total = n_m * n_n;
  const int G = gridDim.x;
  auto get = [&](int i, GemmTile& t) -> bool {
    const int v = xcd_virtual_id(blockIdx.x, G, i);
    if (v >= total) return false;
    int mt, nt;
    tile_coords<8>(v, n_m, n_n, mt, nt);
    const int64_t a0 = (int64_t)mt * BM;
    t.a = h + a0 * d;
    t.a_rows = (int)min((int64_t)BM, T - a0);
    t.n0 = nt * BN;
    t.b = wt + (int64_t)t.n0 * d;
    t.c_row = a0;
    t.nk = d / 64;
    return true;
  };
  TG::run_tiles(get, E_pad, d, logits, E, lds, bias, E);
}

// CU count per device, looked up once (concurrent first calls may both look it
// up and store the same value)
static std::atomic<int> g_num_cu[64];

static int num_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = g_num_cu[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    g_num_cu[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

int device_cu_count() { return num_cus(); }

template <int BM, int BN, int WM, int WN>
static hipError_t router_tile_launch(const bf16* h, const bf16* wt, const float* bias,
                                     float* logits, int64_t T, int d, int E, int E_pad,
                                     hipStream_t s) {
  const int n_m = (int)((T + BM - 1) / BM);
  const int n_n = E_pad / BN;
  const int total = n_m * n_n;
  int G = min(((total + 7) / 8) * 8, num_cus());
  G = max(8, G / 8 * 8);
  hipLaunchKernelGGL((router_tile_kernel<BM, BN, WM, WN>), dim3(G), dim3(64 * WM * WN), 0, s, h,
                     wt, bias, logits, T, d, E, E_pad, n_m, n_n);
  return hipGetLastError();
}

hipError_t launch_router_bf16(const bf16* h, const bf16* wt, const float* bias, float* logits,
                              int64_t T, int d, int E, int E_pad, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const unsigned blocks16 = (unsigned)((T + 15) / 16);
  switch (E_pad) {
    case 16:
      hipLaunchKernelGGL(router_skinny_kernel<1>, dim3(blocks16), dim3(64 * kSkinnyWaves), 0, s, h, wt, bias,
                         logits, T, d, E);
      return hipGetLastError();
    case 32:
      hipLaunchKernelGGL(router_skinny_kernel<2>, dim3(blocks16), dim3(64 * kSkinnyWaves), 0, s, h, wt, bias,
                         logits, T, d, E);
      return hipGetLastError();
    case 64: return router_tile_launch<64, 64, 2, 4>(h, wt, bias, logits, T, d, E, E_pad, s);
    case 128: return router_tile_launch<64, 128, 2, 4>(h, wt, bias, logits, T, d, E, E_pad, s);
    default: return router_tile_launch<128, 256, 2, 4>(h, wt, bias, logits, T, d, E, E_pad, s);
  }
}

// ---------------------------------------------------------------------------
// fp32 router: one thread per (token, expert), K summed in order.
__global__ __launch_bounds__(256) void router_f32_kernel(const float* __restrict__ h,
                                                         const float* __restrict__ w,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ logits, int64_t T,
                                                         int d, int E) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * E) return;
  int64_t t = i / E;
  int e = (int)(i - t * E);
  const float* x = h + t * d;
  float acc = 0.f;
  for (int c = 0; c < d; ++c) acc = fmaf(x[c], w[(int64_t)c * E + e], acc);
  if (bias) acc += bias[e];
  logits[i] = acc;
}

hipError_t launch_router_f32(const float* h, const float* w, const float* bias, float* logits,
                             int64_t T, int d, int E, hipStream_t s) {
  int64_t n = T * E;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(router_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, h, w,
                     bias, logits, T, d, E);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k + gates. A token's E scores are spread over a segment of W lanes, V
// scores per lane (W = 16 for 16 < E <= 256, the next power of two >= E below
// that, 64 above). Each score becomes a 64-bit key whose order is the ranking
// order: high 32 bits an order-preserving image of the float (-0 folded onto
// +0, every NaN just below -Inf, absent experts below that), low 32 bits the
// complemented id so equal scores favour the lower id. k rounds of a segment
// max-reduction pick the winners in order; keys are unique, so exactly one
// slot wins each round. Segments of up to 16 lanes reduce with DPP row
// permutations (no LDS traffic); 64-lane segments use cross-lane shuffles.
__device__ __forceinline__ uint32_t score_bits(float x) {
  if (x != x) return 1u;       // NaN: below every number
  if (x == 0.0f) x = 0.0f;     // -0 -> +0
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// inverse of score_bits for a present, non-NaN score
__device__ __forceinline__ float bits_score(uint32_t b) {
  return __uint_as_float((b & 0x80000000u) ? (b & 0x7fffffffu) : ~b);
}

// log sigmoid(s) - log sigmoid(s0) for s <= s0. log sigmoid(s) is
// s - log(1 + e^s) below zero and -log(1 + e^-s) above; when both scores are
// negative the differences s - s0 and of the two log terms are taken
// separately, so the gap keeps full precision for large negative scores.
__device__ __forceinline__ float log_sigmoid_gap(float s, float s0) {
  if (s < 0.0f && s0 < 0.0f) return (s - s0) - (log1pf(expf(s)) - log1pf(expf(s0)));
  const float ls = s < 0.0f ? s - log1pf(expf(s)) : -log1pf(expf(-s));
  const float l0 = s0 < 0.0f ? s0 - log1pf(expf(s0)) : -log1pf(expf(-s0));
  return ls - l0;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}

// DPP patterns that, applied in turn with a commutative op, leave every lane
// of a W-lane segment (W <= 16, aligned in a 16-lane row) with the result.
template <int W, typename F>
__device__ __forceinline__ void seg_dpp_steps(F&& step) {
  if (W >= 2) step(std::integral_constant<int, 0xB1>());   // quad_perm [1,0,3,2]
  if (W >= 4) step(std::integral_constant<int, 0x4E>());   // quad_perm [2,3,0,1]
  if (W >= 8) step(std::integral_constant<int, 0x141>());  // row_half_mirror
  if (W >= 16) step(std::integral_constant<int, 0x140>()); // row_mirror
}

template <int W>
__device__ __forceinline__ uint64_t seg_max(uint64_t v) {
  if (W <= 16) {
    seg_dpp_steps<W>([&](auto c) {
      constexpr int C = decltype(c)::value;
      const uint64_t o = ((uint64_t)dpp<C>((uint32_t)(v >> 32)) << 32) | dpp<C>((uint32_t)v);
      v = o > v ? o : v;
    });
  } else {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) {
      uint64_t w = __shfl_xor(v, o, W);
      v = w > v ? w : v;
    }
  }
  return v;
}

template <int W>
__device__ __forceinline__ float seg_sum(float v) {
  if (W <= 16) {
    seg_dpp_steps<W>([&](auto c) {
      constexpr int C = decltype(c)::value;
      v += __uint_as_float(dpp<C>(__float_as_uint(v)));
    });
  } else {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, W);
  }
  return v;
}

template <int W, int V>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   int32_t* __restrict__ idx,
                                                   float* __restrict__ gate,
                                                   uint32_t* __restrict__ flags, int64_t T, int E,
                                                   int k, int mode) {
  const int sl = threadIdx.x & (W - 1);
  const int64_t t = ((int64_t)blockIdx.x * 256 + threadIdx.x) / W;
  const bool act = t < T;
  const float* row = logits + (act ? t : 0) * (int64_t)E;

  float val[V];
  uint64_t key[V];
  bool bad = false;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = sl + i * W;
    const bool ok = act && e < E;
    const float x = ok ? row[e] : 0.0f;
    val[i] = x;
    bad |= ok && !isfinite(x);
    key[i] = ok ? (((uint64_t)score_bits(x) << 32) | (uint32_t)(~(uint32_t)e)) : 0ull;
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flags, MOE_FLAG_NONFINITE_LOGIT);

  uint32_t taken = 0;
  uint64_t mine = 0;   // lane r < k keeps the key of the r-th winner
  uint64_t first = 0;  // every lane: the top key
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (!(taken & (1u << i)) && key[i] > best) best = key[i];
    const uint64_t win = seg_max<W>(best);
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (key[i] == win && win != 0ull) taken |= 1u << i;
    if (r == 0) first = win;
    if (sl == r) mine = win;
  }

  const bool holder = act && sl < k;
  const int my_id = (int)(~(uint32_t)(mine & 0xffffffffu));
  // winners' scores come back from their keys (a NaN winner re-reads its score)
  const uint32_t mb = (uint32_t)(mine >> 32), fb = (uint32_t)(first >> 32);
  const float my_v = holder ? (mb == 1u ? row[my_id] : bits_score(mb)) : 0.0f;
  const float top = fb == 1u ? __int_as_float(0x7fc00000) : bits_score(fb);
  float g = 0.f;
  if (mode == MOE_GATE_SOFTMAX) {
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = sl + i * W;
      if (act && e < E) part += __expf(val[i] - top);
    }
    const float sum = seg_sum<W>(part);
    g = __expf(my_v - top) / sum;
  } else if (mode == MOE_GATE_SOFTMAX_TOPK_RENORM) {
    const float ex = holder ? __expf(my_v - top) : 0.f;
    const float sum = seg_sum<W>(ex);
    g = ex / sum;
  } else {
    // logistic gates normalised over the chosen k, formed in the log domain:
    // g_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) with l = log sigmoid(s) and
    // slot 0 the top score, so scores far below zero (where sigmoid itself
    // underflows in float32) still give finite gates
    const float ex = holder ? __expf(log_sigmoid_gap(my_v, top)) : 0.f;
    const float sum = seg_sum<W>(ex);
    g = ex / sum;
  }
  if (holder) {
    idx[t * k + sl] = my_id;
    gate[t * k + sl] = g;
  }
}

template <int W, int V>
static hipError_t topk_launch(const float* logits, int32_t* idx, float* gate, uint32_t* flags,
                              int64_t T, int E, int k, int mode, hipStream_t s) {
  int64_t threads = T * W;
  hipLaunchKernelGGL((topk_kernel<W, V>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     s, logits, idx, gate, flags, T, E, k, mode);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int32_t* idx, float* gate, uint32_t* flags,
                       int64_t T, int E, int k, int mode, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (E <= 1) return topk_launch<1, 1>(logits, idx, gate, flags, T, E, k, mode, s);
  if (E <= 2) return topk_launch<2, 1>(logits, idx, gate, flags, T, E, k, mode, s);
  if (E <= 4) return topk_launch<4, 1>(logits, idx, gate, flags, T, E, k, mode, s);
  if (E <= 8) return topk_launch<8, 1>(logits, idx, gate, flags, T, E, k, mode, s);
  if (E <= 16) return topk_launch<16, 1>(logits, idx, gate, flags, T, E, k, mode, s);
  if (E <= 32) return topk_launch<16, 2>(logits, idx, gate, flags, T, E, k, mode, s);
  if (E <= 64) return topk_launch<16, 4>(logits, idx, gate, flags, T, E, k, mode, s);
  if (E <= 128) return topk_launch<16, 8>(logits, idx, gate, flags, T, E, k, mode, s);
  if (E <= 256) return topk_launch<16, 16>(logits, idx, gate, flags, T, E, k, mode, s);
  if (E <= 512) return topk_launch<64, 8>(logits, idx, gate, flags, T, E, k, mode, s);
  return topk_launch<64, 16>(logits, idx, gate, flags, T, E, k, mode, s);
}

}  // namespace moe
