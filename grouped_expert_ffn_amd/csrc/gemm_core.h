// bf16 MFMA tile routine for C = A . B^T on gfx950, used by the router
// (A = token rows, B = router weight transposed) and by the grouped expert
// GEMMs (A = rows of one expert's group, B = that expert's weight rows).
//
// Both operands are K-contiguous, which is the natural layout for
// v_mfma_f32_16x16x32_bf16: every lane feeds 8 consecutive K values of one
// row of each operand. Tiles of A and B are staged through LDS in 64-wide
// K slices (double-buffered, loads for slice k+1 in flight while slice k is
// multiplied). Each 128-byte LDS row holds eight 16-byte chunks stored at
// chunk ^ ((row >> 1) & 7), so the 16 rows a fragment read touches fall in
// distinct banks of the 256-byte-wide LDS.
//
// The MFMA is issued as D = W . X^T (weights as the first operand), so each
// lane ends up holding four consecutive output columns of one row: stores
// of the epilogue are 8-byte (bf16) or 16-byte (fp32) vectors.
#pragma once

#include "common.h"

namespace moe {

enum Epilogue { EPI_STORE_BF16 = 0, EPI_SWIGLU_BF16 = 1, EPI_ROUTER_F32 = 2, EPI_RELU_BF16 = 3 };

constexpr int kBK = 64;  // K slice staged per step (64 bf16 = 128 bytes per row)

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

template <int BM, int BN, int WM, int WN, int EPI>
struct TileGemm {
  static constexpr int NT = 64 * WM * WN;          // threads
  static constexpr int NB = (EPI == EPI_SWIGLU_BF16) ? 2 * BN : BN;  // B rows staged
  static constexpr int WTM = BM / WM;              // wave tile rows (m)
  static constexpr int WTN = BN / WN;              // wave tile cols (n)
  static constexpr int TM = WTM / 16;
  static constexpr int TN = WTN / 16;
  static constexpr int A_CHUNKS = BM * 8;
  static constexpr int B_CHUNKS = NB * 8;
  static constexpr int A_PER = (A_CHUNKS + NT - 1) / NT;
  static constexpr int B_PER = (B_CHUNKS + NT - 1) / NT;
  static constexpr int LDS_BUF = (BM + NB) * kBK;  // bf16 elements per buffer
  static constexpr int LDS_ELEMS = 2 * LDS_BUF;
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
  static constexpr bool GATED = EPI == EPI_SWIGLU_BF16;

  // One output tile.
  //   A      : token rows, row stride K; the tile covers rows a0 .. a0+a_rows-1
  //   B      : weight rows [NBtot, K]; output columns n0 .. n0+BN-1 (< N valid);
  //            gated: gate rows n, up rows N + n
  //   C      : output, row stride ldc, rows a0.., columns n0..
  __device__ static void run(const bf16* __restrict__ A, int64_t a0, int a_rows,
                             const bf16* __restrict__ B, int n0, int N, int K,
                             void* __restrict__ C, int64_t ldc, const float* __restrict__ bias,
                             int n_store, bf16* lds) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;

    // global source pointers for this thread's chunks
    const bf16* a_src[A_PER];
    int a_dst[A_PER];
    bool a_on[A_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      int q = tid + i * NT;
      a_on[i] = q < A_CHUNKS;
      int r = q >> 3, c = q & 7;
      int rr = r < a_rows ? r : a_rows - 1;
      a_src[i] = A + (a0 + rr) * (int64_t)K + c * 8;
      a_dst[i] = r * kBK + swz(r, c) * 8;
    }
    const bf16* b_src[B_PER];
    int b_dst[B_PER];
    bool b_on[B_PER];
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      int q = tid + i * NT;
      b_on[i] = q < B_CHUNKS;
      int r = q >> 3, c = q & 7;
      int n;
      if (GATED) {
        int rl = r < BN ? r : r - BN;
        int nn = n0 + rl;
        nn = nn < N ? nn : N - 1;
        n = r < BN ? nn : N + nn;
      } else {
        n = n0 + r;
        n = n < N ? n : N - 1;
      }
      b_src[i] = B + (int64_t)n * K + c * 8;
      b_dst[i] = BM * kBK + r * kBK + swz(r, c) * 8;
    }

    f32x4 acc[TN][TM];
    f32x4 acc2[GATED ? TN : 1][GATED ? TM : 1];
#pragma unroll
    for (int x = 0; x < TN; ++x)
#pragma unroll
      for (int y = 0; y < TM; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (GATED) {
#pragma unroll
      for (int x = 0; x < (GATED ? TN : 1); ++x)
#pragma unroll
        for (int y = 0; y < (GATED ? TM : 1); ++y) acc2[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    bf16x8 ra[A_PER], rb[B_PER];
    const int nk = K / kBK;

    auto gload = [&](int kt) {
      const int64_t ko = (int64_t)kt * kBK;
#pragma unroll
      for (int i = 0; i < A_PER; ++i)
        if (a_on[i]) ra[i] = *reinterpret_cast<const bf16x8*>(a_src[i] + ko);
#pragma unroll
      for (int i = 0; i < B_PER; ++i)
        if (b_on[i]) rb[i] = *reinterpret_cast<const bf16x8*>(b_src[i] + ko);
    };
    auto sstore = [&](int buf) {
      bf16* base = lds + buf * LDS_BUF;
#pragma unroll
      for (int i = 0; i < A_PER; ++i)
        if (a_on[i]) *reinterpret_cast<bf16x8*>(base + a_dst[i]) = ra[i];
#pragma unroll
      for (int i = 0; i < B_PER; ++i)
        if (b_on[i]) *reinterpret_cast<bf16x8*>(base + b_dst[i]) = rb[i];
    };

    gload(0);
    sstore(0);
    __syncthreads();

    const int lr = lane & 15;
    const int lq = lane >> 4;
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) gload(kt + 1);
      const bf16* As = lds + (kt & 1) * LDS_BUF;
      const bf16* Bs = As + BM * kBK;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int ci = ks * 4 + lq;
        bf16x8 yf[TM];
#pragma unroll
        for (int y = 0; y < TM; ++y) {
          int r = wm * WTM + y * 16 + lr;
          yf[y] = *reinterpret_cast<const bf16x8*>(As + r * kBK + swz(r, ci) * 8);
        }
#pragma unroll
        for (int x = 0; x < TN; ++x) {
          int r = wn * WTN + x * 16 + lr;
          bf16x8 wf = *reinterpret_cast<const bf16x8*>(Bs + r * kBK + swz(r, ci) * 8);
#pragma unroll
          for (int y = 0; y < TM; ++y)
            acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, yf[y], acc[x][y], 0, 0, 0);
          if (GATED) {
            int r2 = BN + r;
            bf16x8 wu = *reinterpret_cast<const bf16x8*>(Bs + r2 * kBK + swz(r2, ci) * 8);
#pragma unroll
            for (int y = 0; y < (GATED ? TM : 1); ++y)
              acc2[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wu, yf[y], acc2[x][y], 0, 0, 0);
          }
        }
      }
      if (kt + 1 < nk) sstore((kt + 1) & 1);
      __syncthreads();
    }

    // epilogue: lane holds D[n = 4*lq + i][m = lr] of every 16x16 sub-tile
#pragma unroll
    for (int y = 0; y < TM; ++y) {
      const int m = wm * WTM + y * 16 + lr;
      if (m >= a_rows) continue;
      const int64_t row = a0 + m;
#pragma unroll
      for (int x = 0; x < TN; ++x) {
        const int n = n0 + wn * WTN + x * 16 + lq * 4;
        if (EPI == EPI_ROUTER_F32) {
          float* out = reinterpret_cast<float*>(C) + row * ldc;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (n + i < n_store) {
              float v = acc[x][y][i];
              if (bias) v += bias[n + i];
              out[n + i] = v;
            }
          }
        } else {
          if (n >= n_store) continue;
          bf16x4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = acc[x][y][i];
            if (GATED) v = silu_f(v) * acc2[(GATED ? x : 0)][(GATED ? y : 0)][i];
            if (EPI == EPI_RELU_BF16) v = fmaxf(v, 0.0f);
            o[i] = (bf16)v;
          }
          *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(C) + row * ldc + n) = o;
        }
      }
    }
  }
};

// Workgroup -> tile order. Workgroups are dealt round-robin to the 8 XCDs;
// remap so that the workgroups one XCD runs at the same time get
// consecutive virtual tile ids, then walk tiles GROUP_M m-tiles at a time
// per n-column so neighbours share operand rows in that XCD's L2.
__device__ __forceinline__ int xcd_virtual_id(int b, int G, int iter) {
  return iter * G + (b & 7) * (G >> 3) + (b >> 3);
}

template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int v, int n_m, int n_n, int& mt, int& nt) {
  const int per_group = GROUP_M * n_n;
  const int g = v / per_group;
  const int first = g * GROUP_M;
  const int gm = min(n_m - first, GROUP_M);
  const int r = v - g * per_group;
  mt = first + r % gm;
  nt = r / gm;
}

}  // namespace moe
