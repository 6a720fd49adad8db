// bf16 MFMA tile routine for C = A . B^T on gfx950, used by the router
// (A = token rows, B = router weight transposed) and by the grouped expert
// GEMMs (A = rows of one expert's group, B = that expert's weight rows).
//
// Both operands are K-contiguous, the natural layout for the bf16 MFMAs:
// every lane feeds 8 consecutive K values of one row of each operand. K
// slices of A and B stream from global memory straight into LDS
// (global_load_lds_dwordx4), double-buffered. Each LDS row holds 16-byte
// chunks stored at chunk ^ (row-dependent key), so the 16 rows one fragment
// read touches fall in distinct banks of the 256-byte-wide LDS.
//
// The MFMA is issued as D = W . X^T (weights as the first operand), so each
// lane ends up holding four consecutive output columns of one row: stores of
// the epilogue are 8-byte (bf16) or 16-byte (fp32) vectors.
#pragma once

#include <type_traits>

#include "common.h"

namespace moe {

enum Epilogue { EPI_STORE_BF16 = 0, EPI_SWIGLU_BF16 = 1, EPI_ROUTER_F32 = 2, EPI_RELU_BF16 = 3 };

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// ---------------------------------------------------------------------------
// The tile: K slices of A and B go from global memory straight into LDS
// (global_load_lds_dwordx4: each lane's 16 bytes land at LDS base + 16 *
// lane), so no VGPRs or ds_write instructions are spent on staging; STAGES
// slices are kept in flight (STAGES-1 ahead of the one being multiplied).
// One such load fills 1 KiB of consecutive LDS rows; the XOR swizzle of the
// 16-byte chunks is kept by choosing which global chunk each lane fetches.
template <int BK>
struct SliceLayout {
  static constexpr int CPR = BK / 8;            // 16-byte chunks per LDS row
  static constexpr int RPL = 64 / CPR;          // rows filled by one 1 KiB load
  static constexpr int RPB = 16 / CPR;          // rows per 256-byte bank line
  __device__ static int swz(int row, int chunk) { return chunk ^ ((row / RPB) & (CPR - 1)); }
};

// Workgroup barrier that orders LDS traffic only: this wave's LDS reads and
// writes are complete, then all waves meet. Unlike __syncthreads() it does not
// drain outstanding global loads, so slices prefetched into LDS by
// global_load_lds stay in flight across it (their completion is awaited
// explicitly with wait_vmcnt before the barrier that publishes them).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt with vmcnt <= N and no wait on the other counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int BM, int BN, int WM, int WN, int EPI, int BK = 64, int STAGES = 2, int MF = 16>
struct TileGemmDL {
  using L = SliceLayout<BK>;
  static constexpr int NT = 64 * WM * WN;
  static constexpr int NW = WM * WN;
  static constexpr bool GATED = EPI == EPI_SWIGLU_BF16;
  static constexpr int NB = GATED ? 2 * BN : BN;
  static constexpr int ROWS = BM + NB;             // LDS rows per K slice
  static constexpr int LOADS = ROWS / L::RPL;      // 1 KiB loads per slice
  static constexpr int LPW = LOADS / NW;           // loads per wave per slice
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / MF, TN = WTN / MF;   // MFMA tiles per wave
  static constexpr int LDS_BUF = ROWS * BK;
  static constexpr int LDS_ELEMS = STAGES * LDS_BUF;
  using Acc = typename std::conditional<MF == 32, f32x16, f32x4>::type;
  static constexpr int NACC = MF == 32 ? 16 : 4;
  static_assert(MF == 16 || MF == 32, "MFMA shape");
  static_assert(LOADS % NW == 0, "loads must split evenly over waves");
  static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must be a multiple of the MFMA tile");
  static_assert(BK % 32 == 0 && STAGES >= 2, "K slice and stage count");
  static_assert((STAGES - 2) * LPW < 64, "vmcnt range");

  // C is bf16 (row stride ldc) for the expert epilogues; for EPI_ROUTER_F32 it
  // is float, bias (or null) is added and only columns < n_store are written.
  __device__ __forceinline__ static void run(const bf16* __restrict__ A, int64_t a0, int a_rows,
                                             const bf16* __restrict__ B, int n0, int N, int K,
                                             void* __restrict__ Cv, int64_t ldc, bf16* lds,
                                             const float* __restrict__ bias = nullptr,
                                             int n_store = 0) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wm = wave / WN;
    const int wn = wave % WN;

    // per-lane element offset of each of this wave's loads, relative to the
    // tile's first A row (loads into A rows) or first weight row (B rows);
    // rows past the end are clamped onto the last valid row
    const bf16* Ab = A + a0 * (int64_t)K;
    const bf16* Bb = B + (int64_t)n0 * K;
    uint32_t off[LPW];
    bool is_a[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int r = (wave * LPW + i) * L::RPL + lane / L::CPR;  // LDS row
      const int c = L::swz(r, lane % L::CPR);                   // global chunk kept in that slot
      is_a[i] = r < BM;
      int row;
      if (r < BM) {
        row = r < a_rows ? r : a_rows - 1;
      } else {
        const int q = r - BM;
        const int ql = (GATED && q >= BN) ? q - BN : q;
        const int nn = n0 + ql < N ? ql : N - 1 - n0;
        row = (GATED && q >= BN) ? N + nn : nn;
      }
      off[i] = (uint32_t)row * (uint32_t)K + (uint32_t)(c * 8);
    }

    Acc acc[TN][TM];
    Acc acc2[GATED ? TN : 1][GATED ? TM : 1];
#pragma unroll
    for (int x = 0; x < TN; ++x)
#pragma unroll
      for (int y = 0; y < TM; ++y)
#pragma unroll
        for (int q = 0; q < NACC; ++q) acc[x][y][q] = 0.f;
    if (GATED) {
#pragma unroll
      for (int x = 0; x < (GATED ? TN : 1); ++x)
#pragma unroll
        for (int y = 0; y < (GATED ? TM : 1); ++y)
#pragma unroll
          for (int q = 0; q < NACC; ++q) acc2[x][y][q] = 0.f;
    }

    auto issue = [&](int kt, int buf) {
      bf16* base = lds + buf * LDS_BUF + wave * LPW * L::RPL * BK;
      const int ko = kt * BK;
#pragma unroll
      for (int i = 0; i < LPW; ++i)
        __builtin_amdgcn_global_load_lds((is_a[i] ? Ab : Bb) + (off[i] + ko),
                                         base + i * L::RPL * BK, 16, 0, 0);
    };

    // MFMA operand lanes: lane feeds row (lane % MF) and the 8 K values of
    // 16-byte chunk (lane / MF) of the current K sub-step
    const int lr = lane % MF;
    const int lq = lane / MF;
    auto mma = [&](const bf16x8& w, const bf16x8& x, Acc& c) {
      if constexpr (MF == 32)
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, x, c, 0, 0, 0);
      else
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, x, c, 0, 0, 0);
    };
    constexpr int KSUB = MF == 32 ? 16 : 32;       // K per MFMA
    constexpr int CPS = KSUB / 8;                  // 16-byte chunks per sub-step
    auto compute = [&](int buf) {
      const bf16* As = lds + buf * LDS_BUF;
      const bf16* Bs = As + BM * BK;
#pragma unroll
      for (int ks = 0; ks < BK / KSUB; ++ks) {
        const int ci = ks * CPS + lq;
        bf16x8 yf[TM];
#pragma unroll
        for (int y = 0; y < TM; ++y) {
          const int r = wm * WTM + y * MF + lr;
          yf[y] = *reinterpret_cast<const bf16x8*>(As + r * BK + L::swz(r, ci) * 8);
        }
#pragma unroll
        for (int x = 0; x < TN; ++x) {
          const int r = wn * WTN + x * MF + lr;
          const bf16x8 wf = *reinterpret_cast<const bf16x8*>(Bs + r * BK + L::swz(r, ci) * 8);
#pragma unroll
          for (int y = 0; y < TM; ++y) mma(wf, yf[y], acc[x][y]);
          if (GATED) {
            const int r2 = BN + r;
            const bf16x8 wu = *reinterpret_cast<const bf16x8*>(Bs + r2 * BK + L::swz(r2, ci) * 8);
#pragma unroll
            for (int y = 0; y < (GATED ? TM : 1); ++y) mma(wu, yf[y], acc2[(GATED ? x : 0)][y]);
          }
        }
      }
    };

    const int nk = K / BK;
    if (STAGES == 2) {
      // slice kt+1 streams into the other buffer while slice kt is multiplied;
      // the closing barrier also frees the buffer just read for the next load
      issue(0, 0);
      wait_vmcnt<0>();
      lds_barrier();
      for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) issue(kt + 1, (kt + 1) & 1);
        compute(kt & 1);
        wait_vmcnt<0>();
        lds_barrier();
      }
    } else {
      // the previous tile's LDS reads and global stores are finished first
      wait_vmcnt<0>();
      lds_barrier();
#pragma unroll
      for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk) issue(s, s);
      for (int kt = 0; kt < nk; ++kt) {
        if (kt + STAGES - 1 <= nk)
          wait_vmcnt<(STAGES - 2) * LPW>();
        else
          wait_vmcnt<0>();
        lds_barrier();
        if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
        compute(kt % STAGES);
      }
    }

    // epilogue: lane holds D[n][m = lr] for n = 8*g + 4*lq + i (32x32 tiles,
    // g = 0..3) or n = 4*lq + i (16x16 tiles), four consecutive columns at a time
#pragma unroll
    for (int y = 0; y < TM; ++y) {
      const int m = wm * WTM + y * MF + lr;
      if (m >= a_rows) continue;
#pragma unroll
      for (int x = 0; x < TN; ++x) {
#pragma unroll
        for (int g = 0; g < NACC / 4; ++g) {
          const int n = n0 + wn * WTN + x * MF + (MF == 32 ? 8 * g + 4 * lq : 4 * lq);
          if constexpr (EPI == EPI_ROUTER_F32) {
            float* out = reinterpret_cast<float*>(Cv) + (a0 + m) * ldc;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (n + i < n_store) out[n + i] = acc[x][y][4 * g + i] + (bias ? bias[n + i] : 0.0f);
          } else {
            if (n >= N) continue;
            bf16* out = reinterpret_cast<bf16*>(Cv) + (a0 + m) * ldc;
            bf16x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float v = acc[x][y][4 * g + i];
              if (GATED) v = silu_f(v) * acc2[(GATED ? x : 0)][(GATED ? y : 0)][4 * g + i];
              if (EPI == EPI_RELU_BF16) v = fmaxf(v, 0.0f);
              o[i] = (bf16)v;
            }
            *reinterpret_cast<bf16x4*>(out + n) = o;
          }
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
