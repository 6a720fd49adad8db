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

#include <type_traits>

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
  __device__ __forceinline__ static void run(const bf16* __restrict__ A, int64_t a0, int a_rows,
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

// ---------------------------------------------------------------------------
// Large-tile variant for the expert GEMMs: K slices of A and B go from global
// memory straight into LDS (global_load_lds_dwordx4: each lane's 16 bytes
// land at LDS base + 16 * lane), so no VGPRs or ds_write instructions are
// spent on staging, and STAGES slices are kept in flight (STAGES-1 ahead of
// the one being multiplied) to cover memory latency. One such load fills
// 1 KiB of consecutive LDS rows; the XOR swizzle of the 16-byte chunks is
// kept by choosing which global chunk each lane fetches.
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

  __device__ __forceinline__ static void run(const bf16* __restrict__ A, int64_t a0, int a_rows,
                                             const bf16* __restrict__ B, int n0, int N, int K,
                                             bf16* __restrict__ C, int64_t ldc, bf16* lds) {
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
      bf16* out = C + (a0 + m) * ldc;
#pragma unroll
      for (int x = 0; x < TN; ++x) {
#pragma unroll
        for (int g = 0; g < NACC / 4; ++g) {
          const int n = n0 + wn * WTN + x * MF + (MF == 32 ? 8 * g + 4 * lq : 4 * lq);
          if (n >= N) continue;
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
