// bf16 MFMA tile routine for C = A . B^T on gfx950, used by the router
// (A = token rows, B = router weight transposed) and by the grouped expert
// GEMMs (A = rows of one expert's group, B = that expert's weight rows).
//
// Both operands are K-contiguous, the natural layout for the bf16 MFMAs:
// every lane feeds 8 consecutive K values of one row of each operand. K
// slices of A and B stream from global memory straight into LDS (buffer
// loads with the LDS bit, 16 bytes per lane) through two to five slice
// buffers. Each LDS row holds 16-byte chunks stored at chunk ^
// (row-dependent key), so the 16 rows one fragment read touches fall in
// distinct banks of the 256-byte-wide LDS.
//
// The MFMA is issued as D = W . X^T (weights as the first operand), so each
// lane ends up holding four consecutive output columns of one row: stores of
// the epilogue are 16-byte vectors (bf16, after a lane swap between column
// tiles; 8-byte where a wave has a single column tile) or fp32 vectors.
#pragma once

#include <type_traits>

#include "common.h"

namespace moe {

// EPI_SLOTS_BF16 stores like EPI_STORE_BF16, but grouped row r goes to output
// row o_tok[r] * o_k + o_slot[r] (the row of its (token, slot) pair)
enum Epilogue {
  EPI_STORE_BF16 = 0,
  EPI_SWIGLU_BF16 = 1,
  EPI_ROUTER_F32 = 2,
  EPI_RELU_BF16 = 3,
  EPI_SLOTS_BF16 = 4
};

// SiLU with the hardware reciprocal (about 1 ulp): g * 1 / (1 + e^-g)
__device__ __forceinline__ float silu_f(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// ---------------------------------------------------------------------------
// The tile: K slices of A and B go from global memory straight into LDS
// (loads with the LDS bit: each lane's 16 bytes land at LDS base + 16 *
// lane), so no VGPRs or ds_write instructions are spent on staging; two
// slices are kept in LDS, the next one in flight while one is multiplied.
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
// drain outstanding global loads, so slices prefetched into LDS by the
// direct loads stay in flight across it (their completion is awaited
// explicitly with wait_vmcnt before the barrier that publishes them).
// The lgkmcnt wait goes through the builtin so the compiler's own wait
// insertion knows that every earlier LDS read has returned; the barrier itself
// is an asm statement with a memory clobber, so no LDS access moves across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt: no wait
  asm volatile("s_barrier" ::: "memory");
}

// Cache-policy operand of a buffer load on this GPU family: bit 1 marks the
// access non-temporal.
constexpr int kNonTemporal = 2;

// s_waitcnt with vmcnt <= N and no wait on the other counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One output tile as the persistent loop sees it.
struct GemmTile {
  const bf16* a;    // first A row of the tile (row stride K)
  const bf16* b;    // weight row n0 (row stride K); with the gated epilogue the
                    // matching up-projection rows sit N rows further on
  int a_rows;       // valid A rows, 1..BM (rows past them are not stored)
  int n0;           // first output column
  int64_t c_row;    // output row of the tile's first A row
  int nk;           // K slices (of BK) to multiply
  const int32_t* rows;   // gathered A rows only: the tile's A row i is row rows[i]
                         // of the matrix at `a` (then `a` is that matrix's base)
  const int32_t* o_tok;  // EPI_SLOTS_BF16 only: token and slot of each grouped row
  const int32_t* o_slot;
  int o_k;
  // weight slices loaded non-temporal (no reuse expected in the last-level
  // cache), so that they do not evict data a later kernel reads
  bool nt_w = false;
  // rider: up to 16 more rows of the same expert (the short remainder of its
  // group), multiplied with this tile's weight slices and stored beside its
  // rows; r_rows = 0: none. ra: rider row 0 (row stride K), or with gathered
  // rows the matrix base, rrows then holding the rider's row indices; r_crow:
  // output row of rider row 0
  int r_rows = 0;
  const bf16* ra = nullptr;
  const int32_t* rrows = nullptr;
  int64_t r_crow = 0;
};

// Persistent tile loop of one workgroup: run_tiles(get, ...) multiplies the
// tiles get(0), get(1), ... until get returns false. K slices stream through
// NBUF LDS buffers as one sequence that runs across tile boundaries: the
// next tile's first slices are already in flight while the current tile's
// epilogue converts and stores its accumulators.
//
// A tile whose valid rows all fall in the lower half of the wave grid
// (a_rows <= BM / 2 with two wave rows) leaves the upper waves idle: they
// still fetch their share of each slice and meet every barrier, but issue no
// MFMAs, so the lower waves have their SIMDs to themselves.
//
// RIDE: a tile may carry a rider (GemmTile::r_rows), 16 rows of the same
// expert that would otherwise form a short tile of their own, which would
// stream the whole weight block again for a few rows. The rider's rows come
// into a 16-row area after each slice (one extra load per wave, 16 lanes),
// and every wave multiplies them with its own weight fragments for half of
// its column tiles (the two wave rows take one half each): the same MFMAs,
// operands and K order as in a tile of their own, so the same bits.
template <int BM, int BN, int WM, int WN, int EPI, int BK = 64, int MF = 16, bool GA = false,
          int NBUF = 2, bool RIDE = false>
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
  static constexpr int RR = RIDE ? 16 : 0;          // rider rows per slice
  static constexpr int LDS_BUF = (ROWS + RR) * BK;
  static constexpr int LDS_ELEMS = NBUF * LDS_BUF;
  static constexpr int LPWR = LPW + (RIDE ? 1 : 0);  // loads per wave per slice
  static constexpr int RX = TN >= 2 ? TN / 2 : 1;    // rider column tiles per wave
  using Acc = typename std::conditional<MF == 32, f32x16, f32x4>::type;
  static constexpr int NACC = MF == 32 ? 16 : 4;
  static constexpr int KSUB = MF == 32 ? 16 : 32;  // K per MFMA
  static constexpr int CPS = KSUB / 8;             // 16-byte chunks per sub-step
  static constexpr int NSUB = BK / KSUB;           // sub-steps per slice
  static constexpr int TU = GATED ? TN : 1;
  static_assert(MF == 16 || MF == 32, "MFMA shape");
  static_assert(NBUF >= 2 && NBUF <= 5, "two to five slice buffers");
  static_assert((NBUF - 2) * LPWR < 64, "slices in flight must fit the vmcnt field");
  // a rider: 16-row MFMA tiles, two rider rows per wave, two wave rows
  static_assert(!RIDE || (MF == 16 && BK == 64 && WM == 2 && 2 * NW == RR &&
                          EPI != EPI_ROUTER_F32),
                "rider layout");
  static_assert(LOADS % NW == 0, "loads must split evenly over waves");
  static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must be a multiple of the MFMA tile");
  static_assert(BK % 32 == 0 && NSUB >= 2, "two or more MFMA sub-steps per K slice");
  static_assert(BM % L::RPL == 0, "a load must not straddle the A and B rows");
  // gathered A rows keep one swizzle key per load parity (16 rows per key cycle)
  static_assert(!GA || 2 * L::RPL == L::RPB * L::CPR, "gathered rows need BK = 64");

  // C is bf16 (row stride ldc) for the expert epilogues; for EPI_ROUTER_F32 it
  // is float, bias (or null) is added and only columns < n_store are written.
  // N is the weight's output width (rows past it are clamped onto row N-1 and
  // their columns not stored); K is the operands' row stride, every tile has
  // nk >= 1 slices of BK, and every operand byte a tile reads must lie within
  // 4 GiB of its a / b pointer.
  template <class GetTile>
  __device__ __forceinline__ static void run_tiles(GetTile get, int N, int K,
                                                   void* __restrict__ Cv, int64_t ldc, bf16* lds,
                                                   const float* __restrict__ bias = nullptr,
                                                   int n_store = 0) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wm = wave / WN;
    const int wn = wave % WN;

    // ---- global -> LDS loads. Load i of this wave fills LDS rows
    // (wave * LPW + i) * RPL .. + RPL - 1 of a slice; whether those are A or
    // weight rows is uniform across the wave (RPL divides BM).
    bool is_a[LPW];
    // per-lane byte offset from the tile's a / b pointer; for gathered A rows
    // the row index itself, made a byte offset when the slice is fetched (so
    // the row-index load has a whole slice of MFMAs to arrive)
    uint32_t off[LPW];
    // rider load: byte offset from the tile's ra (gathered rows: the row
    // index, and the chunk's byte offset in rchunk)
    uint32_t roff = 0, rchunk = 0;
#pragma unroll
    for (int i = 0; i < LPW; ++i) is_a[i] = (wave * LPW + i) * L::RPL < BM;
    // gathered A rows: byte offset of this lane's 16-byte chunk, for loads of
    // even and odd index in the slice
    const uint32_t chunk_even = GA ? (uint32_t)(L::swz(lane / L::CPR, lane % L::CPR) * 16) : 0u;
    const uint32_t chunk_odd =
        GA ? (uint32_t)(L::swz(L::RPL + lane / L::CPR, lane % L::CPR) * 16) : 0u;
    auto set_offsets = [&](const GemmTile& t) {
      // the lane id is re-read here (volatile, so it stays inside the tile
      // loop); otherwise the compiler keeps every load's row and chunk live
      // across the loop for the next call, which costs 16 VGPRs
      int ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int r = (wave * LPW + i) * L::RPL + ln / L::CPR;  // LDS row
        const int c = L::swz(r, ln % L::CPR);                   // global chunk kept in that slot
        int row;
        if (is_a[i]) {
          row = r < t.a_rows ? r : t.a_rows - 1;
          if constexpr (GA) {
            off[i] = (uint32_t)t.rows[row];
            continue;
          }
        } else {
          const int q = r - BM;
          const int ql = (GATED && q >= BN) ? q - BN : q;
          const int nn = t.n0 + ql < N ? ql : N - 1 - t.n0;
          row = (GATED && q >= BN) ? N + nn : nn;
        }
        off[i] = ((uint32_t)row * (uint32_t)K + (uint32_t)(c * 8)) * 2u;
      }
      if constexpr (RIDE) {
        // rider row rr (two per wave; lanes 2 * CPR and up load nothing),
        // clamped onto the last rider row; a tile without a rider points
        // its unused rider load at its own first row
        const int rr = wave * 2 + (ln / L::CPR) % 2;
        const int c = L::swz(rr, ln % L::CPR);
        const int src = t.r_rows > 0 ? (rr < t.r_rows ? rr : t.r_rows - 1) : 0;
        if constexpr (GA) {
          roff = (uint32_t)(t.r_rows > 0 ? t.rrows[src] : t.rows[0]);
          rchunk = (uint32_t)(c * 16);
        } else {
          roff = ((uint32_t)src * (uint32_t)K + (uint32_t)(c * 8)) * 2u;
        }
      }
    };
    // When a wave's loads are all token rows or all weight rows (RPL * LPW
    // divides BM), they go through one buffer resource per slice: base = the
    // tile's a or b pointer, slice offset in the scalar offset, 32-bit lane
    // offset in the VGPR, LDS destination in M0 (buffer_load_dwordx4 ... lds).
    // Buffer loads rather than global_load_lds because the compiler's wait
    // insertion treats a global load into LDS as an access that may hit both
    // counters and then turns every LDS-read wait into a full drain while one
    // is outstanding; with buffer loads its LDS-read waits stay exact.
    // Resource word 3 = 0x00020000 (32-bit data format, the raw-buffer setting
    // of this GPU family); the record count is the maximum, so no clamping.
    // A wave whose loads straddle the A and weight rows keeps a resource for
    // each and picks one per load (a scalar select; which rows a load fills
    // depends only on the wave and the load's index).
    constexpr bool WAVE_UNIFORM = BM % (LPW * L::RPL) == 0;
    const bool wave_a = wave * LPW * L::RPL < BM;
    auto issue = [&](const GemmTile& t, int kt, int buf) {
      bf16* base = lds + buf * LDS_BUF + wave * LPW * L::RPL * BK;
      const uint32_t ko = (uint32_t)kt * (BK * 2);
      if constexpr (WAVE_UNIFORM) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16*>(wave_a ? t.a : t.b), (short)0, -1, 0x00020000);
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
          uint32_t o = off[i];
          if (GA && wave_a)
            o = o * (uint32_t)(K * 2) + (((wave * LPW + i) & 1) ? chunk_odd : chunk_even);
          if (!wave_a && t.nt_w)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void*)(base + i * L::RPL * BK), 16, o, ko,
                0, kNonTemporal);
          else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void*)(base + i * L::RPL * BK), 16, o, ko,
                0, 0);
        }
        return;
      }
      const __amdgpu_buffer_rsrc_t ra =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(t.a), (short)0, -1, 0x00020000);
      const __amdgpu_buffer_rsrc_t rb =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(t.b), (short)0, -1, 0x00020000);
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        uint32_t o = off[i];
        if (GA && is_a[i])
          o = o * (uint32_t)(K * 2) + (((wave * LPW + i) & 1) ? chunk_odd : chunk_even);
        if (!is_a[i] && t.nt_w)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rb, (__attribute__((address_space(3))) void*)(base + i * L::RPL * BK), 16, o, ko, 0,
              kNonTemporal);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              is_a[i] ? ra : rb, (__attribute__((address_space(3))) void*)(base + i * L::RPL * BK),
              16, o, ko, 0, 0);
      }
    };
    // load cursor: the tile and slice fetched next
    GemmTile lt;
    int l_idx = 0, l_k = 0, tiles_end = 0x7fffffff;
    bool l_live = get(0, lt);
    if (!l_live) return;
    GemmTile ct = lt;   // tile being multiplied
    set_offsets(lt);
    // the buffer the next slice goes to; slices issued so far (the slices of
    // all tiles form one sequence)
    int l_buf = 0, l_issued = 0;
    // the rider's two rows of this wave for slice kt (16 lanes, 256 bytes,
    // after the slice's A and weight rows in the buffer). With two buffers
    // every slice wait is a full drain, so only tiles with a rider issue it;
    // with more buffers the waits count loads, so every slice of every tile
    // issues it and each wave's load count per slice stays fixed
    auto issue_rider = [&](const GemmTile& t, int kt, int buf) {
      if constexpr (RIDE) {
        if (NBUF == 2 && t.r_rows == 0) return;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16*>(t.r_rows > 0 ? t.ra : t.a), (short)0, -1, 0x00020000);
        const uint32_t o = GA ? roff * (uint32_t)(K * 2) + rchunk : roff;
        bf16* base = lds + buf * LDS_BUF + ROWS * BK + wave * 2 * BK;
        if (lane < 2 * L::CPR)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, (__attribute__((address_space(3))) void*)base, 16, o, (uint32_t)kt * (BK * 2), 0,
              0);
      }
    };
    auto issue_next = [&]() {
      if (!l_live) return;
      issue(lt, l_k, l_buf);
      issue_rider(lt, l_k, l_buf);
      ++l_issued;
      l_buf = l_buf + 1 == NBUF ? 0 : l_buf + 1;
      if (++l_k == lt.nk) {
        l_k = 0;
        l_live = get(++l_idx, lt);
        if (l_live)
          set_offsets(lt);
        else
          tiles_end = l_idx;
      }
    };

    // ---- MFMA side. Lane feeds row (lane % MF) and the 8 K values of
    // 16-byte chunk (lane / MF) of the current K sub-step.
    Acc acc[TN][TM];
    Acc acc2[TU][GATED ? TM : 1];
    auto zero_acc = [&]() {
#pragma unroll
      for (int x = 0; x < TN; ++x)
#pragma unroll
        for (int y = 0; y < TM; ++y)
#pragma unroll
          for (int q = 0; q < NACC; ++q) acc[x][y][q] = 0.f;
      if (GATED) {
#pragma unroll
        for (int x = 0; x < TU; ++x)
#pragma unroll
          for (int y = 0; y < (GATED ? TM : 1); ++y)
#pragma unroll
            for (int q = 0; q < NACC; ++q) acc2[x][y][q] = 0.f;
      }
    };
    // rider accumulators: half of this wave's column tiles, the lower half on
    // the lower wave row and the upper half on the upper one (each SIMD runs
    // one wave of each row, so each takes the same extra work); with a single
    // column tile only the lower wave row has a rider part
    Acc accr[RX];
    Acc accr2[GATED ? RX : 1];
    const bool r_wave = TN >= 2 || wm == 0;
    const int xb = TN >= 2 ? wm * RX : 0;
    auto zero_acc_r = [&]() {
#pragma unroll
      for (int x = 0; x < RX; ++x)
#pragma unroll
        for (int q = 0; q < NACC; ++q) {
          accr[x][q] = 0.f;
          if (GATED) accr2[GATED ? x : 0][q] = 0.f;
        }
    };
    const int lr = lane % MF;
    const int lq = lane / MF;
    auto mma = [&](const bf16x8& w, const bf16x8& x, Acc& c) {
      if constexpr (MF == 32)
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, x, c, 0, 0, 0);
      else
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, x, c, 0, 0, 0);
    };
    // Operand fragments. The weight fragments of one K sub-step (TN, plus TU
    // up-projection ones) are double-buffered; the TM token-row fragments are
    // not: each is re-read for the next sub-step right after the last MFMA
    // that uses it, into the same registers.
    struct FragsB {
      bf16x8 w[TN], u[TU];
    };
    bf16x8 fy[TM];
    bf16x8 fr;   // the rider's token-row fragment
    auto read_r = [&](int buf, int ks) -> bf16x8 {
      const bf16* Rs = lds + buf * LDS_BUF + ROWS * BK;
      const int ci = ks * CPS + lq;
      return *reinterpret_cast<const bf16x8*>(Rs + lr * BK + L::swz(lr, ci) * 8);
    };
    auto read_a = [&](int buf, int ks, int y) -> bf16x8 {
      const bf16* As = lds + buf * LDS_BUF;
      const int ci = ks * CPS + lq;
      const int r = wm * WTM + y * MF + lr;
      return *reinterpret_cast<const bf16x8*>(As + r * BK + L::swz(r, ci) * 8);
    };
    auto read_b = [&](int buf, int ks, FragsB& f) {
      const bf16* Bs = lds + buf * LDS_BUF + BM * BK;
      const int ci = ks * CPS + lq;
#pragma unroll
      for (int x = 0; x < TN; ++x) {
        const int r = wn * WTN + x * MF + lr;
        f.w[x] = *reinterpret_cast<const bf16x8*>(Bs + r * BK + L::swz(r, ci) * 8);
        if (GATED) {
          const int r2 = BN + r;
          f.u[GATED ? x : 0] = *reinterpret_cast<const bf16x8*>(Bs + r2 * BK + L::swz(r2, ci) * 8);
        }
      }
    };
    // multiply one sub-step (token fragments fy, weight fragments cur); with
    // RD, read sub-step nks of buffer nbuf into fy and nxt meanwhile; a
    // tile's rider MFMAs (and rider fragment read) follow
    bool has_r = false;   // the tile being multiplied carries a rider (uniform)
    auto step = [&](auto rd, const FragsB& cur, FragsB& nxt, int nbuf, int nks) {
      constexpr bool RD = decltype(rd)::value;
      if (RD) read_b(nbuf, nks, nxt);
#pragma unroll
      for (int y = 0; y < TM; ++y) {
#pragma unroll
        for (int x = 0; x < TN; ++x) {
          mma(cur.w[x], fy[y], acc[x][y]);
          if (GATED) mma(cur.u[GATED ? x : 0], fy[y], acc2[GATED ? x : 0][y]);
        }
        if (RD) fy[y] = read_a(nbuf, nks, y);
      }
      // issue order (sched_group_barrier masks: MFMA 0x008, DS read 0x100):
      // the first token row's MFMAs each followed by one weight read, then
      // every token row's MFMAs followed by that row's re-read
      constexpr int NRB = TN + (GATED ? TU : 0);     // weight reads
      constexpr int MPY = TN * (GATED ? 2 : 1);      // MFMAs per token row
      if constexpr (RD && NRB == MPY) {
#pragma unroll
        for (int i = 0; i < NRB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int y = 1; y < TM; ++y) {
          __builtin_amdgcn_sched_group_barrier(0x008, MPY, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      if constexpr (RIDE) {
        // the rider's MFMAs and fragment read come after the sub-step's own,
        // fenced off so that they leave its issue order alone; the wave row's
        // half of the weight fragments is a select (wm is wave-uniform), not a
        // branch. Tiles with a rider are the rare case: that code sits out of
        // line.
        __builtin_amdgcn_sched_barrier(0);
        if (__builtin_expect(has_r, 0)) {
#pragma unroll
          for (int x = 0; x < RX; ++x) {
            const bf16x8 w = (TN >= 2 && wm != 0) ? cur.w[TN >= 2 ? RX + x : 0] : cur.w[x];
            mma(w, fr, accr[x]);
            if constexpr (GATED) {
              const bf16x8 u = (TN >= 2 && wm != 0) ? cur.u[TN >= 2 ? RX + x : 0] : cur.u[x];
              mma(u, fr, accr2[x]);
            }
          }
          if (RD) fr = read_r(nbuf, nks);
        }
      }
    };

    // ---- epilogue: lane holds D[n][m = lr] for n = 8*g + 4*lq + i (32x32
    // tiles, g = 0..3) or n = 4*lq + i (16x16 tiles), four consecutive
    // columns at a time
    // one 16x16 tile's four columns of this lane as bf16 (activation applied),
    // packed in two 32-bit words
    auto pack4 = [&](int x, int y, uint32_t* p) {
      bf16x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = acc[x][y][i];
        if (GATED) v = silu_f(v) * acc2[GATED ? x : 0][GATED ? y : 0][i];
        if (EPI == EPI_RELU_BF16) v = fmaxf(v, 0.0f);
        o[i] = (bf16)v;
      }
      __builtin_memcpy(p, &o, 8);
    };
    auto epilogue = [&](const GemmTile& t) {
      // bf16 outputs of 16x16 tiles, column tiles in pairs: the lane-swap
      // instruction trades the four columns that lanes of 16-lane row q hold
      // of tile x+1 (q even) against those of tile x (q odd) with the
      // neighbouring row, so that each lane holds eight consecutive columns:
      // row 0 columns 0-7 of tile x, row 1 columns 0-7 of tile x+1, rows 2
      // and 3 columns 8-15 of each. One 16-byte store then covers 16 output
      // rows by 64 bytes, half the store instructions of 8-byte stores (the
      // store burst at the end of a tile is what short-K GEMMs wait for).
      // Every lane takes part in the swaps; rows past a_rows only skip the
      // store. The values are the same conversions, so the bits are too.
      if constexpr (EPI != EPI_ROUTER_F32 && MF == 16 && TN % 2 == 0) {
#pragma unroll
        for (int y = 0; y < TM; ++y) {
          const int m = wm * WTM + y * MF + lr;
          const bool row_ok = m < t.a_rows;
          int64_t orow = t.c_row + m;
          if constexpr (EPI == EPI_SLOTS_BF16)
            orow = row_ok ? (int64_t)t.o_tok[orow] * t.o_k + t.o_slot[orow] : 0;
          bf16* out = reinterpret_cast<bf16*>(Cv) + orow * ldc;
#pragma unroll
          for (int p = 0; p < TN / 2; ++p) {
            uint32_t pa[2], pb[2];
            pack4(2 * p, y, pa);
            pack4(2 * p + 1, y, pb);
            const auto s0 = __builtin_amdgcn_permlane16_swap(pa[0], pb[0], false, false);
            const auto s1 = __builtin_amdgcn_permlane16_swap(pa[1], pb[1], false, false);
            const int n = t.n0 + wn * WTN + (2 * p + (lq & 1)) * MF + 8 * (lq >> 1);
            if (row_ok && n < N) {
              const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
              *reinterpret_cast<u32x4*>(out + n) = v;
            }
          }
        }
        return;
      }
#pragma unroll
      for (int y = 0; y < TM; ++y) {
        const int m = wm * WTM + y * MF + lr;
        if (m >= t.a_rows) continue;
        int64_t orow = t.c_row + m;
        if constexpr (EPI == EPI_SLOTS_BF16)
          orow = (int64_t)t.o_tok[orow] * t.o_k + t.o_slot[orow];
#pragma unroll
        for (int x = 0; x < TN; ++x) {
#pragma unroll
          for (int g = 0; g < NACC / 4; ++g) {
            const int n = t.n0 + wn * WTN + x * MF + (MF == 32 ? 8 * g + 4 * lq : 4 * lq);
            if constexpr (EPI == EPI_ROUTER_F32) {
              float* out = reinterpret_cast<float*>(Cv) + (t.c_row + m) * ldc;
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (n + i < n_store) out[n + i] = acc[x][y][4 * g + i] + (bias ? bias[n + i] : 0.0f);
            } else {
              if (n >= N) continue;
              bf16* out = reinterpret_cast<bf16*>(Cv) + orow * ldc;
              bf16x4 o;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                float v = acc[x][y][4 * g + i];
                if (GATED) v = silu_f(v) * acc2[GATED ? x : 0][GATED ? y : 0][4 * g + i];
                if (EPI == EPI_RELU_BF16) v = fmaxf(v, 0.0f);
                o[i] = (bf16)v;
              }
              *reinterpret_cast<bf16x4*>(out + n) = o;
            }
          }
        }
      }
    };

    // the rider's rows: lane holds D[n = 4*lq + i][m = lr] of each 16 x 16 tile
    auto epilogue_r = [&](const GemmTile& t) {
      if constexpr (RIDE) {
#pragma unroll
        for (int x = 0; x < RX; ++x) {
          const int n = t.n0 + wn * WTN + (xb + x) * MF + 4 * lq;
          if (!r_wave || lr >= t.r_rows || n >= N) continue;
          int64_t orow = t.r_crow + lr;
          if constexpr (EPI == EPI_SLOTS_BF16)
            orow = (int64_t)t.o_tok[orow] * t.o_k + t.o_slot[orow];
          bf16* out = reinterpret_cast<bf16*>(Cv) + orow * ldc;
          bf16x4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = accr[x][i];
            if constexpr (GATED) v = silu_f(v) * accr2[x][i];
            if (EPI == EPI_RELU_BF16) v = fmaxf(v, 0.0f);
            o[i] = (bf16)v;
          }
          *reinterpret_cast<bf16x4*>(out + n) = o;
        }
      }
    };

    // ---- the tile and slice loops. Global slice g sits in LDS buffer
    // g % NBUF. Fragment reads are software-pipelined across the slice
    // barrier: sub-step 1 is read while sub-step 0 is multiplied, and sub-step
    // 0 of slice g+1 is read right after the barrier that publishes it, while
    // sub-step 1 of slice g is multiplied. Slice g+NBUF is fetched into the
    // buffer slice g just left, so it has NBUF-1 slices of MFMAs to arrive
    // (NBUF-2 whole slices, and the sub-steps around the barriers).
    // sched_barrier fences keep the compiler from moving MFMAs across the
    // slice barrier, which would leave the reads before it uncovered.
    static_assert(NSUB % 2 == 0, "the loop below alternates two fragment sets");
    using Yes = std::integral_constant<bool, true>;
    using No = std::integral_constant<bool, false>;
    // Wait until slice t, which the next barrier publishes, has landed from
    // this wave: the slices issued after it (at most NBUF - 2) may stay in
    // flight. Only loads are outstanding at these waits (the epilogue's
    // stores are drained at the first barrier of the next tile), and loads
    // complete in order.
    auto wait_slice = [&](int t) {
      const int n = l_issued - 1 - t;
      if (NBUF >= 5 && n >= 3)
        wait_vmcnt<(NBUF >= 5 ? 3 * LPWR : 0)>();
      else if (NBUF >= 4 && n >= 2)
        wait_vmcnt<(NBUF >= 4 ? 2 * LPWR : 0)>();
      else if (NBUF >= 3 && n >= 1)
        wait_vmcnt<(NBUF >= 3 ? LPWR : 0)>();
      else
        wait_vmcnt<0>();
    };
    auto next_buf = [](int b) { return b + 1 == NBUF ? 0 : b + 1; };
    for (int i = 0; i < NBUF - 1; ++i) issue_next();
    wait_slice(0);
    lds_barrier();
    issue_next();
    FragsB b0, b1;
    int cb = 0;   // LDS buffer of the slice being multiplied
    int gc = 0;   // its index in the slice sequence
    // The slice loop is rotated so that its head follows a slice barrier,
    // where no LDS read is outstanding: the compiler's wait insertion is
    // exact inside a loop body but waits for everything at a loop head that
    // outstanding reads reach through the back edge.
    for (int c_idx = 0;; ++c_idx) {
      if constexpr (RIDE) has_r = ct.r_rows > 0;
      // upper wave row with no valid row of this tile (wave-uniform): it
      // skips the fragment reads, MFMAs and epilogue below (a tile with a
      // rider keeps every wave busy)
      const bool busy = has_r || !(WM == 2 && wm == 1 && ct.a_rows <= WTM);
      // the tile's first slice is in LDS buffer cb
      if (busy) {
        zero_acc();
        if (RIDE && has_r && r_wave) zero_acc_r();
        read_b(cb, 0, b0);
#pragma unroll
        for (int y = 0; y < TM; ++y) fy[y] = read_a(cb, 0, y);
        if (RIDE && has_r && r_wave) fr = read_r(cb, 0);
        // sub-steps 0 .. NSUB-2 of the first slice, each reading the next
        if constexpr (NSUB == 2) {
          step(Yes{}, b0, b1, cb, 1);
        } else {
#pragma unroll
          for (int j = 1; j < NSUB; ++j) {
            if (j & 1)
              step(Yes{}, b0, b1, cb, j);
            else
              step(Yes{}, b1, b0, cb, j);
            if (j + 1 < NSUB) __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // slice g fully read by this wave; slice g+1 landed from this wave (and
      // the previous tile's stores drained)
      wait_vmcnt<0>();
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      for (int ck = 0; ck < ct.nk - 1; ++ck) {
        const int nb = next_buf(cb);
        issue_next();                          // slice g+NBUF into the buffer g left
        if (busy) {
          step(Yes{}, b1, b0, nb, 0);          // last sub-step of g, reads g+1
          if constexpr (NSUB == 2) {
            __builtin_amdgcn_sched_barrier(0);
            step(Yes{}, b0, b1, nb, 1);        // sub-step 0 of g+1, reads its sub-step 1
          } else {
#pragma unroll
            for (int j = 1; j < NSUB; ++j) {   // sub-step j-1 of g+1, reads sub-step j
              __builtin_amdgcn_sched_barrier(0);
              if (j & 1)
                step(Yes{}, b0, b1, nb, j);
              else
                step(Yes{}, b1, b0, nb, j);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_slice(gc + 2);                    // slice g+2 landed from this wave ...
        lds_barrier();                         // ... and slice g+1 read by every wave
        __builtin_amdgcn_sched_barrier(0);
        cb = nb;
        ++gc;
      }
      // the tile's last slice; its epilogue runs while the next tile's first
      // slices load, and that tile's first fragments are read after it
      issue_next();
      if (busy) step(No{}, b1, b0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      cb = next_buf(cb);
      ++gc;
      if (busy) epilogue(ct);
      if (RIDE && has_r) epilogue_r(ct);
      // the load cursor has already looked up the tile after this one
      if (c_idx + 1 >= tiles_end) break;
      get(c_idx + 1, ct);
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
