// Grouped expert FFN over ragged groups: one launch per GEMM covers every
// local expert's rows ("Dropless MoE Is a Runtime Problem as Much as a Model
// Design", grouped GEMM paragraph: a collection of expert shapes in one
// implementation, no per-expert launches, no padding to a common capacity).
//
// The group sizes live only on the device. A one-workgroup kernel turns the
// expert offsets into a table of M-tiles (local expert, first row, end row);
// the GEMM kernels are persistent grids that walk that table, so no host
// sync and no padded rows. bf16 runs on MFMA with float32 accumulation; the
// SwiGLU gate and up products share one pass over the activation tile and
// are combined in float32 before the single bf16 rounding of `act`.
#include "gemm_core.h"

namespace moe {

int device_cu_count();

// ---------------------------------------------------------------------------
// Tile tables, one per expert GEMM: for local expert i, rows
// [offsets[lo+i], offsets[lo+i+1]) clamped to max_rows, cut into BM-row
// tiles, in expert order. Table length (the same for both) at the end,
// then one word per GEMM: the most rows any of its leftover tiles holds when
// all of them are short tiles moved there (see below), else 0.
//
// An expert's last tile is short when it holds at most BM / 2 rows; the
// GEMMs run a short tile on the lower half of their waves. The tiles past
// the last whole round of a persistent grid of G workgroups go to a second
// launch (when they fill at most half a round), cut into pieces. For each
// GEMM (n_n column tiles per M-tile, grid G; G = 0: no reordering) with
// such leftover tiles, the last k short M-tiles move to the end of its
// table, k = enough whole groups of group_m M-tiles (the GEMMs walk the
// table group_m M-tiles per column) to hold every leftover tile. That
// launch then gets cheap tiles, and so does the round before it when the
// moved tiles reach into it. Short tiles elsewhere keep their place beside
// their expert's full tiles (a layer without leftover tiles keeps the plain
// expert order).
//
// ride: an expert's short last tile of s rows instead rides on its full
// tiles, 16 rows on each of ceil(s / 16) of them per column tile (entry
// fields x and w; set_rider picks the tiles), when it has that many full
// tiles (and fewer than 2^14); it then needs no weight pass of its own.
__global__ __launch_bounds__(1024) void tile_map_kernel(const int32_t* __restrict__ offsets,
                                                        int e_lo, int E_loc, int64_t max_rows,
                                                        int BM, int4* __restrict__ tiles1,
                                                        int4* __restrict__ tiles2,
                                                        int* __restrict__ n_tiles_out, int n_n1,
                                                        int G1, int n_n2, int G2, int group_m,
                                                        uint32_t* __restrict__ flags, int ride) {
  // one thread per local expert (64 per wave); scans within a wave by
  // shuffles, across waves through LDS
  __shared__ int wsum_m[16], wsum_s[16], wmax[2][16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nw = (int)(blockDim.x >> 6);
  // local rows past max_rows are not computed: report them
  if (tid == 0 && flags && (int64_t)offsets[e_lo + E_loc] > max_rows)
    atomicOr(flags, MOE_FLAG_ROW_OVERFLOW);
  int r0 = 0, r1 = 0, mt = 0, sh = 0;
  int rb = 0, r_first = 0;   // rider row blocks, first rider row
  if (tid < E_loc) {
    r0 = (int)min((int64_t)offsets[e_lo + tid], max_rows);
    r1 = (int)min((int64_t)offsets[e_lo + tid + 1], max_rows);
    mt = r1 > r0 ? (r1 - r0 + BM - 1) / BM : 0;
    sh = (mt > 0 && r1 - r0 - (mt - 1) * BM <= BM / 2) ? 1 : 0;
    if (ride && sh && mt >= 2 && mt <= (1 << 14) - 1) {
      const int need = (r1 - r0 - (mt - 1) * BM + 15) / 16;
      if (need <= mt - 1) {
        rb = need;
        mt -= 1;
        sh = 0;
        r_first = r0 + mt * BM;
      }
    }
  }
  int im = mt, is = sh;   // inclusive scans within the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int am = __shfl_up(im, o), as = __shfl_up(is, o);
    if (lane >= o) {
      im += am;
      is += as;
    }
  }
  if (lane == 63) {
    wsum_m[wv] = im;
    wsum_s[wv] = is;
  }
  __syncthreads();
  int M = 0, S = 0;
  for (int w = 0; w < nw; ++w) {
    if (w < wv) {
      im += wsum_m[w];
      is += wsum_s[w];
    }
    M += wsum_m[w];
    S += wsum_s[w];
  }
  for (int g = 0; g < 2; ++g) {
    const int n_n = g ? n_n2 : n_n1, G = g ? G2 : G1;
    int4* tab = g ? tiles2 : tiles1;
    int k = 0, need = 0;
    if (G > 0 && M > 0) {
      const int left = (int)((int64_t)M * n_n % G);
      if (left > 0 && 2 * left <= G) {
        const int last = M - (M - 1) / group_m * group_m;   // M-tiles in the last group
        const int more = max(0, left - last * n_n);        // leftover tiles before it
        need = last + (more + group_m * n_n - 1) / (group_m * n_n) * group_m;
        k = min(S, need);
      }
    }
    // short M-tiles j = 0..S-1 in expert order; those with j >= S - k move
    const int j = is - sh;   // short M-tiles of the experts before this one
    const int mv = (sh && j >= S - k) ? 1 : 0;
    const int moved_before = max(0, j - (S - k));
    const int start = im - mt - moved_before;
    for (int m = 0; m < mt - mv; ++m) {
      const int a = r0 + m * BM;
      if (rb)
        tab[start + m] = make_int4(tid | ((r1 - r_first) << 10) | (mt << 18), a, a + BM, r_first);
      else
        tab[start + m] = make_int4(tid, a, min(a + BM, r1), 0);
    }
    int rows_mv = 0;
    if (mv) {
      tab[M - k + j - (S - k)] = make_int4(tid, r0 + (mt - 1) * BM, r1, 0);
      rows_mv = r1 - r0 - (mt - 1) * BM;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) rows_mv = max(rows_mv, __shfl_xor(rows_mv, o));
    if (lane == 0) wmax[g][wv] = (need > 0 && k == need) ? rows_mv : 0;
  }
  __syncthreads();
  if (tid == 0) {
    n_tiles_out[0] = M;
    for (int g = 0; g < 2; ++g) {
      int r = 0;
      for (int w = 0; w < nw; ++w) r = max(r, wmax[g][w]);
      n_tiles_out[1 + g] = r;
    }
  }
}

// ---------------------------------------------------------------------------
// One tile-table entry (uniform), read with a scalar load. The persistent
// loops look it up right after a slice barrier or after an epilogue, where
// no LDS read is outstanding, so waiting for the scalar load costs only its
// own latency; a vector load would also wait for every slice load in flight.
// Entry fields: x = local expert | s << 10 | m << 18, y = first row, z = end
// row, w = first row past the expert's full tiles. s > 0: the expert's last
// s rows (s <= 128) ride on its m full tiles (see tile_map_kernel).
__device__ __forceinline__ int4 tile_entry(const int4* __restrict__ tiles, int mt) {
  using CInt = const __attribute__((address_space(4))) int;
  CInt* p = (CInt*)tiles + 4 * mt;
  return make_int4(p[0], p[1], p[2], p[3]);
}

__device__ __forceinline__ int entry_expert(const int4& e) { return e.x & 0x3ff; }

// The rider of full tile e in column tile nt, for A (gathered: rows) with row
// stride K: the expert's s remainder rows form rb = ceil(s / 16) blocks of 16,
// and in column tile nt block i rides on the expert's full tile
// (i + rb * (nt + nt / S)) mod m. A workgroup of the persistent walk keeps
// its place in the M-tile group from round to round while its column tile
// moves on by S (the grid's column tiles per round), so the nt / S term
// shifts the rb riding tiles by rb places from round to round, and no
// workgroup carries a rider in every round.
template <bool GA, int BM>
__device__ __forceinline__ void set_rider(GemmTile& t, const int4& e, int nt, int S,
                                          const bf16* A, const int32_t* rows, int K) {
  t.r_rows = 0;
  const int s = (e.x >> 10) & 0xff;
  if (s == 0) return;
  const int m = (int)((uint32_t)e.x >> 18);
  const int rb = (s + 15) / 16;
  const int ml = m - (e.w - e.y) / BM;    // this tile's index among the m
  int i = (ml - rb * (nt % m + nt / S % m) % m) % m;
  if (i < 0) i += m;
  if (i >= rb) return;
  t.r_rows = min(16, s - 16 * i);
  t.r_crow = e.w + 16 * i;
  t.ra = GA ? A : A + t.r_crow * K;
  t.rrows = GA ? rows + t.r_crow : nullptr;
}

// Tiles that do not fill a whole round of the persistent grid: when they
// would occupy at most half of it, the main kernel stops after the whole
// rounds and a second launch runs each leftover tile cut into pieces (rows
// and columns, or columns only for short tiles), which keeps more CUs busy.
// Cutting by rows and columns leaves every output's K accumulation order
// unchanged, so results do not depend on it.
constexpr int cmax(int a, int b, int c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }

__device__ __forceinline__ int main_tile_end(int total, int G) {
  const int full = total / G * G;
  const int tail = total - full;
  return (tail > 0 && 2 * tail <= G) ? full : total;
}

// GA (gathered A): A row i of the grouped operand is row rows[i] of A, so the
// token rows need not be copied into expert order first (the fused layer
// call's dispatch); otherwise A is the expert-ordered matrix itself.
template <int BM, int BN, int WM, int WN, int EPI, int BK, int GROUP_M, int MF, bool GA,
          bool RIDE>
__global__ __launch_bounds__(64 * WM * WN) void grouped_gemm_dl_kernel(
    const bf16* __restrict__ A, const int32_t* __restrict__ rows, const bf16* __restrict__ W,
    bf16* __restrict__ C, const int4* __restrict__ tiles, const int* __restrict__ n_mt_ptr,
    int N, int K, int64_t w_stride, int n_n, int64_t ldc, const int32_t* __restrict__ o_tok,
    const int32_t* __restrict__ o_slot, int o_k) {
  // two slice buffers, or three where they fit in the 160 KiB of LDS (the
  // 128-wide tile without the gated pair: 48 KiB slices, so a third one
  // gives each slice two slices of MFMAs to arrive)
  using TG2 = TileGemmDL<BM, BN, WM, WN, EPI, BK, MF, GA, 2, RIDE>;
  using TG = TileGemmDL<BM, BN, WM, WN, EPI, BK, MF, GA,
                        TG2::LDS_BUF * 2 * 3 <= 160 * 1024 ? 3 : 2, RIDE>;
  __shared__ __attribute__((aligned(1024))) bf16 lds[TG::LDS_ELEMS];
  const int n_m = *n_mt_ptr;
  const int G = gridDim.x;
  const int end = main_tile_end(n_m * n_n, G);
  const int nk = K / BK;
  // this workgroup's i-th tile, in XCD-major, GROUP_M-grouped order
  auto get = [&](int i, GemmTile& t) -> bool {
    const int v = xcd_virtual_id(blockIdx.x, G, i);
    if (v >= end) return false;
    int mt, nt;
    tile_coords<GROUP_M>(v, n_m, n_n, mt, nt);
    const int4 e = tile_entry(tiles, mt);
    const int ex = entry_expert(e), ey = e.y, ez = e.z;
    t.a = GA ? A : A + (int64_t)ey * K;
    t.rows = GA ? rows + ey : nullptr;
    t.a_rows = ez - ey;
    t.n0 = nt * BN;
    t.b = W + (int64_t)ex * w_stride + (int64_t)t.n0 * K;
    t.c_row = ey;
    t.nk = nk;
    t.o_tok = o_tok;
    t.o_slot = o_slot;
    t.o_k = o_k;
    if constexpr (RIDE) set_rider<GA, BM>(t, e, nt, max(1, G / GROUP_M), A, rows, K);
    return true;
  };
  TG::run_tiles(get, N, K, C, ldc, lds);
}

// The leftover tiles of the kernel above (same tile table, same order),
// each cut into S = SM * SN pieces of BM / SM rows by BN / SN columns: unit
// u is piece u % S of tile main_tile_end + u / S. One piece per workgroup.
// A piece has few MFMAs per K slice (fewer still on a short tile), so its
// loop waits on memory rather than on the MFMAs: it keeps as many slice
// buffers (up to five, four slices in flight) as fit in the 160 KiB of LDS.
template <int SM, int SN, int BM, int BN, int WM, int WN, int EPI, int BK, int GROUP_M, int MF,
          bool GA, bool RIDE>
struct TailPieces {
  static constexpr int HM = BM / SM, HN = BN / SN, S = SM * SN;
  static constexpr int BUF_BYTES =
      TileGemmDL<HM, HN, WM, WN, EPI, BK, MF, GA, 2, RIDE>::LDS_BUF * 2;
  static constexpr int NB = 160 * 1024 / BUF_BYTES;
  using TG = TileGemmDL<HM, HN, WM, WN, EPI, BK, MF, GA, NB >= 5 ? 5 : NB < 2 ? 2 : NB, RIDE>;
  __device__ __forceinline__ static void run(const bf16* A, const int32_t* rows, const bf16* W,
                                             bf16* C, const int4* tiles, int n_m, int first,
                                             int left, int N, int K, int64_t w_stride, int n_n,
                                             int64_t ldc, const int32_t* o_tok,
                                             const int32_t* o_slot, int o_k, bf16* lds) {
    const int units = S * left;
    const int nk = K / BK;
    const int slot = xcd_virtual_id(blockIdx.x, gridDim.x, 0);
    auto get = [&](int i, GemmTile& t) -> bool {
      // units <= gridDim.x; pieces that fall entirely past the tile's rows
      // or the weight's columns are skipped
      for (int u = slot + i * (int)gridDim.x; u < units; u += gridDim.x) {
        int mt, nt;
        tile_coords<GROUP_M>(first + u / S, n_m, n_n, mt, nt);
        const int part = u % S;
        const int4 e = tile_entry(tiles, mt);
        const int ex = entry_expert(e), ey = e.y + (part % SM) * HM, ez = e.z;
        if (ey >= ez) continue;
        const int n0 = nt * BN + (part / SM) * HN;
        if (n0 >= N) continue;
        t.a = GA ? A : A + (int64_t)ey * K;
        t.rows = GA ? rows + ey : nullptr;
        t.a_rows = min(ez - ey, HM);
        t.n0 = n0;
        t.b = W + (int64_t)ex * w_stride + (int64_t)n0 * K;
        t.c_row = ey;
        t.nk = nk;
        t.o_tok = o_tok;
        t.o_slot = o_slot;
        t.o_k = o_k;
        // a tile's rider goes with its first row piece of each column piece
        if constexpr (RIDE) {
          if (part % SM == 0)
            set_rider<GA, BM>(t, e, nt, max(1, (int)gridDim.x / GROUP_M), A, rows, K);
          else
            t.r_rows = 0;
        }
        return true;
      }
      return false;
    };
    TG::run_tiles(get, N, K, C, ldc, lds);
  }
};

// Leftover tiles that are all short, with at most HMQ rows each (HMQ = BM/4
// or BM/2): each is cut by columns only into SN pieces of HMQ rows by BN / SN
// columns (unit u is column piece u % SN of tile main_tile_end + u / SN), so
// no piece is empty and fewer duplicate token rows are staged. These pieces
// stream weight slices with little math; spreading them over more CUs and
// XCDs is what makes them fast (deeper buffering beyond five slices is not).
template <int HMQ, int SN, int BM, int BN, int WM, int WN, int EPI, int BK, int GROUP_M, int MF,
          bool GA>
struct TailShort {
  static constexpr int HN = BN / SN;
  static constexpr bool VALID = HN % (WN * MF) == 0;   // every wave keeps an MFMA column tile
  static constexpr int BUF_BYTES =
      TileGemmDL<HMQ, VALID ? HN : WN * MF, WM, WN, EPI, BK, MF, GA, 2>::LDS_BUF * 2;
  static constexpr int NB = 160 * 1024 / BUF_BYTES;
  using TG = TileGemmDL<HMQ, VALID ? HN : WN * MF, WM, WN, EPI, BK, MF, GA,
                        NB >= 5 ? 5 : NB < 2 ? 2 : NB>;
  __device__ __forceinline__ static void run(const bf16* A, const int32_t* rows, const bf16* W,
                                             bf16* C, const int4* tiles, int n_m, int first,
                                             int left, int N, int K, int64_t w_stride, int n_n,
                                             int64_t ldc, const int32_t* o_tok,
                                             const int32_t* o_slot, int o_k, bf16* lds,
                                             bool nt_w) {
    if constexpr (VALID) {
      const int units = SN * left;
      const int nk = K / BK;
      // consecutive units on consecutive workgroups, which the hardware deals
      // round-robin to the XCDs: the pieces share little, so they should
      // spread over every XCD's L2 and memory path rather than fill a few
      const int slot = blockIdx.x;
      auto get = [&](int i, GemmTile& t) -> bool {
        for (int u = slot + i * (int)gridDim.x; u < units; u += gridDim.x) {
          int mt, nt;
          tile_coords<GROUP_M>(first + u / SN, n_m, n_n, mt, nt);
          const int4 e = tile_entry(tiles, mt);   // a short tile: no rider
          const int n0 = nt * BN + (u % SN) * HN;
          if (n0 >= N) continue;
          t.a = GA ? A : A + (int64_t)e.y * K;
          t.rows = GA ? rows + e.y : nullptr;
          t.a_rows = min(e.z - e.y, HMQ);
          t.n0 = n0;
          t.b = W + (int64_t)entry_expert(e) * w_stride + (int64_t)n0 * K;
          t.c_row = e.y;
          t.nk = nk;
          t.o_tok = o_tok;
          t.o_slot = o_slot;
          t.o_k = o_k;
          t.nt_w = nt_w;
          return true;
        }
        return false;
      };
      TG::run_tiles(get, N, K, C, ldc, lds);
    }
  }
};

// The leftover tiles with the finest split S in {2, 4, 8} for which
// S * leftover <= G (G: the main kernel's grid size, also this grid's).
// Splitting by rows and columns leaves every output's K order unchanged.
template <int BM, int BN, int WM, int WN, int EPI, int BK, int GROUP_M, int MF, bool GA,
          bool RIDE>
__global__ __launch_bounds__(64 * WM * WN) void grouped_gemm_tail_kernel(
    const bf16* __restrict__ A, const int32_t* __restrict__ rows, const bf16* __restrict__ W,
    bf16* __restrict__ C, const int4* __restrict__ tiles, const int* __restrict__ n_mt_ptr,
    int N, int K, int64_t w_stride, int n_n, int64_t ldc, const int32_t* __restrict__ o_tok,
    const int32_t* __restrict__ o_slot, int o_k, int G, const int* __restrict__ short_rows,
    int nt_w) {
  using P2 = TailPieces<2, 1, BM, BN, WM, WN, EPI, BK, GROUP_M, MF, GA, RIDE>;
  using P4 = TailPieces<2, 2, BM, BN, WM, WN, EPI, BK, GROUP_M, MF, GA, RIDE>;
  using P8 = TailPieces<4, 2, BM, BN, WM, WN, EPI, BK, GROUP_M, MF, GA, RIDE>;
  // all-short leftovers: 64- or 128-row pieces, column quarters, halves or whole
  using Q4 = TailShort<BM / 4, 4, BM, BN, WM, WN, EPI, BK, GROUP_M, MF, GA>;
  using Q2 = TailShort<BM / 4, 2, BM, BN, WM, WN, EPI, BK, GROUP_M, MF, GA>;
  using Q1 = TailShort<BM / 4, 1, BM, BN, WM, WN, EPI, BK, GROUP_M, MF, GA>;
  using H4 = TailShort<BM / 2, 4, BM, BN, WM, WN, EPI, BK, GROUP_M, MF, GA>;
  using H2 = TailShort<BM / 2, 2, BM, BN, WM, WN, EPI, BK, GROUP_M, MF, GA>;
  using H1 = TailShort<BM / 2, 1, BM, BN, WM, WN, EPI, BK, GROUP_M, MF, GA>;
  // 64-row pieces with K slices twice as deep: half the barriers per K, which
  // helps the few short pieces of a small layer; the gathered-row path keeps
  // its own slice depth
  constexpr int BKW = GA ? BK : 2 * BK;
  using W4 = TailShort<BM / 4, 4, BM, BN, WM, WN, EPI, BKW, GROUP_M, MF, GA>;
  using W2 = TailShort<BM / 4, 2, BM, BN, WM, WN, EPI, BKW, GROUP_M, MF, GA>;
  using W1 = TailShort<BM / 4, 1, BM, BN, WM, WN, EPI, BKW, GROUP_M, MF, GA>;
  constexpr int ELEMS = cmax(cmax(P2::TG::LDS_ELEMS, P4::TG::LDS_ELEMS, P8::TG::LDS_ELEMS),
                             cmax(cmax(Q4::TG::LDS_ELEMS, Q2::TG::LDS_ELEMS, Q1::TG::LDS_ELEMS),
                                  cmax(W4::TG::LDS_ELEMS, W2::TG::LDS_ELEMS, W1::TG::LDS_ELEMS),
                                  0),
                             cmax(H4::TG::LDS_ELEMS, H2::TG::LDS_ELEMS, H1::TG::LDS_ELEMS));
  __shared__ __attribute__((aligned(1024))) bf16 lds[ELEMS];
  const int n_m = *n_mt_ptr;
  const int total = n_m * n_n;
  const int first = main_tile_end(total, G);
  const int left = total - first;
  if (left == 0) return;
  const int srows = short_rows ? *short_rows : 0;
  if (srows > 0) {
    // the finest valid column split with a piece per workgroup
    const bool quarter = srows <= BM / 4;
    const bool deep = !GA && K % BKW == 0;
    if (quarter && deep) {
      if (W4::VALID && 4 * left <= G)
        W4::run(A, rows, W, C, tiles, n_m, first, left, N, K, w_stride, n_n, ldc, o_tok, o_slot,
                o_k, lds,
                nt_w != 0);
      else if (W2::VALID)
        W2::run(A, rows, W, C, tiles, n_m, first, left, N, K, w_stride, n_n, ldc, o_tok, o_slot,
                o_k, lds,
                nt_w != 0);
      else
        W1::run(A, rows, W, C, tiles, n_m, first, left, N, K, w_stride, n_n, ldc, o_tok, o_slot,
                o_k, lds,
                nt_w != 0);
    } else if (Q4::VALID && 4 * left <= G) {
      if (quarter)
        Q4::run(A, rows, W, C, tiles, n_m, first, left, N, K, w_stride, n_n, ldc, o_tok, o_slot,
                o_k, lds,
                nt_w != 0);
      else
        H4::run(A, rows, W, C, tiles, n_m, first, left, N, K, w_stride, n_n, ldc, o_tok, o_slot,
                o_k, lds,
                nt_w != 0);
    } else if (Q2::VALID) {
      if (quarter)
        Q2::run(A, rows, W, C, tiles, n_m, first, left, N, K, w_stride, n_n, ldc, o_tok, o_slot,
                o_k, lds,
                nt_w != 0);
      else
        H2::run(A, rows, W, C, tiles, n_m, first, left, N, K, w_stride, n_n, ldc, o_tok, o_slot,
                o_k, lds,
                nt_w != 0);
    } else if (quarter) {
      Q1::run(A, rows, W, C, tiles, n_m, first, left, N, K, w_stride, n_n, ldc, o_tok, o_slot,
              o_k, lds,
                nt_w != 0);
    } else {
      H1::run(A, rows, W, C, tiles, n_m, first, left, N, K, w_stride, n_n, ldc, o_tok, o_slot,
              o_k, lds,
                nt_w != 0);
    }
  } else if (8 * left <= G)
    P8::run(A, rows, W, C, tiles, n_m, first, left, N, K, w_stride, n_n, ldc, o_tok, o_slot, o_k,
            lds);
  else if (4 * left <= G)
    P4::run(A, rows, W, C, tiles, n_m, first, left, N, K, w_stride, n_n, ldc, o_tok, o_slot, o_k,
            lds);
  else
    P2::run(A, rows, W, C, tiles, n_m, first, left, N, K, w_stride, n_n, ldc, o_tok, o_slot, o_k,
            lds);
}

// Persistent grid of the bf16 expert GEMMs: per_cu workgroups per CU, at
// most the tile count's upper bound, a multiple of 8 (one share per XCD).
static int gemm_grid(int64_t max_mtiles, int n_n, int per_cu) {
  const int64_t ub = max_mtiles * n_n;
  const int64_t G = min(((ub + 7) / 8) * 8, (int64_t)device_cu_count() * per_cu);
  return (int)max((int64_t)8, G / 8 * 8);
}

template <int BM, int BN, int WM, int WN, int EPI, int BK, int GROUP_M, int MF, bool GA = false,
          bool RIDE = true>
static hipError_t grouped_gemm_dl_launch(const bf16* A, const int32_t* rows, const bf16* W,
                                         bf16* C, const int4* tiles, const int* n_mt, int N,
                                         int K, int64_t w_stride, int64_t ldc,
                                         int64_t max_mtiles, int per_cu, hipStream_t s,
                                         const int* short_rows, bool nt_w,
                                         const int32_t* o_tok = nullptr,
                                         const int32_t* o_slot = nullptr, int o_k = 0) {
  const int n_n = (N + BN - 1) / BN;
  const int G = gemm_grid(max_mtiles, n_n, per_cu);
  hipLaunchKernelGGL((grouped_gemm_dl_kernel<BM, BN, WM, WN, EPI, BK, GROUP_M, MF, GA, RIDE>),
                     dim3((unsigned)G), dim3(64 * WM * WN), 0, s, A, rows, W, C, tiles, n_mt, N,
                     K, w_stride, n_n, ldc, o_tok, o_slot, o_k);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((grouped_gemm_tail_kernel<BM, BN, WM, WN, EPI, BK, GROUP_M, MF, GA, RIDE>),
                     dim3((unsigned)G), dim3(64 * WM * WN), 0, s, A, rows, W, C, tiles, n_mt, N,
                     K, w_stride, n_n, ldc, o_tok, o_slot, o_k, (int)G, short_rows, (int)nt_w);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// float32 grouped GEMM (small layers): 64x64 output tiles, 256 threads each
// computing a 4x4 block, K in slices of 16 through LDS. Epilogue 0 = store,
// 1 = ReLU, 2 = SwiGLU (gate rows n, up rows N + n).
constexpr int kF32BM = 64;

template <int EPI>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ a_rows, const float* __restrict__ W,
    float* __restrict__ C, const int4* __restrict__ tiles, const int* __restrict__ n_mt_ptr,
    int N, int K, int64_t w_stride, int64_t ldc, const int32_t* __restrict__ o_tok,
    const int32_t* __restrict__ o_slot, int o_k) {
  const int mt = blockIdx.x;
  if (mt >= *n_mt_ptr) return;
  const int4 t = tiles[mt];
  const int rows = t.z - t.y;
  const int n0 = blockIdx.y * 64;
  const float* Wb = W + (int64_t)t.x * w_stride;
  __shared__ float As[16][65], Bs[16][65], Us[16][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {}, accu[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int q = threadIdx.x; q < 64 * 16; q += 256) {
      int r = q >> 4, kk = q & 15;
      int k = k0 + kk;
      const int64_t ar = r < rows ? (a_rows ? a_rows[t.y + r] : t.y + r) : 0;
      As[kk][r] = (r < rows && k < K) ? A[ar * K + k] : 0.f;
      int n = n0 + r;
      Bs[kk][r] = (n < N && k < K) ? Wb[(int64_t)n * K + k] : 0.f;
      if (EPI == 2) Us[kk][r] = (n < N && k < K) ? Wb[(int64_t)(N + n) * K + k] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4], u[4];
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
      if (EPI == 2)
        for (int j = 0; j < 4; ++j) u[j] = Us[kk][tx * 4 + j];
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
          if (EPI == 2) accu[i][j] = fmaf(a[i], u[j], accu[i][j]);
        }
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i) {
    int m = ty * 4 + i;
    if (m >= rows) continue;
    // o_tok: output row of grouped row r is the row of its (token, slot) pair
    const int64_t r = t.y + m;
    const int64_t orow = o_tok ? (int64_t)o_tok[r] * o_k + o_slot[r] : r;
    for (int j = 0; j < 4; ++j) {
      int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float v = acc[i][j];
      if (EPI == 1) v = fmaxf(v, 0.f);
      if (EPI == 2) v = v / (1.0f + expf(-v)) * accu[i][j];
      C[orow * ldc + n] = v;
    }
  }
}

template <int EPI>
static hipError_t grouped_gemm_f32_launch(const float* A, const int32_t* a_rows, const float* W,
                                          float* C, const int4* tiles, const int* n_mt, int N,
                                          int K, int64_t w_stride, int64_t ldc,
                                          int64_t max_mtiles, hipStream_t s,
                                          const int32_t* o_tok = nullptr,
                                          const int32_t* o_slot = nullptr, int o_k = 0) {
  dim3 grid((unsigned)max_mtiles, (unsigned)((N + 63) / 64));
  hipLaunchKernelGGL(grouped_gemm_f32_kernel<EPI>, grid, dim3(256), 0, s, A, a_rows, W, C, tiles,
                     n_mt, N, K, w_stride, ldc, o_tok, o_slot, o_k);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16 expert GEMMs: 256-row M tiles, 8 waves (2 x 4), each wave a 128 x 64
// block of 16x16x32 MFMAs; K slices of 64 stream into LDS by direct loads.
// GEMM1 (SwiGLU) stages 128 gate + 128 up weight rows per tile and writes
// 128 activation columns; GEMM2 stages 256 weight rows (128 for small layers,
// where wave tiles are 128 x 32). Tiles are walked
// 8 M-tiles per N column (GROUP_M = 8) in XCD-major order.
constexpr int kGemmBM = 256;
constexpr int kGemmGroupM = 8;

int64_t gemm_max_mtiles(const moe_layer_desc_t& d) {
  const int64_t el = d.E / d.ep_size;
  const int64_t rows = d.max_rows;
  return (rows + kF32BM - 1) / kF32BM + el;  // the smallest BM of any path
}

// threads of the tile-map launch: one per local expert, whole waves
static unsigned tile_map_threads(int el) { return 64u * (unsigned)((max(el, 1) + 63) / 64); }

// x_perm: the expert-ordered rows, or (gathered, rows != null) the token rows
// h, read through rows = src_token. o_tok == null: grouped row r of the output
// goes to row r of y_perm; otherwise to row o_tok[r] * k + o_slot[r].
hipError_t launch_grouped_ffn(const moe_layer_desc_t& desc, const void* x_perm,
                              const int32_t* rows, const int32_t* offsets, const void* w1,
                              const void* w2, void* y_perm, void* act, int4* tiles,
                              uint32_t* flags, hipStream_t s, const int32_t* o_tok,
                              const int32_t* o_slot) {
  const int el = desc.E / desc.ep_size;
  const int e_lo = desc.ep_rank * el;
  const int64_t max_mt = gemm_max_mtiles(desc);
  int4* tiles2 = tiles + max_mt;   // the down GEMM's tile table
  int* n_mt = reinterpret_cast<int*>(tiles + 2 * max_mt);
  const int d = desc.d, dff = desc.d_ff;
  const bool swiglu = desc.act == MOE_ACT_SWIGLU;
  const int w1_rows = swiglu ? 2 * dff : dff;
  hipError_t err;
  if (desc.dtype == MOE_DTYPE_BF16) {
    const int64_t mt_ub = (desc.max_rows + kGemmBM - 1) / kGemmBM + el;
    const int n_n1 = (dff + (swiglu ? 127 : 255)) / (swiglu ? 128 : 256);   // GEMM1 BN
    // down GEMM column tiles: 256 wide, or 128 wide when even the most tiles
    // the layer can have (from max_rows, not from the routing) would leave
    // part of one round of the grid idle; the K order of every output is the
    // same either way
    const bool narrow2 = mt_ub * ((d + 255) / 256) < device_cu_count();
    // The leftover launches stream the weights of short tiles once. When the
    // local experts' weights cannot stay in the 256 MiB last-level cache
    // between layers anyway, those loads go non-temporal, so that they leave
    // the down GEMM's output there for the combine; smaller layers keep their
    // weights cached.
    const int64_t w_bytes = (int64_t)el * (w1_rows + dff) * d * 2;   // W1 and W2 per expert
    const bool nt_w = w_bytes > (int64_t)256 << 20;
    const int n_n2 = narrow2 ? (d + 127) / 128 : (d + 255) / 256;
    hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(tile_map_threads(el)), 0, s, offsets,
                       e_lo, el, desc.max_rows, kGemmBM, tiles, tiles2, n_mt, n_n1,
                       gemm_grid(mt_ub, n_n1, 1), n_n2, gemm_grid(mt_ub, n_n2, 1), kGemmGroupM,
                       flags, 1);
    const bf16* X = (const bf16*)x_perm;
    const bf16* W1 = (const bf16*)w1;
    bf16* H = (bf16*)act;
    const int64_t s1 = (int64_t)w1_rows * d;
    if (swiglu && rows)
      err = grouped_gemm_dl_launch<kGemmBM, 128, 2, 4, EPI_SWIGLU_BF16, 64, kGemmGroupM, 16, true>(
          X, rows, W1, H, tiles, n_mt, dff, d, s1, dff, mt_ub, 1, s, n_mt + 1, nt_w);
    else if (swiglu)
      err = grouped_gemm_dl_launch<kGemmBM, 128, 2, 4, EPI_SWIGLU_BF16, 64, kGemmGroupM, 16>(
          X, nullptr, W1, H, tiles, n_mt, dff, d, s1, dff, mt_ub, 1, s, n_mt + 1, nt_w);
    else if (rows)
      err = grouped_gemm_dl_launch<kGemmBM, 256, 2, 4, EPI_RELU_BF16, 64, kGemmGroupM, 16, true>(
          X, rows, W1, H, tiles, n_mt, dff, d, s1, dff, mt_ub, 1, s, n_mt + 1, nt_w);
    else
      err = grouped_gemm_dl_launch<kGemmBM, 256, 2, 4, EPI_RELU_BF16, 64, kGemmGroupM, 16>(
          X, nullptr, W1, H, tiles, n_mt, dff, d, s1, dff, mt_ub, 1, s, n_mt + 1, nt_w);
    if (err != hipSuccess) return err;
    const bf16* W2 = (const bf16*)w2;
    bf16* Y = (bf16*)y_perm;
    const int64_t s2 = (int64_t)d * dff;
    if (o_tok && narrow2)
      return grouped_gemm_dl_launch<kGemmBM, 128, 2, 4, EPI_SLOTS_BF16, 64, kGemmGroupM, 16>(
          H, nullptr, W2, Y, tiles2, n_mt, d, dff, s2, d, mt_ub, 1, s, n_mt + 2, nt_w, o_tok, o_slot,
          desc.k);
    if (o_tok)
      return grouped_gemm_dl_launch<kGemmBM, 256, 2, 4, EPI_SLOTS_BF16, 64, kGemmGroupM, 16>(
          H, nullptr, W2, Y, tiles2, n_mt, d, dff, s2, d, mt_ub, 1, s, n_mt + 2, nt_w, o_tok, o_slot,
          desc.k);
    if (narrow2)
      return grouped_gemm_dl_launch<kGemmBM, 128, 2, 4, EPI_STORE_BF16, 64, kGemmGroupM, 16>(
          H, nullptr, W2, Y, tiles2, n_mt, d, dff, s2, d, mt_ub, 1, s, n_mt + 2, nt_w);
    return grouped_gemm_dl_launch<kGemmBM, 256, 2, 4, EPI_STORE_BF16, 64, kGemmGroupM, 16>(
        H, nullptr, W2, Y, tiles2, n_mt, d, dff, s2, d, mt_ub, 1, s, n_mt + 2, nt_w);
  }
  hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(tile_map_threads(el)), 0, s, offsets, e_lo,
                     el, desc.max_rows, kF32BM, tiles, tiles2, n_mt, 0, 0, 0, 0, 1, flags, 0);
  const float* X = (const float*)x_perm;
  float* H = (float*)act;
  if (swiglu)
    err = grouped_gemm_f32_launch<2>(X, rows, (const float*)w1, H, tiles, n_mt, dff, d,
                                     (int64_t)w1_rows * d, dff, max_mt, s);
  else
    err = grouped_gemm_f32_launch<1>(X, rows, (const float*)w1, H, tiles, n_mt, dff, d,
                                     (int64_t)w1_rows * d, dff, max_mt, s);
  if (err != hipSuccess) return err;
  return grouped_gemm_f32_launch<0>(H, nullptr, (const float*)w2, (float*)y_perm, tiles, n_mt, d,
                                    dff, (int64_t)d * dff, d, max_mt, s, o_tok, o_slot, desc.k);
}

}  // namespace moe
