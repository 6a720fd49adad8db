// Permute plan, row permute and unpermute + combine.
//
// The plan follows "MoE Token Dispatch: Why an All-Reduce Result Does Not
// Describe the Exchange", section "Follow one documented dispatch and return
// path" (per-expert counts and communication splits from the routing map,
// tokens rearranged into per-expert groups, outputs restored to their
// origin) and the capacity rule of "How does dropless MoE dispatch differ
// from capacity factor token dropping?" (section "Why per-expert buffers
// exist in expert-parallel training"): an expert keeps at most `capacity`
// assignments; the repeatability page has capacity resolved in request
// order, read here as ascending (token, slot) order.
//
// Everything stays on the device: a tile histogram, one scan workgroup, a
// stable in-tile rank by wave ballots, then bandwidth-bound row copies. All
// integer results are independent of scheduling (the only atomics are
// integer counts and flag ORs).
#include <algorithm>

#include "common.h"

namespace moe {

// ---------------------------------------------------------------------------
// 1. Per-tile expert histogram of the (token, slot) assignments.
__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx,
                                                   int32_t* __restrict__ tile_hist, int64_t T,
                                                   int E, int k, uint32_t* __restrict__ flags) {
  __shared__ int32_t h[kMaxE];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t a0 = (int64_t)blockIdx.x * kTokTile * k;
  const int64_t a1 = min(T * k, a0 + (int64_t)kTokTile * k);
  bool bad = false;
  for (int64_t a = a0 + threadIdx.x; a < a1; a += 256) {
    int e = idx[a];
    if (e >= 0 && e < E)
      atomicAdd(&h[e], 1);
    else
      bad = true;
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flags, MOE_FLAG_BAD_EXPERT_ID);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) tile_hist[(int64_t)blockIdx.x * E + e] = h[e];
}

// ---------------------------------------------------------------------------
// 2. One workgroup: tile counts -> exclusive prefix over tiles (in place),
//    counts, capacity, offsets, expert-parallel splits, flags.
//    Each expert's tiles are split into P parts so all 1024 threads work.
__global__ __launch_bounds__(1024) void scan_kernel(
    int32_t* __restrict__ tile_hist, int n_tiles, int E, int64_t capacity, int64_t max_rows,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int64_t* __restrict__ send_splits, int64_t* __restrict__ send_displs, int ep_size,
    uint32_t* __restrict__ flags) {
  __shared__ int32_t part[1024];
  __shared__ int32_t kept[1024];
  __shared__ int32_t any_drop;
  const int tid = threadIdx.x;
  const int P = 1024 / E;  // parts per expert (E <= 1024)
  const int e = tid % E, p = tid / E;
  const bool worker = p < P;
  const int per = (n_tiles + P - 1) / P;
  const int t0 = min(n_tiles, p * per), t1 = min(n_tiles, t0 + per);
  if (tid == 0) any_drop = 0;
  // each worker's column slice is read in batches of independent loads
  constexpr int kB = 16;
  int32_t s = 0;
  if (worker) {
    for (int t = t0; t < t1; t += kB) {
      int32_t v[kB];
#pragma unroll
      for (int i = 0; i < kB; ++i) v[i] = t + i < t1 ? tile_hist[(int64_t)(t + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kB; ++i) s += v[i];
    }
  }
  part[tid] = s;
  __syncthreads();
  int32_t base = 0;
  if (worker) {
    for (int q = 0; q < p; ++q) base += part[q * E + e];
    int32_t run = base;
    for (int t = t0; t < t1; t += kB) {
      int32_t v[kB];
#pragma unroll
      for (int i = 0; i < kB; ++i) v[i] = t + i < t1 ? tile_hist[(int64_t)(t + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        if (t + i < t1) tile_hist[(int64_t)(t + i) * E + e] = run;
        run += v[i];
      }
    }
  }
  // totals per expert, from the last part's prefix + its own sum
  if (worker && p == P - 1) {
    int32_t total = base + s;
    counts[e] = total;
    int32_t kp = (capacity >= 0 && (int64_t)total > capacity) ? (int32_t)capacity : total;
    if (kp < total) any_drop = 1;
    kept[e] = kp;
  }
  __syncthreads();
  // exclusive scan of kept over experts (Hillis-Steele, E <= 1024)
  int32_t v = tid < E ? kept[tid] : 0;
  part[tid] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    int32_t add = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  if (tid < E) offsets[tid] = part[tid] - v;
  if (tid == E - 1) {
    offsets[E] = part[tid];
    uint32_t f = 0;
    if (any_drop) f |= MOE_FLAG_DROPPED;
    if ((int64_t)part[tid] > max_rows) f |= MOE_FLAG_ROW_OVERFLOW;
    if (f) atomicOr(flags, f);
  }
  __syncthreads();
  if (tid < ep_size) {
    const int el = E / ep_size;
    int32_t lo = tid * el == 0 ? 0 : part[tid * el - 1];
    int32_t hi = part[(tid + 1) * el - 1];
    send_displs[tid] = lo;
    send_splits[tid] = hi - lo;
  }
}

// ---------------------------------------------------------------------------
// 3. Stable rank inside each tile. The tile's assignments are cut into
//    kRankWaves consecutive blocks, one per wave. Each wave first counts its
//    block per expert (LDS integer atomics), so every wave knows where its
//    block starts within each expert: the prefix over earlier tiles plus the
//    counts of the blocks before it. Then each wave ranks its block 64
//    assignments at a time in (token, slot) order: lanes holding the same
//    expert find each other by matching the expert id bit by bit with
//    ballots; a lane's rank is the number of matching lanes below it, added
//    to the expert's running position (updated by the highest matching lane).
constexpr int kRankWaves = 4;
__global__ __launch_bounds__(64 * kRankWaves) void rank_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ tile_prefix,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ dest,
    int32_t* __restrict__ src_token, int32_t* __restrict__ src_slot, int64_t T, int E, int k,
    int ebits, int64_t capacity, int64_t max_rows) {
  __shared__ int32_t run[kRankWaves][kMaxE];
  __shared__ int32_t off[kMaxE];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int q = 0; q < kRankWaves; ++q)
    for (int e = threadIdx.x; e < E; e += 64 * kRankWaves) run[q][e] = 0;
  for (int e = threadIdx.x; e < E; e += 64 * kRankWaves) off[e] = offsets[e];
  const int64_t t0 = (int64_t)blockIdx.x * kTokTile * k;
  const int64_t t1 = min(T * k, t0 + (int64_t)kTokTile * k);
  // this wave's block: a whole number of 64-assignment steps
  const int64_t per = (t1 - t0 + 64 * kRankWaves - 1) / (64 * kRankWaves) * 64;
  const int64_t a0 = min(t1, t0 + w * per);
  const int64_t a1 = min(t1, a0 + per);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // the block's ids, loaded up front so the serial matching loop below never
  // waits on global memory
  constexpr int kMaxIt = kTokTile * kMaxK / (64 * kRankWaves);
  int ids[kMaxIt];
#pragma unroll
  for (int it = 0; it < kMaxIt; ++it) {
    const int64_t my = a0 + (int64_t)it * 64 + lane;
    ids[it] = my < a1 ? idx[my] : -1;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < kMaxIt; ++it) {
    const int e = ids[it];
    if (e >= 0 && e < E) atomicAdd(&run[w][e], 1);
  }
  __syncthreads();
  // counts -> each block's start position within each expert
  for (int e = threadIdx.x; e < E; e += 64 * kRankWaves) {
    int32_t p = tile_prefix[(int64_t)blockIdx.x * E + e];
#pragma unroll
    for (int q = 0; q < kRankWaves; ++q) {
      const int32_t c = run[q][e];
      run[q][e] = p;
      p += c;
    }
  }
  __syncthreads();
  int32_t* wrun = run[w];
#pragma unroll
  for (int it = 0; it < kMaxIt; ++it) {
    const int64_t a = a0 + (int64_t)it * 64;
    if (a >= a1) break;
    const int64_t my = a + lane;
    const bool in = my < a1;
    const int e = ids[it];
    const bool valid = in && e >= 0 && e < E;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t ones = __ballot(bit);
      peers &= bit ? ones : ~ones;
    }
    int pos = 0;
    if (valid) {
      const int rank = __popcll(peers & below);
      const int base = wrun[e];
      pos = base + rank;
      const bool leader = (peers >> lane) == 1ull;  // highest lane of its group
      if (leader) wrun[e] = base + __popcll(peers);
    }
    if (in) {
      int32_t d = -1;
      if (valid && (capacity < 0 || (int64_t)pos < capacity)) {
        const int64_t row = (int64_t)off[e] + pos;
        if (row >= max_rows) {
          d = -2;
        } else {
          d = (int32_t)row;
          src_token[row] = (int32_t)(my / k);
          src_slot[row] = (int32_t)(my - (my / k) * k);
        }
      }
      dest[my] = d;
    }
  }
}

// Exclusive scan over experts of min(total, capacity) by a 256-thread
// workgroup: each thread takes a run of consecutive experts, then the 256 run
// sums are scanned. Writes off[0..E]; returns whether any expert overflowed.
__device__ bool scan_experts_block(const int32_t* tot, int32_t* off, int32_t* wsum, int E,
                                   int64_t capacity) {
  const int tid = threadIdx.x;
  const int per = (E + 255) / 256;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int32_t local = 0;
  bool drop = false;
  for (int e = e0; e < e1; ++e) {
    const int32_t c = tot[e];
    const int32_t kp = (capacity >= 0 && (int64_t)c > capacity) ? (int32_t)capacity : c;
    drop |= kp < c;
    local += kp;
  }
  wsum[tid] = local;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int32_t add = tid >= o ? wsum[tid - o] : 0;
    __syncthreads();
    wsum[tid] += add;
    __syncthreads();
  }
  int32_t run0 = wsum[tid] - local;
  for (int e = e0; e < e1; ++e) {
    off[e] = run0;
    const int32_t c = tot[e];
    run0 += (capacity >= 0 && (int64_t)c > capacity) ? (int32_t)capacity : c;
  }
  if (tid == 255) off[E] = wsum[255];
  return __syncthreads_or(drop);
}

// ---------------------------------------------------------------------------
// 3'. Scan folded into the rank step, for plans up to kFusedPlanMax tile x
//     expert counts: every workgroup (one per tile) reduces the tile
//     histograms itself -- each expert's total and its prefix over earlier
//     tiles, with LDS integer atomics -- so no separate scan launch is needed.
//     Workgroup 0 also writes counts, offsets, splits and flags. The ranking
//     then runs as in rank_kernel, on wave 0.
constexpr int64_t kFusedPlanMax = 1 << 12;

__global__ __launch_bounds__(256) void rank_scan_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ tile_hist, int n_tiles,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ dest,
    int32_t* __restrict__ src_token, int32_t* __restrict__ src_slot,
    int64_t* __restrict__ send_splits, int64_t* __restrict__ send_displs, int ep_size,
    uint32_t* __restrict__ flags, int64_t T, int E, int k, int ebits, int64_t capacity,
    int64_t max_rows) {
  __shared__ int32_t pre[kMaxE];       // prefix over earlier tiles, then the running position
  __shared__ int32_t tot[kMaxE];       // per-expert totals
  __shared__ int32_t off[kMaxE + 1];   // offsets
  __shared__ int32_t wsum[256];
  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  // wave 0 fetches this tile's expert ids first, so their latency overlaps
  // the histogram reduction and the scan
  const int64_t a0 = (int64_t)tile * kTokTile * k;
  const int64_t a1 = min(T * k, a0 + (int64_t)kTokTile * k);
  constexpr int kMaxIt = kTokTile * kMaxK / 64;
  int ids[kMaxIt];
  if (tid < 64) {
#pragma unroll
    for (int it = 0; it < kMaxIt; ++it) {
      const int64_t my = a0 + (int64_t)it * 64 + tid;
      ids[it] = my < a1 ? idx[my] : -1;
    }
  }
  for (int e = tid; e < E; e += 256) {
    pre[e] = 0;
    tot[e] = 0;
  }
  __syncthreads();
  const int n = n_tiles * E;            // <= kFusedPlanMax
#pragma unroll 8
  for (int i = tid; i < n; i += 256) {
    const int v = tile_hist[i];
    if (v) {
      const int t = i / E, e = i - t * E;
      atomicAdd(&tot[e], v);
      if (t < tile) atomicAdd(&pre[e], v);
    }
  }
  __syncthreads();
  // exclusive scan over experts of min(total, capacity)
  bool any_drop;
  if (E <= 64) {
    // one wave, one expert per lane, shuffle scan: no workgroup barriers
    if (tid < 64) {
      const int32_t c = tid < E ? tot[tid] : 0;
      const int32_t kp = (capacity >= 0 && (int64_t)c > capacity) ? (int32_t)capacity : c;
      int32_t incl = kp;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int32_t up = __shfl_up(incl, o);
        if (tid >= o) incl += up;
      }
      if (tid < E) off[tid] = incl - kp;
      if (tid == E - 1) off[E] = incl;
      wsum[0] = __any(kp < c);   // the same value from every lane of wave 0
    }
    __syncthreads();
    any_drop = wsum[0] != 0;
  } else {
    any_drop = scan_experts_block(tot, off, wsum, E, capacity);
  }
  if (tile == 0) {
    for (int e = tid; e < E; e += 256) {
      counts[e] = tot[e];
      offsets[e] = off[e];
    }
    if (tid == 0) {
      offsets[E] = off[E];
      uint32_t f = 0;
      if (any_drop) f |= MOE_FLAG_DROPPED;
      if ((int64_t)off[E] > max_rows) f |= MOE_FLAG_ROW_OVERFLOW;
      if (f) atomicOr(flags, f);
    }
    if (tid < ep_size) {
      const int el = E / ep_size;
      send_displs[tid] = off[tid * el];
      send_splits[tid] = off[(tid + 1) * el] - off[tid * el];
    }
  }
  if (tid >= 64) return;

  const int lane = tid;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int it = 0; it < kMaxIt; ++it) {
    const int64_t a = a0 + (int64_t)it * 64;
    if (a >= a1) break;
    const int64_t my = a + lane;
    const bool in = my < a1;
    const int e = ids[it];
    const bool valid = in && e >= 0 && e < E;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t ones = __ballot(bit);
      peers &= bit ? ones : ~ones;
    }
    int pos = 0;
    if (valid) {
      const int rank = __popcll(peers & below);
      const int base = pre[e];
      pos = base + rank;
      const bool leader = (peers >> lane) == 1ull;  // highest lane of its group
      if (leader) pre[e] = base + __popcll(peers);
    }
    if (in) {
      int32_t d = -1;
      if (valid && (capacity < 0 || (int64_t)pos < capacity)) {
        const int64_t row = (int64_t)off[e] + pos;
        if (row >= max_rows) {
          d = -2;
        } else {
          d = (int32_t)row;
          src_token[row] = (int32_t)(my / k);
          src_slot[row] = (int32_t)(my - (my / k) * k);
        }
      }
      dest[my] = d;
    }
  }
}

hipError_t launch_dispatch_plan(const int32_t* idx, int32_t* tile_hist, int32_t* counts,
                                int32_t* offsets, int32_t* dest, int32_t* src_token,
                                int32_t* src_slot, int64_t* send_splits, int64_t* send_displs,
                                uint32_t* flags, int64_t T, int E, int k, int64_t capacity,
                                int64_t max_rows, int ep_size, hipStream_t s) {
  const int n_tiles = (int)((T + kTokTile - 1) / kTokTile);
  int ebits = 0;
  while ((1 << ebits) < E) ++ebits;
  if (n_tiles > 0)
    hipLaunchKernelGGL(hist_kernel, dim3(n_tiles), dim3(256), 0, s, idx, tile_hist, T, E, k,
                       flags);
  if ((int64_t)n_tiles * E <= kFusedPlanMax) {
    hipLaunchKernelGGL(rank_scan_kernel, dim3(max(n_tiles, 1)), dim3(256), 0, s, idx, tile_hist,
                       n_tiles, counts, offsets, dest, src_token, src_slot, send_splits,
                       send_displs, ep_size, flags, T, E, k, ebits, capacity, max_rows);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, tile_hist, n_tiles, E, capacity,
                     max_rows, counts, offsets, send_splits, send_displs, ep_size, flags);
  if (n_tiles > 0)
    hipLaunchKernelGGL(rank_kernel, dim3(n_tiles), dim3(64 * kRankWaves), 0, s, idx, tile_hist, offsets,
                       dest, src_token, src_slot, T, E, k, ebits, capacity, max_rows);
  return hipGetLastError();
}

int device_cu_count();

// ---------------------------------------------------------------------------
// 4. Row permute, token-major: one wave per token reads the row once in
//    16-byte lanes and writes it to each of the token's materialised rows.
//    U vectors per lane are held at once (U = 16: a whole 16 KiB row), so each
//    destination row is written in one contiguous run.
template <int U>
__global__ __launch_bounds__(256) void permute_rows_kernel(const u32x4* __restrict__ h,
                                                           const int32_t* __restrict__ dest,
                                                           u32x4* __restrict__ x, int64_t T,
                                                           int k, int row_vec) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += nw) {
    const int mine = lane < k ? dest[t * k + lane] : -1;
    int dj[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) dj[j] = __shfl(mine, j);
    const u32x4* src = h + t * row_vec;
    for (int c0 = lane; c0 < row_vec; c0 += 64 * U) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int c = c0 + u * 64;
        if (c < row_vec) v[u] = __builtin_nontemporal_load(src + c);
      }
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (j >= k) break;
        if (dj[j] < 0) continue;
        u32x4* dst = x + (int64_t)dj[j] * row_vec;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          int c = c0 + u * 64;
          if (c < row_vec) dst[c] = v[u];
        }
      }
    }
  }
}

// fp32 rows whose byte size is not a multiple of 16: plain 4-byte copies.
__global__ __launch_bounds__(256) void permute_rows_f32_kernel(const float* __restrict__ h,
                                                               const int32_t* __restrict__ dest,
                                                               float* __restrict__ x, int64_t T,
                                                               int k, int d) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += nw) {
    for (int j = 0; j < k; ++j) {
      int r = dest[t * k + j];
      if (r < 0) continue;
      for (int c = lane; c < d; c += 64) x[(int64_t)r * d + c] = h[t * d + c];
    }
  }
}

hipError_t launch_permute_rows(const void* h, const int32_t* dest, void* x_perm, int64_t T,
                               int k, int row_bytes, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int64_t blocks = min((T + 3) / 4, (int64_t)device_cu_count() * 8);
  if (row_bytes % 16 == 0) {
    hipLaunchKernelGGL(permute_rows_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, s,
                       (const u32x4*)h, dest, (u32x4*)x_perm, T, k, row_bytes / 16);
  } else {
    hipLaunchKernelGGL(permute_rows_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       (const float*)h, dest, (float*)x_perm, T, k, row_bytes / 4);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 4'. Expert-parallel packing with token deduplication: one send row per
//     (destination rank, token) pair. The pairs are planned by the dispatch
//     plan itself, run on a table that keeps, per token, only the first sent
//     slot for each rank (its "expert" id is the rank); the row copy then
//     writes each pair's row once.

// pid[t,j] = rank of slot j if it is sent (dest >= 0) and no earlier slot of
// token t goes to the same rank; -1 otherwise.
__global__ __launch_bounds__(256) void pair_ids_kernel(const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ dest,
                                                       int32_t* __restrict__ pid, int64_t T,
                                                       int k, int el) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  int rk[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j >= k) break;
    const int64_t a = t * k + j;
    const int r = dest[a] >= 0 ? idx[a] / el : -1;
    bool first = r >= 0;
#pragma unroll
    for (int i = 0; i < j; ++i) first = first && rk[i] != r;
    rk[j] = r;
    pid[a] = first ? r : -1;
  }
}

// pair_dest[t,j] = the pair row of slot j's rank (the row planned for the
// token's first slot to that rank), -1 for unsent slots.
__global__ __launch_bounds__(256) void pair_dest_kernel(const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ dest,
                                                        const int32_t* __restrict__ first_row,
                                                        int32_t* __restrict__ pair_dest,
                                                        int64_t T, int k, int el) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  for (int j = 0; j < k; ++j) {
    const int64_t a = t * k + j;
    int32_t row = -1;
    if (dest[a] >= 0) {
      const int r = idx[a] / el;
      for (int i = 0; i <= j; ++i) {
        const int64_t b = t * k + i;
        if (dest[b] >= 0 && idx[b] / el == r) {
          row = first_row[b];
          break;
        }
      }
    }
    pair_dest[a] = row;
  }
}

// recv_rows[i] = pair row holding the token of grouped row i, for the local
// experts' rows offsets[e_lo] .. min(offsets[e_hi], max_rows) - 1.
__global__ __launch_bounds__(256) void recv_rows_kernel(const int32_t* __restrict__ offsets,
                                                        int e_lo, int e_hi, int64_t max_rows,
                                                        const int32_t* __restrict__ src_token,
                                                        const int32_t* __restrict__ src_slot,
                                                        const int32_t* __restrict__ pair_dest,
                                                        int32_t* __restrict__ recv_rows, int k) {
  const int64_t lo = min((int64_t)offsets[e_lo], max_rows);
  const int64_t hi = min((int64_t)offsets[e_hi], max_rows);
  for (int64_t i = lo + (int64_t)blockIdx.x * 256 + threadIdx.x; i < hi;
       i += (int64_t)gridDim.x * 256)
    recv_rows[i] = pair_dest[(int64_t)src_token[i] * k + src_slot[i]];
}

hipError_t launch_pack_dedup(const void* h, const int32_t* idx, const int32_t* dest,
                             const int32_t* src_token, const int32_t* src_slot,
                             const int32_t* offsets, void* send_buf, int32_t* pair_dest,
                             int32_t* pair_token, int64_t* pair_splits, int64_t* pair_displs,
                             int32_t* recv_rows, const DedupScratch& w, int64_t T, int E, int k,
                             int ep_size, int ep_rank, int64_t max_rows, int row_bytes,
                             hipStream_t s) {
  const int el = E / ep_size;
  const unsigned tb = (unsigned)((T + 255) / 256);
  const int64_t max_pairs = T * (int64_t)min(k, ep_size);
  if (T > 0)
    hipLaunchKernelGGL(pair_ids_kernel, dim3(tb), dim3(256), 0, s, idx, dest, w.pid, T, k, el);
  hipError_t err = launch_dispatch_plan(w.pid, w.tile_hist, w.counts, w.offsets, w.first_row,
                                        pair_token, w.pair_slot, pair_splits, pair_displs,
                                        w.flags, T, ep_size, k, -1, max_pairs, ep_size, s);
  if (err != hipSuccess) return err;
  if (T > 0)
    hipLaunchKernelGGL(pair_dest_kernel, dim3(tb), dim3(256), 0, s, idx, dest, w.first_row,
                       pair_dest, T, k, el);
  if (max_rows > 0) {
    const unsigned rb = (unsigned)std::min<int64_t>((max_rows + 255) / 256, 1024);
    hipLaunchKernelGGL(recv_rows_kernel, dim3(rb), dim3(256), 0, s, offsets, ep_rank * el,
                       (ep_rank + 1) * el, max_rows, src_token, src_slot, pair_dest, recv_rows,
                       k);
  }
  return launch_permute_rows(h, w.first_row, send_buf, T, k, row_bytes, s);
}

// ---------------------------------------------------------------------------
// 5. Unpermute + combine, token-major: one wave per token gathers its k
//    rows, weights them by that token's own gates and sums in float32 in
//    slot order, then rounds once.
template <int U>
__global__ __launch_bounds__(256) void combine_bf16_kernel(
    const bf16x8* __restrict__ yp, const int32_t* __restrict__ idx,
    const float* __restrict__ gate, const int32_t* __restrict__ dest, bf16x8* __restrict__ y,
    int64_t T, int k, int row_vec, int e_lo, int e_hi, bool slots) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += nw) {
    int mine = -1;
    float gm = 0.f;
    if (lane < k) {
      int r = dest[t * k + lane];
      int e = idx[t * k + lane];
      if (r >= 0 && e >= e_lo && e < e_hi) {
        mine = slots ? (int)(t * k + lane) : r;
        gm = gate[t * k + lane];
      }
    }
    int rj[kMaxK];
    float gj[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      rj[j] = __shfl(mine, j);
      gj[j] = __shfl(gm, j);
    }
    for (int c0 = lane; c0 < row_vec; c0 += 64 * U) {
      float acc[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (j >= k) break;
        if (rj[j] < 0) continue;
        const bf16x8* src = yp + (int64_t)rj[j] * row_vec;
        bf16x8 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          int c = c0 + u * 64;
          if (c < row_vec) v[u] = src[c];
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[u][i] = fmaf(gj[j], (float)v[u][i], acc[u][i]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int c = c0 + u * 64;
        if (c < row_vec) {
          bf16x8 o;
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i] = (bf16)acc[u][i];
          __builtin_nontemporal_store(o, y + t * row_vec + c);
        }
      }
    }
  }
}

// The same combine for a compile-time k (1, 2, 4): all k rows' loads of a
// chunk are issued before any of them is accumulated (k * U 16-byte loads in
// flight per lane), then summed in slot order exactly as above. For larger k
// the generic kernel already has enough rows in flight per wave.
template <int KT, int U>
__global__ __launch_bounds__(256) void combine_bf16_k_kernel(
    const bf16x8* __restrict__ yp, const int32_t* __restrict__ idx,
    const float* __restrict__ gate, const int32_t* __restrict__ dest, bf16x8* __restrict__ y,
    int64_t T, int row_vec, int e_lo, int e_hi, bool slots) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += nw) {
    int mine = -1;
    float gm = 0.f;
    if (lane < KT) {
      int r = dest[t * KT + lane];
      int e = idx[t * KT + lane];
      if (r >= 0 && e >= e_lo && e < e_hi) {
        mine = slots ? (int)(t * KT + lane) : r;
        gm = gate[t * KT + lane];
      }
    }
    int rj[KT];
    float gj[KT];
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      rj[j] = __builtin_amdgcn_readfirstlane(__shfl(mine, j));
      gj[j] = __shfl(gm, j);
    }
    for (int c0 = lane; c0 < row_vec; c0 += 64 * U) {
      bf16x8 v[KT][U];
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        if (rj[j] < 0) continue;
        const bf16x8* src = yp + (int64_t)rj[j] * row_vec;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          int c = c0 + u * 64;
          if (c < row_vec) v[j][u] = src[c];
        }
      }
      float acc[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        if (rj[j] < 0) continue;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[u][i] = fmaf(gj[j], (float)v[j][u][i], acc[u][i]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int c = c0 + u * 64;
        if (c < row_vec) {
          bf16x8 o;
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i] = (bf16)acc[u][i];
          __builtin_nontemporal_store(o, y + t * row_vec + c);
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(
    const float* __restrict__ yp, const int32_t* __restrict__ idx,
    const float* __restrict__ gate, const int32_t* __restrict__ dest, float* __restrict__ y,
    int64_t T, int k, int d, int e_lo, int e_hi, bool slots) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += nw) {
    for (int c = lane; c < d; c += 64) {
      float acc = 0.f;
      for (int j = 0; j < k; ++j) {
        int r = dest[t * k + j];
        int e = idx[t * k + j];
        const int64_t row = slots ? t * k + j : r;
        if (r >= 0 && e >= e_lo && e < e_hi) acc = fmaf(gate[t * k + j], yp[row * d + c], acc);
      }
      y[t * d + c] = acc;
    }
  }
}

hipError_t launch_combine(const void* y_perm, const int32_t* idx, const float* gate,
                          const int32_t* dest, void* y, int64_t T, int k, int d, int dtype,
                          int e_lo, int e_hi, hipStream_t s, bool slots) {
  if (T == 0) return hipSuccess;
  int64_t blocks = min((T + 3) / 4, (int64_t)device_cu_count() * 16);
  if (dtype == MOE_DTYPE_BF16) {
    const bf16x8* yp = (const bf16x8*)y_perm;
    bf16x8* yo = (bf16x8*)y;
    const int rv = d / 8;
    const dim3 g((unsigned)blocks), b(256);
    switch (k) {
      case 1: hipLaunchKernelGGL((combine_bf16_k_kernel<1, 4>), g, b, 0, s, yp, idx, gate, dest, yo, T, rv, e_lo, e_hi, slots); break;
      case 2: hipLaunchKernelGGL((combine_bf16_k_kernel<2, 4>), g, b, 0, s, yp, idx, gate, dest, yo, T, rv, e_lo, e_hi, slots); break;
      case 4: hipLaunchKernelGGL((combine_bf16_k_kernel<4, 2>), g, b, 0, s, yp, idx, gate, dest, yo, T, rv, e_lo, e_hi, slots); break;
      default:
        hipLaunchKernelGGL(combine_bf16_kernel<4>, g, b, 0, s, yp, idx, gate, dest, yo, T, k, rv,
                           e_lo, e_hi, slots);
    }
  } else {
    hipLaunchKernelGGL(combine_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       (const float*)y_perm, idx, gate, dest, (float*)y, T, k, d, e_lo, e_hi,
                       slots);
  }
  return hipGetLastError();
}

}  // namespace moe
