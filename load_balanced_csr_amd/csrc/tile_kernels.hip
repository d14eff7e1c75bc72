// Column-blocked tiles for the long rows of a merge-path walk plan.
//
// Merge-path ("A Programming Model for GPU Load Balancing", PPoPP'23,
// Section 5.2.1) cuts a row of 50,000 nonzeros into ~50 partitions of
// T = 1024 units, each a run of the row's consecutive nonzeros. With columns
// spread over all of x, every such partition gathers x from a wide span, one
// cache line per product: on MI355X those gathers, not HBM, bind (the RgCSR
// page's results section reports the same effect of caching x, 1.81x on its
// GPU). Here the partitions that lie entirely inside one row (no row end in
// them) are regrouped by column: a long row's interior nonzeros are cut at
// fixed column-block boundaries (BC columns, 16 KiB of x) -- all of such a
// row's nonzeros, those in its first and last partition too --, and a
// workgroup (a tile) takes one column block and the segments of up to
// kTileRows long rows in it: it stages that block of x in LDS once and
// gathers from LDS. Every segment's sum goes to partial[row][block]; a
// reduction adds alpha * sum over blocks, in block order, to each row's y
// after the walk and the carry fix-up. The walk skips the rows' interior
// partitions (their carries are 0) and leaves the rows' nonzeros in their
// first and last partition out (masked), so every nonzero is summed exactly
// once and the result is bitwise reproducible for a fixed plan. The walk
// and the tiles run in one grid, the fix-up and the reduction in another
// (merge_kernels.hip; the tiles' device code is in tile_exec.hpp); this file
// builds the plan's tables.
//
// Correctness never depends on the columns: segments partition each row's
// interior range whatever col_idx holds, and a column outside the tile's
// block is gathered from global x.
#include "device_common.hpp"
#include "internal.hpp"

#include <limits.h>

#include <algorithm>

namespace spmv {
namespace {

// ---- plan: interior runs of long rows ---------------------------------------------

// The partition just past row r's interior run starting at p (its row-end
// partition): the first q > p with split_row[q + 1] > r, by binary search.
__device__ __forceinline__ int64_t run_end(const int32_t* __restrict__ split_row, int64_t p,
                                           int64_t P, int32_t r) {
  int64_t lo = p + 1, hi = P;   // split_row[P] = M > r
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (split_row[mid] > r) hi = mid; else lo = mid + 1;
  }
  return lo - 1;
}

// flags[p] = 1 when partition p starts an interior run whose nonzeros reach
// min_entries (0 past P); nothing unless the plan allows tiles.
__global__ __launch_bounds__(kBlock) void tile_flags_kernel(
    const int32_t* __restrict__ split_row, const int32_t* __restrict__ split_nz, int64_t p_max,
    int32_t M, int64_t min_entries, const int64_t* __restrict__ stats, int32_t* __restrict__ flags) {
  const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (p >= p_max || stats[kStatTileOk] == 0) return;
  const int64_t P = stats[kStatParts];
  int f = 0;
  if (p < P) {
    const int32_t r = split_row[p];
    if (r < M && split_row[p + 1] == r && (p == 0 || split_row[p - 1] != r)) {
      const int64_t q = run_end(split_row, p, P, r);
      f = (int64_t)split_nz[q] - split_nz[p] >= min_entries;
    }
  }
  flags[p] = f;
}

// After the exclusive scan of the flags: the tile-row table (row, its first
// and end nonzero -- the whole row --, the first interior partition and the
// row's end partition), at most cap rows; stats[kStatTileRows] = their
// number, stats[kStatTileEntries] = their nonzeros.
__global__ __launch_bounds__(kBlock) void tile_rows_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ split_row,
    const int32_t* __restrict__ split_nz, int64_t p_max, int32_t M, int64_t min_entries,
    int32_t cap, const int32_t* __restrict__ scan, int64_t* __restrict__ stats,
    int32_t* __restrict__ rows) {
  const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (p >= p_max || stats[kStatTileOk] == 0) return;
  const int64_t P = stats[kStatParts];
  if (p >= P) return;
  const int32_t r = split_row[p];
  int64_t q = -1;
  bool f = false;
  if (r < M && split_row[p + 1] == r && (p == 0 || split_row[p - 1] != r)) {
    q = run_end(split_row, p, P, r);
    f = (int64_t)split_nz[q] - split_nz[p] >= min_entries;
  }
  const int32_t i = scan[p];
  if (f && i < cap) {
    int32_t* t = rows + (int64_t)kTileRowInts * i;
    t[0] = r;
    t[1] = row_ptr[r];
    t[2] = row_ptr[r + 1];
    t[3] = (int32_t)p;
    t[4] = (int32_t)q;
    atomicAdd((unsigned long long*)&stats[kStatTileEntries],
              (unsigned long long)((int64_t)row_ptr[r + 1] - row_ptr[r]));
  }
  if (p == P - 1) stats[kStatTileRows] = min((int64_t)cap, (int64_t)i + (f ? 1 : 0));
}

// Tiles are worth their extra launches only when their rows hold at least
// half of the nonzeros.
__global__ __launch_bounds__(64) void tile_gate_kernel(int64_t nnz, int64_t* stats) {
  if (threadIdx.x != 0) return;
  if (2 * stats[kStatTileEntries] < nnz) stats[kStatTileRows] = 0;
}

// seg[i][b] = first nonzero of tile row i whose column is >= b * bc
// (b = 0..nb; the ends are the row's bounds), made non-decreasing in b so
// that the segments always partition the row.
__global__ __launch_bounds__(kBlock) void tile_seg_kernel(const int32_t* __restrict__ rows,
                                                          const int32_t* __restrict__ col_idx,
                                                          int32_t nb, int32_t bc, int64_t n_max,
                                                          const int64_t* __restrict__ stats,
                                                          int32_t* __restrict__ seg) {
  const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= n_max * (nb + 1)) return;
  const int64_t i = t / (nb + 1);
  const int b = (int)(t - i * (nb + 1));
  if (i >= stats[kStatTileRows]) return;
  const int32_t* row = rows + kTileRowInts * i;
  const int32_t a = row[1], e = row[2];
  int32_t pos;
  if (b == 0) {
    pos = a;
  } else if (b == nb) {
    pos = e;
  } else {
    const int64_t c = (int64_t)b * bc;
    int32_t lo = a, hi = e;
    while (lo < hi) {
      const int32_t mid = (int32_t)(((int64_t)lo + hi) >> 1);
      if (col_idx[mid] < c) lo = mid + 1; else hi = mid;
    }
    pos = lo;
  }
  seg[i * (nb + 1) + b] = pos;
}

// Inclusive running maximum of an int across the wave, in DPP moves (the
// steps of wave_scan_i32 with max in place of +).
__device__ __forceinline__ int wave_max_scan_i32(int x) {
  const int lane = lane_id();
  const int r = lane & 15, row = lane >> 4;
  int t;
  t = dpp_i32<dpp_row_shr(1)>(0, x);
  x = r >= 1 ? max(x, t) : x;
  t = dpp_i32<dpp_row_shr(2)>(0, x);
  x = r >= 2 ? max(x, t) : x;
  t = dpp_i32<dpp_row_shr(4)>(0, x);
  x = r >= 4 ? max(x, t) : x;
  t = dpp_i32<dpp_row_shr(8)>(0, x);
  x = r >= 8 ? max(x, t) : x;
  t = dpp_i32<kDppRowBcast15, 0xA>(0, x);
  x = (row & 1) ? max(x, t) : x;
  t = dpp_i32<kDppRowBcast31, 0xC>(0, x);
  x = row >= 2 ? max(x, t) : x;
  return x;
}

// Running maximum along each tile row's boundaries (only changes anything
// when a row's columns are not sorted); the row's interior partitions marked
// as skipped by the walk kernel, with zero carries that the fix-up adds to
// the row harmlessly; and the row's nonzeros in its first and last
// partition masked off for the walk kernel (so its carry there is 0 and its
// y gets beta * y only). A partition holds at most one tile row's start and
// one tile row's end, so no two threads write the same mask. One wave per
// tile row (a row's bounds and interior partitions number in the
// thousands: one thread per row took 0.5 ms on the bimodal matrix).
__global__ __launch_bounds__(kBlock) void tile_finish_kernel(
    const int32_t* __restrict__ rows, const int32_t* __restrict__ split_nz, int32_t nb,
    int64_t n_max, const int64_t* __restrict__ stats, int32_t* __restrict__ seg,
    int32_t* __restrict__ skip, int32_t* __restrict__ mask_end, int32_t* __restrict__ mask_start,
    int32_t* __restrict__ carry_row, void* carry_val, int vbytes) {
  const int64_t i = ((int64_t)blockIdx.x * kBlock + threadIdx.x) / kWave;
  if (i >= n_max || i >= stats[kStatTileRows]) return;   // wave-uniform
  const int lane = lane_id();
  int32_t* s = seg + i * (nb + 1);
  int32_t run = s[0];
  for (int b0 = 0; b0 <= nb; b0 += kWave) {
    const int b = b0 + lane;
    const int32_t v = max(wave_max_scan_i32(b <= nb ? s[b] : INT_MIN), run);
    if (b <= nb) s[b] = v;
    run = __builtin_amdgcn_readlane(v, kWave - 1);
  }
  const int32_t* row = rows + kTileRowInts * i;
  const int32_t p_first = row[3], p_end = row[4];
  for (int32_t p = p_first + lane; p < p_end; p += kWave) {
    skip[p] = 1;
    carry_row[p] = row[0];
    if (vbytes == 4) static_cast<float*>(carry_val)[p] = 0.f;
    else static_cast<double*>(carry_val)[p] = 0.0;
  }
  if (lane == 0) {
    // the row's start, in the partition before its interior run
    if (p_first > 0 && row[1] < split_nz[p_first]) mask_start[p_first - 1] = row[1];
    // the row's end partition
    if (row[2] > split_nz[p_end]) mask_end[p_end] = row[2];
  }
}

__global__ __launch_bounds__(kBlock) void fill_i32_kernel(int32_t* __restrict__ a, int64_t n,
                                                          int32_t v, const int64_t* enable) {
  if (enable && *enable == 0) return;
  for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < n;
       k += (int64_t)gridDim.x * kBlock)
    a[k] = v;
}

// keep[p] = 1 for the partitions the walk kernel still runs (0 past P)
__global__ __launch_bounds__(kBlock) void tile_keep_kernel(const int32_t* __restrict__ skip,
                                                           int64_t p_max,
                                                           const int64_t* __restrict__ stats,
                                                           int32_t* __restrict__ keep) {
  const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (p >= p_max || stats[kStatTileRows] == 0) return;
  keep[p] = p < stats[kStatParts] && skip[p] == 0;
}

// the walk kernel's dispatch list: the kept partitions in partition order
__global__ __launch_bounds__(kBlock) void tile_list_kernel(const int32_t* __restrict__ skip,
                                                           const int32_t* __restrict__ scan,
                                                           int64_t p_max,
                                                           int64_t* __restrict__ stats,
                                                           int32_t* __restrict__ list) {
  const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (p >= p_max || stats[kStatTileRows] == 0) return;
  const int64_t P = stats[kStatParts];
  if (p >= P) return;
  const bool kept = skip[p] == 0;
  if (kept) list[scan[p]] = (int32_t)p;
  if (p == P - 1) stats[kStatWalkParts] = scan[p] + (kept ? 1 : 0);
}

// ---- exec ------------------------------------------------------------------------

// y[row] += alpha * (sum of the row's block partials, in block order), one
// wave per tile row.
unsigned grid_for(int64_t n, int64_t per) {
  return (unsigned)std::max<int64_t>(1, (n + per - 1) / per);
}

}  // namespace

hipError_t launch_tile_plan(const TilePlan& tp, const int32_t* split_row, const int32_t* split_nz,
                            const int32_t* col_idx, int64_t M, int64_t nnz, int64_t p_max,
                            int64_t* stats, int32_t* carry_row, void* carry_val, int vbytes,
                            hipStream_t s) {
  if (tp.cap <= 0 || p_max <= 0) return hipSuccess;
  const dim3 blk(kBlock);
  hipLaunchKernelGGL(tile_flags_kernel, dim3(grid_for(p_max, kBlock)), blk, 0, s, split_row,
                     split_nz, p_max, (int32_t)M, tp.min_entries, stats, tp.scan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = exclusive_scan_i32(tp.scan, p_max, stats + kStatTileOk, tp.scan_temp, s)) != hipSuccess)
    return e;
  hipLaunchKernelGGL(tile_rows_kernel, dim3(grid_for(p_max, kBlock)), blk, 0, s, tp.row_ptr,
                     split_row, split_nz, p_max, (int32_t)M, tp.min_entries, tp.cap, tp.scan,
                     stats, tp.rows);
  hipLaunchKernelGGL(tile_gate_kernel, dim3(1), dim3(64), 0, s, nnz, stats);
  // segment bounds at every quarter block (a multi-vector product's tiles
  // take narrower blocks of x; the SpMV tiles read every fourth bound)
  const int32_t nq = tp.nb * kTileSub;
  hipLaunchKernelGGL(tile_seg_kernel, dim3(grid_for((int64_t)tp.cap * (nq + 1), kBlock)), blk, 0,
                     s, tp.rows, col_idx, nq, tp.bc / kTileSub, (int64_t)tp.cap, stats, tp.seg);
  const unsigned fill_blocks = std::min<unsigned>(grid_for(p_max, kBlock), 4096);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(fill_blocks), blk, 0, s, tp.skip, p_max, 0,
                     stats + kStatTileRows);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(fill_blocks), blk, 0, s, tp.mask_end, p_max, 0,
                     stats + kStatTileRows);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(fill_blocks), blk, 0, s, tp.mask_start, p_max,
                     INT_MAX, stats + kStatTileRows);
  hipLaunchKernelGGL(tile_finish_kernel, dim3(grid_for((int64_t)tp.cap * kWave, kBlock)), blk, 0,
                     s, tp.rows,
                     split_nz, nq, (int64_t)tp.cap, stats, tp.seg, tp.skip, tp.mask_end,
                     tp.mask_start, carry_row, carry_val, vbytes);
  hipLaunchKernelGGL(tile_keep_kernel, dim3(grid_for(p_max, kBlock)), blk, 0, s, tp.skip, p_max,
                     stats, tp.scan);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = exclusive_scan_i32(tp.scan, p_max, stats + kStatTileRows, tp.scan_temp, s)) !=
      hipSuccess)
    return e;
  hipLaunchKernelGGL(tile_list_kernel, dim3(grid_for(p_max, kBlock)), blk, 0, s, tp.skip, tp.scan,
                     p_max, stats, tp.list);
  return hipGetLastError();
}

}  // namespace spmv
