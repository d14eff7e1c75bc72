// x slabs: the columns of a walk plan cut into one slab of x per XCD.
//
// Merge-path ("A Programming Model for GPU Load Balancing", PPoPP'23,
// Section 5.2.1) balances rows and nonzeros but leaves each product's x
// gather wherever its column falls. The RgCSR page's results section shows
// what an x that stays in cache is worth (1.81x single precision on its
// GPU). On MI355X the x of a power-law matrix with 4M columns (16 MB fp32)
// is four times one XCD's 4 MB L2, so three gathers in four miss it, and
// those misses, not HBM, bound the SpMV.
//
// With slabs, the plan keeps a copy A' of the matrix whose entries are
// ordered slab-major: slab s covers columns [ceil(s N / 8), ceil((s+1) N / 8))
// and holds, row after row, each row's run of entries in those columns (a
// segment). A' is an ordinary CSR matrix of M' segments; the merge-path walk
// runs over it unchanged and deals its partitions to the XCDs in contiguous
// eighths (workgroup b runs on XCD b mod 8), so XCD s gathers only from slab
// s, an eighth of x. A combine kernel then adds the segment sums of every
// row, in slab order, and applies alpha and beta; every sum is taken in a
// fixed order, so the result is bitwise reproducible for the plan.
//
// Planning (before the plan's one read-back): per row, eight lanes find the
// row's slab bounds by binary search over its columns (which must be sorted
// within the row; descending pairs are counted and, if any, the plan keeps
// no slabs), and each workgroup of 32 rows counts entries and segments per
// slab. Prefix sums of those counts give every segment its id and its first
// position in A'. After the read-back (M' known), the copy is written by
// one workgroup per 32 rows.
#include "device_common.hpp"
#include "internal.hpp"

#include <algorithm>

namespace spmv {
namespace {

// First column of slab s: ceil(s N / kSlabs).
__device__ __forceinline__ int64_t slab_col0(int s, int64_t N) {
  return ((int64_t)s * N + kSlabs - 1) / kSlabs;
}

// First entry of [a, e) whose column is >= c (the row's columns sorted).
__device__ __forceinline__ int32_t first_col_at_least(const int32_t* __restrict__ col, int32_t a,
                                                      int32_t e, int64_t c) {
  int32_t lo = a, hi = e;
  while (lo < hi) {
    const int32_t mid = lo + ((hi - lo) >> 1);
    if ((int64_t)col[mid] < c) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// One row seen by its 8 lanes, lane s for slab s: the row's entries [a, e),
// those in slab s [b, bn), and the row's slabs with entries (bit s).
struct SlabLane {
  int32_t a, e;
  int32_t b, bn;
  uint32_t mask;
};

// Every lane of the wave must call this (shuffle and ballot); rows r >= M
// read as empty at row_ptr[M].
__device__ __forceinline__ SlabLane slab_lane(const int32_t* __restrict__ row_ptr,
                                              const int32_t* __restrict__ col, int64_t M,
                                              int64_t N, int64_t r, int s) {
  SlabLane l;
  l.a = row_ptr[r < M ? r : M];
  l.e = r < M ? row_ptr[r + 1] : l.a;
  l.b = s == 0 ? l.a : first_col_at_least(col, l.a, l.e, slab_col0(s, N));
  const int32_t up = __shfl_down(l.b, 1, kSlabs);
  l.bn = s == kSlabs - 1 ? l.e : up;
  const uint64_t ne = __ballot(l.bn > l.b);
  l.mask = (uint32_t)(ne >> (lane_id() & ~(kSlabs - 1))) & 0xffu;
  return l;
}

__global__ __launch_bounds__(kBlock) void slab_rows_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col, int64_t M, int64_t N,
    int32_t* __restrict__ rptr, uint8_t* __restrict__ mask, int32_t* __restrict__ tile_e,
    int32_t* __restrict__ tile_g, int64_t n_tiles, int64_t* __restrict__ stats) {
  if (stats[kStatSlabOk] == 0) return;   // workgroup-uniform
  __shared__ int s_e[kWavesPerBlock][kSlabs], s_g[kWavesPerBlock][kSlabs];
  const int s = threadIdx.x & (kSlabs - 1);
  const int64_t t = blockIdx.x;
  const int64_t r = t * kSlabTileRows + (threadIdx.x >> 3);
  const SlabLane l = slab_lane(row_ptr, col, M, N, r, s);
  // descending neighbours inside the row (the bounds above assume none)
  int desc = 0;
  for (int64_t k = (int64_t)l.a + 1 + s; k < l.e; k += kSlabs) desc += col[k] < col[k - 1];
  if (r < M && s == 0) {
    rptr[r] = __popc(l.mask);
    mask[r] = (uint8_t)l.mask;
  }
  if (t == 0 && threadIdx.x == 0) rptr[M] = 0;
  // entries and segments per slab over the wave's 8 rows (lanes s, s + 8, ...)
  int e = l.bn - l.b, g = l.bn > l.b ? 1 : 0;
  for (int o = kSlabs; o < kWave; o <<= 1) {
    e += __shfl_xor(e, o);
    g += __shfl_xor(g, o);
  }
  for (int o = 1; o < kWave; o <<= 1) desc += __shfl_xor(desc, o);
  const int wave = threadIdx.x / kWave, lane = lane_id();
  if (lane < kSlabs) {
    s_e[wave][lane] = e;
    s_g[wave][lane] = g;
  }
  if (lane == 0 && desc > 0)
    atomicAdd((unsigned long long*)&stats[kStatSlabDescents], (unsigned long long)desc);
  __syncthreads();
  if (threadIdx.x < kSlabs) {
    int te = 0, tg = 0;
    for (int w = 0; w < kWavesPerBlock; ++w) {
      te += s_e[w][threadIdx.x];
      tg += s_g[w][threadIdx.x];
    }
    tile_e[threadIdx.x * n_tiles + t] = te;
    tile_g[threadIdx.x * n_tiles + t] = tg;
  }
}

__global__ __launch_bounds__(64) void slab_total_kernel(const int32_t* rptr, int64_t M,
                                                        int64_t* stats) {
  if (threadIdx.x == 0 && stats[kStatSlabOk] != 0) stats[kStatSlabSegs] = rptr[M];
}

// One workgroup per 32 rows: the rows' slab bounds (as in slab_rows_kernel),
// each (row, slab) run's first position in A' and segment id from the
// prefix sums, then the copy of the tile's entries, 256 at a time, each to
// its run's position plus its offset in the run.
template <typename V>
__global__ __launch_bounds__(kBlock) void slab_emit_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
    const V* __restrict__ val, int64_t M, int64_t N, int64_t nnz,
    const int32_t* __restrict__ rptr, const int32_t* __restrict__ tile_e,
    const int32_t* __restrict__ tile_g, int64_t n_tiles, int32_t* __restrict__ seg_ptr,
    int32_t* __restrict__ col2, V* __restrict__ val2, int32_t* __restrict__ rseg,
    int64_t n_seg) {
  __shared__ int32_t s_rs[kSlabTileRows + 1];          // row starts
  __shared__ int32_t s_b[kSlabTileRows][kSlabs + 1];   // slab bounds of each row
  __shared__ int32_t s_len[kSlabs][kSlabTileRows];     // run lengths
  __shared__ int32_t s_pos[kSlabTileRows][kSlabs];     // first A' position of each run
  const int s = threadIdx.x & (kSlabs - 1);
  const int j = threadIdx.x >> 3;
  const int64_t t = blockIdx.x;
  const int64_t r = t * kSlabTileRows + j;
  const SlabLane l = slab_lane(row_ptr, col, M, N, r, s);
  s_b[j][s] = l.b;
  if (s == kSlabs - 1) s_b[j][kSlabs] = l.e;
  if (s == 0) s_rs[j] = l.a;
  if (threadIdx.x == 0) s_rs[kSlabTileRows] = row_ptr[(t + 1) * kSlabTileRows < M ? (t + 1) * kSlabTileRows : M];
  s_len[s][j] = l.bn - l.b;
  __syncthreads();
  int32_t pos = tile_e[s * n_tiles + t], id = tile_g[s * n_tiles + t];
  for (int q = 0; q < j; ++q) {
    const int32_t n = s_len[s][q];
    pos += n;
    id += n > 0 ? 1 : 0;
  }
  s_pos[j][s] = pos;
  if (r < M && l.bn > l.b) {
    seg_ptr[id] = pos;
    rseg[rptr[r] + __popc(l.mask & ((1u << s) - 1u))] = id;
  }
  if (t == 0 && threadIdx.x == 0) seg_ptr[n_seg] = (int32_t)nnz;
  __syncthreads();
  const int64_t e0 = s_rs[0], e1 = s_rs[kSlabTileRows];
  for (int64_t k = e0 + threadIdx.x; k < e1; k += kBlock) {
    // the last row starting at or before k (rows of the tile past M start
    // at nnz > k and are never chosen), then the last slab bound <= k
    int lo = 0, hi = kSlabTileRows - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_rs[mid] <= k) lo = mid;
      else hi = mid - 1;
    }
    int q = 0;
#pragma unroll
    for (int u = 1; u < kSlabs; ++u) q = s_b[lo][u] <= k ? u : q;
    const int64_t p2 = (int64_t)s_pos[lo][q] + (k - s_b[lo][q]);
    col2[p2] = col[k];
    val2[p2] = val[k];
  }
}

__global__ __launch_bounds__(64) void slab_stats_kernel(int64_t* stats, int ipt, int64_t P) {
  for (int i = threadIdx.x; i < kStatCount; i += 64) stats[i] = 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    stats[kStatIpt] = ipt;
    stats[kStatParts] = P;
  }
}

// One thread per row: its at most kSlabs segment sums, all requested before
// the first is added, added in slab order.
template <typename V>
__global__ __launch_bounds__(kBlock) void slab_combine_kernel(
    const int32_t* __restrict__ rptr, const int32_t* __restrict__ rseg, const V* __restrict__ yp,
    V* __restrict__ y, V alpha, V beta, int beta_nonzero, int32_t M) {
  const int64_t r = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (r >= M) return;
  const int32_t t0 = rptr[r], n = rptr[r + 1] - t0;
  int32_t sg[kSlabs];
#pragma unroll
  for (int u = 0; u < kSlabs; ++u) sg[u] = u < n ? rseg[t0 + u] : -1;
  V v[kSlabs];
#pragma unroll
  for (int u = 0; u < kSlabs; ++u) v[u] = sg[u] >= 0 ? yp[sg[u]] : V(0);
  V acc = V(0);
#pragma unroll
  for (int u = 0; u < kSlabs; ++u) acc += v[u];
  V out = alpha * acc;
  if (beta_nonzero) out = fma(beta, y[r], out);
  y[r] = out;
}

int blocks_for(int64_t n, int64_t per) { return (int)((n + per - 1) / per); }

}  // namespace

hipError_t launch_slab_rows(const SlabRows& t, const int32_t* row_ptr, const int32_t* col_idx,
                            int64_t M, int64_t N, int64_t* stats, hipStream_t s) {
  if (M <= 0 || t.n_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(slab_rows_kernel, dim3((unsigned)t.n_tiles), dim3(kBlock), 0, s, row_ptr,
                     col_idx, M, N, t.rptr, t.mask, t.tile_e, t.tile_g, t.n_tiles, stats);
  hipError_t err = hipGetLastError();
  const int64_t* enable = stats + kStatSlabOk;
  if (err == hipSuccess) err = exclusive_scan_i32(t.rptr, M + 1, enable, t.scan_temp, s);
  if (err == hipSuccess)
    err = exclusive_scan_i32(t.tile_e, kSlabs * t.n_tiles, enable, t.scan_temp, s);
  if (err == hipSuccess)
    err = exclusive_scan_i32(t.tile_g, kSlabs * t.n_tiles, enable, t.scan_temp, s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(slab_total_kernel, dim3(1), dim3(64), 0, s, t.rptr, M, stats);
  return hipGetLastError();
}

hipError_t launch_slab_emit(const SlabRows& t, const SlabMatrix& m, const int32_t* row_ptr,
                            const int32_t* col_idx, const void* values, int vbytes, int64_t M,
                            int64_t N, int64_t nnz, hipStream_t s) {
  if (M <= 0 || t.n_tiles <= 0) return hipSuccess;
  const dim3 g((unsigned)t.n_tiles), b(kBlock);
  if (vbytes == 4)
    hipLaunchKernelGGL(slab_emit_kernel<float>, g, b, 0, s, row_ptr, col_idx,
                       static_cast<const float*>(values), M, N, nnz, t.rptr, t.tile_e, t.tile_g,
                       t.n_tiles, m.seg_ptr, m.col, static_cast<float*>(m.val), m.rseg, m.n_seg);
  else
    hipLaunchKernelGGL(slab_emit_kernel<double>, g, b, 0, s, row_ptr, col_idx,
                       static_cast<const double*>(values), M, N, nnz, t.rptr, t.tile_e,
                       t.tile_g, t.n_tiles, m.seg_ptr, m.col, static_cast<double*>(m.val), m.rseg,
                       m.n_seg);
  return hipGetLastError();
}

hipError_t launch_slab_stats(int64_t* stats, int ipt, int64_t P, hipStream_t s) {
  hipLaunchKernelGGL(slab_stats_kernel, dim3(1), dim3(64), 0, s, stats, ipt, P);
  return hipGetLastError();
}

template <typename V>
hipError_t launch_slab_combine(const int32_t* rptr, const int32_t* rseg, const V* yp, V* y,
                               V alpha, V beta, int beta_nonzero, int64_t M, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(slab_combine_kernel<V>, dim3(blocks_for(M, kBlock)), dim3(kBlock), 0, s,
                     rptr, rseg, yp, y, alpha, beta, beta_nonzero, (int32_t)M);
  return hipGetLastError();
}

template hipError_t launch_slab_combine<float>(const int32_t*, const int32_t*, const float*,
                                               float*, float, float, int, int64_t, hipStream_t);
template hipError_t launch_slab_combine<double>(const int32_t*, const int32_t*, const double*,
                                                double*, double, double, int, int64_t,
                                                hipStream_t);

}  // namespace spmv
