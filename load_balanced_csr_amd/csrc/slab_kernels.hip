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
// row over its slabs and applies alpha and beta; every sum is taken in a
// fixed order, so the result is bitwise reproducible for the plan.
//
// Tables: rows are taken in tiles of 32, eight lanes a row, lane s for slab
// s. Lane s finds the row's first entry in slab s by binary search over the
// row's columns (which assumes them sorted within the row); the bounds are
// made non-decreasing across the lanes, so the runs partition the row and
// every entry is summed once whatever the columns' order -- only the x
// locality depends on it. Runs whose middle entry lies outside their slab
// or below its predecessor are counted, and the automatic choice keeps no
// slabs if there are any. Per tile and slab the entries and segments are counted,
// slab-major, and their prefix sums give every run its first position in A'
// and every segment its id: segment (row r, slab s) is the tile's first
// slab-s id plus the rows before r in the tile with an entry in slab s (the
// rows' slab masks, one byte each). The combine finds the segments the same
// way, so it needs no per-segment table. The copy into A' runs in chunks of
// at most kSlabChunk entries of one tile, so a tile holding a long row is
// shared out.
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

// Every lane of the wave must call this (shuffles and ballot); rows r >= M
// read as empty at row_ptr[M]. The bounds are made non-decreasing across
// the lanes (a running maximum), so [b, bn) partition [a, e) whatever the
// columns' order.
__device__ __forceinline__ SlabLane slab_lane(const int32_t* __restrict__ row_ptr,
                                              const int32_t* __restrict__ col, int64_t M,
                                              int64_t N, int64_t r, int s) {
  SlabLane l;
  l.a = row_ptr[r < M ? r : M];
  l.e = r < M ? row_ptr[r + 1] : l.a;
  int32_t b = s == 0 ? l.a : first_col_at_least(col, l.a, l.e, slab_col0(s, N));
#pragma unroll
  for (int o = 1; o < kSlabs; o <<= 1) {
    const int32_t lower = __shfl_up(b, o, kSlabs);
    b = s >= o ? max(b, lower) : b;
  }
  l.b = b;
  const int32_t up = __shfl_down(b, 1, kSlabs);
  l.bn = s == kSlabs - 1 ? l.e : up;
  const uint64_t ne = __ballot(l.bn > l.b);
  l.mask = (uint32_t)(ne >> (lane_id() & ~(kSlabs - 1))) & 0xffu;
  return l;
}

__global__ __launch_bounds__(kBlock) void slab_rows_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col, int64_t M, int64_t N,
    uint8_t* __restrict__ mask, int32_t* __restrict__ tile_e, int32_t* __restrict__ tile_g,
    int32_t* __restrict__ tile_c, int64_t n_tiles, int64_t* __restrict__ stats) {
  if (stats[kStatSlabOk] == 0) return;   // workgroup-uniform
  __shared__ int s_e[kWavesPerBlock][kSlabs], s_g[kWavesPerBlock][kSlabs];
  __shared__ int s_stray[kWavesPerBlock];
  const int s = threadIdx.x & (kSlabs - 1);
  const int64_t t = blockIdx.x;
  const int64_t r = t * kSlabTileRows + (threadIdx.x >> 3);
  const SlabLane l = slab_lane(row_ptr, col, M, N, r, s);
  // a run whose middle entry lies outside its slab or below its
  // predecessor (a row whose columns are not sorted; the binary search
  // alone keeps each run's first and last column inside the slab)
  int stray = 0;
  if (l.bn > l.b) {
    const int32_t mid = l.b + ((l.bn - l.b) >> 1);
    const int64_t c = col[mid];
    stray = c < slab_col0(s, N) || (s + 1 < kSlabs && c >= slab_col0(s + 1, N)) ||
            (mid > l.b && col[mid - 1] > c);
  }
  if (r < M && s == 0) mask[r] = (uint8_t)l.mask;
  if (t == 0 && threadIdx.x == 0) {
    tile_e[kSlabs * n_tiles] = 0;
    tile_g[kSlabs * n_tiles] = 0;
    tile_c[n_tiles] = 0;
  }
  if (threadIdx.x == 0) {
    const int64_t re = (t + 1) * kSlabTileRows < M ? (t + 1) * kSlabTileRows : M;
    const int64_t n = (int64_t)row_ptr[re] - row_ptr[t * kSlabTileRows];
    tile_c[t] = n > kSlabChunk ? (int32_t)((n + kSlabChunk - 1) / kSlabChunk) : 1;
  }
  // entries and segments per slab over the wave's 8 rows (lanes s, s + 8, ...)
  int e = l.bn - l.b, g = l.bn > l.b ? 1 : 0;
  for (int o = kSlabs; o < kWave; o <<= 1) {
    e += __shfl_xor(e, o);
    g += __shfl_xor(g, o);
  }
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int wave_stray = __popcll(__ballot(stray != 0));
  if (lane < kSlabs) {
    s_e[wave][lane] = e;
    s_g[wave][lane] = g;
  }
  if (lane == 0) s_stray[wave] = wave_stray;
  __syncthreads();
  // one atomic per workgroup, and only where a run strays
  if (threadIdx.x == 0) {
    int n = 0;
    for (int w = 0; w < kWavesPerBlock; ++w) n += s_stray[w];
    if (n > 0) atomicAdd((unsigned long long*)&stats[kStatSlabStray], (unsigned long long)n);
  }
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

__global__ __launch_bounds__(64) void slab_total_kernel(const int32_t* tile_g,
                                                        const int32_t* tile_c, int64_t n_tiles,
                                                        int64_t* stats) {
  if (threadIdx.x == 0 && stats[kStatSlabOk] != 0) {
    stats[kStatSlabSegs] = tile_g[kSlabs * n_tiles];
    stats[kStatSlabChunks] = tile_c[n_tiles];
  }
}

// One workgroup per copy chunk (part i of tile t): the tile's rows' slab
// bounds, each run's first position in A' and, in part 0, each segment's
// first position into seg_ptr; then the chunk's entries, each to its run's
// position plus its offset in the run. Positions and ids outside A' (only
// if col_idx changed since the plan was made) are skipped.
template <typename V>
__global__ __launch_bounds__(kBlock) void slab_emit_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
    const V* __restrict__ val, int64_t M, int64_t N, int64_t nnz,
    const int32_t* __restrict__ tile_e, const int32_t* __restrict__ tile_g,
    const int32_t* __restrict__ tile_c, int64_t n_tiles, int32_t* __restrict__ seg_ptr,
    int32_t* __restrict__ col2, V* __restrict__ val2, int64_t n_seg) {
  __shared__ int32_t s_rs[kSlabTileRows + 1];          // row starts
  __shared__ int32_t s_b[kSlabTileRows][kSlabs + 1];   // slab bounds of each row
  __shared__ int32_t s_len[kSlabs][kSlabTileRows];     // run lengths
  __shared__ int32_t s_pos[kSlabTileRows][kSlabs];     // first A' position of each run
  // the tile whose chunks hold this workgroup: the last t with tile_c[t] <= b
  const int64_t blk = blockIdx.x;
  int64_t lo_t = 0, hi_t = n_tiles - 1;
  while (lo_t < hi_t) {
    const int64_t mid = (lo_t + hi_t + 1) >> 1;
    if (tile_c[mid] <= blk) lo_t = mid;
    else hi_t = mid - 1;
  }
  const int64_t t = lo_t, part = blk - tile_c[t];
  const int s = threadIdx.x & (kSlabs - 1);
  const int j = threadIdx.x >> 3;
  const int64_t r = t * kSlabTileRows + j;
  const SlabLane l = slab_lane(row_ptr, col, M, N, r, s);
  s_b[j][s] = l.b;
  if (s == kSlabs - 1) s_b[j][kSlabs] = l.e;
  if (s == 0) s_rs[j] = l.a;
  if (threadIdx.x == 0)
    s_rs[kSlabTileRows] = row_ptr[(t + 1) * kSlabTileRows < M ? (t + 1) * kSlabTileRows : M];
  s_len[s][j] = l.bn - l.b;
  __syncthreads();
  int32_t pos = tile_e[s * n_tiles + t], id = tile_g[s * n_tiles + t];
  for (int q = 0; q < j; ++q) {
    const int32_t n = s_len[s][q];
    pos += n;
    id += n > 0 ? 1 : 0;
  }
  s_pos[j][s] = pos;
  if (part == 0 && r < M && l.bn > l.b && id < n_seg) seg_ptr[id] = pos;
  if (blk == 0 && threadIdx.x == 0) seg_ptr[n_seg] = (int32_t)nnz;
  __syncthreads();
  const int64_t e0 = s_rs[0] + part * kSlabChunk;
  const int64_t e1 = min((int64_t)s_rs[kSlabTileRows], e0 + kSlabChunk);
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
    if ((uint64_t)p2 < (uint64_t)nnz) {
      col2[p2] = col[k];
      val2[p2] = val[k];
    }
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

// Rows per thread of the combine: a wave takes 4 x 64 consecutive rows, 64
// at a time, so more of its loads are in flight together (power-law: 1 / 4 /
// 8 rows a thread, 32 / 21 / 26 us).
constexpr int kCombineSteps = 4;

// A wave takes kCombineSteps runs of 64 rows (two tiles of 32 each), one
// row per lane per run. The segment id of (row, slab s) is the tile's first
// slab-s id plus the lanes of the tile before this one whose rows have an
// entry in slab s (a ballot). First every lane's masks and old y and, in one
// load, the first ids of the wave's 8 tiles x 8 slabs; then every segment
// sum of the lane's rows; each row's sums are added in slab order.
template <typename V>
__global__ __launch_bounds__(kBlock) void slab_combine_kernel(
    const uint8_t* __restrict__ mask, const int32_t* __restrict__ tile_g, int64_t n_tiles,
    const V* __restrict__ yp, V* __restrict__ y, V alpha, V beta, int beta_nonzero, int32_t M) {
  constexpr int K = kCombineSteps;
  constexpr int TPW = K * kWave / kSlabTileRows;   // tiles of a wave
  constexpr int NG = TPW * kSlabs / kWave;          // first ids per lane
  static_assert(kWave == 2 * kSlabTileRows && NG * kWave == TPW * kSlabs, "ids fill lanes");
  const int lane = lane_id();
  const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  const int64_t r0 = wave * K * kWave;             // the wave's first row (a tile start)
  const int64_t t0 = r0 / kSlabTileRows;
  // gl[j] of lane l: first id of slab l % 8 in tile t0 + 8 j + l / 8
  int32_t gl[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const int64_t tl = min(t0 + (kWave / kSlabs) * j + lane / kSlabs, n_tiles - 1);
    gl[j] = tile_g[(lane % kSlabs) * n_tiles + tl];
  }
  uint32_t m[K];
  V yold[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t r = r0 + k * kWave + lane;
    m[k] = r < M ? mask[r] : 0u;
    yold[k] = beta_nonzero && r < M ? y[r] : V(0);
  }
  const uint64_t half = lane >= kSlabTileRows ? 0xffffffff00000000ull : 0x00000000ffffffffull;
  const uint64_t below = ((1ull << lane) - 1ull) & half;
  V v[K][kSlabs];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int tile = 2 * k + (lane >= kSlabTileRows ? 1 : 0);
#pragma unroll
    for (int s = 0; s < kSlabs; ++s) {
      const bool has = (m[k] >> s) & 1u;
      const int before = __popcll(__ballot(has) & below);
      const int q = tile * kSlabs + s;   // q / 64 is fixed for each step k
      const int32_t g = __shfl(gl[q / kWave], q % kWave);
      v[k][s] = has ? yp[g + before] : V(0);
    }
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t r = r0 + k * kWave + lane;
    V acc = V(0);
#pragma unroll
    for (int s = 0; s < kSlabs; ++s) acc += v[k][s];
    if (r < M) {
      V out = alpha * acc;
      if (beta_nonzero) out = fma(beta, yold[k], out);
      y[r] = out;
    }
  }
}

int blocks_for(int64_t n, int64_t per) { return (int)((n + per - 1) / per); }

}  // namespace

hipError_t launch_slab_rows(const SlabRows& t, const int32_t* row_ptr, const int32_t* col_idx,
                            int64_t M, int64_t N, int64_t nnz, int64_t* stats, hipStream_t s) {
  if (M <= 0 || t.n_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(slab_rows_kernel, dim3((unsigned)t.n_tiles), dim3(kBlock), 0, s, row_ptr,
                     col_idx, M, N, t.mask, t.tile_e, t.tile_g, t.tile_c, t.n_tiles, stats);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t* enable = stats + kStatSlabOk;
  if ((err = exclusive_scan_i32(t.tile_e, kSlabs * t.n_tiles + 1, enable, t.scan_temp, s)) !=
          hipSuccess ||
      (err = exclusive_scan_i32(t.tile_g, kSlabs * t.n_tiles + 1, enable, t.scan_temp, s)) !=
          hipSuccess ||
      (err = exclusive_scan_i32(t.tile_c, t.n_tiles + 1, enable, t.scan_temp, s)) != hipSuccess)
    return err;
  hipLaunchKernelGGL(slab_total_kernel, dim3(1), dim3(64), 0, s, t.tile_g, t.tile_c, t.n_tiles,
                     stats);
  return hipGetLastError();
}

hipError_t launch_slab_emit(const SlabRows& t, const SlabMatrix& m, const int32_t* row_ptr,
                            const int32_t* col_idx, const void* values, int vbytes, int64_t M,
                            int64_t N, int64_t nnz, hipStream_t s) {
  if (M <= 0 || t.n_tiles <= 0 || m.n_chunks <= 0) return hipSuccess;
  if (m.n_chunks > 0x7fffffffll) return hipErrorInvalidValue;
  const dim3 g((unsigned)m.n_chunks), b(kBlock);
  if (vbytes == 4)
    hipLaunchKernelGGL(slab_emit_kernel<float>, g, b, 0, s, row_ptr, col_idx,
                       static_cast<const float*>(values), M, N, nnz, t.tile_e, t.tile_g, t.tile_c,
                       t.n_tiles, m.seg_ptr, m.col, static_cast<float*>(m.val), m.n_seg);
  else
    hipLaunchKernelGGL(slab_emit_kernel<double>, g, b, 0, s, row_ptr, col_idx,
                       static_cast<const double*>(values), M, N, nnz, t.tile_e, t.tile_g,
                       t.tile_c, t.n_tiles, m.seg_ptr, m.col, static_cast<double*>(m.val),
                       m.n_seg);
  return hipGetLastError();
}

hipError_t launch_slab_stats(int64_t* stats, int ipt, int64_t P, hipStream_t s) {
  hipLaunchKernelGGL(slab_stats_kernel, dim3(1), dim3(64), 0, s, stats, ipt, P);
  return hipGetLastError();
}

template <typename V>
hipError_t launch_slab_combine(const SlabRows& t, const V* yp, V* y, V alpha, V beta,
                               int beta_nonzero, int64_t M, hipStream_t s) {
  if (M <= 0 || t.n_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(slab_combine_kernel<V>, dim3(blocks_for(M, kBlock * kCombineSteps)),
                     dim3(kBlock), 0, s,
                     t.mask, t.tile_g, t.n_tiles, yp, y, alpha, beta, beta_nonzero, (int32_t)M);
  return hipGetLastError();
}

template hipError_t launch_slab_combine<float>(const SlabRows&, const float*, float*, float,
                                               float, int, int64_t, hipStream_t);
template hipError_t launch_slab_combine<double>(const SlabRows&, const double*, double*, double,
                                                double, int, int64_t, hipStream_t);

}  // namespace spmv
