// Planning kernels: row-length statistics and bins counted in LDS, the
// exclusive scan of the bin counts, the stable scatter of row ids into bins,
// and the merge-path split search (one binary search per wavefront
// partition).
//
// Binning follows "OpSparse: a Highly Optimized Framework for Sparse General
// Matrix Multiplication on GPUs" (arXiv 2206.07244), Section 5.1: a first
// pass counts the rows of every bin with shared-memory (here LDS) counters
// and tracks the longest row the same way, an exclusive sum turns the counts
// into offsets, and a second pass writes the row ids; when every row falls
// into one bin the second pass is skipped and row ids are used directly.
// Here the counts are kept per workgroup and scanned bin-major, so the
// offsets are deterministic and rows stay in ascending order inside a bin,
// without any global atomics.
//
// The split search follows "A Programming Model for GPU Load Balancing"
// (Osama, Porumbescu, Owens, PPoPP'23), Section 5.2.1: rows and nonzeros are
// units of equal cost, taken in order (a row's nonzeros, then the row's
// end); a worker's start is found by a binary search along its diagonal.
#include "device_common.hpp"
#include "internal.hpp"

#include <limits.h>

#include <algorithm>

namespace spmv {
namespace {

__device__ __forceinline__ int bin_of(int64_t L, const BinEdges& e) {
  int b = 0;
#pragma unroll
  for (int k = 0; k < kMaxBins - 1; ++k)
    b += (k < e.n_bins - 1 && L > e.max_len[k]) ? 1 : 0;
  return b;
}

__global__ __launch_bounds__(64) void clear_stats_kernel(int64_t* stats) {
  if (threadIdx.x < kStatCount) stats[threadIdx.x] = 0;
}

// Pass 1: per-workgroup bin counts, longest row and empty rows, kept in LDS;
// also checks that row_ptr is a valid CSR row pointer array.
__global__ __launch_bounds__(kBlock) void bin_count_kernel(
    const int32_t* __restrict__ row_ptr, int32_t M, int32_t nnz, BinEdges edges,
    int32_t* __restrict__ counts, int32_t* __restrict__ wg_max,
    int32_t* __restrict__ wg_empty, int64_t* stats) {
  __shared__ int32_t s_cnt[kMaxBins];
  __shared__ int32_t s_max, s_empty;
  const int tid = threadIdx.x;
  if (tid < kMaxBins) s_cnt[tid] = 0;
  if (tid == 0) { s_max = 0; s_empty = 0; }
  __syncthreads();
  int my_max = 0, my_empty = 0;
  bool bad = false;
  const int64_t first = (int64_t)blockIdx.x * kBinRowsPerBlock;
#pragma unroll
  for (int k = 0; k < kBinRowsPerBlock / kBlock; ++k) {
    const int64_t r = first + k * kBlock + tid;
    if (r < M) {
      const int32_t a = row_ptr[r], b = row_ptr[r + 1];
      const int32_t L = b - a;
      bad |= (L < 0) | (r == 0 && a != 0) | (r == M - 1 && b != nnz);
      atomicAdd(&s_cnt[bin_of(L, edges)], 1);
      my_max = max(my_max, L);
      my_empty += (L == 0);
    }
  }
  // reduce in the wave first, then one LDS atomic per wave
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    my_max = max(my_max, __shfl_xor(my_max, o, kWave));
    my_empty += __shfl_xor(my_empty, o, kWave);
  }
  if (lane_id() == 0) {
    atomicMax(&s_max, my_max);
    atomicAdd(&s_empty, my_empty);
  }
  if (bad) atomicOr((unsigned long long*)&stats[kStatError], (unsigned long long)kErrRowPtr);
  __syncthreads();
  if (tid < edges.n_bins) counts[(int64_t)tid * gridDim.x + blockIdx.x] = s_cnt[tid];
  if (tid == 0) {
    wg_max[blockIdx.x] = s_max;
    wg_empty[blockIdx.x] = s_empty;
  }
}

// Exclusive scan, in place, of the bin-major [bin][workgroup] counts by one
// workgroup; also reduces the longest row and the empty-row count.
__global__ __launch_bounds__(1024) void bin_scan_kernel(
    int32_t M, int32_t n_wg, int32_t n_bins, int32_t* __restrict__ counts,
    const int32_t* __restrict__ wg_max, const int32_t* __restrict__ wg_empty,
    int64_t* __restrict__ stats) {
  __shared__ int32_t s_wave[16];
  __shared__ int32_t s_max[16];
  __shared__ int64_t s_emp[16];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int64_t E = (int64_t)n_bins * n_wg;
  const int64_t per = (E + 1023) / 1024;
  const int64_t beg = min(E, (int64_t)tid * per), end = min(E, beg + per);
  int32_t local = 0;
  for (int64_t i = beg; i < end; ++i) local += counts[i];
  int32_t v = local;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int32_t t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  if (lane == kWave - 1) s_wave[wave] = v;
  int32_t mx = 0;
  int64_t emp = 0;
  for (int w = tid; w < n_wg; w += 1024) {
    mx = max(mx, wg_max[w]);
    emp += wg_empty[w];
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    mx = max(mx, __shfl_xor(mx, o, kWave));
    emp += __shfl_xor(emp, o, kWave);
  }
  if (lane == 0) { s_max[wave] = mx; s_emp[wave] = emp; }
  __syncthreads();
  int32_t wave_base = 0;
  for (int w = 0; w < wave; ++w) wave_base += s_wave[w];
  int32_t run = v - local + wave_base;
  for (int64_t i = beg; i < end; ++i) {
    const int32_t c = counts[i];
    counts[i] = run;
    run += c;
  }
  __syncthreads();
  if (tid == 0) {
    int32_t m = 0;
    int64_t e = 0;
    for (int w = 0; w < 16; ++w) { m = max(m, s_max[w]); e += s_emp[w]; }
    stats[kStatMaxLen] = m;
    stats[kStatEmpty] = e;
    int nonempty = 0;
    for (int b = 0; b < n_bins; ++b) {
      const int64_t off = counts[(int64_t)b * n_wg];
      const int64_t nxt = b + 1 < n_bins ? counts[(int64_t)(b + 1) * n_wg] : M;
      stats[kStatBinOffset + b] = off;
      nonempty += nxt > off;
    }
    stats[kStatBinOffset + n_bins] = M;
    stats[kStatNonEmptyBins] = nonempty;
  }
}

// Pass 2: stable scatter of row ids into their bins. Ranks inside a wave come
// from ballots, ranks across the 4 waves and the 4 passes from LDS counters.
__global__ __launch_bounds__(kBlock) void bin_scatter_kernel(
    const int32_t* __restrict__ row_ptr, int32_t M, BinEdges edges,
    const int32_t* __restrict__ offsets, const int64_t* __restrict__ stats,
    int32_t* __restrict__ bins) {
  if (stats[kStatNonEmptyBins] <= 1) return;  // one bin: ids are the identity
  __shared__ int32_t s_base[kMaxBins];
  __shared__ int32_t s_wcnt[kWavesPerBlock][kMaxBins];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  if (tid < edges.n_bins) s_base[tid] = offsets[(int64_t)tid * gridDim.x + blockIdx.x];
  __syncthreads();
  const int64_t first = (int64_t)blockIdx.x * kBinRowsPerBlock;
  for (int pass = 0; pass < kBinRowsPerBlock / kBlock; ++pass) {
    const int64_t r = first + pass * kBlock + tid;
    const bool valid = r < M;
    const int bin = valid ? bin_of((int64_t)row_ptr[r + 1] - row_ptr[r], edges) : -1;
    int rank = 0;
    for (int b = 0; b < edges.n_bins; ++b) {
      const uint64_t mask = __ballot(bin == b);
      if (bin == b) rank = lanes_below(mask);
      if (lane == 0) s_wcnt[wave][b] = __popcll(mask);
    }
    __syncthreads();
    if (valid) {
      int pos = s_base[bin] + rank;
      for (int w = 0; w < wave; ++w) pos += s_wcnt[w][bin];
      bins[pos] = (int32_t)r;
    }
    __syncthreads();
    if (tid < edges.n_bins) {
      int add = 0;
      for (int w = 0; w < kWavesPerBlock; ++w) add += s_wcnt[w][tid];
      s_base[tid] += add;
    }
    __syncthreads();
  }
}

// Split coordinates of every partition boundary p: at diagonal
// d = min(p*T, M+nnz), rows_ended = max{ i : row_ptr[i] + i <= d } and
// nonzeros = d - rows_ended.
// Also writes, per boundary, the row and that row's first nonzero, the
// boundaries of the stream reduction (rows never cross its partitions).
__device__ __forceinline__ int64_t split_at(const int32_t* __restrict__ row_ptr, int32_t M,
                                            int32_t nnz, int64_t d) {
  int64_t lo = max((int64_t)0, d - nnz), hi = min(d, (int64_t)M);
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if ((int64_t)row_ptr[mid] + mid <= d) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Decisions the plan takes on the device, so that the host reads the
// statistics back once, at the end. One thread.
//  stage 0 -- items per lane: given by the caller, else from the row lengths:
//    4 (T = 256) when every row has <= 32 entries and the mean is < 12 (short
//    rows: more, smaller partitions keep the tail of the launch short), else
//    16 for fp32 and 8 for fp64 (whose staging needs twice the LDS per unit).
//  stage 1 -- after the split at that size: walk plans (some row longer than
//    T/8) whose x is larger than one XCD's L2 and whose partitions mostly
//    hold row ends are split again at T = 256 (their gathers are bound by the
//    L1 misses in flight, and T = 256 runs twice the waves per CU).
//  stage 3 -- (after the window spans and the tile plan) x slabs, see
//    slab_kernels.hip.
//  stage 2 -- walk plans deal their partitions in column order when at least
//    an eighth of them lie inside one row and every row covers under a
//    quarter of the columns (or when the caller asks for it); and walk plans
//    whose x spans more than one tile block may tile their long rows (the
//    tile plan keeps them, and the partition order, when they hold at least
//    half of the nonzeros).
__global__ __launch_bounds__(64) void plan_choose_kernel(const PlanCtl c, int64_t* stats,
                                                         int stage) {
  if (threadIdx.x != 0) return;
  const int64_t W = c.M + c.nnz;
  const int64_t err = stats[kStatError];
  const int64_t max_len = stats[kStatMaxLen];
  if (stage == 0) {
    int ipt = c.forced_ipt;
    if (ipt == 0) {
      const double avg = c.M > 0 ? (double)c.nnz / (double)c.M : 0.0;
      ipt = (err & kErrRowPtr) ? 4 : (max_len <= 32 && avg < 12.0) ? 4 : c.vbytes == 4 ? 16 : 8;
    }
    stats[kStatIpt] = ipt;
    stats[kStatParts] = (W + kWave * ipt - 1) / (kWave * ipt);
    stats[kStatResplit] = 0;
    stats[kStatOrder] = 0;
  } else if (stage == 1) {
    const int64_t ipt = stats[kStatIpt];
    const int64_t T = kWave * ipt;
    if (c.forced_ipt == 0 && ipt > 4 && !(err & (kErrRowPtr | kErrColumn)) && max_len > T / 8 &&
        c.wide_x && 2 * stats[kStatInterior] < stats[kStatParts]) {
      stats[kStatIpt] = 4;
      stats[kStatParts] = (W + kWave * 4 - 1) / (kWave * 4);
      stats[kStatResplit] = 1;
      stats[kStatInterior] = 0;
    }
  } else if (stage == 2) {
    const int64_t T = kWave * stats[kStatIpt], P = stats[kStatParts];
    const bool walk = c.reduce_req == 1 || (c.reduce_req == 0 && max_len > T / 8);
    int d = c.order_req;
    if (d == 0) d = 8 * stats[kStatInterior] >= P && 4 * max_len < c.N ? 2 : 1;
    stats[kStatOrder] = walk && P > 0 && c.nnz > 0 && !(err & kErrRowPtr) && d == 2;
    // long rows may be tiled by column block (walk plans whose x spans more
    // than one block; their runs are found next)
    const int64_t bc = kTileBytes / c.vbytes;
    stats[kStatTileOk] = walk && c.tiles_req != 1 && c.order_req != 2 && P > 0 && c.nnz > 0 &&
                         !(err & kErrRowPtr) && c.N > bc;
  } else if (stage == 3) {
    // after the window spans and the tile plan: x slabs where the gathers
    // spread over an x wider than one XCD's L2 -- walk plans split again at
    // T = 256 (partitions mostly holding row ends), stream plans whose
    // workgroups' columns fit no x window -- or over an x of 1..4 MiB when
    // rows are long enough to pay for the combine (mid_x: walk plans whose
    // partitions mostly hold row ends, the same stream plans), and no tiles
    // are kept; or whenever the caller asks for them
    const int64_t T = kWave * stats[kStatIpt], P = stats[kStatParts];
    const bool walk = c.reduce_req == 1 || (c.reduce_req == 0 && max_len > T / 8);
    const int64_t S = stats[kStatWindowSamples];
    const bool spread = !walk && S > 0 && 2 * stats[kStatWindowFits] < S &&
                        2 * stats[kStatWindowFitsMulti] < S;
    const bool ok = c.slab_room && c.slabs_req != 1 && P > 0 && c.nnz > 0 &&
                    !(err & (kErrRowPtr | kErrColumn)) && stats[kStatTileRows] == 0;
    const bool wide = c.wide_x && ((walk && stats[kStatResplit] != 0) || spread);
    const bool mid = c.mid_x && ((walk && 2 * stats[kStatInterior] < P) || spread);
    stats[kStatSlabOk] = ok && (c.slabs_req == 2 || wide || mid);
  }
}

__global__ __launch_bounds__(kBlock) void split_search_kernel(
    const int32_t* __restrict__ row_ptr, int32_t M, int32_t nnz, int pass,
    int32_t* __restrict__ split_row, int32_t* __restrict__ split_nz,
    int32_t* __restrict__ row_bounds, int64_t* __restrict__ stats) {
  if (pass == 1 && stats[kStatResplit] == 0) return;
  const int64_t T = kWave * stats[kStatIpt];
  const int64_t P = stats[kStatParts];
  if ((int64_t)blockIdx.x * kBlock > P) return;   // workgroup-uniform
  __shared__ int64_t s_lo[kBlock + 1];
  __shared__ int s_cnt[kWavesPerBlock];
  const int t = threadIdx.x;
  const int64_t p = (int64_t)blockIdx.x * kBlock + t;
  const int64_t W = (int64_t)M + nnz;
  int64_t lo = -1;
  if (p <= P) {
    const int64_t d = min(p * T, W);
    lo = split_at(row_ptr, M, nnz, d);
    split_row[p] = (int32_t)lo;
    split_nz[p] = (int32_t)(d - lo);
    row_bounds[2 * p] = (int32_t)lo;
    row_bounds[2 * p + 1] = row_ptr[lo];
  }
  s_lo[t] = lo;
  // the next block's first boundary, for this block's last partition
  if (t == kBlock - 1) s_lo[kBlock] = p + 1 <= P ? split_at(row_ptr, M, nnz, min((p + 1) * T, W)) : -1;
  __syncthreads();
  // partition p is interior when no row ends in it (same split row at both ends)
  const bool interior = p < P && s_lo[t + 1] == lo;
  const int c = __popcll(__ballot(interior));
  if (lane_id() == 0) s_cnt[t / kWave] = c;
  __syncthreads();
  if (t == 0) {
    int total = 0;
    for (int w = 0; w < kWavesPerBlock; ++w) total += s_cnt[w];
    if (total) atomicAdd((unsigned long long*)&stats[kStatInterior], (unsigned long long)total);
  }
}

// Column dispatch order: key of each walk partition, the column of its
// middle nonzero (0 when it has none). Only when the plan chose that order.
__global__ __launch_bounds__(kBlock) void partition_keys_kernel(
    const int32_t* __restrict__ split_nz, const int32_t* __restrict__ col_idx,
    const int64_t* __restrict__ stats, int32_t* __restrict__ keys) {
  if (stats[kStatOrder] == 0) return;
  const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (p >= stats[kStatParts]) return;
  const int n0 = split_nz[p], n1 = split_nz[p + 1];
  keys[p] = n1 > n0 ? col_idx[n0 + (n1 - n0) / 2] : 0;
}

__global__ __launch_bounds__(kBlock) void check_columns_kernel(
    const int32_t* __restrict__ col_idx, int64_t nnz, int64_t N, int64_t* stats) {
  bool bad = false;
  for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < nnz;
       k += (int64_t)gridDim.x * kBlock) {
    const int32_t c = col_idx[k];
    bad |= (c < 0) | ((int64_t)c >= N);
  }
  if (bad) atomicOr((unsigned long long*)&stats[kStatError], (unsigned long long)kErrColumn);
}

// x window of each group of `group` consecutive stream partitions: up to
// kWinIntervals column intervals that together cover every column of the
// group's nonzero quads (the range widened to whole 16-byte quads, as the
// exec kernel stages it), each widened to whole 16-byte chunks of x (e
// elements) and kept inside x's full chunks, their total within cap entries.
// One interval (the whole span) when that fits; otherwise the span is cut
// into 256 buckets, the runs of buckets that hold columns become the
// intervals (at most kWinIntervals runs), tightened to the exact min and max
// column of each run. Writes win_span[8g ..]: {lo, len} per interval (len 0:
// unused), then the total length and flags (bit 0: the columns fit one
// interval, bit 1: they fit the intervals). This only prepares a
// kernel variant: the exec kernel checks every column against the intervals
// again and gathers from global x when one is outside.
// Whether the plan's stream kernel has a window at all (stream reduction,
// a window at this partition size, a well-formed row_ptr), and its
// capacity in elements.
__device__ __forceinline__ int window_cap(const PlanCtl& c, const int64_t* stats) {
  const int64_t ipt = stats[kStatIpt];
  const bool stream = c.reduce_req == 2 ||
                      (c.reduce_req == 0 && stats[kStatMaxLen] <= kWave * ipt / 8);
  if (!stream || c.nnz == 0 || (stats[kStatError] & kErrRowPtr)) return 0;
  return stream_window_bytes((int)ipt, c.vbytes, kWavesPerBlock) / c.vbytes;
}

__global__ __launch_bounds__(kBlock) void window_span_kernel(
    const PlanCtl ctl, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const int32_t* __restrict__ split_row, const int64_t* __restrict__ stats,
    int32_t* __restrict__ win_span) {
  constexpr int NB = kBlock;            // buckets
  const int cap = window_cap(ctl, stats);
  const int group = kWavesPerBlock;
  const int P = (int)stats[kStatParts];
  if (cap == 0 || (int64_t)blockIdx.x * group >= P) return;   // workgroup-uniform
  const int nnz = (int)ctl.nnz, N = (int)ctl.N, e = 16 / ctl.vbytes;
  __shared__ int32_t s_lo[kWavesPerBlock], s_hi[kWavesPerBlock];
  __shared__ int32_t s_flag[NB], s_run[NB];
  __shared__ int32_t s_rlo[NB], s_rhi[NB];
  __shared__ int32_t s_nrun;
  const int g = blockIdx.x;
  const int t = threadIdx.x;
  const int p0 = g * group, p1 = min(p0 + group, P);
  // 64-bit positions: strides past nnz near 2^31 must not wrap
  int64_t k0 = row_ptr[split_row[p0]], k1 = row_ptr[split_row[p1]];
  if (k1 > k0) {
    k0 &= ~int64_t(3);
    k1 = min((k1 + 3) & ~int64_t(3), (int64_t)nnz);
  }
  int lo = INT_MAX, hi = INT_MIN;
  for (int64_t k = k0 + t; k < k1; k += kBlock) {
    const int c = col_idx[k];
    lo = min(lo, c);
    hi = max(hi, c);
  }
  for (int o = kWave / 2; o > 0; o >>= 1) {
    lo = min(lo, __shfl_xor(lo, o, kWave));
    hi = max(hi, __shfl_xor(hi, o, kWave));
  }
  if (lane_id() == 0) {
    s_lo[t / kWave] = lo;
    s_hi[t / kWave] = hi;
  }
  s_flag[t] = 0;
  s_rlo[t] = INT_MAX;
  s_rhi[t] = INT_MIN;
  __syncthreads();
  lo = min(min(s_lo[0], s_lo[1]), min(s_lo[2], s_lo[3]));
  hi = max(max(s_hi[0], s_hi[1]), max(s_hi[2], s_hi[3]));
  int32_t* out = win_span + (int64_t)kWinTable * g;
  const int last_full = (N / e) * e - 1;   // last column of x's full chunks
  // (lo, hi) are block-uniform from here on
  if (hi < lo) {
    if (t < kWinTable) out[t] = 0;
    return;
  }
  const int alo = lo & ~(e - 1), ahi = hi | (e - 1);
  if (ahi <= last_full && ahi - alo < cap) {            // one interval
    if (t < kWinTable)
      out[t] = t == 0 ? alo : (t == 1 || t == 2 * kWinIntervals) ? ahi - alo + 1
                        : t == kWinTable - 1 ? 3 : 0;
    return;
  }
  // buckets of width w over [lo, hi] (hi - lo < 2^31: columns are int32 and
  // non-negative); mark the ones that hold a column
  const unsigned w = ((unsigned)(hi - lo) + NB) / NB;
  for (int64_t k = k0 + t; k < k1; k += kBlock) s_flag[(unsigned)(col_idx[k] - lo) / w] = 1;
  __syncthreads();
  // runs of marked buckets: run id by a block scan of the run starts
  const int start = s_flag[t] && (t == 0 || !s_flag[t - 1]);
  s_run[t] = start;
  __syncthreads();
  for (int o = 1; o < NB; o <<= 1) {
    const int v = t >= o ? s_run[t - o] : 0;
    __syncthreads();
    s_run[t] += v;
    __syncthreads();
  }
  if (t == NB - 1) s_nrun = s_run[t];
  __syncthreads();
  const int nrun = s_nrun;
  if (nrun <= kWinIntervals) {
    // exact min / max column of each run (run id of bucket b: s_run[b] - 1),
    // per lane, then per wave, then one LDS atomic per wave and run
    int rlo[kWinIntervals], rhi[kWinIntervals];
#pragma unroll
    for (int q = 0; q < kWinIntervals; ++q) {
      rlo[q] = INT_MAX;
      rhi[q] = INT_MIN;
    }
    for (int64_t k = k0 + t; k < k1; k += kBlock) {
      const int c = col_idx[k];
      const int r = s_run[(unsigned)(c - lo) / w] - 1;
#pragma unroll
      for (int q = 0; q < kWinIntervals; ++q) {
        rlo[q] = r == q ? min(rlo[q], c) : rlo[q];
        rhi[q] = r == q ? max(rhi[q], c) : rhi[q];
      }
    }
#pragma unroll
    for (int q = 0; q < kWinIntervals; ++q) {
      for (int o = kWave / 2; o > 0; o >>= 1) {
        rlo[q] = min(rlo[q], __shfl_xor(rlo[q], o, kWave));
        rhi[q] = max(rhi[q], __shfl_xor(rhi[q], o, kWave));
      }
      if (lane_id() == 0 && q < nrun) {
        atomicMin(&s_rlo[q], rlo[q]);
        atomicMax(&s_rhi[q], rhi[q]);
      }
    }
  }
  __syncthreads();
  if (t == 0) {
    int ilo[kWinIntervals], ilen[kWinIntervals], n = 0, total = 0;
    bool ok = nrun <= kWinIntervals;
    for (int r = 0; ok && r < nrun; ++r) {
      int a = s_rlo[r] & ~(e - 1), b = s_rhi[r] | (e - 1);
      if (b > last_full) ok = false;               // a column in x's last partial chunk
      if (n > 0 && a <= ilo[n - 1] + ilen[n - 1]) {   // touches the previous one: merge
        a = ilo[n - 1];
        total -= ilen[n - 1];
        --n;
      }
      ilo[n] = a;
      ilen[n] = b - a + 1;
      total += ilen[n];
      ++n;
    }
    ok = ok && total <= cap;
    for (int k = 0; k < kWinIntervals; ++k) {
      out[2 * k] = ok && k < n ? ilo[k] : 0;
      out[2 * k + 1] = ok && k < n ? ilen[k] : 0;
    }
    out[2 * kWinIntervals] = ok ? total : 0;
    for (int k = 2 * kWinIntervals + 1; k < kWinTable - 1; ++k) out[k] = 0;
    out[kWinTable - 1] = ok ? 2 : 0;
  }
}

// Sums the window table's flags into the statistics block: groups examined,
// groups that fit one interval, groups that fit the intervals. A grid-stride
// pass with one global atomic per workgroup and counter (thousands of groups
// each adding to one address would serialise on it).
__global__ __launch_bounds__(kBlock) void window_count_kernel(const PlanCtl ctl,
                                                              const int32_t* __restrict__ win_span,
                                                              int64_t* stats) {
  if (window_cap(ctl, stats) == 0) return;
  const int groups = (int)((stats[kStatParts] + kWavesPerBlock - 1) / kWavesPerBlock);
  __shared__ int s_sum[3][kWavesPerBlock];
  int cnt[3] = {0, 0, 0};   // groups, fit one interval, fit the intervals
  for (int g = blockIdx.x * kBlock + threadIdx.x; g < groups; g += gridDim.x * kBlock) {
    const int f = win_span[(int64_t)kWinTable * g + kWinTable - 1];
    cnt[0] += 1;
    cnt[1] += f & 1;
    cnt[2] += (f >> 1) & 1;
  }
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    for (int o = kWave / 2; o > 0; o >>= 1) cnt[q] += __shfl_xor(cnt[q], o, kWave);
    if (lane_id() == 0) s_sum[q][threadIdx.x / kWave] = cnt[q];
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    const int q = threadIdx.x;
    unsigned long long sum = 0;
    for (int i = 0; i < kWavesPerBlock; ++i) sum += (unsigned)s_sum[q][i];
    const int slot = q == 0 ? kStatWindowSamples : q == 1 ? kStatWindowFits : kStatWindowFitsMulti;
    atomicAdd((unsigned long long*)&stats[slot], sum);
  }
}

// COO input, "A Programming Model for GPU Load Balancing" (PPoPP'23),
// Section 3.1: the same atoms (nonzeros) and tiles (rows), given one row
// index per atom instead of row offsets. With the row indices sorted, row r's
// atoms start at the first index >= r: row_ptr[r] = lower_bound(row_idx, r),
// one binary search per row, and every CSR step then applies unchanged.
__global__ __launch_bounds__(kBlock) void coo_row_ptr_kernel(const int32_t* __restrict__ row_idx,
                                                             int32_t nnz, int32_t M,
                                                             int32_t* __restrict__ row_ptr) {
  const int64_t r = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (r > M) return;
  int lo = 0, hi = nnz;
  while (lo < hi) {
    const int mid = (int)(((int64_t)lo + hi) >> 1);
    if (row_idx[mid] < r) lo = mid + 1;
    else hi = mid;
  }
  row_ptr[r] = lo;
}

// flag |= 1 when a row index is outside [0, M) or smaller than its
// predecessor (the offsets above need them sorted)
__global__ __launch_bounds__(kBlock) void coo_check_kernel(const int32_t* __restrict__ row_idx,
                                                           int64_t nnz, int32_t M,
                                                           int64_t* stats) {
  bool bad = false;
  for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < nnz;
       e += (int64_t)gridDim.x * kBlock) {
    const int32_t r = row_idx[e];
    bad |= r < 0 || r >= M || (e + 1 < nnz && row_idx[e + 1] < r);
  }
  if (__ballot(bad) != 0 && lane_id() == 0)
    atomicOr((unsigned long long*)&stats[kStatError], (unsigned long long)kErrCooRows);
}

__global__ __launch_bounds__(64) void fold_flag_kernel(const int32_t* flag, int64_t bits,
                                                       int64_t* stats) {
  if (threadIdx.x == 0 && *flag != 0)
    atomicOr((unsigned long long*)&stats[kStatError], (unsigned long long)bits);
}

// flag |= 1 unless row_ptr[0] = 0, row_ptr[M] = nnz and row_ptr never
// decreases
__global__ __launch_bounds__(kBlock) void csr_check_kernel(const int32_t* __restrict__ row_ptr,
                                                           int64_t M, int64_t nnz, int32_t* flag) {
  bool bad = false;
  for (int64_t r = (int64_t)blockIdx.x * kBlock + threadIdx.x; r <= M;
       r += (int64_t)gridDim.x * kBlock) {
    const int32_t v = row_ptr[r];
    bad |= (r == 0 && v != 0) || (r == M && v != nnz) || (r < M && row_ptr[r + 1] < v);
  }
  if (__ballot(bad) != 0 && lane_id() == 0) atomicOr(flag, 1);
}

// Entries of A^T in column order of A: entry t of the sorted order is A's
// entry perm[t]; its column in A^T is the row of A holding it (the last row
// whose start is <= the entry), its value is copied.
template <typename V>
__global__ __launch_bounds__(kBlock) void transpose_gather_kernel(
    const int32_t* __restrict__ row_ptr, int32_t M, const int32_t* __restrict__ perm,
    const V* __restrict__ values, int64_t nnz, int32_t* __restrict__ col_t, V* __restrict__ val_t) {
  for (int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x; t < nnz;
       t += (int64_t)gridDim.x * kBlock) {
    const int32_t e = perm[t];
    int lo = 0, hi = M;   // last row r with row_ptr[r] <= e
    while (lo < hi) {
      const int mid = (int)(((int64_t)lo + hi + 1) >> 1);
      if (row_ptr[mid] <= e) lo = mid;
      else hi = mid - 1;
    }
    col_t[t] = lo;
    val_t[t] = values[e];
  }
}

int n_blocks(int64_t n, int64_t per) { return (int)((n + per - 1) / per); }

}  // namespace

hipError_t launch_clear_stats(int64_t* stats, hipStream_t s) {
  hipLaunchKernelGGL(clear_stats_kernel, dim3(1), dim3(64), 0, s, stats);
  return hipGetLastError();
}

hipError_t launch_bin_count(const int32_t* row_ptr, int64_t M, int64_t nnz,
                            const BinEdges& edges, int32_t* counts, int32_t* wg_max,
                            int32_t* wg_empty, int64_t* stats, hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(bin_count_kernel, dim3(n_blocks(M, kBinRowsPerBlock)), dim3(kBlock), 0, s,
                     row_ptr, (int32_t)M, (int32_t)nnz, edges, counts, wg_max, wg_empty, stats);
  return hipGetLastError();
}

hipError_t launch_bin_scan(int64_t M, const BinEdges& edges, int32_t* counts,
                           const int32_t* wg_max, const int32_t* wg_empty, int64_t* stats,
                           hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(bin_scan_kernel, dim3(1), dim3(1024), 0, s, (int32_t)M,
                     n_blocks(M, kBinRowsPerBlock), edges.n_bins, counts, wg_max, wg_empty,
                     stats);
  return hipGetLastError();
}

hipError_t launch_bin_scatter(const int32_t* row_ptr, int64_t M, const BinEdges& edges,
                              const int32_t* offsets, const int64_t* stats, int32_t* bins,
                              hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(bin_scatter_kernel, dim3(n_blocks(M, kBinRowsPerBlock)), dim3(kBlock), 0,
                     s, row_ptr, (int32_t)M, edges, offsets, stats, bins);
  return hipGetLastError();
}

hipError_t launch_plan_choose(const PlanCtl& c, int64_t* stats, int stage, hipStream_t s) {
  hipLaunchKernelGGL(plan_choose_kernel, dim3(1), dim3(64), 0, s, c, stats, stage);
  return hipGetLastError();
}

hipError_t launch_partition_keys(const int32_t* split_nz, const int32_t* col_idx, int64_t p_max,
                                 const int64_t* stats, int32_t* keys, hipStream_t s) {
  if (p_max <= 0) return hipSuccess;
  hipLaunchKernelGGL(partition_keys_kernel, dim3(n_blocks(p_max, kBlock)), dim3(kBlock), 0, s,
                     split_nz, col_idx, stats, keys);
  return hipGetLastError();
}

hipError_t launch_split_search(const int32_t* row_ptr, int64_t M, int64_t nnz, int64_t p_max,
                               int pass, int32_t* split_row, int32_t* split_nz,
                               int32_t* row_bounds, int64_t* stats, hipStream_t s) {
  hipLaunchKernelGGL(split_search_kernel, dim3(n_blocks(p_max + 1, kBlock)), dim3(kBlock), 0, s,
                     row_ptr, (int32_t)M, (int32_t)nnz, pass, split_row, split_nz, row_bounds,
                     stats);
  return hipGetLastError();
}

hipError_t launch_window_spans(const PlanCtl& c, const int32_t* row_ptr, const int32_t* col_idx,
                               const int32_t* split_row, int64_t p_max, int32_t* win_span,
                               int64_t* stats, hipStream_t s) {
  if (p_max <= 0 || c.nnz == 0) return hipSuccess;
  const int64_t groups = (p_max + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(window_span_kernel, dim3((unsigned)groups), dim3(kBlock), 0, s, c, row_ptr,
                     col_idx, split_row, stats, win_span);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(window_count_kernel, dim3((int)std::min<int64_t>(n_blocks(groups, kBlock), 64)),
                     dim3(kBlock), 0, s, c, win_span, stats);
  return hipGetLastError();
}

hipError_t launch_fold_flag(const int32_t* flag, int64_t bits, int64_t* stats, hipStream_t s) {
  hipLaunchKernelGGL(fold_flag_kernel, dim3(1), dim3(64), 0, s, flag, bits, stats);
  return hipGetLastError();
}

hipError_t launch_coo_row_ptr(const int32_t* row_idx, int64_t nnz, int64_t M, int32_t* row_ptr,
                              int64_t* stats, hipStream_t s) {
  if (nnz > 0) {
    const int blocks = (int)std::min<int64_t>(n_blocks(nnz, kBlock), 8192);
    hipLaunchKernelGGL(coo_check_kernel, dim3(blocks), dim3(kBlock), 0, s, row_idx, nnz,
                       (int32_t)M, stats);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(coo_row_ptr_kernel, dim3(n_blocks(M + 1, kBlock)), dim3(kBlock), 0, s,
                     row_idx, (int32_t)nnz, (int32_t)M, row_ptr);
  return hipGetLastError();
}

hipError_t launch_csr_check(const int32_t* row_ptr, int64_t M, int64_t nnz, int32_t* flag,
                            hipStream_t s) {
  const int blocks = (int)std::min<int64_t>(n_blocks(M + 1, kBlock), 8192);
  hipLaunchKernelGGL(csr_check_kernel, dim3(blocks), dim3(kBlock), 0, s, row_ptr, M, nnz, flag);
  return hipGetLastError();
}

hipError_t launch_transpose_gather(const int32_t* row_ptr, int64_t M, const int32_t* perm,
                                   const void* values, int vbytes, int64_t nnz, int32_t* col_t,
                                   void* val_t, hipStream_t s) {
  if (nnz == 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>(n_blocks(nnz, kBlock), 65536);
  if (vbytes == 4)
    hipLaunchKernelGGL(transpose_gather_kernel<float>, dim3(blocks), dim3(kBlock), 0, s, row_ptr,
                       (int32_t)M, perm, static_cast<const float*>(values), nnz, col_t,
                       static_cast<float*>(val_t));
  else
    hipLaunchKernelGGL(transpose_gather_kernel<double>, dim3(blocks), dim3(kBlock), 0, s,
                       row_ptr, (int32_t)M, perm, static_cast<const double*>(values), nnz,
                       col_t, static_cast<double*>(val_t));
  return hipGetLastError();
}

hipError_t launch_check_columns(const int32_t* col_idx, int64_t nnz, int64_t N,
                                int64_t* stats, hipStream_t s) {
  if (nnz == 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>(n_blocks(nnz, kBlock), 8192);
  hipLaunchKernelGGL(check_columns_kernel, dim3(blocks), dim3(kBlock), 0, s, col_idx, nnz, N,
                     stats);
  return hipGetLastError();
}

}  // namespace spmv
