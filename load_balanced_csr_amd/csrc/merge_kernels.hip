// Merge-path CSR SpMV for gfx950: y = alpha * A x + beta * y.
//
// Schedule: "A Programming Model for GPU Load Balancing" (Osama, Porumbescu,
// Owens, PPoPP'23), Section 5.2.1. Every nonzero and every row end is one
// unit of work; the M + nnz units, taken in order (a row's nonzeros, then its
// end), are cut into partitions of T units. A partition's start (rows ended,
// nonzeros consumed) comes from the plan's split search. Rows cut by a
// partition boundary are completed by the segmented fix-up step that the
// page's Sidebar 1 describes for the CUB implementation.
//
// MI355X mapping (not the page's): one 64-lane wavefront owns one partition
// of T = 64 * IPT units. It
//   1. stages its row-end offsets and its products val[k] * x[col[k]] in LDS,
//      loading col_idx/values with coalesced 64-lane non-temporal loads, all
//      IPT loads of a lane issued before the first use;
//   2. lets each lane find its own start inside the partition by a binary
//      search in LDS and walk IPT units in order, keeping a running sum;
//   3. combines the lanes' open-row sums with a wave segmented scan keyed by
//      row (no LDS atomics, no float atomics);
//   4. writes the finished rows' y with coalesced stores, applying alpha and
//      beta once, and leaves the sum of the row still open at its end as the
//      partition's carry.
// The fix-up kernel adds alpha * (carries of a row) to that row, combining a
// row's carries with a wave segmented scan, deterministically.
#include "device_common.hpp"
#include "internal.hpp"
#include "tile_exec.hpp"

#include <limits.h>

namespace spmv {
namespace {

// LDS of one wave's partition: row ends (int32) and sums / products (V),
// T + 8 of each.
template <typename V, int IPT>
constexpr int walk_lds_bytes() { return kWavesPerBlock * (kWave * IPT + 8) * (4 + (int)sizeof(V)); }

// One wave walks partition slot `slot` of the dispatch (all P partitions,
// or the n_dispatch of the plan's list), with its LDS at s_end / s_val.
// MASK: with long-row tiles, a partition leaves the nonzeros outside
// [mask_end[p], mask_start[p]) to them (their products are 0 here).
template <typename V, int IPT, bool MASK>
__device__ __forceinline__ void walk_partition(const MergeArgs<V>& a, int slot, int32_t* s_end,
                                               V* s_val) {
  constexpr int T = kWave * IPT;
  constexpr int RQ = (T / 4 + 2 + kWave - 1) / kWave;   // quad rounds per array
  const int lane = lane_id();
  int p = slot;
  if (p >= (a.n_dispatch ? a.n_dispatch : a.P)) return;
  // column dispatch order, or the partitions that long-row tiles leave: the
  // plan's list of partitions (a uniform read of a table nothing here writes)
  if (a.part_order) p = a.part_order[p];

  const int r0 = a.split_row[p], r1 = a.split_row[p + 1];
  const int n0 = a.split_nz[p], n1 = a.split_nz[p + 1];
  const int nrows = r1 - r0, nnzc = n1 - n0, total = nrows + nnzc;

  // ---- 1. stage row ends and products with 16-byte loads ---------------------
  // re[k]: local nonzero offset where row r0+k ends (row_ptr[r0+1+k] - n0).
  // vb holds the finished rows' sums at [0, nrows) and, at its far end, the
  // products of the quads covering [n0, n1): nrows + nnzc <= T keeps the two
  // regions apart.
  const int qr0 = (r0 + 1) >> 2;
  const int nqr = nrows > 0 ? ((r1 >> 2) - qr0 + 1) : 0;
  const int qn0 = n0 >> 2;
  const int nqn = nnzc > 0 ? (((n1 - 1) >> 2) - qn0 + 1) : 0;
  int32_t* re = s_end + ((r0 + 1) & 3);
  V* vb = s_val;
  V* prod_q = vb + (T + 8 - 4 * nqn);
  V* prod = prod_q + (n0 & 3);
  const int mlo = MASK ? a.mask_end[p] : 0;
  const int mhi = MASK ? a.mask_start[p] : INT_MAX;
  stage_partition<V, RQ, RQ, MASK>(a.row_ptr, a.M + 1, qr0, nqr, n0, a.col_idx, a.val, a.x,
                                   a.nnz, qn0, nqn, s_end, prod_q, mlo, mhi);
  wave_sync();

  // ---- 2. per-lane start by binary search, then walk IPT units --------------
  const int d = min(lane * IPT, total);
  int lo = max(0, d - nnzc), hi = min(d, nrows);
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (re[mid - 1] + mid - 1 < d) lo = mid; else hi = mid - 1;
  }
  int ri = lo, ni = d - lo;
  const int cnt = min(IPT, total - d);
  int next_end = ri < nrows ? re[ri] : INT_MAX;
  V acc = V(0);
  int first_row = -1;
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    if (it < cnt) {
      if (next_end <= ni) {            // unit = end of row ri
        vb[ri] = acc;
        first_row = first_row < 0 ? ri : first_row;
        acc = V(0);
        ++ri;
        next_end = ri < nrows ? re[ri] : INT_MAX;
      } else {                         // unit = nonzero ni
        acc += prod[ni];
        ++ni;
      }
    }
  }

  // ---- 3. combine open-row sums across lanes ---------------------------------
  // Lane l starts inside the row lane l-1 ended in, so the sum flowing into
  // lane l's first finished row is the segmented scan value of lane l-1
  // (DPP moves only: the scan keys are the lanes' open rows, which never
  // decrease across the lanes).
  const V s = wave_segscan_keys(acc, ri);
  const V incoming = lane_prev(s);
  if (first_row >= 0) vb[first_row] += incoming;
  wave_sync();

  // ---- 4. finished rows, then the carry of the open row -----------------------
  for (int k = lane; k < nrows; k += kWave) {
    V out = a.alpha * vb[k];
    if (a.beta_nonzero) out = fma(a.beta, ld_stream(a.y + r0 + k), out);
    st_stream(a.y + r0 + k, out);
  }
  if (lane == kWave - 1) {
    a.carry_row[p] = r1;
    a.carry_val[p] = s;
  }
}

template <typename V, int IPT>
__global__ __launch_bounds__(kBlock) void merge_spmv_kernel(const MergeArgs<V> a) {
  constexpr int T = kWave * IPT;
  __shared__ __attribute__((aligned(16))) int32_t s_end[kWavesPerBlock][T + 8];
  __shared__ __attribute__((aligned(16))) V s_val[kWavesPerBlock][T + 8];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int blk = a.xcd_remap ? xcd_tile(blockIdx.x, 0, gridDim.x) : (int)blockIdx.x;
  walk_partition<V, IPT, false>(a, blk * kWavesPerBlock + wave, s_end[wave], s_val[wave]);
}

// The walk over the partitions long-row tiles leave and the tiles
// themselves, in one grid: workgroups [0, walk_blocks) walk (one partition
// per wave, masked), the rest each take one tile. The two share no output
// (tiles write only their block partials). Workgroups are dispatched about
// in index order, so the walk of the short rows runs first, with the tiles
// filling the CUs as its workgroups end, in one launch. One LDS buffer
// serves either role.
template <typename V, int IPT>
__global__ __launch_bounds__(kBlock) void walk_tile_kernel(const MergeArgs<V> a,
                                                           const TileArgs<V> t, int walk_blocks) {
  constexpr int T = kWave * IPT;
  constexpr int LDS = walk_lds_bytes<V, IPT>() > kTileBytes ? walk_lds_bytes<V, IPT>() : kTileBytes;
  __shared__ __attribute__((aligned(16))) char lds[LDS];
  const int b = blockIdx.x;
  if (b < walk_blocks) {   // workgroup-uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int blk = a.xcd_remap ? xcd_tile(b, 0, walk_blocks) : b;
    int32_t* ends = reinterpret_cast<int32_t*>(lds) + wave * (T + 8);
    V* vals = reinterpret_cast<V*>(lds + kWavesPerBlock * (T + 8) * 4) + wave * (T + 8);
    walk_partition<V, IPT, true>(a, blk * kWavesPerBlock + wave, ends, vals);
  } else {
    tile_block<V>(t, xcd_tile(b, walk_blocks, (int)gridDim.x - walk_blocks),
                  reinterpret_cast<V*>(lds));
  }
}

// Stream reduction, used when every row holds at most T/8 entries. The
// partitions keep the merge-path row coordinate (rows ended before the
// diagonal) but start their nonzeros at that row's start, so no row crosses a
// partition: a partition owns rows [r0, r1) whole and nonzeros
// [row_ptr[r0], row_ptr[r1]); rows + nonzeros <= T + T/8 (the row cut by the
// diagonal moves forward entirely). There are no carries and no fix-up.
//
// The kernel is bound by latency x occupancy, so it keeps one small LDS
// buffer per wave: products at the front, row ends (int32) at the back.
// With WIN, each workgroup first fetches the span of x its entries use
// (recorded by the plan) straight into LDS with direct-to-LDS 16-byte loads,
// which need no registers and overlap the partition's own loads; the gathers
// then read LDS. Groups of G lanes sum each row (strided by G, then a
// butterfly), 64 / G rows per round.
// An x window of up to three column intervals, packed in LDS in column
// order. The bounds are wave-uniform (scalar registers); an unused interval
// has length 0.
struct WindowBounds {
  int lo[kWinIntervals], len[kWinIntervals];
  // LDS slot of column col, or -1 when no interval holds it: the column
  // belongs to the last non-empty interval starting at or below it.
  template <int WK>
  __device__ __forceinline__ int slot(int col) const {
    if (WK == 1) return (unsigned)(col - lo[0]) < (unsigned)len[0] ? col - lo[0] : -1;
    const bool a1 = len[1] > 0 && col >= lo[1];
    const bool a2 = len[2] > 0 && col >= lo[2];
    const int l = a2 ? lo[2] : a1 ? lo[1] : lo[0];
    const int n = a2 ? len[2] : a1 ? len[1] : len[0];
    const int base = a2 ? len[0] + len[1] : a1 ? len[0] : 0;
    return (unsigned)(col - l) < (unsigned)n ? base + (col - l) : -1;
  }
};

template <typename V, int NR, int NN, int WK>
__device__ __forceinline__ void stream_stage(const MergeArgs<V>& a, int qr0, int nqr, int n0,
                                             int qn0, int nqn, int32_t* ends, V* prods,
                                             const V* xs, const int* win_meta) {
  constexpr bool WIN = WK > 0;
  const int lane = lane_id();
  i32x4 e[NR > 0 ? NR : 1];
  i32x4 c[NN > 0 ? NN : 1];
  Quad<V> v[NN > 0 ? NN : 1];
  // all column quads, then all value quads, then the row ends (needed last,
  // for the LDS store): the gathers wait only for the columns, and nothing
  // computed from the row ends sits in front of the other loads
  // (partition-relative 32-bit byte offsets from wave-uniform bases)
  const int32_t* cb = a.col_idx + 4 * (int64_t)qn0;
  const V* vb = a.val + 4 * (int64_t)qn0;
  const int32_t* eb = a.row_ptr + 4 * (int64_t)qr0;
#pragma unroll
  for (int r = 0; r < NN; ++r)
    c[r] = ld_stream_at<i32x4>(cb, 16u * (uint32_t)min(lane + kWave * r, nqn - 1));
#pragma unroll
  for (int r = 0; r < NN; ++r) {
    const uint32_t off = 16u * (uint32_t)min(lane + kWave * r, nqn - 1);
    if constexpr (sizeof(V) == 4) {
      v[r].v = ld_stream_at<f32x4>(vb, off);
    } else {
      v[r].lo = ld_stream_at<f64x2>(vb, 2 * off);
      v[r].hi = ld_stream_at<f64x2>(vb, 2 * off + 16);
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r)
    e[r] = ld_stream_at<i32x4>(eb, 16u * (uint32_t)min(lane + kWave * r, nqr - 1));
  bool from_lds = false;
  if (WIN) {
    // The window's direct-to-LDS loads went out before this partition's
    // NR + NN + NN * (sizeof(V) / 4) loads (the caller orders them), and
    // vector loads retire in order: once no more than that many are in
    // flight, this wave's share of the window has landed. The barrier then
    // covers the other waves' shares; the partition's own loads stay in
    // flight across it (no fence: nothing but the window is shared), and the
    // columns are only looked at after it.
    // The window bounds are read back from LDS after the barrier, so the
    // column checks cannot be hoisted above it.
    memory_order_point();
    wait_vmcnt_lds<NR + NN + NN * (int)(sizeof(V) / 4)>();
    __builtin_amdgcn_s_barrier();
    memory_order_point();
    WindowBounds w;
#pragma unroll
    for (int k = 0; k < kWinIntervals; ++k) {
      w.lo[k] = k < WK ? __builtin_amdgcn_readfirstlane(win_meta[2 * k]) : 0;
      w.len[k] = k < WK ? __builtin_amdgcn_readfirstlane(win_meta[2 * k + 1]) : 0;
    }
    bool inside = true;
#pragma unroll
    for (int r = 0; r < NN; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) inside &= w.slot<WK>(c[r][j]) >= 0;
    from_lds = __ballot(!inside) == 0;
    if (from_lds) {
#pragma unroll
      for (int r = 0; r < NN; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) v[r].set(j, v[r][j] * xs[w.slot<WK>(c[r][j])]);
    }
  }
  if (!from_lds) {
#pragma unroll
    for (int r = 0; r < NN; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[r].set(j, v[r][j] * a.x[c[r][j]]);
  }
  // clamped lanes rewrite the last quad with the same values: unconditional
  // stores keep the loads from being sunk into (and serialised by) branches
#pragma unroll
  for (int r = 0; r < NR; ++r)
    *reinterpret_cast<i32x4*>(ends + 4 * min(lane + kWave * r, nqr - 1)) = e[r] - n0;
#pragma unroll
  for (int r = 0; r < NN; ++r) store_quad(prods, min(lane + kWave * r, nqn - 1), v[r]);
}

template <typename V, int NR, int RQN, int WK>
__device__ __forceinline__ void stream_stage_nn(const MergeArgs<V>& a, int qr0, int nqr, int n0,
                                                int qn0, int nqn, int32_t* ends, V* prods,
                                                const V* xs, const int* win_meta) {
  const int rounds = (nqn + kWave - 1) / kWave;
  if (rounds == 0)
    stream_stage<V, NR, 0, WK>(a, qr0, nqr, n0, qn0, nqn, ends, prods, xs, win_meta);
  else if (rounds == 1 || RQN < 2)
    stream_stage<V, NR, (RQN < 1 ? 0 : 1), WK>(a, qr0, nqr, n0, qn0, nqn, ends, prods, xs,
                                               win_meta);
  else if (rounds == 2 || RQN < 3)
    stream_stage<V, NR, 2, WK>(a, qr0, nqr, n0, qn0, nqn, ends, prods, xs, win_meta);
  else if (rounds == 3 || RQN < 4)
    stream_stage<V, NR, (RQN < 3 ? 2 : 3), WK>(a, qr0, nqr, n0, qn0, nqn, ends, prods, xs,
                                               win_meta);
  else if (rounds == 4 || RQN < 5)
    stream_stage<V, NR, (RQN < 4 ? 2 : 4), WK>(a, qr0, nqr, n0, qn0, nqn, ends, prods, xs,
                                               win_meta);
  else
    stream_stage<V, NR, (RQN < 5 ? 2 : 5), WK>(a, qr0, nqr, n0, qn0, nqn, ends, prods, xs,
                                               win_meta);
}

// Reduction of a staged stream partition: groups of G lanes sum each row,
// 64 / G rows per round; alpha and beta are applied once per row. re[k] is
// the local end of row r0 + k, prod[i] the product of the partition's
// nonzero i. With one lane per row the lane sums its row in order; in wider
// groups each lane reads U products per iteration (strided by G), all in
// flight together; reads past the row end reread the row's last product and
// add 0. The group's partial sums meet by DPP moves.
template <typename V, int G>
__device__ __forceinline__ void stream_reduce_g(const MergeArgs<V>& a, int r0, int nrows,
                                                const int32_t* re, const V* prod) {
  constexpr int U = G <= 4 ? 8 : 4;
  const int lane = lane_id();
  const int gl = lane & (G - 1);
  constexpr int RPR = kWave / G;   // rows per round
  const int grp = lane / G;
  for (int base = 0; base < nrows; base += RPR) {
    const int k = base + grp;
    V acc = V(0);
    if (k < nrows) {
      const int s = k > 0 ? re[k - 1] : 0, t = re[k];
      if (G == 1) {
        // one lane per row (short rows): the plain loop is cheapest
        for (int i = s; i < t; ++i) acc += prod[i];
      } else {
      for (int i = s + gl; i < t; i += U * G) {
        V p[U];
#pragma unroll
        for (int u = 0; u < U; ++u) p[u] = prod[min(i + u * G, t - 1)];
        V part = p[0];
#pragma unroll
        for (int u = 1; u < U; ++u) part += i + u * G < t ? p[u] : V(0);
        acc += part;
      }
      }
    }
    acc = group_sum_dpp<G>(acc);
    if (k < nrows && gl == 0) {
      V out = a.alpha * acc;
      if (a.beta_nonzero) out = fma(a.beta, a.y[r0 + k], out);
      a.y[r0 + k] = out;   // cached store: L2 merges the partial lines of neighbours
    }
  }
}

// Wider groups (32, 64 lanes per row): the group's partial sums meet in its
// last lane by DPP moves (rows of 16, then row 0 into 1 and 2 into 3; for 64
// lanes also lane 31 into rows 2 and 3).
template <typename V, int G>
__device__ __forceinline__ void stream_reduce_wide(const MergeArgs<V>& a, int r0, int nrows,
                                                   const int32_t* re, const V* prod) {
  static_assert(G == 32 || G == 64, "wide groups");
  const int lane = lane_id();
  const int gl = lane & (G - 1);
  constexpr int RPR = kWave / G;
  const int grp = lane / G;
  for (int base = 0; base < nrows; base += RPR) {
    const int k = base + grp;
    V acc = V(0);
    if (k < nrows) {
      const int s = k > 0 ? re[k - 1] : 0, t = re[k];
      for (int i = s + gl; i < t; i += G) acc += prod[i];
    }
    if (G == 64) {
      acc = wave_sum_to_last(acc);
    } else {
      acc = group_sum_dpp<16>(acc);
      const V up = dpp_move<kDppRowBcast15, 0xA>(acc);
      acc = ((lane >> 4) & 1) ? acc + up : acc;
    }
    if (k < nrows && gl == G - 1) {
      V out = a.alpha * acc;
      if (a.beta_nonzero) out = fma(a.beta, a.y[r0 + k], out);
      a.y[r0 + k] = out;
    }
  }
}

template <typename V>
__device__ __forceinline__ void stream_reduce(const MergeArgs<V>& a, int r0, int nrows,
                                              const int32_t* re, const V* prod) {
  switch (a.stream_lanes) {
    case 1: stream_reduce_g<V, 1>(a, r0, nrows, re, prod); break;
    case 2: stream_reduce_g<V, 2>(a, r0, nrows, re, prod); break;
    case 4: stream_reduce_g<V, 4>(a, r0, nrows, re, prod); break;
    case 8: stream_reduce_g<V, 8>(a, r0, nrows, re, prod); break;
    case 16: stream_reduce_g<V, 16>(a, r0, nrows, re, prod); break;
    case 32: stream_reduce_wide<V, 32>(a, r0, nrows, re, prod); break;
    default: stream_reduce_wide<V, 64>(a, r0, nrows, re, prod); break;
  }
}

// WK: x window of 0, 1 or kWinIntervals column intervals; WPB waves per
// workgroup.
template <typename V, int IPT, int WK, int WPB>
__global__ __launch_bounds__(WPB * kWave, stream_min_waves(sizeof(V), IPT, WK > 0)) void merge_stream_kernel(
    const MergeArgs<V> a, const int32_t* __restrict__ rb, const int32_t* __restrict__ wt) {
  constexpr bool WIN = WK > 0;
  constexpr int T = kWave * IPT;
  constexpr int CAP = T + T / 8;            // rows + nonzeros of one partition
  constexpr int BUF = stream_buf_elems(IPT);  // per-wave buffer, elements of V
  constexpr int RQN = (CAP / 4 + 2 + kWave - 1) / kWave;
  constexpr int RQR = (T / 4 + 2 + kWave - 1) / kWave;
  // 16-byte chunks of the x window
  constexpr int WCHUNKS = WIN ? stream_window_bytes(IPT, sizeof(V), WPB) / 16 : 1;
  static_assert(!WIN || WCHUNKS > 0, "window kernel instantiated without window room");
  constexpr int E = 16 / sizeof(V);           // elements per chunk
  static_assert(RQN <= 5, "at most 5 nonzero rounds");
  __shared__ __attribute__((aligned(16))) V s_buf[WPB][BUF];
  __shared__ __attribute__((aligned(16))) V s_x[WIN ? WCHUNKS * E : E];

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int blk = a.xcd_remap ? xcd_tile(blockIdx.x, 0, gridDim.x) : (int)blockIdx.x;
  const int p = blk * WPB + wave;
  // one descriptor read, {r0, row_ptr[r0]} and {r1, row_ptr[r1]}: a uniform
  // read of a table nothing in the kernel writes, so it is a scalar load
  // (neighbouring waves share scalar cache lines; the vector memory path
  // carries only the matrix)
  int r0 = 0, r1 = 0, n0 = 0, n1 = 0;
  if (p < a.P) {
    r0 = rb[2 * p];
    n0 = rb[2 * p + 1];
    r1 = rb[2 * p + 2];
    n1 = rb[2 * p + 3];
  }
  const int nrows = r1 - r0;
  // with the window every wave must reach the block's barrier
  if (!WIN && nrows == 0) return;

  __shared__ int s_win[kWinTable];
  if (WIN) {
    // the window's intervals: chunk aligned and inside x (the plan guarantees
    // it), packed one after the other in LDS; like the bounds, a scalar read
    const int32_t* ws = wt + (int64_t)kWinTable * blk;
    const int lo0 = ws[0], len0 = ws[1];
    const int lo1 = WK > 1 ? ws[2] : 0, len1 = WK > 1 ? ws[3] : 0;
    const int lo2 = WK > 1 ? ws[4] : 0, len2 = WK > 1 ? ws[5] : 0;
    if (threadIdx.x == 0) {
      s_win[0] = lo0;
      s_win[1] = len0;
      if (WK > 1) {
        s_win[2] = lo1;
        s_win[3] = len1;
        s_win[4] = lo2;
        s_win[5] = len2;
      }
    }
    const int c1 = len0 / E, c2 = c1 + len1 / E;         // first chunk of intervals 1, 2
    const int nch = c2 + len2 / E;
#pragma unroll
    for (int r = 0; r < (WCHUNKS + WPB * kWave - 1) / (WPB * kWave); ++r) {
      const int first = WPB * kWave * r + kWave * wave;   // this wave's first chunk
      const int ch = first + lane;
      if (first < nch && ch < nch) {
        const int src = WK == 1 ? lo0 + E * ch
                        : ch >= c2 ? lo2 + E * (ch - c2)
                        : ch >= c1 ? lo1 + E * (ch - c1) : lo0 + E * ch;
        lds_dma16(a.x + src, s_x + E * first);
      }
    }
    // the staging loads must be issued after these (the window wait counts them)
    memory_order_point();
  }

  const int nnzc = n1 - n0;
  const int qr0 = (r0 + 1) >> 2;
  const int nqr = nrows > 0 ? (r1 >> 2) - qr0 + 1 : 0;
  const int qn0 = n0 >> 2;
  const int nqn = nnzc > 0 ? (((n0 + nnzc - 1) >> 2) - qn0 + 1) : 0;
  V* buf = s_buf[wave];
  // products of quads [qn0, qn0 + nqn) at the front, row-end quads at the back
  int32_t* ends_q = reinterpret_cast<int32_t*>(buf + BUF) - 4 * nqr;
  const int32_t* re = ends_q + ((r0 + 1) & 3);   // re[k]: local end of row r0 + k
  const V* prod = buf + (n0 & 3);

  const bool tail = (nqr > 0 && ((a.M + 1) & 3) && qr0 + nqr - 1 == a.M >> 2) ||
                    (nqn > 0 && (a.nnz & 3) && qn0 + nqn - 1 == (a.nnz - 1) >> 2);
  if (tail) {
    if (WIN) {
      wait_vmem();
      __syncthreads();
    }
    stage_safe<V, RQR, RQN>(a.row_ptr, a.M + 1, qr0, nqr, n0, a.col_idx, a.val, a.x, a.nnz,
                            qn0, nqn, ends_q, buf);
  } else if (nqr == 0) {
    stream_stage<V, 0, 0, WK>(a, qr0, nqr, n0, qn0, nqn, ends_q, buf, s_x, s_win);
  } else if (nqr <= kWave || RQR < 2) {
    stream_stage_nn<V, 1, RQN, WK>(a, qr0, nqr, n0, qn0, nqn, ends_q, buf, s_x, s_win);
  } else {
    stream_stage_nn<V, RQR, RQN, WK>(a, qr0, nqr, n0, qn0, nqn, ends_q, buf, s_x, s_win);
  }
  if (nrows == 0) return;
  wave_sync();

  stream_reduce(a, r0, nrows, re, prod);
}

// Adds alpha * sum(carries) to every row that partitions left open. One wave
// handles 64 consecutive partitions; a row's carries are contiguous, so they
// form a segment of equal keys, summed by the wave's DPP segmented scan. The
// wave that holds a segment's first carry owns it and, if the segment runs
// past its 64 partitions, keeps reading, eight windows of 64 per step, until
// the step where the key changes. Every lane of the wave stays active up to
// the scans (the early return is wave-uniform).
template <typename V, bool TILED>
__device__ __forceinline__ void fixup_chunks(const int32_t* __restrict__ carry_row,
                                             const int32_t* __restrict__ skip,
                                             const V* __restrict__ carry_val, int32_t P,
                                             int32_t M, V* __restrict__ y, V alpha, int blk) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t base = ((int64_t)blk * kWavesPerBlock + wave) * kWave;
  if (base >= P) return;
  const int64_t p = base + lane;
  const int key = p < P ? carry_key<TILED>(carry_row, skip, p, P, M) : INT_MAX;
  const V v = p < P ? carry_val[p] : V(0);
  const V s = wave_segscan_keys(v, key);

  // the key after this lane's (the next chunk's first for lane 63)
  const int next_key = lane_next(
      key, base + kWave < P ? carry_key<TILED>(carry_row, skip, base + kWave, P, M) : INT_MAX - 1);
  // wave-uniform: the chunk's first key and the key before the chunk
  const int key0 = __builtin_amdgcn_readfirstlane(key);
  const int prev0 = base > 0 ? carry_key<TILED>(carry_row, skip, base - 1, P, M) : -1;
  // a segment is owned here unless it starts at lane 0 and continues from
  // the previous chunk
  const bool owned = !(key == key0 && prev0 == key0);
  const bool tail = next_key != key;
  if (tail && owned && key < M) y[key] += alpha * s;

  const int key63 = __builtin_amdgcn_readlane(key, kWave - 1);
  const bool cont63 = __builtin_amdgcn_readlane((int)(!tail && owned), kWave - 1) != 0;
  if (cont63 && key63 < M) {
    // kFixupWindows windows of 64 partitions per step, every load of a step
    // in flight together; the row's carries are a prefix of the step, so it
    // goes on only if the step's last window is still all the row's
    constexpr int kFixupWindows = 8;
    V extra = V(0);
    for (int64_t q = base + kWave;; q += kWave * kFixupWindows) {
      int kq[kFixupWindows];
#pragma unroll
      for (int u = 0; u < kFixupWindows; ++u) {
        const int64_t pp = q + kWave * u + lane;
        kq[u] = pp < P ? carry_key<TILED>(carry_row, skip, pp, P, M) : -1;
      }
      V w[kFixupWindows];
#pragma unroll
      for (int u = 0; u < kFixupWindows; ++u)
        w[u] = kq[u] == key63 ? carry_val[q + kWave * u + lane] : V(0);
#pragma unroll
      for (int u = 0; u < kFixupWindows; ++u) extra += w[u];
      if (__ballot(kq[kFixupWindows - 1] == key63) != ~0ull) break;
    }
    // lane 63 holds both the wave's total and the chunk's part of the row
    extra = wave_sum_to_last(extra);
    if (lane == kWave - 1) y[key63] += alpha * (s + extra);
  }
}

template <typename V>
__global__ __launch_bounds__(kBlock) void merge_fixup_kernel(
    const int32_t* __restrict__ carry_row, const V* __restrict__ carry_val, int32_t P,
    int32_t M, V* __restrict__ y, V alpha) {
  fixup_chunks<V, false>(carry_row, nullptr, carry_val, P, M, y, alpha, (int)blockIdx.x);
}

// The fix-up and, on a plan with long-row tiles, the tiles' reduction in
// one launch: blocks [0, fix_blocks) take the carries as above (tile rows'
// keyed past the last row), the others one wave per tile row, which adds
// alpha * (the row's block partials, summed in a fixed order) to its y. So
// the two parts write different rows.
template <typename V>
__global__ __launch_bounds__(kBlock) void fixup_tile_reduce_kernel(
    const int32_t* __restrict__ carry_row, const V* __restrict__ carry_val, int32_t P,
    int32_t M, V* __restrict__ y, V alpha, const TileArgs<V> t, int fix_blocks) {
  if ((int)blockIdx.x < fix_blocks) {   // workgroup-uniform
    fixup_chunks<V, true>(carry_row, t.skip, carry_val, P, M, y, alpha, (int)blockIdx.x);
    return;
  }
  const int64_t i = ((int64_t)(blockIdx.x - fix_blocks) * kBlock + threadIdx.x) / kWave;
  if (i >= t.n_rows) return;   // wave-uniform
  const int lane = lane_id();
  V acc = V(0);
  for (int b = lane; b < t.nb; b += kWave) acc += t.partial[i * t.nb + b];
  acc = wave_sum_to_last(acc);
  if (lane == kWave - 1) {
    const int32_t r = t.rows[kTileRowInts * i];
    t.y[r] += t.alpha * acc;
  }
}

template <typename V, int IPT, int WK>
hipError_t launch_window(const MergeArgs<V>& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  constexpr int WPB = kWavesPerBlock;
  if constexpr (stream_window_bytes(IPT, sizeof(V), WPB) > 0) {
    launch_timed(merge_stream_kernel<V, IPT, WK, WPB>, dim3((a.P + WPB - 1) / WPB),
                 dim3(WPB * kWave), 0, s, ev0, ev1, a, a.row_bounds, a.win_span);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;   // the plan never asks for it
}

template <typename V, int IPT>
hipError_t launch_main(const MergeArgs<V>& a, const TileArgs<V>* tiles, hipStream_t s,
                       hipEvent_t ev0, hipEvent_t ev1) {
  const int slots = a.stream || !a.n_dispatch ? a.P : a.n_dispatch;
  const int blocks = (slots + kWavesPerBlock - 1) / kWavesPerBlock;
  if (tiles) {
    if (a.stream || !a.mask_end || !a.n_dispatch) return hipErrorInvalidValue;
    const int64_t n_tiles = (int64_t)tiles->ngroups * tiles->nb;
    if (n_tiles + blocks > 0x7fffffffll) return hipErrorInvalidValue;
    launch_timed(walk_tile_kernel<V, IPT>, dim3((unsigned)(blocks + n_tiles)), dim3(kBlock), 0, s,
                 ev0, ev1, a, *tiles, blocks);
  } else if (a.stream && a.x_window == 1) {
    return launch_window<V, IPT, 1>(a, s, ev0, ev1);
  } else if (a.stream && a.x_window > 1) {
    return launch_window<V, IPT, kWinIntervals>(a, s, ev0, ev1);
  } else if (a.stream) {
    launch_timed(merge_stream_kernel<V, IPT, 0, kWavesPerBlock>, dim3(blocks), dim3(kBlock), 0,
                 s, ev0, ev1, a, a.row_bounds, a.win_span);
  } else if (a.mask_end) {
    return hipErrorInvalidValue;   // masked partitions run only beside their tiles
  } else {
    launch_timed(merge_spmv_kernel<V, IPT>, dim3(blocks), dim3(kBlock), 0, s, ev0, ev1, a);
  }
  return hipGetLastError();
}

}  // namespace

template <typename V>
hipError_t launch_merge(const MergeArgs<V>& a, int ipt, hipStream_t s, hipEvent_t ev0,
                        hipEvent_t ev1, const TileArgs<V>* tiles) {
  if (a.P <= 0) return hipSuccess;
  hipError_t err;
  // ev0 / ev1 bracket the main kernel alone (recorded by its dispatch)
  switch (ipt) {
    case 4: err = launch_main<V, 4>(a, tiles, s, ev0, ev1); break;
    case 7: err = launch_main<V, 7>(a, tiles, s, ev0, ev1); break;
    case 8: err = launch_main<V, 8>(a, tiles, s, ev0, ev1); break;
    case 16: err = launch_main<V, 16>(a, tiles, s, ev0, ev1); break;
    default: return hipErrorInvalidValue;
  }
  if (err != hipSuccess) return err;
  const int64_t chunks = ((int64_t)a.P + kWave - 1) / kWave;
  const int fix_blocks =
      a.P > 1 && !a.stream ? (int)((chunks + kWavesPerBlock - 1) / kWavesPerBlock) : 0;
  const int64_t red_blocks =
      tiles && tiles->n_rows > 0 ? ((int64_t)tiles->n_rows * kWave + kBlock - 1) / kBlock : 0;
  if (red_blocks > 0) {
    hipLaunchKernelGGL((fixup_tile_reduce_kernel<V>), dim3((unsigned)(fix_blocks + red_blocks)),
                       dim3(kBlock), 0, s, a.carry_row, a.carry_val, a.P, a.M, a.y, a.alpha,
                       *tiles, fix_blocks);
    err = hipGetLastError();
  } else if (fix_blocks > 0) {
    hipLaunchKernelGGL((merge_fixup_kernel<V>), dim3(fix_blocks), dim3(kBlock), 0, s,
                       a.carry_row, a.carry_val, a.P, a.M, a.y, a.alpha);
    err = hipGetLastError();
  }
  return err;
}

template hipError_t launch_merge<float>(const MergeArgs<float>&, int, hipStream_t, hipEvent_t,
                                        hipEvent_t, const TileArgs<float>*);
template hipError_t launch_merge<double>(const MergeArgs<double>&, int, hipStream_t,
                                         hipEvent_t, hipEvent_t, const TileArgs<double>*);

}  // namespace spmv
