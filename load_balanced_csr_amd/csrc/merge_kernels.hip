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

#include <limits.h>

namespace spmv {
namespace {

template <typename V, int IPT>
__global__ __launch_bounds__(kBlock) void merge_spmv_kernel(const MergeArgs<V> a) {
  constexpr int T = kWave * IPT;
  constexpr int RQ = (T / 4 + 2 + kWave - 1) / kWave;   // quad rounds per array
  __shared__ __attribute__((aligned(16))) int32_t s_end[kWavesPerBlock][T + 8];
  __shared__ __attribute__((aligned(16))) V s_val[kWavesPerBlock][T + 8];

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int blk = a.xcd_remap ? xcd_tile(blockIdx.x, 0, gridDim.x) : (int)blockIdx.x;
  const int p = blk * kWavesPerBlock + wave;
  if (p >= a.P) return;

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
  int32_t* re = s_end[wave] + ((r0 + 1) & 3);
  V* vb = s_val[wave];
  V* prod_q = vb + (T + 8 - 4 * nqn);
  V* prod = prod_q + (n0 & 3);
  stage_partition<V, RQ, RQ>(a.row_ptr, a.M + 1, qr0, nqr, n0, a.col_idx, a.val, a.x, a.nnz,
                             qn0, nqn, s_end[wave], prod_q);
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
  // lane l's first finished row is the segmented scan value of lane l-1.
  const V s = wave_segscan(acc, ri);
  V incoming = __shfl_up(s, 1, kWave);
  if (lane == 0) incoming = V(0);
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

// Stream reduction, used when every row holds at most T/4 entries. The
// partitions keep the merge-path row coordinate (rows ended before the
// diagonal) but start their nonzeros at that row's start, so no row crosses a
// partition: a partition owns rows [r0, r1) whole and nonzeros
// [row_ptr[r0], row_ptr[r1]), at most T + T/4 of them (the row cut by the
// diagonal moves forward entirely). There are no carries and no fix-up.
// After staging the products in LDS, groups of G lanes each sum one row
// (strided by G, then a butterfly), 64 / G rows per round.
template <typename V, int IPT>
__global__ __launch_bounds__(kBlock) void merge_stream_kernel(const MergeArgs<V> a) {
  constexpr int T = kWave * IPT;
  constexpr int CAP = T + T / 4;           // nonzeros one partition can hold
  constexpr int RQN = (CAP / 4 + 2 + kWave - 1) / kWave;
  constexpr int RQR = (T / 4 + 2 + kWave - 1) / kWave;
  __shared__ __attribute__((aligned(16))) int32_t s_end[kWavesPerBlock][T + 8];
  __shared__ __attribute__((aligned(16))) V s_prod[kWavesPerBlock][CAP + 8];

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int blk = a.xcd_remap ? xcd_tile(blockIdx.x, 0, gridDim.x) : (int)blockIdx.x;
  const int p = blk * kWavesPerBlock + wave;
  if (p >= a.P) return;
  const int r0 = a.split_row[p], r1 = a.split_row[p + 1];
  const int nrows = r1 - r0;
  if (nrows == 0) return;
  const int n0 = a.row_ptr[r0];
  const int nnzc = a.row_ptr[r1] - n0;

  // ---- stage row ends and products with 16-byte loads ------------------------
  const int qr0 = (r0 + 1) >> 2;
  const int nqr = (r1 >> 2) - qr0 + 1;
  const int qn0 = n0 >> 2;
  const int nqn = nnzc > 0 ? (((n0 + nnzc - 1) >> 2) - qn0 + 1) : 0;
  int32_t* re = s_end[wave] + ((r0 + 1) & 3);  // re[k]: local end of row r0 + k
  V* prod = s_prod[wave] + (n0 & 3);
  stage_partition<V, RQR, RQN>(a.row_ptr, a.M + 1, qr0, nqr, n0, a.col_idx, a.val, a.x,
                               a.nnz, qn0, nqn, s_end[wave], s_prod[wave]);
  wave_sync();

  // ---- G lanes per row ---------------------------------------------------------
  const int G = a.stream_lanes;
  const int gl = lane & (G - 1);
  const int rows_per_round = kWave / G;
  const int grp = lane / G;
  for (int base = 0; base < nrows; base += rows_per_round) {
    const int k = base + grp;
    V acc = V(0);
    if (k < nrows) {
      const int s = k > 0 ? re[k - 1] : 0, t = re[k];
      for (int i = s + gl; i < t; i += G) acc += prod[i];
    }
    for (int o = G >> 1; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
    if (k < nrows && gl == 0) {
      V out = a.alpha * acc;
      if (a.beta_nonzero) out = fma(a.beta, ld_stream(a.y + r0 + k), out);
      st_stream(a.y + r0 + k, out);
    }
  }
}

// Adds alpha * sum(carries) to every row that partitions left open. One wave
// handles 64 consecutive partitions; a row's carries are contiguous, so they
// form a segment of equal keys. The wave that holds a segment's first carry
// owns it and, if the segment runs past its 64 partitions, keeps reading
// until the key changes.
template <typename V>
__global__ __launch_bounds__(kBlock) void merge_fixup_kernel(
    const int32_t* __restrict__ carry_row, const V* __restrict__ carry_val, int32_t P,
    int32_t M, V* __restrict__ y, V alpha) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t base = ((int64_t)blockIdx.x * kWavesPerBlock + wave) * kWave;
  if (base >= P) return;
  const int64_t p = base + lane;
  const int key = p < P ? carry_row[p] : INT_MAX;
  const V v = p < P ? carry_val[p] : V(0);
  const V s = wave_segscan(v, key);

  int next_key = __shfl_down(key, 1, kWave);
  if (lane == kWave - 1) next_key = p + 1 < P ? carry_row[p + 1] : INT_MAX - 1;
  const int key0 = __shfl(key, 0, kWave);
  const int prev0 = base > 0 ? carry_row[base - 1] : -1;
  // a segment is owned here unless it starts at lane 0 and continues from
  // the previous chunk
  const bool owned = !(key == key0 && prev0 == key0);
  const bool tail = next_key != key;
  if (tail && owned && key < M) y[key] += alpha * s;

  const int key63 = __shfl(key, kWave - 1, kWave);
  const bool cont63 = __shfl((int)(!tail && owned), kWave - 1, kWave);
  if (cont63 && key63 < M) {
    V extra = V(0);
    for (int64_t q = base + kWave;; q += kWave) {
      const int64_t pp = q + lane;
      const bool match = pp < P && carry_row[pp] == key63;
      extra += match ? carry_val[pp] : V(0);
      if (__ballot(match) != ~0ull) break;
    }
    extra = group_sum<kWave>(extra);
    const V s63 = __shfl(s, kWave - 1, kWave);
    if (lane == 0) y[key63] += alpha * (s63 + extra);
  }
}

template <typename V, int IPT>
hipError_t launch_main(const MergeArgs<V>& a, hipStream_t s) {
  const int blocks = (a.P + kWavesPerBlock - 1) / kWavesPerBlock;
  if (a.stream)
    hipLaunchKernelGGL((merge_stream_kernel<V, IPT>), dim3(blocks), dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((merge_spmv_kernel<V, IPT>), dim3(blocks), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace

template <typename V>
hipError_t launch_merge(const MergeArgs<V>& a, int ipt, hipStream_t s, hipEvent_t ev0,
                        hipEvent_t ev1) {
  if (a.P <= 0) return hipSuccess;
  hipError_t err;
  if (ev0 && (err = hipEventRecord(ev0, s)) != hipSuccess) return err;
  switch (ipt) {
    case 4: err = launch_main<V, 4>(a, s); break;
    case 8: err = launch_main<V, 8>(a, s); break;
    case 16: err = launch_main<V, 16>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  if (err != hipSuccess) return err;
  if (ev1 && (err = hipEventRecord(ev1, s)) != hipSuccess) return err;
  if (a.P > 1 && !a.stream) {
    const int64_t chunks = ((int64_t)a.P + kWave - 1) / kWave;
    const int blocks = (int)((chunks + kWavesPerBlock - 1) / kWavesPerBlock);
    hipLaunchKernelGGL((merge_fixup_kernel<V>), dim3(blocks), dim3(kBlock), 0, s,
                       a.carry_row, a.carry_val, a.P, a.M, a.y, a.alpha);
    err = hipGetLastError();
  }
  return err;
}

template hipError_t launch_merge<float>(const MergeArgs<float>&, int, hipStream_t, hipEvent_t,
                                        hipEvent_t);
template hipError_t launch_merge<double>(const MergeArgs<double>&, int, hipStream_t,
                                         hipEvent_t, hipEvent_t);

}  // namespace spmv
