// Binned CSR SpMV for gfx950: rows grouped by length, each bin run by the
// row mapping that suits its length, all bins in ONE launch.
//
// Row mappings: thread-mapped (one lane per row) and warp/block-mapped (a
// group of lanes, a wavefront, or a workgroup strides a row's nonzeros and
// reduces), "A Programming Model for GPU Load Balancing" (PPoPP'23),
// Sections 4.2 and 5.2.2; the scalar and vector CSR kernels that "New
// Row-grouped CSR format..." (arXiv 1012.2270) Section 3 discusses. Rows come
// grouped by the plan's bins ("OpSparse", arXiv 2206.07244, Section 5.1);
// OpSparse launches the kernels of the bins with the largest rows first so
// the short-row work fills the machine behind them.
//
// MI355X mapping: instead of one kernel per bin on several streams, the bins
// are segments of a single grid. Workgroups are dispatched in index order,
// and the segments are ordered longest rows first, so the long-row
// workgroups start first; there is no inter-kernel gap. Inside a segment the
// workgroup index is renumbered so each XCD walks a contiguous run of rows.
#include "device_common.hpp"
#include "internal.hpp"

namespace spmv {
namespace {

template <typename V>
__device__ __forceinline__ void store_row(const BinnedArgs<V>& a, int r, V acc) {
  V out = a.alpha * acc;
  if (a.beta_nonzero) out = fma(a.beta, a.y[r], out);
  a.y[r] = out;
}

// The sum over row entries [s, e) of the quads q0 + t, q0 + t + G, ...
// (q0 = s / 4, t = this lane's place among the G lanes of the row), NQ
// quads a step (one for rows of up to 8 entries on 1 or 2 lanes, two
// otherwise): 16-byte loads of columns and values (element loads for the
// array's last, partial quad), then the x gathers; entries of a quad outside
// [s, e) are masked to exactly 0 (their gather reads x[0]). Four running
// sums, one per entry of a quad, added in a fixed order.
template <typename V, int G>
__device__ __forceinline__ V quad_row_sum(const BinnedArgs<V>& a, int32_t s, int32_t e, int t) {
  // unsigned: 4q + 3 may pass 2^31 - 1 near the largest nnz
  const uint32_t q1 = ((uint32_t)e + 3u) >> 2;
  const uint32_t nnz = (uint32_t)a.nnz;
  constexpr int NQ = G <= 2 ? 1 : 2;
  V acc[4] = {V(0), V(0), V(0), V(0)};
  for (uint32_t q = ((uint32_t)s >> 2) + (uint32_t)t; q < q1; q += (uint32_t)(NQ * G)) {
    uint32_t qq[NQ];
#pragma unroll
    for (int h = 0; h < NQ; ++h) qq[h] = min(q + (uint32_t)(h * G), q1 - 1u);
    i32x4 c[NQ];
    Quad<V> v[NQ];
#pragma unroll
    for (int h = 0; h < NQ; ++h) {
      const bool full = 4u * qq[h] + 3u < nnz;
      c[h] = full ? load_quad<false>(a.col_idx, (int)qq[h], 0)
                  : load_quad<true>(a.col_idx, (int)qq[h], (int)nnz);
      v[h] = full ? load_quad<false>(a.val, (int)qq[h], 0)
                  : load_quad<true>(a.val, (int)qq[h], (int)nnz);
    }
#pragma unroll
    for (int h = 0; h < NQ; ++h) {
      const bool live = q + (uint32_t)(h * G) < q1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t k = 4u * qq[h] + (uint32_t)j;
        const bool in = live && k >= (uint32_t)s && k < (uint32_t)e;
        acc[j] += masked_product(in, v[h][j], a.x, c[h][j]);
      }
    }
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// G lanes per row (G = 1, 2, ..., 64), 256 / G rows per workgroup.
template <typename V, int G>
__device__ __forceinline__ void group_rows(const BinnedArgs<V>& a, const BinLaunch& L,
                                           int tile) {
  constexpr int kRows = kBlock / G;
  const int grp = threadIdx.x / G, gl = threadIdx.x % G;
  const int idx = tile * kRows + grp;
  if (idx >= L.n_rows) return;  // whole groups leave together
  const int r = a.identity ? L.row_begin + idx : a.bins[L.row_begin + idx];
  const int s = a.row_ptr[r], e = a.row_ptr[r + 1];
  V acc = quad_row_sum<V, G>(a, s, e, gl);
  if (G > 1) acc = group_sum<G>(acc);
  if (gl == 0) store_row(a, r, acc);
}

// One 256-thread workgroup per row.
template <typename V>
__device__ __forceinline__ void block_row(const BinnedArgs<V>& a, const BinLaunch& L,
                                          int tile) {
  __shared__ V s_part[kWavesPerBlock];
  const int r = a.identity ? L.row_begin + tile : a.bins[L.row_begin + tile];
  const int s = a.row_ptr[r], e = a.row_ptr[r + 1];
  V acc = group_sum<kWave>(quad_row_sum<V, kBlock>(a, s, e, threadIdx.x));
  if (lane_id() == 0) s_part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) store_row(a, r, (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]));
}

template <typename V>
__global__ __launch_bounds__(kBlock) void binned_spmv_kernel(const BinnedArgs<V> a) {
  const int b = blockIdx.x;
  int d = 0;
#pragma unroll
  for (int k = 1; k < kMaxBins; ++k) d += (k < a.n_launch && b >= a.bin[k].block_begin) ? 1 : 0;
  d = __builtin_amdgcn_readfirstlane(d);
  const BinLaunch L = a.bin[d];
  const int tile = a.xcd_remap ? xcd_tile(b, L.block_begin, L.n_blocks) : b - L.block_begin;
  switch (L.lanes) {
    case 1: group_rows<V, 1>(a, L, tile); break;
    case 2: group_rows<V, 2>(a, L, tile); break;
    case 4: group_rows<V, 4>(a, L, tile); break;
    case 8: group_rows<V, 8>(a, L, tile); break;
    case 16: group_rows<V, 16>(a, L, tile); break;
    case 32: group_rows<V, 32>(a, L, tile); break;
    case 64: group_rows<V, 64>(a, L, tile); break;
    default: block_row<V>(a, L, tile); break;
  }
}

}  // namespace

template <typename V>
hipError_t launch_binned(const BinnedArgs<V>& a, int total_blocks, hipStream_t s,
                         hipEvent_t ev0, hipEvent_t ev1) {
  if (total_blocks <= 0) return hipSuccess;
  launch_timed(binned_spmv_kernel<V>, dim3(total_blocks), dim3(kBlock), 0, s, ev0, ev1, a);
  return hipGetLastError();
}

template hipError_t launch_binned<float>(const BinnedArgs<float>&, int, hipStream_t, hipEvent_t,
                                         hipEvent_t);
template hipError_t launch_binned<double>(const BinnedArgs<double>&, int, hipStream_t,
                                          hipEvent_t, hipEvent_t);

}  // namespace spmv
