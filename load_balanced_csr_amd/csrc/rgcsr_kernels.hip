// Row-grouped CSR ("New Row-grouped CSR format for storing the sparse
// matrices on GPU with implementation in CUDA", arXiv 1012.2270, Section 4):
// rows are taken in groups of G consecutive rows; inside a group the entries
// are stored column-interleaved -- entry k of the group's row i at
// group_base + k * G + i -- to the width of the group's longest row, so one
// thread per row reads its k-th entries with the whole group's threads
// touching consecutive addresses. The page keeps groupPointers (the group
// bases) and rowLength (entries per row); the same two arrays here, plus the
// group widths.
//
// MI355X mapping: a 64-lane wavefront takes 64 consecutive rows (64 / G
// groups); each lane walks its own row's entries four at a time (all loads of
// a step issued before the first use) and skips the padding; the wavefront
// loops while any of its lanes has entries left.
#include "device_common.hpp"
#include "internal.hpp"

#include <limits.h>

namespace spmv {
namespace {

// Group widths (longest row of each group) and, summed over the grid, the
// entries the format stores for the rows that exist (width x rows).
__global__ __launch_bounds__(kBlock) void rg_width_kernel(const int32_t* __restrict__ row_ptr,
                                                          int32_t M, int32_t G, int32_t ngroups,
                                                          int32_t* __restrict__ gw,
                                                          unsigned long long* stored) {
  const int g = blockIdx.x * kBlock + threadIdx.x;
  unsigned long long mine = 0;
  if (g < ngroups) {
    const int r0 = g * G, r1 = (int)min((int64_t)r0 + G, (int64_t)M);
    int w = 0;
    for (int r = r0; r < r1; ++r) w = max(w, row_ptr[r + 1] - row_ptr[r]);
    gw[g] = w;
    mine = (unsigned long long)w * (unsigned long long)(r1 - r0);
  }
  for (int o = kWave / 2; o > 0; o >>= 1) mine += __shfl_xor(mine, o, kWave);
  __shared__ unsigned long long s_sum[kWavesPerBlock];
  if (lane_id() == 0) s_sum[threadIdx.x / kWave] = mine;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long t = 0;
    for (int i = 0; i < kWavesPerBlock; ++i) t += s_sum[i];
    atomicAdd(stored, t);
  }
}

// Group bases: exclusive prefix sum of width x G over the groups (int64),
// one workgroup, each thread a contiguous chunk; base[ngroups] = total.
__global__ __launch_bounds__(1024) void rg_base_kernel(const int32_t* __restrict__ gw,
                                                       int32_t ngroups, int32_t G,
                                                       int64_t* __restrict__ base) {
  __shared__ int64_t s_part[1024];
  const int t = threadIdx.x;
  const int64_t per = ((int64_t)ngroups + 1023) / 1024;
  const int64_t b = min((int64_t)ngroups, t * per), e = min((int64_t)ngroups, b + per);
  int64_t local = 0;
  for (int64_t g = b; g < e; ++g) local += (int64_t)gw[g] * G;
  s_part[t] = local;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int64_t v = t >= o ? s_part[t - o] : 0;
    __syncthreads();
    s_part[t] += v;
    __syncthreads();
  }
  int64_t run = s_part[t] - local;
  for (int64_t g = b; g < e; ++g) {
    base[g] = run;
    run += (int64_t)gw[g] * G;
  }
  if (t == 1023) base[ngroups] = s_part[1023];
}

// Column-interleaved copy: entry k of row r at base[g] + k * G + (r - g G);
// padding (k past the row's length, up to the group width) holds the row's
// last column (or 0) and the value 0. Also the row lengths.
template <typename V>
__global__ __launch_bounds__(kBlock) void rg_fill_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const V* __restrict__ values, int32_t M, int32_t G, const int32_t* __restrict__ gw,
    const int64_t* __restrict__ base, int32_t* __restrict__ rl, int32_t* __restrict__ col_rg,
    V* __restrict__ val_rg) {
  const int r = blockIdx.x * kBlock + threadIdx.x;
  if (r >= M) return;
  const int g = r / G;
  const int w = gw[g];
  const int a = row_ptr[r], L = row_ptr[r + 1] - a;
  rl[r] = L;
  const int pad_col = L > 0 ? col_idx[a + L - 1] : 0;
  int64_t at = base[g] + (r - g * G);
  for (int k = 0; k < w; ++k, at += G) {
    col_rg[at] = k < L ? col_idx[a + k] : pad_col;
    val_rg[at] = k < L ? values[a + k] : V(0);
  }
}

template <typename V>
__global__ __launch_bounds__(kBlock) void rg_spmv_kernel(const RgArgs<V> a) {
  constexpr int U = 4;
  const int64_t r64 = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const bool live = r64 < a.M;
  const int r = live ? (int)r64 : a.M - 1;
  const int g = r / a.G;
  // unsigned: stepping past a row of nearly 2^31 entries must not wrap
  const unsigned L = live ? (unsigned)a.rl[r] : 0u;
  const int64_t at = a.base[g] + (r - (int64_t)g * a.G);
  V acc = V(0);
  for (unsigned k = 0; __ballot(k < L) != 0; k += U) {
    int c[U];
    V v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = k + u < L;
      c[u] = ok ? ld_stream(a.col + at + (int64_t)(k + u) * a.G) : 0;
      v[u] = ok ? ld_stream(a.val + at + (int64_t)(k + u) * a.G) : V(0);
    }
    // every gather in flight before the first FMA; a padded step reads x[0]
    // and adds nothing (a select, not 0 * x)
    V xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) xv[u] = a.x[c[u]];
#pragma unroll
    for (int u = 0; u < U; ++u) acc = k + u < L ? fma(v[u], xv[u], acc) : acc;
  }
  if (!live) return;
  V out = a.alpha * acc;
  if (a.beta_nonzero) out = fma(a.beta, a.y[r], out);
  a.y[r] = out;
}

}  // namespace

hipError_t launch_rg_build(const int32_t* row_ptr, const int32_t* col_idx, const void* values,
                           int vbytes, int64_t M, int32_t G, int32_t* gw, int64_t* base,
                           int32_t* rl, int32_t* col_rg, void* val_rg, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int blocks = (int)((M + kBlock - 1) / kBlock);
  if (vbytes == 4)
    hipLaunchKernelGGL(rg_fill_kernel<float>, dim3(blocks), dim3(kBlock), 0, s, row_ptr, col_idx,
                       static_cast<const float*>(values), (int32_t)M, G, gw, base, rl, col_rg,
                       static_cast<float*>(val_rg));
  else
    hipLaunchKernelGGL(rg_fill_kernel<double>, dim3(blocks), dim3(kBlock), 0, s, row_ptr,
                       col_idx, static_cast<const double*>(values), (int32_t)M, G, gw, base, rl,
                       col_rg, static_cast<double*>(val_rg));
  return hipGetLastError();
}

hipError_t launch_rg_widths(const int32_t* row_ptr, int64_t M, int32_t G, int32_t* gw,
                            int64_t* base, unsigned long long* stored, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int ngroups = (int)((M + G - 1) / G);
  hipLaunchKernelGGL(rg_width_kernel, dim3((ngroups + kBlock - 1) / kBlock), dim3(kBlock), 0, s,
                     row_ptr, (int32_t)M, G, ngroups, gw, stored);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(rg_base_kernel, dim3(1), dim3(1024), 0, s, gw, ngroups, G, base);
  return hipGetLastError();
}

template <typename V>
hipError_t launch_rg_spmv(const RgArgs<V>& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if (a.M == 0) return hipSuccess;
  launch_timed(rg_spmv_kernel<V>, dim3((a.M + kBlock - 1) / kBlock), dim3(kBlock), 0, s, ev0, ev1,
               a);
  return hipGetLastError();
}

template hipError_t launch_rg_spmv<float>(const RgArgs<float>&, hipStream_t, hipEvent_t,
                                          hipEvent_t);
template hipError_t launch_rg_spmv<double>(const RgArgs<double>&, hipStream_t, hipEvent_t,
                                           hipEvent_t);

}  // namespace spmv
