// Measurement aids, for reports that put an SpMV's time beside what simpler
// access patterns reach on the same GPU. None of them computes any part of
// the SpMV.
//
//  * read probe: the achievable streaming-read bandwidth. Every wavefront
//    reads one 4 KiB block once (64 lanes x 4 x 16-byte non-temporal loads,
//    all issued before the first use) and exits: on gfx950 this one-shot
//    pattern streams faster than a grid-stride loop.
//  * gather probe: a matrix's column indices read once, in storage order, and
//    x gathered at each of them, nothing else (the cost of the gathers an
//    SpMV of that matrix cannot avoid, with the matrix's own locality).
//  * stream probe: the SpMV's own access mix without x: each wavefront
//    streams one partition's share of row_ptr, col_idx and values (T units
//    of rows + nonzeros, cut evenly) and writes its share of y.
// Loaded values are folded into one word that is stored only if it equals a
// key known at run time alone, so the compiler cannot drop the loads. Every
// index is clamped into its array, so the probes never read or write outside
// the caller's buffers whatever they hold.
#include "device_common.hpp"
#include "internal.hpp"

namespace spmv {
namespace {

__global__ __launch_bounds__(kBlock) void read_probe_kernel(const i32x4* __restrict__ a,
                                                            int64_t n16, int32_t key,
                                                            int32_t* sink) {
  const int64_t w = ((int64_t)blockIdx.x * kBlock + threadIdx.x) / kWave;
  const int64_t base = w * 4 * kWave + lane_id();
  i32x4 v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t i = base + (int64_t)k * kWave;
    v[k] = i < n16 ? ld_stream(a + i) : i32x4{0, 0, 0, 0};
  }
  int32_t s = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) s ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  if (s == key) sink[0] = s;
}

// the bits of a probe's folded value, compared with the key
__device__ __forceinline__ int32_t fold_bits(float v) { return __float_as_int(v); }
__device__ __forceinline__ int32_t fold_bits(double v) {
  const int64_t b = __double_as_longlong(v);
  return (int32_t)b ^ (int32_t)(b >> 32);
}

// One wavefront per 1,024 column indices: 4 rounds of 16-byte quads, every
// load in flight before the first gather.
template <typename V>
__global__ __launch_bounds__(kBlock) void gather_probe_kernel(const int32_t* __restrict__ col,
                                                              int64_t nnz,
                                                              const V* __restrict__ x,
                                                              uint32_t n_x, int32_t key,
                                                              int32_t* sink) {
  const int64_t w = ((int64_t)blockIdx.x * kBlock + threadIdx.x) / kWave;
  i32x4 c[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t q = w * 4 * kWave + (int64_t)k * kWave + lane_id();
    if (4 * q + 3 < nnz) {
      c[k] = ld_stream(reinterpret_cast<const i32x4*>(col) + q);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) c[k][j] = 4 * q + j < nnz ? col[4 * q + j] : 0;
    }
  }
  V s = V(0);
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j) s += x[min((uint32_t)c[k][j], n_x - 1)];
  if (fold_bits(s) == key) sink[0] = key;
}

// X-row gathers as the SpMM kernels issue them: a wavefront is 64 / KL
// slots of KL lanes, a slot takes one column index per round and its lanes
// read the 16-byte parts of that row of X (rows of 16 KL bytes); 8 rounds,
// every load in flight before the first use. The column indices come
// straight from global memory (one line per round for the whole wave).
template <int KL>
__global__ __launch_bounds__(kBlock) void gather_rows_probe_kernel(const int32_t* __restrict__ col,
                                                                   int64_t nnz,
                                                                   const char* __restrict__ X,
                                                                   uint32_t n_rows, int32_t key,
                                                                   int32_t* sink) {
  constexpr int S = kWave / KL, U = 8;
  const int64_t w = ((int64_t)blockIdx.x * kBlock + threadIdx.x) / kWave;
  const int lane = lane_id();
  const int s = lane / KL, part = lane % KL;
  const int64_t base = w * S * U;
  int c[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t e = base + (int64_t)S * u + s;
    c[u] = e < nnz ? col[e] : 0;
  }
  i32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t r = min((uint32_t)c[u], n_rows - 1);
    v[u] = *reinterpret_cast<const i32x4*>(X + (r * KL + part) * 16);
  }
  int32_t acc = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  if (acc == key) sink[0] = key;
}

// One wavefront per partition of T = 64 * IPT units, P = ceil((M + nnz) / T):
// rows [p R, (p+1) R) and nonzeros [p Z, (p+1) Z), R = ceil(M / P) and
// Z = ceil(nnz / P), clipped to the arrays.
// Every quad of the three arrays is loaded first (16-byte non-temporal loads,
// clamped to the arrays' full quads: a partial last quad is read as the full
// one before it, since the probe times bytes, not values), then the rows of y
// are written with a value folded from the loads (cached stores, as the
// stream kernel writes y).
template <typename V, int IPT>
__global__ __launch_bounds__(kBlock) void stream_probe_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
    const V* __restrict__ val, int64_t M, int64_t nnz, int64_t P, int64_t rows_per,
    int64_t nnz_per, V* __restrict__ y) {
  constexpr int RQ = (kWave * IPT / 4 + 2 + kWave - 1) / kWave;
  const int64_t p = ((int64_t)blockIdx.x * kBlock + threadIdx.x) / kWave;
  if (p >= P) return;
  const int lane = lane_id();
  // equal shares (the last one shorter), no division on the device
  const int64_t r0 = min(M, p * rows_per), r1 = min(M, r0 + rows_per);
  const int64_t n0 = min(nnz, p * nnz_per), n1 = min(nnz, n0 + nnz_per);
  const int64_t nqn = nnz / 4, nqr = (M + 1) / 4;
  const int64_t qn0 = n0 / 4, qn1 = max(qn0 + 1, (n1 + 3) / 4);
  const int64_t qr0 = r0 / 4, qr1 = (r1 + 4) / 4;
  i32x4 c[RQ], e[RQ];
  Quad<V> v[RQ];
#pragma unroll
  for (int k = 0; k < RQ; ++k) {
    const int q = (int)max((int64_t)0, min(min(qn0 + k * kWave + lane, qn1 - 1), nqn - 1));
    c[k] = nqn > 0 ? ld_stream(reinterpret_cast<const i32x4*>(col) + q) : i32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int k = 0; k < RQ; ++k) {
    const int q = (int)max((int64_t)0, min(min(qn0 + k * kWave + lane, qn1 - 1), nqn - 1));
    if (nqn > 0) {
      v[k] = load_quad<false>(val, q, 0);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[k].set(j, V(0));
    }
  }
#pragma unroll
  for (int k = 0; k < RQ; ++k) {
    const int q = (int)max((int64_t)0, min(min(qr0 + k * kWave + lane, qr1 - 1), nqr - 1));
    e[k] = nqr > 0 ? ld_stream(reinterpret_cast<const i32x4*>(row_ptr) + q) : i32x4{0, 0, 0, 0};
  }
  V s = V(0);
#pragma unroll
  for (int k = 0; k < RQ; ++k) s += (V)(c[k][0] ^ c[k][3] ^ e[k][0] ^ e[k][3]) + v[k][0] + v[k][3];
  for (int64_t r = r0 + lane; r < r1; r += kWave) y[r] = s;
}

}  // namespace

hipError_t launch_gather_probe(const int32_t* col_idx, int64_t nnz, const void* x, int64_t n_x,
                               int vbytes, int32_t key, int32_t* sink, hipStream_t s) {
  const int64_t waves = (nnz + 4 * 4 * kWave - 1) / (4 * 4 * kWave);
  const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks <= 0 || n_x <= 0) return hipSuccess;
  if (blocks > 0x7fffffffll || n_x > 0xffffffffll) return hipErrorInvalidValue;
  if (vbytes == 4)
    hipLaunchKernelGGL(gather_probe_kernel<float>, dim3((unsigned)blocks), dim3(kBlock), 0, s,
                       col_idx, nnz, static_cast<const float*>(x), (uint32_t)n_x, key, sink);
  else
    hipLaunchKernelGGL(gather_probe_kernel<double>, dim3((unsigned)blocks), dim3(kBlock), 0, s,
                       col_idx, nnz, static_cast<const double*>(x), (uint32_t)n_x, key, sink);
  return hipGetLastError();
}

hipError_t launch_gather_rows_probe(const int32_t* col_idx, int64_t nnz, const void* X,
                                    int64_t n_rows, int row_bytes, int32_t key, int32_t* sink,
                                    hipStream_t s) {
  const int kl = row_bytes / 16;
  const int64_t per_wave = (int64_t)(kWave / kl) * 8;
  const int64_t waves = (nnz + per_wave - 1) / per_wave;
  const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffll || n_rows <= 0 || n_rows > 0xffffffffll) return hipErrorInvalidValue;
  const dim3 g((unsigned)blocks), b(kBlock);
  const char* xb = static_cast<const char*>(X);
  switch (kl) {
    case 1: hipLaunchKernelGGL(gather_rows_probe_kernel<1>, g, b, 0, s, col_idx, nnz, xb, (uint32_t)n_rows, key, sink); break;
    case 2: hipLaunchKernelGGL(gather_rows_probe_kernel<2>, g, b, 0, s, col_idx, nnz, xb, (uint32_t)n_rows, key, sink); break;
    case 4: hipLaunchKernelGGL(gather_rows_probe_kernel<4>, g, b, 0, s, col_idx, nnz, xb, (uint32_t)n_rows, key, sink); break;
    case 8: hipLaunchKernelGGL(gather_rows_probe_kernel<8>, g, b, 0, s, col_idx, nnz, xb, (uint32_t)n_rows, key, sink); break;
    case 16: hipLaunchKernelGGL(gather_rows_probe_kernel<16>, g, b, 0, s, col_idx, nnz, xb, (uint32_t)n_rows, key, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename V>
hipError_t launch_stream_probe_t(const int32_t* row_ptr, const int32_t* col, const V* val,
                                 int64_t M, int64_t nnz, int ipt, V* y, hipStream_t s) {
  const int64_t T = (int64_t)kWave * ipt;
  const int64_t P = (M + nnz + T - 1) / T;
  const int64_t blocks = (P + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffll) return hipErrorInvalidValue;
  const int64_t R = (M + P - 1) / P, Z = (nnz + P - 1) / P;   // R + Z <= T + 2
  const dim3 g((unsigned)blocks), b(kBlock);
  switch (ipt) {
    case 4: hipLaunchKernelGGL((stream_probe_kernel<V, 4>), g, b, 0, s, row_ptr, col, val, M, nnz, P, R, Z, y); break;
    case 8: hipLaunchKernelGGL((stream_probe_kernel<V, 8>), g, b, 0, s, row_ptr, col, val, M, nnz, P, R, Z, y); break;
    case 16: hipLaunchKernelGGL((stream_probe_kernel<V, 16>), g, b, 0, s, row_ptr, col, val, M, nnz, P, R, Z, y); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_stream_probe(const int32_t* row_ptr, const int32_t* col_idx, const void* values,
                               int64_t M, int64_t nnz, int vbytes, int ipt, void* y,
                               hipStream_t s) {
  if (vbytes == 4)
    return launch_stream_probe_t(row_ptr, col_idx, static_cast<const float*>(values), M, nnz,
                                 ipt, static_cast<float*>(y), s);
  return launch_stream_probe_t(row_ptr, col_idx, static_cast<const double*>(values), M, nnz, ipt,
                               static_cast<double*>(y), s);
}

hipError_t launch_read_probe(const void* data, int64_t bytes, int32_t key, int32_t* sink,
                             hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int64_t waves = (n16 + 4 * kWave - 1) / (4 * kWave);
  const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffll) return hipErrorInvalidValue;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s,
                     static_cast<const i32x4*>(data), n16, key, sink);
  return hipGetLastError();
}

}  // namespace spmv
