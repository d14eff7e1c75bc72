// spmv_exec_noalloc: one SpMV, y = alpha * A x + beta * y, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc). It runs what spmv_plan +
// spmv_exec run for a merge-path walk plan at a fixed partition size -- the
// split search, the walk kernel and the carry fix-up -- with the plan's
// scratch (statistics, split coordinates, carries) in a file-scope device
// array instead of a plan workspace. Nothing here allocates, frees or
// synchronises.
//
// The array is a host-side stand-in in host code: its device address, which
// differs per GPU, is looked up once per device with hipGetSymbolAddress and
// kept; kernels receive that address, never the array's name.
#include "spmv.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <mutex>

#include "internal.hpp"

namespace {

using namespace spmv;

// 32 MiB: the statistics block plus, per partition, two split coordinates,
// one row-bounds pair, a carry row and a carry value (24 bytes for fp32,
// 28 for fp64): about 1.19M partitions, M + nnz up to ~1.2e9 (fp32, T = 1024)
// or ~0.6e9 (fp64, T = 512).
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
char* g_scratch_ptr[kMaxDevices] = {};

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

// Scratch bytes for P partitions with values of vbytes bytes; the layout
// used below, in this order.
size_t scratch_need(int64_t P, size_t vbytes) {
  return round256(sizeof(int64_t) * kStatCount) + 2 * round256(sizeof(int32_t) * (P + 1)) +
         round256(sizeof(int32_t) * 2 * (P + 1)) + round256(sizeof(int32_t) * P) +
         round256(vbytes * P);
}

}  // namespace

namespace spmv {
// the library's thread-local error text (api.hip)
void set_last_error(const char* text);
}

extern "C" {

spmv_status_t spmv_exec_noalloc(int64_t M, int64_t N, int64_t nnz, const int32_t* row_ptr,
                                const int32_t* col_idx, const void* values, spmv_dtype_t dtype,
                                const void* x, void* y, double alpha, double beta,
                                hipStream_t stream) {
  auto fail = [](spmv_status_t st, const char* msg) {
    spmv::set_last_error(msg);
    return st;
  };
  if (dtype != SPMV_F32 && dtype != SPMV_F64) return fail(SPMV_ERR_INVALID_ARG, "unknown dtype");
  if (M < 0 || N < 0 || nnz < 0) return fail(SPMV_ERR_INVALID_ARG, "negative size");
  if ((M == 0 || N == 0) && nnz != 0)
    return fail(SPMV_ERR_INVALID_ARG, "M = 0 or N = 0 needs nnz = 0");
  if (nnz > 2147483647ll) return fail(SPMV_ERR_INVALID_ARG, "nnz beyond int32 indices");
  if (M >= 2147483647ll || N > 2147483647ll || M + nnz > 2147483647ll - 64)
    return fail(SPMV_ERR_UNSUPPORTED, "sizes beyond the int32 item model");
  if (M == 0) return SPMV_SUCCESS;
  if (!row_ptr || !y || (nnz > 0 && (!col_idx || !values || !x)))
    return fail(SPMV_ERR_INVALID_ARG, "NULL array");
  if ((reinterpret_cast<uintptr_t>(row_ptr) | reinterpret_cast<uintptr_t>(col_idx) |
       reinterpret_cast<uintptr_t>(values)) & 15)
    return fail(SPMV_ERR_INVALID_ARG, "row_ptr, col_idx and values must be 16-byte aligned");
  const size_t vs = dtype == SPMV_F32 ? 4 : 8;
  if (x && N > 0) {
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(x), x1 = x0 + (uintptr_t)N * vs;
    const uintptr_t y0 = reinterpret_cast<uintptr_t>(y), y1 = y0 + (uintptr_t)M * vs;
    if (x0 < y1 && y0 < x1) return fail(SPMV_ERR_INVALID_ARG, "x and y overlap");
  }
  const int ipt = dtype == SPMV_F32 ? 16 : 8;
  const int64_t T = (int64_t)kWave * ipt;
  const int64_t P = (M + nnz + T - 1) / T;
  if (scratch_need(P, vs) > kScratchBytes) {
    char msg[160];
    std::snprintf(msg, sizeof msg,
                  "M + nnz = %lld needs %zu bytes of scratch, more than the %zu it has",
                  (long long)(M + nnz), scratch_need(P, vs), kScratchBytes);
    return fail(SPMV_ERR_UNSUPPORTED, msg);
  }

  // this device's copy of the scratch array (looked up once per device)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SPMV_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SPMV_ERR_UNSUPPORTED, "device index >= 64");
  char* base;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) {
        (void)hipGetLastError();
        return fail(SPMV_ERR_HIP, "hipGetSymbolAddress of the scratch array failed");
      }
      g_scratch_ptr[dev] = static_cast<char*>(p);
    }
    base = g_scratch_ptr[dev];
  }
  size_t off = 0;
  auto take = [&](size_t bytes) { char* q = base + off; off += round256(bytes); return q; };
  int64_t* stats = reinterpret_cast<int64_t*>(take(sizeof(int64_t) * kStatCount));
  int32_t* split_row = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (P + 1)));
  int32_t* split_nz = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (P + 1)));
  int32_t* row_bounds = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * 2 * (P + 1)));
  int32_t* carry_row = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * P));
  void* carry_val = take(vs * P);

  // statistics cleared by a kernel (the split search adds to a counter),
  // the partition size fixed, the split, then the walk kernel and fix-up
  PlanCtl ctl;
  std::memset(&ctl, 0, sizeof ctl);
  ctl.M = M;
  ctl.N = N;
  ctl.nnz = nnz;
  ctl.vbytes = (int32_t)vs;
  ctl.forced_ipt = ipt;
  ctl.reduce_req = 1;
  ctl.order_req = 1;
  if ((e = launch_clear_stats(stats, stream)) != hipSuccess ||
      (e = launch_plan_choose(ctl, stats, 0, stream)) != hipSuccess ||
      (e = launch_split_search(row_ptr, M, nnz, P, 0, split_row, split_nz, row_bounds, stats,
                               stream)) != hipSuccess)
    return fail(SPMV_ERR_HIP, hipGetErrorString(e));
  if (dtype == SPMV_F32) {
    MergeArgs<float> a;
    std::memset(&a, 0, sizeof a);
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    a.val = static_cast<const float*>(values);
    a.x = static_cast<const float*>(x);
    a.y = static_cast<float*>(y);
    a.split_row = split_row;
    a.split_nz = split_nz;
    a.row_bounds = row_bounds;
    a.carry_row = carry_row;
    a.carry_val = static_cast<float*>(carry_val);
    a.alpha = (float)alpha;
    a.beta = (float)beta;
    a.beta_nonzero = beta != 0.0;
    a.P = (int32_t)P;
    a.M = (int32_t)M;
    a.nnz = (int32_t)nnz;
    a.xcd_remap = 1;
    e = launch_merge<float>(a, ipt, stream, nullptr, nullptr);
  } else {
    MergeArgs<double> a;
    std::memset(&a, 0, sizeof a);
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    a.val = static_cast<const double*>(values);
    a.x = static_cast<const double*>(x);
    a.y = static_cast<double*>(y);
    a.split_row = split_row;
    a.split_nz = split_nz;
    a.row_bounds = row_bounds;
    a.carry_row = carry_row;
    a.carry_val = static_cast<double*>(carry_val);
    a.alpha = alpha;
    a.beta = beta;
    a.beta_nonzero = beta != 0.0;
    a.P = (int32_t)P;
    a.M = (int32_t)M;
    a.nnz = (int32_t)nnz;
    a.xcd_remap = 1;
    e = launch_merge<double>(a, ipt, stream, nullptr, nullptr);
  }
  if (e != hipSuccess) return fail(SPMV_ERR_HIP, hipGetErrorString(e));
  return SPMV_SUCCESS;
}

}  // extern "C"
