// Achievable streaming-read bandwidth of the device, for reports that put an
// SpMV's bytes per second beside what plain reads reach on the same GPU.
//
// Every wavefront reads one 4 KiB block once (64 lanes x 4 x 16-byte
// non-temporal loads, all issued before the first use) and exits: on gfx950
// this one-shot pattern streams faster than a grid-stride loop. The loaded
// values are folded into one word that is stored only if it equals a key
// known at run time alone, so the compiler cannot drop the loads.
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

}  // namespace

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
