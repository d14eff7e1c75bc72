// Device-side helpers shared by the gfx950 kernels of libspmv.so.
//
// Everything here is written for CDNA4 wave64: a wavefront is 64 lanes that
// execute in lockstep, so lanes of one wave can hand data to each other
// through LDS with only a compiler/memory fence (no s_barrier).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"

namespace spmv {

// LDS hand-off between lanes of the same wave.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Workgroups are handed to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8). Renumber the workgroups of the range [begin, begin + n) so that the
// ones landing on one XCD take a contiguous run of tiles: neighbouring tiles
// then share that XCD's L2 (x entries of banded and stencil matrices).
__device__ __forceinline__ int xcd_tile(int b, int begin, int n) {
  const int j = b - begin;
  const int xcd = b % kXcds;
  const int j0 = (xcd - begin % kXcds + kXcds) % kXcds;  // first j on this XCD
  int before = 0;                                        // tiles of lower XCDs
#pragma unroll
  for (int k = 0; k < kXcds; ++k) {
    const int jk = (k - begin % kXcds + kXcds) % kXcds;
    const int ck = jk < n ? (n - jk + kXcds - 1) / kXcds : 0;
    before += k < xcd ? ck : 0;
  }
  return before + (j - j0) / kXcds;
}

// Streaming (read-once) loads and stores: non-temporal, so they do not push
// the gathered vector out of L2.
template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
  return __builtin_nontemporal_load(p);
}
template <typename T>
__device__ __forceinline__ void st_stream(T* p, T v) {
  __builtin_nontemporal_store(v, p);
}

// Segmented inclusive scan across the wave: lanes with equal `key` that are
// contiguous form a segment (keys must be non-decreasing across lanes).
template <typename V>
__device__ __forceinline__ V wave_segscan(V v, int key) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const V t = __shfl_up(v, o, kWave);
    const int kt = __shfl_up(key, o, kWave);
    if (lane >= o && kt == key) v += t;
  }
  return v;
}

// Sum over aligned groups of G lanes (G a power of two <= 64); every lane of
// the group gets the total.
template <int G, typename V>
__device__ __forceinline__ V group_sum(V v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace spmv
