// Device-side helpers shared by the gfx950 kernels of libspmv.so.
//
// Everything here is written for CDNA4 wave64: a wavefront is 64 lanes that
// execute in lockstep, so lanes of one wave can hand data to each other
// through LDS with only a compiler/memory fence (no s_barrier).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <limits.h>

#include "internal.hpp"

namespace spmv {

// LDS hand-off between lanes of the same wave.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// gfx950 direct-to-LDS load: this lane's 16 bytes at g land at
// lds_wave_base + 16 * lane (lds_wave_base must be wave-uniform). The load is
// counted by vmcnt like any vector load; the compiler does not track the LDS
// write, so readers wait with wait_vmem() and a barrier. (The builtin exists
// only for the device target; the host pass never runs this code.)
__device__ __forceinline__ void lds_dma16(const void* g, void* lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base,
                                   16, 0, 0);
#endif
}
__device__ __forceinline__ void wait_vmem() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(0);
#endif
}
// Wait until at most N vector memory instructions of this wave are in
// flight (they retire in order: everything older than the last N is done);
// LDS, scalar and export counters are not waited for. gfx9 encoding:
// vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
#endif
}
// The same, and every LDS access of this wave done (lgkmcnt 0).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
#endif
}
// Keeps the compiler from moving memory accesses across this point.
__device__ __forceinline__ void memory_order_point() { asm volatile("" ::: "memory"); }

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

// Streamed load of a T at byte offset off from base. With a wave-uniform
// base (held in scalar registers) and a 32-bit offset the load takes the
// scalar-base address form: one VGPR per address instead of a 64-bit pair,
// and loads of several arrays at the same offset share it.
template <typename T>
__device__ __forceinline__ T ld_stream_at(const void* base, uint32_t off) {
  return __builtin_nontemporal_load(
      reinterpret_cast<const T*>(static_cast<const char*>(base) + off));
}

// 16-byte vectors for quad loads.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

// Four consecutive values of type V (one 16-byte load for fp32, two for fp64).
template <typename V> struct Quad;
template <> struct Quad<float> {
  f32x4 v;
  __device__ __forceinline__ float operator[](int j) const { return v[j]; }
  __device__ __forceinline__ void set(int j, float a) { v[j] = a; }
};
template <> struct Quad<double> {
  f64x2 lo, hi;
  __device__ __forceinline__ double operator[](int j) const { return j < 2 ? lo[j] : hi[j - 2]; }
  __device__ __forceinline__ void set(int j, double a) {
    if (j < 2) lo[j] = a; else hi[j - 2] = a;
  }
};

// Elements [4q, 4q + 4) of a 16-byte aligned array of n elements, streamed
// (n < 2^31; the bound is compared unsigned, since 4q + 3 may pass 2^31 - 1).
// SAFE = false: the caller guarantees 4q + 3 < n (one or two 16-byte loads).
// SAFE = true: elements at or past n read as 0 and nothing past the array is
// touched (element-wise loads); used only by the wave that holds the array's
// last, partial quad, so the fast path has no per-lane branch.
template <bool SAFE>
__device__ __forceinline__ i32x4 load_quad(const int32_t* a, int q, int n) {
  if (!SAFE) return ld_stream(reinterpret_cast<const i32x4*>(a) + q);
  i32x4 r = {0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (4u * (uint32_t)q + j < (uint32_t)n) r[j] = a[4 * (int64_t)q + j];
  return r;
}
template <bool SAFE>
__device__ __forceinline__ Quad<float> load_quad(const float* a, int q, int n) {
  Quad<float> r;
  if (!SAFE) {
    r.v = ld_stream(reinterpret_cast<const f32x4*>(a) + q);
  } else {
    r.v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4u * (uint32_t)q + j < (uint32_t)n) r.v[j] = a[4 * (int64_t)q + j];
  }
  return r;
}
template <bool SAFE>
__device__ __forceinline__ Quad<double> load_quad(const double* a, int q, int n) {
  Quad<double> r;
  if (!SAFE) {
    r.lo = ld_stream(reinterpret_cast<const f64x2*>(a) + 2 * q);
    r.hi = ld_stream(reinterpret_cast<const f64x2*>(a) + 2 * q + 1);
  } else {
    r.lo = f64x2{0.0, 0.0};
    r.hi = f64x2{0.0, 0.0};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4u * (uint32_t)q + j < (uint32_t)n) r.set(j, a[4 * (int64_t)q + j]);
  }
  return r;
}
__device__ __forceinline__ void store_quad(float* lds, int i, const Quad<float>& v) {
  *reinterpret_cast<f32x4*>(lds + 4 * i) = v.v;
}
__device__ __forceinline__ void store_quad(double* lds, int i, const Quad<double>& v) {
  reinterpret_cast<f64x2*>(lds + 4 * i)[0] = v.lo;
  reinterpret_cast<f64x2*>(lds + 4 * i)[1] = v.hi;
}

// p when `in`, else exactly +0 (whatever p is: NaN and infinities too), by
// clearing its bits rather than by a select the compiler could turn into a
// branch.
__device__ __forceinline__ float mask_zero(bool in, float p) {
  return __int_as_float(__float_as_int(p) & (in ? -1 : 0));
}
__device__ __forceinline__ double mask_zero(bool in, double p) {
  return __longlong_as_double(__double_as_longlong(p) & (in ? -1ll : 0ll));
}

// val * x[col] when `in`, else exactly +0, without a branch: a gather under
// a branch is waited for before the branch joins, which would serialise a
// partition's gathers. Masked lanes read x[0] (one cache line for all).
template <typename V>
__device__ __forceinline__ V masked_product(bool in, V v, const V* __restrict__ x, int col) {
  return mask_zero(in, v * x[in ? col : 0]);
}

// Stage, with 16-byte loads, the row ends and the products of one partition:
//   ends[4 * (q - qr0) + j] = row_ptr[4q + j] - sub     for quads [qr0, qr0 + nqr)
//   prods[4 * (q - qn0) + j] = val[k] * x[col[k]], k = 4q + j, for [qn0, qn0 + nqn)
// row_ptr (m elements), col and val (nnz elements) are 16-byte aligned.
// Entries of the edge quads outside the caller's range are valid matrix
// entries (or 0 past the end of an array), so every gather stays inside x.
//
// Fast path: NR row rounds and NN nonzero rounds of 64 quads each, fixed at
// compile time, lane quads clamped into range (a clamped lane repeats the
// last quad, which costs no extra cache lines), so the code is straight-line
// and every load is issued before the first use.
// MASK: the products of nonzeros k outside [lo, hi) are 0, without a gather
// (nonzeros another kernel sums).
template <typename V, int NR, int NN, bool MASK>
__device__ __forceinline__ void stage_fast(const int32_t* __restrict__ row_ptr, int qr0, int nqr,
                                           int sub, const int32_t* __restrict__ col,
                                           const V* __restrict__ val,
                                           const V* __restrict__ x, int qn0, int nqn,
                                           int32_t* ends, V* prods, int lo, int hi) {
  const int lane = lane_id();
  i32x4 e[NR > 0 ? NR : 1];
  i32x4 c[NN > 0 ? NN : 1];
  Quad<V> v[NN > 0 ? NN : 1];
  // wave-uniform bases and 32-bit byte offsets; all column quads, then all
  // value quads, then the row ends (needed last)
  const int32_t* cb = col + 4 * (int64_t)qn0;
  const V* vbase = val + 4 * (int64_t)qn0;
  const int32_t* eb = row_ptr + 4 * (int64_t)qr0;
#pragma unroll
  for (int r = 0; r < NN; ++r)
    c[r] = ld_stream_at<i32x4>(cb, 16u * (uint32_t)min(lane + kWave * r, nqn - 1));
#pragma unroll
  for (int r = 0; r < NN; ++r) {
    const uint32_t off = 16u * (uint32_t)min(lane + kWave * r, nqn - 1);
    if constexpr (sizeof(V) == 4) {
      v[r].v = ld_stream_at<f32x4>(vbase, off);
    } else {
      v[r].lo = ld_stream_at<f64x2>(vbase, 2 * off);
      v[r].hi = ld_stream_at<f64x2>(vbase, 2 * off + 16);
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r)
    e[r] = ld_stream_at<i32x4>(eb, 16u * (uint32_t)min(lane + kWave * r, nqr - 1));
#pragma unroll
  for (int r = 0; r < NN; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (MASK) {
        const int k = 4 * (qn0 + min(lane + kWave * r, nqn - 1)) + j;
        v[r].set(j, masked_product(k >= lo && k < hi, v[r][j], x, c[r][j]));
      } else {
        v[r].set(j, v[r][j] * x[c[r][j]]);
      }
    }
  // clamped lanes rewrite the last quad with the same values: unconditional
  // stores keep the loads from being sunk into (and serialised by) branches
#pragma unroll
  for (int r = 0; r < NR; ++r)
    *reinterpret_cast<i32x4*>(ends + 4 * min(lane + kWave * r, nqr - 1)) = e[r] - sub;
#pragma unroll
  for (int r = 0; r < NN; ++r) store_quad(prods, min(lane + kWave * r, nqn - 1), v[r]);
}

// Slow path for the one partition that reaches an array's last, partial
// quad: element-wise guarded loads, exec-masked rounds.
template <typename V, int RQR, int RQN, bool MASK = false>
__device__ __forceinline__ void stage_safe(const int32_t* __restrict__ row_ptr, int m, int qr0,
                                        int nqr, int sub, const int32_t* __restrict__ col,
                                        const V* __restrict__ val, const V* __restrict__ x,
                                        int nnz, int qn0, int nqn, int32_t* ends, V* prods,
                                        int lo = 0, int hi = INT_MAX) {
  const int lane = lane_id();
  for (int r = 0; r < RQR; ++r)
    if (lane + kWave * r < nqr) {
      const i32x4 e = load_quad<true>(row_ptr, qr0 + lane + kWave * r, m);
      *reinterpret_cast<i32x4*>(ends + 4 * (lane + kWave * r)) = e - sub;
    }
  for (int r = 0; r < RQN; ++r)
    if (lane + kWave * r < nqn) {
      const i32x4 c = load_quad<true>(col, qn0 + lane + kWave * r, nnz);
      Quad<V> v = load_quad<true>(val, qn0 + lane + kWave * r, nnz);
      for (int j = 0; j < 4; ++j) {
        const int k = 4 * (qn0 + lane + kWave * r) + j;
        v.set(j, MASK ? masked_product(k >= lo && k < hi, v[j], x, c[j]) : v[j] * x[c[j]]);
      }
      store_quad(prods, lane + kWave * r, v);
    }
}

template <typename V, int NR, int RQN, bool MASK>
__device__ __forceinline__ void stage_dispatch_nn(const int32_t* row_ptr, int qr0, int nqr,
                                                  int sub, const int32_t* col, const V* val,
                                                  const V* x, int qn0, int nqn, int32_t* ends,
                                                  V* prods, int lo, int hi) {
  const int rounds = (nqn + kWave - 1) / kWave;
  if (rounds == 0)
    stage_fast<V, NR, 0, MASK>(row_ptr, qr0, nqr, sub, col, val, x, qn0, nqn, ends, prods, lo, hi);
  else if (rounds == 1 || RQN < 2)
    stage_fast<V, NR, 1, MASK>(row_ptr, qr0, nqr, sub, col, val, x, qn0, nqn, ends, prods, lo, hi);
  else if (rounds == 2 || RQN < 3)
    stage_fast<V, NR, (RQN < 2 ? 1 : 2), MASK>(row_ptr, qr0, nqr, sub, col, val, x, qn0, nqn, ends, prods, lo, hi);
  else if (rounds == 3 || RQN < 4)
    stage_fast<V, NR, (RQN < 3 ? 1 : 3), MASK>(row_ptr, qr0, nqr, sub, col, val, x, qn0, nqn, ends, prods, lo, hi);
  else if (rounds == 4 || RQN < 5)
    stage_fast<V, NR, (RQN < 4 ? 1 : 4), MASK>(row_ptr, qr0, nqr, sub, col, val, x, qn0, nqn, ends, prods, lo, hi);
  else if (rounds == 5 || RQN < 6)
    stage_fast<V, NR, (RQN < 5 ? 1 : 5), MASK>(row_ptr, qr0, nqr, sub, col, val, x, qn0, nqn, ends, prods, lo, hi);
  else
    stage_fast<V, NR, (RQN < 6 ? 1 : 6), MASK>(row_ptr, qr0, nqr, sub, col, val, x, qn0, nqn, ends, prods, lo, hi);
}

// Stage one partition (see stage_fast). RQR / RQN bound the rounds.
template <typename V, int RQR, int RQN, bool MASK = false>
__device__ __forceinline__ void stage_partition(const int32_t* __restrict__ row_ptr, int m,
                                                int qr0, int nqr, int sub,
                                                const int32_t* __restrict__ col,
                                                const V* __restrict__ val,
                                                const V* __restrict__ x, int nnz, int qn0,
                                                int nqn, int32_t* ends, V* prods, int lo = 0,
                                                int hi = INT_MAX) {
  static_assert(RQN <= 6, "at most 6 nonzero rounds");
  // does this partition reach an array's last, partial quad? (wave-uniform)
  const bool tail = (nqr > 0 && (m & 3) && qr0 + nqr - 1 == (m - 1) >> 2) ||
                    (nqn > 0 && (nnz & 3) && qn0 + nqn - 1 == (nnz - 1) >> 2);
  if (tail) {
    stage_safe<V, RQR, RQN, MASK>(row_ptr, m, qr0, nqr, sub, col, val, x, nnz, qn0, nqn, ends,
                                  prods, lo, hi);
    return;
  }
  const int rrounds = (nqr + kWave - 1) / kWave;
  if (rrounds == 0)
    stage_dispatch_nn<V, 0, RQN, MASK>(row_ptr, qr0, nqr, sub, col, val, x, qn0, nqn, ends, prods, lo, hi);
  else if (rrounds == 1 || RQR < 2)
    stage_dispatch_nn<V, 1, RQN, MASK>(row_ptr, qr0, nqr, sub, col, val, x, qn0, nqn, ends, prods, lo, hi);
  else
    stage_dispatch_nn<V, RQR, RQN, MASK>(row_ptr, qr0, nqr, sub, col, val, x, qn0, nqn, ends, prods, lo, hi);
}

// ---- cross-lane moves in DPP form (gfx9 encodings) ---------------------------
// A DPP move reads another lane's register as an operand modifier of a VALU
// instruction: no LDS traffic and no wait, unlike a ds_bpermute shuffle.
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7 - i within 8
constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15 - i within 16
constexpr int kDppWaveShl1 = 0x130;       // lane i <- lane i + 1 (lane 63: none)
constexpr int kDppWaveShr1 = 0x138;       // lane i <- lane i - 1 (lane 0: none)
constexpr int kDppRowBcast15 = 0x142;     // rows 1, 3 <- lane 15 of rows 0, 2
constexpr int kDppRowBcast31 = 0x143;     // rows 2, 3 <- lane 31
constexpr int dpp_row_shr(int n) { return 0x110 + n; }  // lane i <- i - n in its row of 16

// this lane's copy of lane src(CTRL)'s v; lanes that CTRL gives no source
// (or whose row is outside ROWS) keep `old`. Callers never rely on `old` for
// those lanes: they test the lane position themselves. Every lane of the
// wave must execute the move (never call it under a condition or on one
// side of || or ?:): a lane reading from a lane masked off gets no value.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp_i32(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(dpp_i32<CTRL, ROWS>(0, __float_as_int(v)));
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ double dpp_move(double v) {
  const int64_t b = __double_as_longlong(v);
  const int lo = dpp_i32<CTRL, ROWS>(0, (int)(uint32_t)b);
  const int hi = dpp_i32<CTRL, ROWS>(0, (int)(b >> 32));
  return __longlong_as_double(((int64_t)hi << 32) | (uint32_t)lo);
}

// lane l - 1's value (lane 0: `first`) and lane l + 1's (lane 63: `last`)
__device__ __forceinline__ int lane_prev(int v, int first) {
  const int t = dpp_i32<kDppWaveShr1>(first, v);
  return lane_id() == 0 ? first : t;
}
__device__ __forceinline__ int lane_next(int v, int last) {
  const int t = dpp_i32<kDppWaveShl1>(last, v);
  return lane_id() == kWave - 1 ? last : t;
}
template <typename V>
__device__ __forceinline__ V lane_prev(V v) {
  const V t = dpp_move<kDppWaveShr1>(v);
  return lane_id() == 0 ? V(0) : t;
}

// One step of a segmented inclusive scan (Hillis-Steele over (value, head
// flag) pairs): when the lane's covered range holds no segment head, the
// range just before it (from lane src(CTRL)) is added, and the flags merge.
// `valid` says whether CTRL gives this lane a source in this step.
template <int CTRL, int ROWS, typename V>
__device__ __forceinline__ void segscan_step(V& v, int& f, bool valid) {
  // selects, not branches: every lane executes the moves
  const V t = dpp_move<CTRL, ROWS>(v);
  const int tf = dpp_i32<CTRL, ROWS>(0, f);
  v = valid && !f ? v + t : v;
  f = valid ? (f | tf) : f;
}

// Segmented inclusive scan across the wave, entirely in DPP moves: a segment
// starts at every lane whose `head` is set (and at lane 0). Shifts of 1, 2, 4
// and 8 lanes inside each row of 16, then the last lane of row 0 (2) into
// row 1 (3), then lane 31 into rows 2 and 3: after the six steps lane l holds
// the sum from the last head at or before l up to l. This is the wave-level
// form of the segmented reduction the PPoPP'23 load-balancing page's
// Sidebar 1 describes for the carry fix-up.
template <typename V>
__device__ __forceinline__ V wave_segscan(V v, bool head) {
  const int lane = lane_id();
  const int r = lane & 15, row = lane >> 4;
  int f = head || lane == 0;
  segscan_step<dpp_row_shr(1), 0xF>(v, f, r >= 1);
  segscan_step<dpp_row_shr(2), 0xF>(v, f, r >= 2);
  segscan_step<dpp_row_shr(4), 0xF>(v, f, r >= 4);
  segscan_step<dpp_row_shr(8), 0xF>(v, f, r >= 8);
  segscan_step<kDppRowBcast15, 0xA>(v, f, (row & 1) != 0);
  segscan_step<kDppRowBcast31, 0xC>(v, f, row >= 2);
  return v;
}

// Segments given by a key that does not decrease across the lanes: a lane
// heads a segment when its key differs from the previous lane's.
template <typename V>
__device__ __forceinline__ V wave_segscan_keys(V v, int key) {
  return wave_segscan(v, lane_prev(key, key) != key);
}

// Inclusive prefix sum of an int across the wave in DPP moves (integer
// sums: exact in any order).
__device__ __forceinline__ int wave_scan_i32(int x) {
  const int lane = lane_id();
  const int r = lane & 15, row = lane >> 4;
  int t;
  t = dpp_i32<dpp_row_shr(1)>(0, x);
  x += r >= 1 ? t : 0;
  t = dpp_i32<dpp_row_shr(2)>(0, x);
  x += r >= 2 ? t : 0;
  t = dpp_i32<dpp_row_shr(4)>(0, x);
  x += r >= 4 ? t : 0;
  t = dpp_i32<dpp_row_shr(8)>(0, x);
  x += r >= 8 ? t : 0;
  t = dpp_i32<kDppRowBcast15, 0xA>(0, x);
  x += (row & 1) ? t : 0;
  t = dpp_i32<kDppRowBcast31, 0xC>(0, x);
  x += row >= 2 ? t : 0;
  return x;
}

// Sum over the whole wave in DPP moves; the total lands in lane 63 (rows of
// 16 first, then row 0 into 1 and 2 into 3, then lane 31 into rows 2 and 3).
template <typename V>
__device__ __forceinline__ V wave_sum_to_last(V v) {
  const int row = lane_id() >> 4;
  v += dpp_move<kDppQuadXor1>(v);
  v += dpp_move<kDppQuadXor2>(v);
  v += dpp_move<kDppRowHalfMirror>(v);
  v += dpp_move<kDppRowMirror>(v);
  const V a = dpp_move<kDppRowBcast15, 0xA>(v);
  v = (row & 1) ? v + a : v;
  const V b = dpp_move<kDppRowBcast31, 0xC>(v);
  v = row >= 2 ? v + b : v;
  return v;
}

// Sum over aligned groups of G lanes, G in {1, 2, 4, 8, 16}, with DPP moves
// (no LDS traffic); every lane of the group gets the total. After the two
// quad steps all lanes of a quad hold its sum, so mirroring 8 (16) lanes
// pairs each lane with one of the other quad (other half).
template <int G, typename V>
__device__ __forceinline__ V group_sum_dpp(V v) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "DPP groups up to 16");
  if (G >= 2) v += dpp_move<kDppQuadXor1>(v);
  if (G >= 4) v += dpp_move<kDppQuadXor2>(v);
  if (G >= 8) v += dpp_move<kDppRowHalfMirror>(v);
  if (G >= 16) v += dpp_move<kDppRowMirror>(v);
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

// The row a partition's carry belongs to. On a plan with long-row tiles
// (skip: 1 for the partitions the walk skips), the carries of a tile row --
// those of its interior partitions, which the walk skips, and of the
// partition just before them, whose open row it is -- are all 0 and are
// keyed past the last row (M), so no fix-up writes a tile row's y: its
// tiles' reduction does, in the same launch. The skip flags decide, not the
// stored keys, which a multi-vector product without tiles rewrites.
template <bool TILED>
__device__ __forceinline__ int carry_key(const int32_t* __restrict__ carry_row,
                                         const int32_t* __restrict__ skip, int64_t p,
                                         int32_t P, int32_t M) {
  if (TILED && (skip[p] != 0 || (p + 1 < P && skip[p + 1] != 0))) return M;
  return carry_row[p];
}

}  // namespace spmv
