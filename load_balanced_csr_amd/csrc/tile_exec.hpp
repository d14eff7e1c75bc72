// Column-blocked tiles of long rows, the device side of their execution:
// one workgroup per tile, a tile being one block of kTileBytes of x (staged
// in LDS) and up to kTileRows long rows, whose entries in that block's
// columns it sums into partial[row][block]. The plan's tile kernels build
// the rows and segments; the kernel that runs the tiles shares its grid with
// the merge-path walk over the partitions the tiles leave.
#pragma once

#include "device_common.hpp"
#include "internal.hpp"

namespace spmv {
namespace {

// x at a quad's four columns, for the entries `in` the segment: from the
// staged block in LDS (read unconditionally at a clamped index, so the read
// stays an LDS read and waits for no global load), or, for a column outside
// the block, from global memory. Only rows with unsorted columns have such
// entries in a segment; the wave takes that branch only when one of its
// lanes needs it.
template <typename V>
__device__ __forceinline__ void tile_x4(V (&xv)[4], const i32x4& c, const bool (&in)[4],
                                        const V* xs, const V* __restrict__ x, int c0, int clen) {
  bool out = false;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const unsigned lc = (unsigned)(c[e] - c0);
    const bool inb = lc < (unsigned)clen;
    xv[e] = xs[inb ? lc : 0u];
    out = out || (in[e] && !inb);
  }
  if (__builtin_amdgcn_ballot_w64(out) != 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (in[e] && (unsigned)(c[e] - c0) >= (unsigned)clen) xv[e] = x[c[e]];
  }
}

// Quads covering entries [s0, s1): the end quad, (s1 + 3) / 4, and whether
// entry 4q + e lies in [s0, s1), in unsigned arithmetic (nnz may come within
// a few entries of 2^31, where 4q + e overflows int32; as unsigned it stays
// below 2^32).
__device__ __forceinline__ int quad_end(int32_t s1) { return (int)(((uint32_t)s1 + 3u) >> 2); }
__device__ __forceinline__ bool in_segment(int q, int e, int32_t s0, int32_t s1) {
  const uint32_t k = 4u * (uint32_t)q + (uint32_t)e;
  return k >= (uint32_t)s0 && k < (uint32_t)s1;
}

// One tile row's segment in one column block, one quad per lane per step,
// for a segment that holds the array's last, partial quad (element loads
// there, nothing past the array touched). Returns the sum in lane 63.
template <typename V>
__device__ V tile_segment_safe(const TileArgs<V>& a, const V* xs, int32_t s0, int32_t s1, int c0,
                               int clen) {
  const int lane = lane_id();
  const int q1 = quad_end(s1);
  V acc = V(0);
  for (int q = (s0 >> 2) + lane; q < q1; q += kWave) {
    // q < q1 <= 2^29: 4q + 3 < 2^31 + 3, compared unsigned
    const bool full = 4u * (uint32_t)q + 3u < (uint32_t)a.nnz;
    const i32x4 c = full ? ld_stream(reinterpret_cast<const i32x4*>(a.col_idx) + q)
                         : load_quad<true>(a.col_idx, q, a.nnz);
    const Quad<V> v = full ? load_quad<false>(a.val, q, 0) : load_quad<true>(a.val, q, a.nnz);
    bool in[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) in[e] = in_segment(q, e, s0, s1);
    V xv[4];
    tile_x4(xv, c, in, xs, a.x, c0, clen);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += mask_zero(in[e], v[e] * xv[e]);
  }
  return wave_sum_to_last(acc);
}

// One workgroup's tile t (column block b, group g of kTileRows tile rows):
// the block of x staged in xs, kTileBytes of LDS (direct-to-LDS 16-byte
// loads when x is 16-byte aligned), while each wave loads the segment bounds
// of its rows (every
// kWavesPerBlock-th row of the group) into one register; then each wave
// streams the segments of kTileBatch rows at a time in 16-byte quads, the
// quads of all of them requested before any is used (indices clamped into
// the segment, entries outside it masked, so no load sits under a branch),
// sums lane-wise and across the wave by DPP moves; lane 63 writes
// partial[row][b]. Each lane adds its quads' products in element order,
// the same order for any batch size.
template <typename V>
__device__ __forceinline__ void tile_block(const TileArgs<V>& a, int t, V* xs) {
  constexpr int BC = kTileBytes / (int)sizeof(V);
  constexpr int E = 16 / (int)sizeof(V);   // elements per 16-byte chunk
  constexpr int RW = kTileRows / kWavesPerBlock;
  constexpr int NB = kTileBatch;
  static_assert(2 * RW <= kWave && RW % NB == 0, "segment bounds of a wave's rows in one register");
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // group-major: consecutive tiles take consecutive blocks of the same
  // rows, so a run of tiles streams each row's segments in memory order
  // (block-major, sharing one x block instead, measured 2% slower)
  const int g = t / a.nb, b = t - g * a.nb;
  const int c0 = b * BC;   // < N
  const int clen = min(BC, a.N - c0);
  // lane 2k + e: the bound of block b + e of row k of this wave (every
  // kTileSub-th of the row's quarter-block bounds; rows past the end clamped
  // to the last, their bounds not used)
  const int i0 = g * kTileRows + wave;
  const int ri = min(i0 + kWavesPerBlock * min(lane >> 1, RW - 1), a.n_rows - 1);
  const int32_t sb = a.seg[(int64_t)ri * (a.nb * kTileSub + 1) + kTileSub * (b + (lane & 1))];
  if (a.x_aligned) {
    const int nch = clen / E;
#pragma unroll
    for (int r = 0; r < BC / E / kBlock; ++r) {
      const int first = r * kBlock + wave * kWave;
      if (first < nch && first + lane < nch) lds_dma16(a.x + c0 + E * (first + lane), xs + E * first);
    }
    if ((int)threadIdx.x < clen - E * nch) xs[E * nch + threadIdx.x] = a.x[c0 + E * nch + threadIdx.x];
  } else {
    for (int k = threadIdx.x; k < clen; k += kBlock) xs[k] = a.x[c0 + k];
  }
  wait_vmem();
  __syncthreads();
  for (int m = 0; m < RW; m += NB) {
    if (i0 + kWavesPerBlock * m >= a.n_rows) break;   // wave-uniform
    int32_t s0[NB], s1[NB], q0[NB], q1[NB];
    int nit = 0;
    bool full = true;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const bool row = i0 + kWavesPerBlock * (m + j) < a.n_rows;
      s0[j] = __builtin_amdgcn_readlane(sb, 2 * (m + j));
      s1[j] = row ? __builtin_amdgcn_readlane(sb, 2 * (m + j) + 1) : s0[j];
      q0[j] = s0[j] >> 2;
      q1[j] = quad_end(s1[j]);
      nit = max(nit, (q1[j] - q0[j] + kWave - 1) / kWave);
      full = full && 4u * (uint32_t)max(q1[j], 1) <= (uint32_t)a.nnz;
    }
    V acc[NB];
    if (full) {
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[j] = V(0);
      for (int it = 0; it < nit; ++it) {
        i32x4 c[NB];
        Quad<V> v[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int qc = max(min(q0[j] + it * kWave + lane, q1[j] - 1), 0);
          c[j] = ld_stream(reinterpret_cast<const i32x4*>(a.col_idx) + qc);
          v[j] = load_quad<false>(a.val, qc, 0);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int q = q0[j] + it * kWave + lane;
          bool in[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) in[e] = in_segment(q, e, s0[j], s1[j]);
          V xv[4];
          tile_x4(xv, c[j], in, xs, a.x, c0, clen);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[j] += mask_zero(in[e], v[j][e] * xv[e]);
        }
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[j] = wave_sum_to_last(acc[j]);
    } else {
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[j] = tile_segment_safe(a, xs, s0[j], s1[j], c0, clen);
    }
    if (lane == kWave - 1) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int i = i0 + kWavesPerBlock * (m + j);
        if (i < a.n_rows) a.partial[(int64_t)i * a.nb + b] = acc[j];
      }
    }
  }
}

}  // namespace
}  // namespace spmv
