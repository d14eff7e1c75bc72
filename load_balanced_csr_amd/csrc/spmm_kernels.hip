// Multi-vector CSR SpMV (SpMM) for gfx950: Y = alpha * A X + beta * Y with
// X (N x k) and Y (M x k) dense and row-major, k <= 64 per launch.
//
// What is computed: "A Programming Model for GPU Load Balancing" (Osama,
// Porumbescu, Owens, PPoPP'23), Section 5.3, Listing 4 -- the SpMV of its
// Listing 3 with a loop over the dense matrix's columns added, every output
// column the sum over a row's atoms of value times the dense entry in the
// atom's column index row.
//
// Schedule: the plan's merge-path partitions, unchanged (Section 5.2.1 of
// the same page): a partition is T units, each nonzero and each row end one
// unit. MI355X mapping (not the page's): one 64-lane wavefront per
// partition, split into S = 64 / KL slots of KL lanes; lane l of a slot
// holds output columns [VE l, VE l + VE), VE = 16 bytes' worth when X and Y
// allow 16-byte accesses (else 1). The partition's units are cut again, merge-path
// style, into S equal runs, one per slot, so every slot does the same work
// however long the rows are. A slot walks its run in order; per batch of 8
// nonzeros it first issues all their X-row loads (KL consecutive elements
// per nonzero: one coalesced access per slot), then adds the products,
// finishing rows as their ends come by (one 16-byte load per lane and
// nonzero). A row wholly inside one run is
// written by that slot; the pieces of rows cut between runs are combined in
// slot order afterwards, and a row cut at the partition's end leaves a
// k-wide carry that the fix-up kernel adds, in partition order. No float
// atomics: for a fixed plan the result is bitwise reproducible.
#include "device_common.hpp"
#include "internal.hpp"

#include <limits.h>

#include <type_traits>

namespace spmv {
namespace {

constexpr int kSpmmBatch = 4;

// Bytes of the per-slot records of the merge kernel's slot combine (head /
// tail vectors, 64 lanes x 16 bytes each, and 5 x 64 int32), which overlay
// the staged partition once the walk is done.
constexpr int kSpmmRecordBytes = 2 * kWave * 16 + 5 * kWave * 4;

// LDS of one wave's partition (bytes), both kernels: a partition holds at
// most cap - 8 rows plus nonzeros (walk: T; stream: T + T/8), and staging an
// array of n words takes at most n + 7, so the row pointers and the column
// indices share one region of cap + 12 words (the columns start at the
// first 16-byte boundary past the row pointers); the values follow it.
// Two thirds of the footprint of three separate regions.
__host__ __device__ constexpr int spmm_wave_lds(int cap, int vbytes) {
  return (cap + 12) * 4 + cap * vbytes > kSpmmRecordBytes ? (cap + 12) * 4 + cap * vbytes
                                                          : kSpmmRecordBytes;
}

// VE consecutive elements of V (a 16-byte vector when VE * sizeof(V) = 16).
template <typename V, int VE>
struct Vec {
  V v[VE];
};
template <typename V, int VE>
__device__ __forceinline__ Vec<V, VE> vec_load(const V* p) {
  Vec<V, VE> r;
  if constexpr (VE > 1 && (VE * sizeof(V) == 16 || VE * sizeof(V) == 8)) {
    typedef V v4 __attribute__((ext_vector_type(VE)));
    const v4 t = *reinterpret_cast<const v4*>(p);
#pragma unroll
    for (int q = 0; q < VE; ++q) r.v[q] = t[q];
  } else {
#pragma unroll
    for (int q = 0; q < VE; ++q) r.v[q] = p[q];
  }
  return r;
}

// a[beg, beg + cnt) (int32 words, n in the array) into LDS dst so that
// a[beg + t] lands at dst[(beg & 3) + t]: whole 16-byte quads by direct-to-LDS
// loads (no registers; all in flight together), the array's last, partial
// quad by element loads. dst is 16-byte aligned with room for cnt + 7
// entries. The caller waits for the loads (vmcnt 0) and syncs the wave
// before reading dst.
__device__ __forceinline__ void stage_dma(int32_t* dst, const int32_t* a, int64_t beg, int cnt,
                                          int64_t n) {
  if (cnt <= 0) return;
  const int lane = lane_id();
  const int64_t q0 = beg >> 2;
  const int nq = (int)(((beg + cnt - 1) >> 2) - q0 + 1);
  for (int r = 0; kWave * r < nq; ++r) {
    const int t = kWave * r + lane;
    const int64_t q = q0 + t;
    if (t < nq && 4 * q + 3 < n) lds_dma16(a + 4 * q, dst + 4 * kWave * r);
  }
  const int64_t ql = q0 + nq - 1;
  if (4 * ql + 3 >= n && lane == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[4 * (nq - 1) + j] = 4 * ql + j < n ? a[4 * ql + j] : 0;
  }
}

// X addressing of the SpMM kernels (XA): 0, a 64-bit element offset; 1,
// a 32-bit byte offset from a wave-uniform base (X spans < 4 GiB), the row
// stride a run-time multiply; 2, the same with rows of exactly KL * VE
// elements (contiguous X), so the stride is a shift (a 32-bit multiply is a
// quarter-rate instruction, one per X-row load).
constexpr int ilog2c(int v) { return v <= 1 ? 0 : 1 + ilog2c(v / 2); }
template <typename V, int KL, int VE, int XA>
__device__ __forceinline__ Vec<V, VE> x_row(const char* xbase, const V* xcol, uint32_t c,
                                            uint32_t xrow_bytes, uint32_t xcol_bytes,
                                            int64_t ldx) {
  constexpr int SH = ilog2c(KL * VE * (int)sizeof(V));
  if constexpr (XA == 2)
    return vec_load<V, VE>(reinterpret_cast<const V*>(xbase + ((c << SH) + xcol_bytes)));
  else if constexpr (XA == 1)
    return vec_load<V, VE>(reinterpret_cast<const V*>(xbase + (c * xrow_bytes + xcol_bytes)));
  else
    return vec_load<V, VE>(xcol + (int64_t)c * ldx);
}

// Y[row, col .. col + VE) = alpha * acc + beta * Y (Y not read when beta = 0)
template <typename V, int VE>
__device__ __forceinline__ void spmm_store(const SpmmArgs<V>& a, int row, int col,
                                           const Vec<V, VE>& acc) {
  V* yp = a.Y + (int64_t)row * a.ldy + col;
  Vec<V, VE> out;
  if (a.beta_nonzero) {
    const Vec<V, VE> old = vec_load<V, VE>(yp);
#pragma unroll
    for (int q = 0; q < VE; ++q) out.v[q] = fma(a.beta, old.v[q], a.alpha * acc.v[q]);
  } else {
#pragma unroll
    for (int q = 0; q < VE; ++q) out.v[q] = a.alpha * acc.v[q];
  }
  if constexpr (VE > 1 && (VE * sizeof(V) == 16 || VE * sizeof(V) == 8)) {
    typedef V v4 __attribute__((ext_vector_type(VE)));
    v4 t;
#pragma unroll
    for (int q = 0; q < VE; ++q) t[q] = out.v[q];
    *reinterpret_cast<v4*>(yp) = t;
  } else {
#pragma unroll
    for (int q = 0; q < VE; ++q) yp[q] = out.v[q];
  }
}

// XA: the X addressing (x_row): a 32-bit offset from a wave-uniform base
// when X spans less than 4 GiB (one VGPR per address instead of two), a
// shift for contiguous rows.
template <typename V, int KL, int VE, int XA>
__global__ __launch_bounds__(kBlock) void spmm_merge_kernel(const SpmmArgs<V> a) {
  constexpr int S = kWave / KL;   // slots per wave
  constexpr int B = kSpmmBatch;
  typedef Vec<V, VE> VV;
  extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int blk = a.xcd_remap ? xcd_tile(blockIdx.x, 0, gridDim.x) : (int)blockIdx.x;
  int p = blk * kWavesPerBlock + wave;
  if (p >= (a.n_dispatch ? a.n_dispatch : a.P)) return;
  // the plan's column dispatch order (walk plans), as in the SpMV kernel,
  // or the partitions long-row tiles leave
  if (a.part_order) p = a.part_order[p];

  // partition p: rows [r0, r1) end inside it; nonzeros [n0, n1). In the
  // stream layout the nonzeros start and stop at row boundaries; otherwise
  // row r1 is open at the end (its part here becomes the carry) and row r0
  // may have started in an earlier partition.
  int r0, r1, n0, n1;
  if (a.stream) {
    r0 = a.row_bounds[2 * p];
    n0 = a.row_bounds[2 * p + 1];
    r1 = a.row_bounds[2 * p + 2];
    n1 = a.row_bounds[2 * p + 3];
  } else {
    r0 = a.split_row[p];
    r1 = a.split_row[p + 1];
    n0 = a.split_nz[p];
    n1 = a.split_nz[p + 1];
  }
  const int R = r1 - r0, nloc = n1 - n0, tot = R + nloc;

  // every partition holds at most cap - 8 rows plus nonzeros (walk: T; stream:
  // T + T/8), which the shared LDS region relies on; never stage past it
  if (tot > a.cap - 8) return;
  unsigned char* base = s_dyn + (size_t)wave * spmm_wave_lds(a.cap, sizeof(V));
  int32_t* s_rp = reinterpret_cast<int32_t*>(base);
  int32_t* s_col = s_rp + ((R + 8 + 3) & ~3);
  int32_t* s_val = s_rp + (a.cap + 12);   // cap entries of V, staged as int32 words

  // row pointers rp[r0 .. r1] (row r1's start ends the last closed row), the
  // partition's column indices and values: coalesced 16-byte loads
  constexpr int W = sizeof(V) / 4;   // int32 words per value
  stage_dma(s_rp, a.row_ptr, r0, R + 1, a.M + 1);
  stage_dma(s_col, a.col_idx, n0, nloc, a.nnz);
  stage_dma(s_val, reinterpret_cast<const int32_t*>(a.val), (int64_t)W * n0, W * nloc,
            (int64_t)W * a.nnz);
  wait_vmem();
  wave_sync();
  memory_order_point();
  const int32_t* rpl = s_rp + (r0 & 3);    // rpl[i] = row_ptr[r0 + i]
  const int32_t* coll = s_col + (n0 & 3);  // coll[t] = col_idx[n0 + t]
  const V* vall = reinterpret_cast<const V*>(s_val + ((W * n0) & 3));   // vall[t] = val[n0 + t]
  // (W * n0 may wrap in int32 for fp64; its low two bits are still right)
  // a partition a tiled row starts or ends in: that row's entries belong to
  // the tiles, so their staged columns become -1: the walk reads X row 0 for
  // them and adds nothing (whatever X row 0 holds)
  if (a.mask_end) {
    const int mlo = a.mask_end[p], mhi = a.mask_start[p];
    if (mlo > n0 || mhi < n1) {   // wave-uniform
      int32_t* cw = s_col + (n0 & 3);
      for (int t = lane; t < nloc; t += kWave) {
        const int gk = n0 + t;
        if (gk < mlo || gk >= mhi) cw[t] = -1;
      }
      wave_sync();
    }
  }

  const int s = lane / KL;
  const int col = (lane % KL) * VE;          // first output column of this lane
  const bool colok = col < a.k;
  const int D = (tot + S - 1) / S;
  const int d0 = min(s * D, tot), d1 = min(d0 + D, tot);
  // merge-path coordinate of unit d: rows whose end unit comes before d
  // (row i's end is unit rpl[i + 1] - n0 + i) and the nonzeros consumed
  auto rows_before = [&](int d) {
    int lo = 0, hi = R;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (rpl[mid + 1] - n0 + mid < d) lo = mid + 1;
      else hi = mid;
    }
    return lo;
  };
  int i = rows_before(d0);
  const int iend = rows_before(d1);
  const int jbeg = d0 - i, jend = d1 - iend;
  const int i0 = i;
  // the slot owns its first row when no earlier slot holds a piece of it
  // (slot 0 always: earlier partitions' pieces come in as carries)
  bool owned = s == 0 || rpl[i] - n0 >= jbeg;
  bool head_ends = false;
  VV acc, head;
#pragma unroll
  for (int q = 0; q < VE; ++q) acc.v[q] = head.v[q] = V(0);
  int e = i < R ? rpl[i + 1] - n0 : INT_MAX;   // local end of row i
  const char* xbase = reinterpret_cast<const char*>(a.X);
  const uint32_t xrow_bytes = (uint32_t)a.ldx * (uint32_t)sizeof(V);

  // rows ending at unit position jj (before nonzero jj): written when this
  // slot holds all of them, else kept as the head piece
  auto finish_rows = [&](int jj) {
    while (i < iend && e == jj) {
      if (owned) {
        if (colok) spmm_store<V, VE>(a, r0 + i, col, acc);
      } else {
        head = acc;
        head_ends = true;
      }
      owned = true;
#pragma unroll
      for (int q = 0; q < VE; ++q) acc.v[q] = V(0);
      ++i;
      e = i < R ? rpl[i + 1] - n0 : INT_MAX;
    }
  };

  // lanes past k read column 0 of the same X rows (in bounds; never stored)
  const int lcol = colok ? col : 0;
  const V* xcol = a.X + lcol;
  const uint32_t xcol_bytes = (uint32_t)lcol * (uint32_t)sizeof(V);
  for (int jb = jbeg; jb < jend; jb += B) {
    // the batch's column indices first (LDS), then every X-row load: past the
    // run's end a lane re-reads its last nonzero's row, and a masked entry
    // (column -1) reads row 0; neither adds anything (a select, not a
    // product with 0, so an Inf or NaN in X stays out of other rows)
    int cs[B];
#pragma unroll
    for (int u = 0; u < B; ++u) cs[u] = coll[min(jb + u, jend - 1)];
    VV xv[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      xv[u] = x_row<V, KL, VE, XA>(xbase, xcol, (uint32_t)max(cs[u], 0), xrow_bytes,
                                   xcol_bytes, a.ldx);
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int jj = jb + u;
      finish_rows(jj);
      const bool live = jj < jend && cs[u] >= 0;
      const V v = vall[min(jj, jend - 1)];
#pragma unroll
      for (int q = 0; q < VE; ++q) acc.v[q] = live ? fma(v, xv[u].v[q], acc.v[q]) : acc.v[q];
    }
  }
  finish_rows(jend);

  // records: the piece of the first row (when another slot started it and it
  // ended here) and the piece of the row open at the run's end, over the
  // staging area (every lane is done reading it)
  wave_sync();
  VV* head_vec = reinterpret_cast<VV*>(base);                 // [64] (16 bytes each)
  VV* tail_vec = reinterpret_cast<VV*>(base + kWave * 16);    // [64]
  int32_t* rec = reinterpret_cast<int32_t*>(base + 2 * kWave * 16);   // [5][64]
  head_vec[lane] = head;
  tail_vec[lane] = acc;
  if (lane % KL == 0) {
    rec[s] = head_ends;
    rec[kWave + s] = owned;
    rec[2 * kWave + s] = d0 < d1;
    rec[3 * kWave + s] = i0;
    rec[4 * kWave + s] = iend;
  }
  wave_sync();
  if (lane < KL) {
    // slot order: a running piece of the current cut row
    bool run = false;
    VV rv;
#pragma unroll
    for (int q = 0; q < VE; ++q) rv.v[q] = V(0);
    for (int t = 0; t < S; ++t) {
      if (!rec[2 * kWave + t]) break;   // only trailing slots are empty
      const VV hv = head_vec[t * KL + lane];
      const VV tv = tail_vec[t * KL + lane];
      if (rec[t]) {
        VV v;
#pragma unroll
        for (int q = 0; q < VE; ++q) v.v[q] = (run ? rv.v[q] : V(0)) + hv.v[q];
        if (colok) spmm_store<V, VE>(a, r0 + rec[3 * kWave + t], col, v);
        run = false;
      }
      if (rec[kWave + t]) {
        run = true;
        rv = tv;
      } else {
#pragma unroll
        for (int q = 0; q < VE; ++q) rv.v[q] += tv.v[q];
      }
    }
    if (!a.stream) {
      if (colok) {
#pragma unroll
        for (int q = 0; q < VE; ++q) a.carry_vec[(int64_t)p * a.k + col + q] = run ? rv.v[q] : V(0);
      }
      if (lane == 0) a.carry_row[p] = r1;
    }
  }
}

// The same product for plans whose partitions hold whole rows (every row
// <= T/8 entries, the stream layout): one wave per partition, staging its
// row pointers, columns and values in LDS (direct-to-LDS loads; row
// pointers and columns share one region). Rows go to slots instead of
// equal runs: G slots share a row when the partition has fewer rows than
// slots (G the largest power of two with rows * G <= slots), each taking
// every G-th of the row's nonzeros in batches of 8 (all X-row loads first),
// and meet by cross-lane adds. A round finishes S / G rows at once, so Y
// rows are written together (coalesced) and no slot walks a row end alone.
// The kernel is bound by the rate of X-row gathers that miss the CU's L1:
// a workgroup holds PPB consecutive partitions, so the waves of a CU walk
// neighbouring rows together and share the X rows around them in L1
// (banded, 8 RHS: 1 partition per workgroup 5.0 ms, 4: 4.2 ms, 8: 3.2 ms).
template <typename V, int KL, int VE, int XA, int PPB>
__global__ __launch_bounds__(PPB * kWave) void spmm_rows_kernel(const SpmmArgs<V> a) {
  constexpr int S = kWave / KL;   // slots per wave
  constexpr int B = 8;
  typedef Vec<V, VE> VV;
  extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];

  const int lane = lane_id();
  const int wave = PPB == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int blk = a.xcd_remap ? xcd_tile(blockIdx.x, 0, gridDim.x) : (int)blockIdx.x;
  const int p = blk * PPB + wave;
  if (p >= a.P) return;   // wave-uniform; the waves never wait for each other
  const int r0 = a.row_bounds[2 * p];
  const int n0 = a.row_bounds[2 * p + 1];
  const int r1 = a.row_bounds[2 * p + 2];
  const int n1 = a.row_bounds[2 * p + 3];
  const int R = r1 - r0, nloc = n1 - n0;
  if (R == 0) return;
  // a stream partition holds at most T + T/8 = cap - 8 rows plus nonzeros,
  // which the shared LDS region relies on; never stage past it
  if (R + nloc > a.cap - 8) return;

  // row pointers, then the columns from the next 16-byte boundary (rows +
  // nonzeros <= cap - 8, each staged array takes at most its count + 7
  // words), in one region of cap + 12 words; the values after it
  int32_t* s_rp =
      reinterpret_cast<int32_t*>(s_dyn + (size_t)wave * spmm_wave_lds(a.cap, sizeof(V)));
  int32_t* s_col = s_rp + ((R + 1 + 7 + 3) & ~3);
  int32_t* s_val = s_rp + a.cap + 12;
  constexpr int W = sizeof(V) / 4;
  stage_dma(s_rp, a.row_ptr, r0, R + 1, a.M + 1);
  stage_dma(s_col, a.col_idx, n0, nloc, a.nnz);
  stage_dma(s_val, reinterpret_cast<const int32_t*>(a.val), (int64_t)W * n0, W * nloc,
            (int64_t)W * a.nnz);
  wait_vmem();
  wave_sync();
  memory_order_point();
  const int32_t* rpl = s_rp + (r0 & 3);
  const int32_t* coll = s_col + (n0 & 3);
  const V* vall = reinterpret_cast<const V*>(s_val + ((W * n0) & 3));

  const int s = lane / KL;
  const int col = (lane % KL) * VE;
  const bool colok = col < a.k;
  const int lcol = colok ? col : 0;
  const char* xbase = reinterpret_cast<const char*>(a.X);
  const uint32_t xrow_bytes = (uint32_t)a.ldx * (uint32_t)sizeof(V);
  const uint32_t xcol_bytes = (uint32_t)lcol * (uint32_t)sizeof(V);
  const V* xcol = a.X + lcol;

  int G = 1;
  while (G < S && R * (2 * G) <= S) G *= 2;
  const int rpr = S / G;                 // rows per round
  const int part = s % G, grp = s / G;
  for (int rb = 0; rb < R; rb += rpr) {
    const int rr = rb + grp;
    const bool live = rr < R;
    const int rs = live ? rpl[rr] - n0 : 0;
    const int re = live ? rpl[rr + 1] - n0 : 0;
    VV acc;
#pragma unroll
    for (int q = 0; q < VE; ++q) acc.v[q] = V(0);
    // one batch of B of the row's nonzeros (every G-th): all X-row loads
    // first, then the FMAs. Only a row's last batch runs past its end; there
    // a lane re-reads the row's last nonzero and adds nothing for it (a
    // select, so an Inf or NaN in that X row does not turn the sum into
    // NaN), the full batches before it need no select.
    auto batch = [&](int jb, auto tail) {
      int cs[B];
#pragma unroll
      for (int u = 0; u < B; ++u) cs[u] = coll[min(jb + G * u, re - 1)];
      VV xv[B];
#pragma unroll
      for (int u = 0; u < B; ++u) {
        xv[u] = x_row<V, KL, VE, XA>(xbase, xcol, (uint32_t)cs[u], xrow_bytes, xcol_bytes,
                                     a.ldx);
      }
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int jj = jb + G * u;
        const V v = vall[min(jj, re - 1)];
#pragma unroll
        for (int q = 0; q < VE; ++q) {
          if (decltype(tail)::value)
            acc.v[q] = jj < re ? fma(v, xv[u].v[q], acc.v[q]) : acc.v[q];
          else
            acc.v[q] = fma(v, xv[u].v[q], acc.v[q]);
        }
      }
    };
    int jb = rs + part;
    for (; jb + G * (B - 1) < re; jb += G * B) batch(jb, std::false_type{});
    if (jb < re) batch(jb, std::true_type{});
    for (int g = 1; g < G; g <<= 1) {
#pragma unroll
      for (int q = 0; q < VE; ++q) acc.v[q] += __shfl_xor(acc.v[q], KL * g, kWave);
    }
    if (live && part == 0 && colok) spmm_store<V, VE>(a, r0 + rr, col, acc);
  }
}

// Y[r] += alpha * (sum of the carries of r) for every row that partitions
// left open. A wave holds G = 64 / kl consecutive partitions (kl the power
// of two covering k), laid out column by column: lane c * G + g takes
// partition base + g, column c, so each column's G partitions are adjacent
// lanes. A row's carries are contiguous: one DPP segmented scan over the
// wave (a segment starts at g = 0 and where the row changes) sums each row's
// carries inside the chunk, and the lane holding a segment's last carry
// updates the row, unless the segment began in an earlier chunk (that
// chunk's wave owns it). A segment owned here that runs past the chunk is
// read on by the whole wave, kFixupSlices slices of G partitions per step
// with every load of a step in flight together, until the step where it
// ends; a second segmented scan (a segment per column) then adds the slices
// up in each column's last lane. The order of the adds depends only on the
// plan and k.
constexpr int kFixupSlices = 8;

template <typename V, bool TILED>
__device__ __forceinline__ void spmm_fixup_chunk(const SpmmArgs<V>& a, const int32_t* skip,
                                                 int blk) {
  const int lane = lane_id();
  const int lg = a.k <= 1 ? 0 : 32 - __builtin_clz((unsigned)(a.k - 1));   // log2 kl
  const int G = kWave >> lg;
  const int g = lane & (G - 1);
  const int c = lane >> (6 - lg);
  const bool col = c < a.k;
  const int64_t base =
      ((int64_t)blk * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave)) * G;
  if (base >= a.P) return;   // wave-uniform: every lane takes part in the scans below
  const int32_t* cr = a.carry_row;
  const int64_t p = base + g;
  const int key = p < a.P ? carry_key<TILED>(cr, skip, p, a.P, a.M) : INT_MAX;
  V s = p < a.P && col ? a.carry_vec[p * a.k + c] : V(0);
  // wave-uniform: the chunk's first row, the row before the chunk, the row
  // after it
  const int key0 = carry_key<TILED>(cr, skip, base, a.P, a.M);
  const int prev0 = base > 0 ? carry_key<TILED>(cr, skip, base - 1, a.P, a.M) : -1;
  const int after = base + G < a.P ? carry_key<TILED>(cr, skip, base + G, a.P, a.M) : INT_MAX - 1;
  // the neighbours' rows, read by DPP moves that every lane executes (a move
  // under a lane mask would read stale values from the masked lanes)
  const int key_prev = lane_prev(key, key);
  const int key_next = lane_next(key, after);
  s = wave_segscan(s, g == 0 || key_prev != key);
  const int next = g == G - 1 ? after : key_next;
  const bool owned = !(key == key0 && prev0 == key0);
  const bool tail = next != key;
  if (tail && owned && key < a.M && col) {
    V* yp = a.Y + (int64_t)key * a.ldy + c;
    *yp = fma(a.alpha, s, *yp);
  }
  // the last partition's segment, when it is owned here and goes on
  // (wave-uniform)
  const int r = base + G - 1 < a.P ? carry_key<TILED>(cr, skip, base + G - 1, a.P, a.M) : INT_MAX;
  const bool cont = after == r && !(r == key0 && prev0 == key0);
  if (!cont || r >= a.M) return;
  V extra = V(0);
  for (int64_t q = base + G;; q += (int64_t)G * kFixupSlices) {
    int kq[kFixupSlices];
#pragma unroll
    for (int u = 0; u < kFixupSlices; ++u) {
      const int64_t pp = q + u * G + g;
      kq[u] = pp < a.P ? carry_key<TILED>(cr, skip, pp, a.P, a.M) : -1;
    }
    V v[kFixupSlices];
#pragma unroll
    for (int u = 0; u < kFixupSlices; ++u) {
      const int64_t pp = q + u * G + g;
      v[u] = kq[u] == r && col ? a.carry_vec[pp * a.k + c] : V(0);
    }
#pragma unroll
    for (int u = 0; u < kFixupSlices; ++u) extra += v[u];
    // the row's carries are a prefix of the step: it goes on only if the
    // step's last partition is still the row's
    if (__ballot(kq[kFixupSlices - 1] == r) != ~0ull) break;
  }
  extra = wave_segscan(extra, g == 0);   // column totals in each column's last lane
  if (g != G - 1 || !col) return;
  V* yp = a.Y + (int64_t)r * a.ldy + c;
  *yp = fma(a.alpha, s + extra, *yp);
}

template <typename V>
__global__ __launch_bounds__(kBlock) void spmm_fixup_kernel(const SpmmArgs<V> a) {
  spmm_fixup_chunk<V, false>(a, nullptr, (int)blockIdx.x);
}

// ---- long-row tiles (plans with tiles, X rows of at most 32 bytes) --------------

// The end quad of entries [., s1), (s1 + 3) / 4, and whether entry 4q + e
// lies in [s0, s1), in unsigned arithmetic (4q + e may pass 2^31 - 1).
__device__ __forceinline__ int quad_end(int32_t s1) { return (int)(((uint32_t)s1 + 3u) >> 2); }

// The 16-byte quad (columns or values) of the partner lane (this lane xor
// 1): one DPP move per word.
__device__ __forceinline__ i32x4 quad_of_partner(const i32x4& v) {
  i32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = dpp_i32<kDppQuadXor1>(0, v[j]);
  return r;
}
template <typename V>
__device__ __forceinline__ Quad<V> quad_of_partner(const Quad<V>& v) {
  Quad<V> r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r.set(j, dpp_move<kDppQuadXor1>(v[j]));
  return r;
}

// acc += the products of quad q (entries 4q..4q+3, those in [s0, s1)) with
// this lane's VE columns of their X rows: from the staged block in LDS, or,
// for a column outside it (only in a row with unsorted columns), from
// global X, in a branch the wave takes only when one of its lanes needs it.
// An entry outside the segment reads the zero row past the block (row
// zrow) and its value is taken as 0, so its FMAs add exactly 0 whatever X
// and the values hold elsewhere.
template <typename V, int VE, int K>
__device__ __forceinline__ void tile_quad_products(Vec<V, VE>& acc, const i32x4& c,
                                                   const Quad<V>& v, int q, int32_t s0,
                                                   int32_t s1, const V* xs,
                                                   const SpmmTileArgs<V>& t, int64_t c0,
                                                   int clen, int zrow, int lcol) {
  bool in[4], out = false;
  Vec<V, VE> xv[4];
  // entry 4q + e is in [s0, s1) when 4q + e - s0 < s1 - s0, unsigned (4q
  // stays below 2^32: q is at most one segment's quads past the other's end)
  const uint32_t d = 4u * (uint32_t)q - (uint32_t)s0, len = (uint32_t)(s1 - s0);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    in[e] = d + (uint32_t)e < len;
    const unsigned lc = (unsigned)((int64_t)c[e] - c0);
    const bool inb = lc < (unsigned)clen;
    // X rows of K values in LDS: a compile-time row stride
    xv[e] = vec_load<V, VE>(xs + (in[e] && inb ? lc : (unsigned)zrow) * (unsigned)K + lcol);
    out = out || (in[e] && !inb);
  }
  if (__builtin_amdgcn_ballot_w64(out) != 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (in[e] && (unsigned)((int64_t)c[e] - c0) >= (unsigned)clen)
        xv[e] = vec_load<V, VE>(t.X + (int64_t)c[e] * t.ldx + lcol);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const V ve = in[e] ? v[e] : V(0);
#pragma unroll
    for (int r = 0; r < VE; ++r) acc.v[r] = fma(ve, xv[e].v[r], acc.v[r]);
  }
}

// One workgroup of W waves per tile: sub-block b of bck X rows, group g of
// TR = W RW tile rows, taken block-major (an XCD's run of tiles then reads
// its own run of X blocks into its L2; X of k columns does not fit one L2
// whole). The tiles of sub-block 0 first zero the carries of their rows'
// interior partitions, which the merge kernel does not walk but its fix-up
// reads. The block's X rows are staged in LDS (direct-to-LDS loads when
// they are contiguous and aligned), with one zero row past them. Each wave
// takes every W-th row of the group, two at a time, one per half-wave, NP
// such pairs per batch: a lane loads one 16-byte quad of its row's segment
// (columns and values; 32 quads per half and step); with KL = 2 lanes a
// slot (X rows of 32 bytes), partners swap their quads by DPP, and each
// lane multiplies all 4 KL entries by its VE columns of their X rows (from
// LDS). The NP pairs' loads are all requested before any is used. Eight waves a workgroup and at most
// 128 registers let two workgroups share a CU (LDS allows two): measured
// on the bimodal matrix at k = 8, 4 waves of 16 rows took 237 us, 8 waves
// of 16 rows 155 us, and 8 of 32 rows less again (X staged half as often).
// Each lane adds in a fixed order; the half's slots then meet by a
// butterfly of cross-lane adds, and its first slot writes
// partial[row][b][columns].
template <typename V, int KL, int VE, int W, int RW>
__global__ __launch_bounds__(W * kWave) __attribute__((amdgpu_waves_per_eu(2 * W / 4)))
void spmm_tile_kernel(const SpmmTileArgs<V> t) {
  constexpr int TR = W * RW;                       // rows per tile
  constexpr int NT = W * kWave;                    // threads per workgroup
  constexpr int HL = kWave / 2;                    // lanes per row (a half-wave)
  // row pairs per batch: as many as fit 128 registers (two workgroups a CU)
  constexpr int NP = (KL == 2 && sizeof(V) == 8) ? 1 : 2;
  static_assert(2 * RW <= kWave && KL <= 2 && (RW / 2) % NP == 0, "tile layout");
  typedef Vec<V, VE> VV;
  extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];
  V* xs = reinterpret_cast<V*>(s_dyn);
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nbs = t.nb * t.m;
  const int sub = kTileSub / t.m;   // quarter-block bounds per sub-block
  const int tile = xcd_tile(blockIdx.x, 0, gridDim.x);
  const int b = tile / t.ngroups, g = tile - b * t.ngroups;
  if (b == 0) {   // workgroup-uniform
    for (int r = 0; r < TR; ++r) {
      const int i = g * TR + r;
      if (i >= t.n_rows) break;
      const int32_t pf = t.rows[kTileRowInts * i + 3], pe = t.rows[kTileRowInts * i + 4];
      const int64_t n = (int64_t)(pe - pf) * t.k;
      for (int64_t e = threadIdx.x; e < n; e += NT) t.carry_vec[(int64_t)pf * t.k + e] = V(0);
    }
  }
  const int64_t c0 = (int64_t)b * t.bck;
  const int clen = (int)max((int64_t)0, min((int64_t)t.bck, (int64_t)t.N - c0));
  // lane 2r + e: the bound of sub-block b + e of row r of this wave (rows
  // past the end clamped to the last; their bounds are not used)
  const int i0 = g * TR + wave;
  const int ri = min(i0 + W * min(lane >> 1, RW - 1), t.n_rows - 1);
  const int32_t sb = t.seg[(int64_t)ri * (t.nb * kTileSub + 1) + sub * (b + (lane & 1))];
  const int64_t nel = (int64_t)clen * t.k;
  if (t.x_dma) {
    // k values of a row are a whole number of 16-byte chunks
    const int nch = (int)(nel * (int64_t)sizeof(V) / 16);
    const char* src = reinterpret_cast<const char*>(t.X + c0 * t.k);
    for (int first = wave * kWave; first < nch; first += NT)
      if (first + lane < nch)
        lds_dma16(src + 16 * (int64_t)(first + lane), reinterpret_cast<char*>(xs) + 16 * first);
  } else {
    for (int64_t e = threadIdx.x; e < nel; e += NT) {
      const int64_t r = e / t.k;
      xs[e] = t.X[(c0 + r) * t.ldx + (e - r * t.k)];
    }
  }
  // the zero row past the block, for the entries outside a segment
  const int zrow = t.bck;
  for (int e = threadIdx.x; e < t.k; e += NT) xs[(int64_t)zrow * t.k + e] = V(0);
  wait_vmem();
  __syncthreads();
  const int h = lane / HL, hl = lane % HL;
  const int col = (hl % KL) * VE;
  const bool colok = col < t.k;
  const int lcol = colok ? col : 0;
  for (int pb = 0; pb < RW / 2; pb += NP) {
    if (i0 + W * 2 * pb >= t.n_rows) break;   // wave-uniform
    int32_t s0[NP], s1[NP];
    int nit = 0;
    bool full = true;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int ra = 2 * (pb + j), rb = ra + 1;   // rows of the pair, in this wave
      const bool va = i0 + W * ra < t.n_rows;
      const bool vb = i0 + W * rb < t.n_rows;
      const int32_t a0 = __builtin_amdgcn_readlane(sb, 2 * ra);
      const int32_t a1 = va ? __builtin_amdgcn_readlane(sb, 2 * ra + 1) : a0;
      const int32_t b0 = __builtin_amdgcn_readlane(sb, 2 * rb);
      const int32_t b1 = vb ? __builtin_amdgcn_readlane(sb, 2 * rb + 1) : b0;
      s0[j] = h ? b0 : a0;
      s1[j] = h ? b1 : a1;
      const int qa = quad_end(a1) - (a0 >> 2), qb = quad_end(b1) - (b0 >> 2);
      nit = max(nit, (max(qa, qb) + HL - 1) / HL);
      full = full && 4u * (uint32_t)max(quad_end(max(a1, b1)), 1) <= (uint32_t)t.nnz;
    }
    VV acc[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j)
#pragma unroll
      for (int r = 0; r < VE; ++r) acc[j].v[r] = V(0);
    for (int it = 0; it < nit; ++it) {
      i32x4 cq[NP];
      Quad<V> vq[NP];
      int qb0[NP];   // quad of lane hl = 0 of this half at this step
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        qb0[j] = (s0[j] >> 2) + it * HL;
        const int qc = max(min(qb0[j] + hl, quad_end(s1[j]) - 1), 0);
        if (full) {
          cq[j] = ld_stream(reinterpret_cast<const i32x4*>(t.col_idx) + qc);
          vq[j] = load_quad<false>(t.val, qc, 0);
        } else {   // the array's last, partial quad is among them
          cq[j] = load_quad<true>(t.col_idx, qc, t.nnz);
          vq[j] = load_quad<true>(t.val, qc, t.nnz);
        }
      }
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        tile_quad_products<V, VE, KL * VE>(acc[j], cq[j], vq[j], qb0[j] + hl, s0[j], s1[j], xs,
                                           t, c0, clen, zrow, lcol);
        if (KL == 2)
          tile_quad_products<V, VE, KL * VE>(acc[j], quad_of_partner(cq[j]),
                                             quad_of_partner(vq[j]), qb0[j] + (hl ^ 1), s0[j],
                                             s1[j], xs, t, c0, clen, zrow, lcol);
      }
    }
    // the half's slots meet (offsets below HL keep each half apart)
    for (int off = KL; off < HL; off <<= 1) {
#pragma unroll
      for (int j = 0; j < NP; ++j)
#pragma unroll
        for (int r = 0; r < VE; ++r) acc[j].v[r] += __shfl_xor(acc[j].v[r], off, kWave);
    }
    if (hl < KL && colok) {
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int i = i0 + W * (2 * (pb + j) + h);
        if (i < t.n_rows) {
          V* dst = t.partial + ((int64_t)i * nbs + b) * t.k + col;
#pragma unroll
          for (int r = 0; r < VE; ++r) dst[r] = acc[j].v[r];
        }
      }
    }
  }
}

// Y[row][c] += alpha * (sum of the row's sub-block partials of column c),
// one wave per tile row: lane l takes column l % KC (KC the power of two
// covering k) and sub-blocks l / KC, l / KC + 64 / KC, ...; the lanes of a
// column then meet by a butterfly of cross-lane adds (a fixed order).
template <typename V>
__device__ __forceinline__ void spmm_tile_reduce_rows(const SpmmTileArgs<V>& t, int kc, int blk) {
  const int64_t i = ((int64_t)blk * kBlock + threadIdx.x) / kWave;
  if (i >= t.n_rows) return;   // wave-uniform
  const int lane = lane_id();
  const int c = lane % kc, bl = lane / kc, nbl = kWave / kc;
  const int nbs = t.nb * t.m;
  // eight running sums, so eight loads are in flight; added in a fixed order
  V a8[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) a8[u] = V(0);
  if (c < t.k) {
    const V* pr = t.partial + (int64_t)i * nbs * t.k + c;
    int b = bl;
    for (; b + 7 * nbl < nbs; b += 8 * nbl) {
#pragma unroll
      for (int u = 0; u < 8; ++u) a8[u] += pr[(int64_t)(b + u * nbl) * t.k];
    }
#pragma unroll
    for (int u = 0; u < 7; ++u)
      if (b + u * nbl < nbs) a8[u] += pr[(int64_t)(b + u * nbl) * t.k];
  }
  V acc = ((a8[0] + a8[1]) + (a8[2] + a8[3])) + ((a8[4] + a8[5]) + (a8[6] + a8[7]));
  for (int off = kc; off < kWave; off <<= 1) acc += __shfl_xor(acc, off, kWave);
  if (bl == 0 && c < t.k) {
    V* yp = t.Y + (int64_t)t.rows[kTileRowInts * i] * t.ldy + c;
    *yp += t.alpha * acc;
  }
}

// The merge kernel's fix-up and the tiles' reduction in one launch: blocks
// [0, fix_blocks) take the carries (those of tile rows keyed past the last
// row, so skipped), the others the tile rows. The two write different rows.
template <typename V>
__global__ __launch_bounds__(kBlock) void spmm_fixup_tile_reduce_kernel(const SpmmArgs<V> a,
                                                                        const SpmmTileArgs<V> t,
                                                                        int fix_blocks, int kc) {
  if ((int)blockIdx.x < fix_blocks) {   // workgroup-uniform
    spmm_fixup_chunk<V, true>(a, t.skip, (int)blockIdx.x);
    return;
  }
  spmm_tile_reduce_rows(t, kc, (int)blockIdx.x - fix_blocks);
}

template <typename V, int KL, int VE, int XA>
void launch_rows(const SpmmArgs<V>& a, int ppb, size_t lds_wave, hipStream_t s, hipEvent_t ev0,
                 hipEvent_t ev1) {
  const dim3 g((a.P + ppb - 1) / ppb);
  const size_t lds = (size_t)ppb * lds_wave;
  switch (ppb) {
    case 8: launch_timed(spmm_rows_kernel<V, KL, VE, XA, 8>, g, dim3(8 * kWave), lds, s, ev0, ev1, a); break;
    case 4: launch_timed(spmm_rows_kernel<V, KL, VE, XA, 4>, g, dim3(4 * kWave), lds, s, ev0, ev1, a); break;
    case 2: launch_timed(spmm_rows_kernel<V, KL, VE, XA, 2>, g, dim3(2 * kWave), lds, s, ev0, ev1, a); break;
    default: launch_timed(spmm_rows_kernel<V, KL, VE, XA, 1>, g, dim3(kWave), lds, s, ev0, ev1, a); break;
  }
}

template <typename V, int KL, int VE>
hipError_t launch_kl(const SpmmArgs<V>& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  // bytes from X to the end of its last row's k columns
  const uint64_t xspan = (uint64_t)a.ldx * sizeof(V) * (uint64_t)(a.N > 0 ? a.N : 1);
  const bool off32 = xspan < (1ull << 32);
  const bool contig = off32 && a.ldx == KL * VE;   // rows of exactly KL * VE elements
  const size_t lds_wave = (size_t)spmm_wave_lds(a.cap, sizeof(V));
  if (a.stream) {
    // up to 8 consecutive partitions per workgroup, as many as one CU's LDS
    // holds (16 measured no better: banded 3.15 against 3.19 ms, fp64
    // Laplacian 0.186 against 0.171 ms)
    int ppb = 8;
    while (ppb > 1 && (size_t)ppb * lds_wave > (size_t)kLdsBytes) ppb >>= 1;
    if (contig) launch_rows<V, KL, VE, 2>(a, ppb, lds_wave, s, ev0, ev1);
    else if (off32) launch_rows<V, KL, VE, 1>(a, ppb, lds_wave, s, ev0, ev1);
    else launch_rows<V, KL, VE, 0>(a, ppb, lds_wave, s, ev0, ev1);
    return hipGetLastError();
  }
  const int slots = a.n_dispatch ? a.n_dispatch : a.P;
  const dim3 g((slots + kWavesPerBlock - 1) / kWavesPerBlock), b(kBlock);
  const size_t lds = (size_t)kWavesPerBlock * lds_wave;
  if (contig)
    launch_timed(spmm_merge_kernel<V, KL, VE, 2>, g, b, lds, s, ev0, ev1, a);
  else if (off32)
    launch_timed(spmm_merge_kernel<V, KL, VE, 1>, g, b, lds, s, ev0, ev1, a);
  else
    launch_timed(spmm_merge_kernel<V, KL, VE, 0>, g, b, lds, s, ev0, ev1, a);
  return hipGetLastError();
}

// lanes per slot: the smallest power of two covering k columns, VE per lane
template <typename V, int VE>
hipError_t launch_ve(const SpmmArgs<V>& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const int lanes = (a.k + VE - 1) / VE;
  if (lanes <= 1) return launch_kl<V, 1, VE>(a, s, ev0, ev1);
  if (lanes <= 2) return launch_kl<V, 2, VE>(a, s, ev0, ev1);
  if (lanes <= 4) return launch_kl<V, 4, VE>(a, s, ev0, ev1);
  if (lanes <= 8) return launch_kl<V, 8, VE>(a, s, ev0, ev1);
  if (lanes <= 16) return launch_kl<V, 16, VE>(a, s, ev0, ev1);
  if (lanes <= 32) return launch_kl<V, 32, VE>(a, s, ev0, ev1);
  return launch_kl<V, 64, VE>(a, s, ev0, ev1);
}

}  // namespace

template <typename V>
int spmm_fixup_blocks(const SpmmArgs<V>& a) {
  if (a.stream || a.P <= 1) return 0;
  // one wave per 64 / kl partitions
  const int lg = a.k <= 1 ? 0 : 32 - __builtin_clz((unsigned)(a.k - 1));
  const int64_t waves = ((int64_t)a.P + (kWave >> lg) - 1) / (kWave >> lg);
  return (int)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
}

template <typename V>
hipError_t launch_spmm(const SpmmArgs<V>& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1,
                       bool fixup) {
  if (a.P <= 0 || a.k <= 0) return hipSuccess;
  if (a.k > kWave || a.cap < spmm_stage_cap(a.T)) return hipErrorInvalidValue;
  // 16-byte lanes when every row of X and Y starts 16-byte aligned and k
  // fills whole vectors; for fp32, 8-byte lanes (two columns) when k, the
  // strides and the 8-byte alignment allow; otherwise one element per lane
  constexpr int VE = 16 / sizeof(V);
  const uintptr_t xy = reinterpret_cast<uintptr_t>(a.X) | reinterpret_cast<uintptr_t>(a.Y);
  const bool vec = a.k % VE == 0 && a.ldx % VE == 0 && a.ldy % VE == 0 && (xy & 15) == 0;
  hipError_t err;
  if (vec) {
    err = launch_ve<V, VE>(a, s, ev0, ev1);
  } else if constexpr (VE == 4) {
    const bool vec2 = a.k % 2 == 0 && a.ldx % 2 == 0 && a.ldy % 2 == 0 && (xy & 7) == 0;
    err = vec2 ? launch_ve<V, 2>(a, s, ev0, ev1) : launch_ve<V, 1>(a, s, ev0, ev1);
  } else {
    err = launch_ve<V, 1>(a, s, ev0, ev1);
  }
  const int fb = spmm_fixup_blocks(a);
  if (err != hipSuccess || !fixup || fb == 0) return err;
  hipLaunchKernelGGL((spmm_fixup_kernel<V>), dim3((unsigned)fb), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_spmm<float>(const SpmmArgs<float>&, hipStream_t, hipEvent_t,
                                       hipEvent_t, bool);
template hipError_t launch_spmm<double>(const SpmmArgs<double>&, hipStream_t, hipEvent_t,
                                        hipEvent_t, bool);

int spmm_tile_split(int k, int vbytes, int bc) {
  const int ve = 16 / vbytes;
  // X rows of at most 32 bytes: at 64 (fp32 k = 16) a row's segment in a
  // sub-block fills under half of a half-wave's quads, and the bimodal
  // matrix measured 0.45 ms tiled against 0.38 ms untiled
  if (k <= 0 || k % ve != 0 || k * vbytes > 32) return 0;
  int m = 1;
  while ((int64_t)(bc / m) * k * vbytes > kSpmmTileBytes) m *= 2;
  return m <= kTileSub ? m : 0;   // the plan keeps bounds at quarter blocks
}

template <typename V>
size_t spmm_tile_workspace(int n_rows, int nb, int m, int k) {
  return (sizeof(V) * (size_t)n_rows * nb * m * k + 255) & ~size_t(255);
}

template <typename V, int W, int RW>
hipError_t launch_spmm_tiles_w(const SpmmTileArgs<V>& t, hipStream_t s);

int spmm_tile_rows_per_wave(int n_rows, int nb, int m) {
  for (int rw = 32; rw > 8; rw /= 2) {
    const int64_t tr = (int64_t)kSpmmTileWaves * rw;
    if ((n_rows + tr - 1) / tr * nb * m >= kSpmmTileMinGrid) return rw;
  }
  return 8;
}
template <typename V>
hipError_t launch_spmm_tiles(const SpmmTileArgs<V>& t, hipStream_t s) {
  if (t.n_rows <= 0 || t.m <= 0) return hipSuccess;
  if (kTileSub % t.m != 0) return hipErrorInvalidValue;
  // the most rows per wave that still leaves kSpmmTileMinGrid tiles (more
  // rows a tile stage its X block fewer times)
  const int rw = spmm_tile_rows_per_wave(t.n_rows, t.nb, t.m);
  if (rw == 32) return launch_spmm_tiles_w<V, kSpmmTileWaves, 32>(t, s);
  if (rw == 16) return launch_spmm_tiles_w<V, kSpmmTileWaves, 16>(t, s);
  return launch_spmm_tiles_w<V, kSpmmTileWaves, 8>(t, s);
}
template <typename V, int W, int RW>
hipError_t launch_spmm_tiles_w(const SpmmTileArgs<V>& t, hipStream_t s) {
  SpmmTileArgs<V> u = t;
  u.ngroups = (t.n_rows + W * RW - 1) / (W * RW);
  const int64_t tiles = (int64_t)u.ngroups * t.nb * t.m;
  if (tiles > 0x7fffffffll) return hipErrorInvalidValue;
  constexpr int VE = 16 / (int)sizeof(V);
  const int lanes = t.k / VE;   // k is a multiple of VE (spmm_tile_split)
  // the kernel takes X rows of exactly KL * VE values
  if (t.k % VE != 0 || lanes < 1 || lanes > 2) return hipErrorInvalidValue;
  // the block's X rows and one zero row (just past 64 KiB at the widest)
  const size_t lds = ((size_t)t.bck + 1) * t.k * sizeof(V);
  const dim3 g((unsigned)tiles), b(W * kWave);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, g, b, lds, s, u);
    return hipGetLastError();
  };
  if (lanes <= 1) return go(spmm_tile_kernel<V, 1, VE, W, RW>);
  if (lanes <= 2) return go(spmm_tile_kernel<V, 2, VE, W, RW>);
  return hipErrorInvalidValue;
}

template <typename V>
hipError_t launch_spmm_fixup_tile_reduce(const SpmmArgs<V>& a, const SpmmTileArgs<V>& t,
                                         hipStream_t s) {
  if (t.n_rows <= 0 || t.m <= 0) return hipSuccess;
  int kc = 1;
  while (kc < t.k) kc *= 2;
  if (kc > kWave || a.k != t.k || !t.skip) return hipErrorInvalidValue;
  const int fb = spmm_fixup_blocks(a);
  const int64_t rb = ((int64_t)t.n_rows * kWave + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(spmm_fixup_tile_reduce_kernel<V>, dim3((unsigned)(fb + rb)), dim3(kBlock), 0,
                     s, a, t, fb, kc);
  return hipGetLastError();
}

template size_t spmm_tile_workspace<float>(int, int, int, int);
template size_t spmm_tile_workspace<double>(int, int, int, int);
template hipError_t launch_spmm_tiles<float>(const SpmmTileArgs<float>&, hipStream_t);
template hipError_t launch_spmm_tiles<double>(const SpmmTileArgs<double>&, hipStream_t);
template hipError_t launch_spmm_fixup_tile_reduce<float>(const SpmmArgs<float>&,
                                                         const SpmmTileArgs<float>&, hipStream_t);
template hipError_t launch_spmm_fixup_tile_reduce<double>(const SpmmArgs<double>&,
                                                          const SpmmTileArgs<double>&,
                                                          hipStream_t);

}  // namespace spmv
