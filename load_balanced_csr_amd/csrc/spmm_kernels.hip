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
// holds output column l. The partition's units are cut again, merge-path
// style, into S equal runs, one per slot, so every slot does the same work
// however long the rows are. A slot walks its run in order; per batch of 8
// nonzeros it first issues all their X-row loads (KL consecutive elements
// per nonzero: one coalesced access per slot), then adds the products,
// finishing rows as their ends come by. A row wholly inside one run is
// written by that slot; the pieces of rows cut between runs are combined in
// slot order afterwards, and a row cut at the partition's end leaves a
// k-wide carry that the fix-up kernel adds, in partition order. No float
// atomics: for a fixed plan the result is bitwise reproducible.
#include "device_common.hpp"
#include "internal.hpp"

#include <limits.h>

namespace spmv {
namespace {

constexpr int kSpmmBatch = 8;

// LDS of one wave (bytes): head / tail vectors (64 V each), the staged row
// pointers and column indices (cap int32 each, 16-byte aligned), and the
// per-slot records (5 x 64 int32).
__host__ __device__ constexpr int spmm_wave_lds(int vbytes, int cap) {
  return (2 * kWave * vbytes + 2 * cap * 4 + 5 * kWave * 4 + 15) / 16 * 16;
}

// a[beg, beg + cnt) (int32, n elements in all) into dst so that a[beg + t]
// lands at dst[(beg & 3) + t]. 16-byte loads where the quad lies inside the
// array, element loads for the array's last, partial quad. dst is 16-byte
// aligned with room for cnt + 7 entries.
__device__ __forceinline__ void stage_i32(int32_t* dst, const int32_t* a, int beg, int cnt,
                                          int n) {
  if (cnt <= 0) return;
  const int q0 = beg >> 2;
  const int nq = ((beg + cnt - 1) >> 2) - q0 + 1;
  for (int t = lane_id(); t < nq; t += kWave) {
    const int q = q0 + t;
    i32x4 v;
    if (4 * q + 3 < n) {
      v = ld_stream(reinterpret_cast<const i32x4*>(a) + q);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = 4 * q + j < n ? a[4 * q + j] : 0;
    }
    *reinterpret_cast<i32x4*>(dst + 4 * t) = v;
  }
}

template <typename V>
__device__ __forceinline__ void spmm_store(const SpmmArgs<V>& a, int row, int col, V acc) {
  V* yp = a.Y + (int64_t)row * a.ldy + col;
  V out = a.alpha * acc;
  if (a.beta_nonzero) out = fma(a.beta, *yp, out);
  *yp = out;
}

template <typename V, int KL>
__global__ __launch_bounds__(kBlock) void spmm_merge_kernel(const SpmmArgs<V> a) {
  constexpr int S = kWave / KL;   // slots per wave
  constexpr int B = kSpmmBatch;
  extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int blk = a.xcd_remap ? xcd_tile(blockIdx.x, 0, gridDim.x) : (int)blockIdx.x;
  const int p = blk * kWavesPerBlock + wave;
  if (p >= a.P) return;

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

  unsigned char* base = s_dyn + (size_t)wave * spmm_wave_lds(sizeof(V), a.cap);
  V* head_vec = reinterpret_cast<V*>(base);
  V* tail_vec = head_vec + kWave;
  int32_t* s_rp = reinterpret_cast<int32_t*>(tail_vec + kWave);
  int32_t* s_col = s_rp + a.cap;
  int32_t* rec = s_col + a.cap;   // [5][64]: head ends, tail owned, used, head row, tail row

  // row pointers rp[r0 .. r1] (row r1's start ends the last closed row) and
  // the partition's column indices
  stage_i32(s_rp, a.row_ptr, r0, R + 1, a.M + 1);
  stage_i32(s_col, a.col_idx, n0, nloc, a.nnz);
  wave_sync();
  const int32_t* rpl = s_rp + (r0 & 3);    // rpl[i] = row_ptr[r0 + i]
  const int32_t* coll = s_col + (n0 & 3);  // coll[t] = col_idx[n0 + t]

  const int s = lane / KL, cl = lane % KL;
  const bool colok = cl < a.k;
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
  V acc = V(0), head = V(0);
  int e = i < R ? rpl[i + 1] - n0 : INT_MAX;   // local end of row i

  for (int jb = jbeg; jb < jend; jb += B) {
    V xv[B], vv[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int jj = jb + u;
      const bool ok = jj < jend;
      const int c = ok ? coll[jj] : 0;
      vv[u] = ok ? a.val[n0 + jj] : V(0);
      xv[u] = ok && colok ? a.X[(int64_t)c * a.ldx + cl] : V(0);
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int jj = jb + u;
      while (i < iend && e == jj) {   // rows ending before nonzero jj
        if (owned) {
          if (colok) spmm_store(a, r0 + i, cl, acc);
        } else {
          head = acc;
          head_ends = true;
        }
        owned = true;
        acc = V(0);
        ++i;
        e = i < R ? rpl[i + 1] - n0 : INT_MAX;
      }
      if (jj < jend) acc = fma(vv[u], xv[u], acc);
    }
  }
  while (i < iend) {                   // rows ending at the run's end
    if (owned) {
      if (colok) spmm_store(a, r0 + i, cl, acc);
    } else {
      head = acc;
      head_ends = true;
    }
    owned = true;
    acc = V(0);
    ++i;
  }

  // records: the piece of the first row (when another slot started it and it
  // ended here) and the piece of the row open at the run's end
  head_vec[lane] = head;
  tail_vec[lane] = acc;
  if (cl == 0) {
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
    V rv = V(0);
    for (int t = 0; t < S; ++t) {
      if (!rec[2 * kWave + t]) break;   // only trailing slots are empty
      if (rec[t]) {
        const V v = (run ? rv : V(0)) + head_vec[t * KL + cl];
        if (colok) spmm_store(a, r0 + rec[3 * kWave + t], cl, v);
        run = false;
      }
      if (rec[kWave + t]) {
        run = true;
        rv = tail_vec[t * KL + cl];
      } else {
        rv += tail_vec[t * KL + cl];
      }
    }
    if (!a.stream) {
      if (colok) a.carry_vec[(int64_t)p * a.k + cl] = run ? rv : V(0);
      if (lane == 0) a.carry_row[p] = r1;
    }
  }
}

// Y[r] += alpha * (sum of the carries of r), one wave per partition: the
// wave holding the first carry of a row sums that row's carries in
// partition order (they are contiguous) and updates the row once.
template <typename V>
__global__ __launch_bounds__(kBlock) void spmm_fixup_kernel(const SpmmArgs<V> a) {
  const int lane = lane_id();
  const int p = blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (p >= a.P) return;
  const int r = a.carry_row[p];
  if (r >= a.M || (p > 0 && a.carry_row[p - 1] == r)) return;
  if (lane >= a.k) return;
  V sum = V(0);
  for (int q = p; q < a.P && a.carry_row[q] == r; ++q) sum += a.carry_vec[(int64_t)q * a.k + lane];
  V* yp = a.Y + (int64_t)r * a.ldy + lane;
  *yp = fma(a.alpha, sum, *yp);
}

template <typename V, int KL>
hipError_t launch_kl(const SpmmArgs<V>& a, hipStream_t s) {
  const int blocks = (a.P + kWavesPerBlock - 1) / kWavesPerBlock;
  const size_t lds = (size_t)kWavesPerBlock * spmm_wave_lds(sizeof(V), a.cap);
  hipLaunchKernelGGL((spmm_merge_kernel<V, KL>), dim3(blocks), dim3(kBlock), lds, s, a);
  return hipGetLastError();
}

}  // namespace

size_t spmm_lds_bytes(int vbytes, int T) {
  return (size_t)kWavesPerBlock * spmm_wave_lds(vbytes, spmm_stage_cap(T));
}

template <typename V>
hipError_t launch_spmm(const SpmmArgs<V>& a, hipStream_t s) {
  if (a.P <= 0 || a.k <= 0) return hipSuccess;
  if (a.k > kWave || a.cap < spmm_stage_cap(a.T)) return hipErrorInvalidValue;
  hipError_t err;
  if (a.k <= 1) err = launch_kl<V, 1>(a, s);
  else if (a.k <= 2) err = launch_kl<V, 2>(a, s);
  else if (a.k <= 4) err = launch_kl<V, 4>(a, s);
  else if (a.k <= 8) err = launch_kl<V, 8>(a, s);
  else if (a.k <= 16) err = launch_kl<V, 16>(a, s);
  else if (a.k <= 32) err = launch_kl<V, 32>(a, s);
  else err = launch_kl<V, 64>(a, s);
  if (err != hipSuccess || a.stream || a.P <= 1) return err;
  hipLaunchKernelGGL((spmm_fixup_kernel<V>), dim3((a.P + kWavesPerBlock - 1) / kWavesPerBlock),
                     dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_spmm<float>(const SpmmArgs<float>&, hipStream_t);
template hipError_t launch_spmm<double>(const SpmmArgs<double>&, hipStream_t);

}  // namespace spmv
