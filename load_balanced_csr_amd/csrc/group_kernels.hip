// Group-mapped SpMV ("A Programming Model for GPU Load Balancing", Osama,
// Porumbescu, Owens, PPoPP'23, Section 5.2.3): a group of threads takes an
// equal share of the tiles (here: a run of consecutive rows), builds the
// prefix sum of its tiles' atom counts in scratchpad memory -- for CSR rows
// that prefix sum is the row pointer itself, so it is read rather than
// summed -- whose last element is the group's atom count, and its threads
// then take the group's atoms in turn; get_tile(atom) is a binary search in
// that prefix array.
//
// MI355X mapping: the group is a workgroup of GW wavefronts (1, 2 or 4). The
// atoms are processed in chunks of 512 per wavefront: each thread multiplies its
// atoms (contiguous in the CSR arrays, so the loads are coalesced) into an
// LDS product buffer; then each row's part of the chunk is summed in atom
// order -- by one lane for short parts, by a wavefront for long ones -- and
// added to the row's accumulator, so the result does not depend on timing
// (no float atomics); get_tile finds the first and last rows a chunk
// touches. y is written once per row at the end.
#include "device_common.hpp"
#include "internal.hpp"

#include <limits.h>

namespace spmv {
namespace {

constexpr int kGroupShort = 16;        // parts up to this many atoms: one lane

template <typename V, int GW>
__global__ __launch_bounds__(GW * kWave) void group_spmv_kernel(const GroupArgs<V> a) {
  constexpr int NT = GW * kWave;
  constexpr int CH = kGroupChunkPerWave * GW;     // atoms per LDS chunk
  constexpr int MAXR = kGroupRowsPerWave * GW;    // rows a group may take
  __shared__ int32_t s_pref[MAXR + 1];
  __shared__ V s_prod[CH];
  __shared__ V s_acc[MAXR];

  const int t = threadIdx.x;
  const int lane = lane_id();
  const int wave = t / kWave;
  const int64_t r0 = (int64_t)blockIdx.x * a.rows_per_group;
  if (r0 >= a.M) return;
  const int R = (int)min((int64_t)a.rows_per_group, (int64_t)a.M - r0);
  // the tiles' atom counts, prefix-summed: row_ptr relative to the group start
  const int64_t n0 = a.row_ptr[r0];
  for (int i = t; i <= R; i += NT) s_pref[i] = (int32_t)(a.row_ptr[r0 + i] - n0);
  for (int i = t; i < R; i += NT) s_acc[i] = V(0);
  __syncthreads();
  const int A = s_pref[R];   // the group's atoms

  // get_tile: the row holding atom j (last i with s_pref[i] <= j)
  auto get_tile = [&](int j) {
    int lo = 0, hi = R - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= j) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };

  // chunks counted, not strided: base + CH must not wrap for A near 2^31
  const int nchunks = A / CH + (A % CH != 0);
  for (int c = 0; c < nchunks; ++c) {
    const int base = c * CH;
    const int cnt = min(CH, A - base);
    // products of the chunk's atoms, coalesced: a thread's CH / NT atoms
    // (t, t + NT, ...) are loaded together, then gathered together, before
    // the first product is stored (atoms past the chunk re-read its last one
    // and store nothing)
    {
      constexpr int U = CH / NT;
      int cu[U];
      V vu[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t e = n0 + base + min(t + u * NT, cnt - 1);
        cu[u] = ld_stream(a.col_idx + e);
        vu[u] = ld_stream(a.val + e);
      }
      V xu[U];
#pragma unroll
      for (int u = 0; u < U; ++u) xu[u] = a.x[cu[u]];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (t + u * NT < cnt) s_prod[t + u * NT] = vu[u] * xu[u];
    }
    __syncthreads();
    // rows whose atoms meet this chunk: [first, last]
    const int first = get_tile(base), last = get_tile(base + cnt - 1);
    // short parts: one lane each, in atom order
    for (int i = first + t; i <= last; i += NT) {
      const int b = max(s_pref[i], base) - base, e = min(s_pref[i + 1], base + cnt) - base;
      if (e - b <= kGroupShort) {
        V s = V(0);
        for (int j = b; j < e; ++j) s += s_prod[j];
        s_acc[i] += s;
      }
    }
    // long parts: one wavefront each, lanes strided, then a butterfly
    for (int i = first + wave; i <= last; i += GW) {
      const int b = max(s_pref[i], base) - base, e = min(s_pref[i + 1], base + cnt) - base;
      if (e - b > kGroupShort) {   // uniform over the wavefront
        V s = V(0);
        for (int j = b + lane; j < e; j += kWave) s += s_prod[j];
        for (int o = kWave / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
        if (lane == 0) s_acc[i] += s;
      }
    }
    __syncthreads();
  }
  for (int i = t; i < R; i += NT) {
    V out = a.alpha * s_acc[i];
    if (a.beta_nonzero) out = fma(a.beta, a.y[r0 + i], out);
    a.y[r0 + i] = out;
  }
}

}  // namespace

template <typename V>
hipError_t launch_group(const GroupArgs<V>& a, int group_waves, hipStream_t s, hipEvent_t ev0,
                        hipEvent_t ev1) {
  if (a.M == 0) return hipSuccess;
  if (a.rows_per_group < 1 || a.rows_per_group > kGroupRowsPerWave * group_waves)
    return hipErrorInvalidValue;
  const int64_t groups = ((int64_t)a.M + a.rows_per_group - 1) / a.rows_per_group;
  switch (group_waves) {
    case 1:
      launch_timed(group_spmv_kernel<V, 1>, dim3((unsigned)groups), dim3(kWave), 0, s, ev0, ev1, a);
      break;
    case 2:
      launch_timed(group_spmv_kernel<V, 2>, dim3((unsigned)groups), dim3(2 * kWave), 0, s, ev0,
                   ev1, a);
      break;
    case 4:
      launch_timed(group_spmv_kernel<V, 4>, dim3((unsigned)groups), dim3(4 * kWave), 0, s, ev0,
                   ev1, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t launch_group<float>(const GroupArgs<float>&, int, hipStream_t, hipEvent_t,
                                        hipEvent_t);
template hipError_t launch_group<double>(const GroupArgs<double>&, int, hipStream_t, hipEvent_t,
                                         hipEvent_t);

}  // namespace spmv
