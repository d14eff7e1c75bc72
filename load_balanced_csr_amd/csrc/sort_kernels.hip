// Stable LSD radix sort of (int32 key, int32 value) pairs, and the exclusive
// scan it uses, for plan-time orderings: the column dispatch order of walk
// partitions (keys: a partition's middle column) and the transpose of a CSR
// matrix (keys: column indices, values: entry positions).
//
// One pass per 8-bit digit of the keys' low `bits` bits:
//   1. each workgroup counts the digits of its tile of keys in LDS and writes
//      its 256 counts digit-major ([digit][tile]);
//   2. an exclusive scan of those counts gives, for every (digit, tile), the
//      first output position (digit-major order makes the result stable);
//   3. each workgroup re-reads its tile in order, 256 keys per round; inside
//      a wave, lanes with the same digit find each other with eight ballots
//      (one per digit bit), a lane's rank is the number of such lanes below
//      it, and the waves' counts per digit are combined in LDS; every key
//      goes to its digit's running position plus its rank.
// No global atomics; the result depends only on the input. The element count
// and an enable flag may live in device memory (written by earlier kernels
// of the same plan), so the host needs no read-back to launch the passes.
#include "device_common.hpp"
#include "internal.hpp"

#include <algorithm>

namespace spmv {
namespace {

constexpr int kSortThreads = 256;
constexpr int kSortRound = kSortThreads;             // keys per round
constexpr int kSortRounds = 16;                      // rounds per tile
constexpr int kSortTile = kSortRound * kSortRounds;  // keys per sub-tile
constexpr int64_t kSortMaxTiles = 32768;             // workgroups per pass
constexpr int kScanChunk = 4096;                     // scan elements per workgroup
constexpr int kScanTopMax = 8192;                    // chunks the one-workgroup scan takes

__device__ __forceinline__ bool sort_enabled(const int64_t* enable) {
  return enable == nullptr || *enable != 0;
}
__device__ __forceinline__ int64_t sort_count(int64_t n, const int64_t* n_dev) {
  return n_dev ? *n_dev : n;
}

// Exclusive scan of one int per thread across a workgroup of kSortThreads;
// returns this thread's exclusive prefix, *total gets the workgroup's sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int x = wave_scan_i32(v);   // inclusive, DPP moves
  if (lane == kWave - 1) s_wave[wave] = x;
  __syncthreads();
  int before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kSortThreads / kWave; ++w) {
    const int c = s_wave[w];
    before += w < wave ? c : 0;
    sum += c;
  }
  __syncthreads();   // s_wave may be reused by the caller
  *total = sum;
  return before + x - v;
}

// Digit counts of each tile, digit-major: counts[d * tiles + tile].
__global__ __launch_bounds__(kSortThreads) void radix_count_kernel(
    const int32_t* __restrict__ keys, int64_t n, const int64_t* n_dev, const int64_t* enable,
    int shift, int iters, int32_t tiles, int32_t* __restrict__ counts) {
  if (!sort_enabled(enable)) return;
  n = sort_count(n, n_dev);
  __shared__ int s_hist[256];
  s_hist[threadIdx.x] = 0;
  __syncthreads();
  const int64_t first = (int64_t)blockIdx.x * iters * kSortTile;
  for (int64_t i = first + threadIdx.x; i < first + (int64_t)iters * kSortTile && i < n;
       i += kSortThreads)
    atomicAdd(&s_hist[(keys[i] >> shift) & 255], 1);
  __syncthreads();
  counts[(int64_t)threadIdx.x * tiles + blockIdx.x] = s_hist[threadIdx.x];
}

// Three-phase exclusive scan, in place, of e int32 (total < 2^31).
__global__ __launch_bounds__(kSortThreads) void scan_reduce_kernel(
    const int32_t* __restrict__ data, int64_t e, const int64_t* enable, int32_t* __restrict__ sums) {
  if (!sort_enabled(enable)) return;
  __shared__ int s_wave[kSortThreads / kWave];
  const int64_t first = (int64_t)blockIdx.x * kScanChunk;
  int v = 0;
  for (int64_t i = first + threadIdx.x; i < first + kScanChunk && i < e; i += kSortThreads)
    v += data[i];
  int total;
  (void)block_exclusive_scan(v, s_wave, &total);
  if (threadIdx.x == 0) sums[blockIdx.x] = total;
}

__global__ __launch_bounds__(1024) void scan_top_kernel(int32_t* __restrict__ sums, int32_t n,
                                                        const int64_t* enable) {
  if (!sort_enabled(enable)) return;
  constexpr int PER = kScanTopMax / 1024;
  __shared__ int s_wave[16];
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  int v[PER], local = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = threadIdx.x * PER + k;
    v[k] = i < n ? sums[i] : 0;
    local += v[k];
  }
  const int x = wave_scan_i32(local);
  if (lane == kWave - 1) s_wave[wave] = x;
  __syncthreads();
  int run = x - local;
  for (int w = 0; w < wave; ++w) run += s_wave[w];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = threadIdx.x * PER + k;
    if (i < n) sums[i] = run;
    run += v[k];
  }
}

__global__ __launch_bounds__(kSortThreads) void scan_down_kernel(
    int32_t* __restrict__ data, int64_t e, const int64_t* enable, const int32_t* __restrict__ sums) {
  if (!sort_enabled(enable)) return;
  constexpr int PER = kScanChunk / kSortThreads;
  __shared__ int s_wave[kSortThreads / kWave];
  const int64_t first = (int64_t)blockIdx.x * kScanChunk + (int64_t)threadIdx.x * PER;
  int v[PER], local = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    v[k] = first + k < e ? data[first + k] : 0;
    local += v[k];
  }
  int total;
  int run = sums[blockIdx.x] + block_exclusive_scan(local, s_wave, &total);
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (first + k < e) data[first + k] = run;
    run += v[k];
  }
}

// Stable scatter of one digit pass. vals_in == nullptr: the value of key i
// is i (the first pass of an index sort).
__global__ __launch_bounds__(kSortThreads) void radix_scatter_kernel(
    const int32_t* __restrict__ keys_in, const int32_t* __restrict__ vals_in, int64_t n,
    const int64_t* n_dev, const int64_t* enable, int shift, int iters, int32_t tiles,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ keys_out,
    int32_t* __restrict__ vals_out) {
  if (!sort_enabled(enable)) return;
  n = sort_count(n, n_dev);
  constexpr int kWaves = kSortThreads / kWave;
  __shared__ int s_base[256];          // next output position of each digit
  __shared__ int s_cnt[kWaves][256];   // this round: keys of each digit per wave
  __shared__ int s_pre[kWaves][256];   // ... and each wave's first position
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  s_base[tid] = offsets[(int64_t)tid * tiles + blockIdx.x];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s_cnt[w][tid] = 0;
  __syncthreads();
  const int64_t first = (int64_t)blockIdx.x * iters * kSortTile;
  for (int sub = 0; sub < iters; ++sub) {
    const int64_t tile0 = first + (int64_t)sub * kSortTile;
    if (tile0 >= n) break;   // block-uniform
    for (int round = 0; round < kSortRounds; ++round) {
      const int64_t i = tile0 + (int64_t)round * kSortRound + tid;
      const bool valid = i < n;
      const int32_t key = valid ? keys_in[i] : 0;
      const int32_t val = valid ? (vals_in ? vals_in[i] : (int32_t)i) : 0;
      const int d = (key >> shift) & 255;
      uint64_t peers = __ballot(valid);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const uint64_t m = __ballot((d >> b) & 1);
        peers &= ((d >> b) & 1) ? m : ~m;
      }
      const int rank = lanes_below(peers);
      if (valid && rank == 0) s_cnt[wave][d] = __popcll(peers);
      __syncthreads();
      {
        int run = s_base[tid];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          s_pre[w][tid] = run;
          run += s_cnt[w][tid];
          s_cnt[w][tid] = 0;
        }
        s_base[tid] = run;
      }
      __syncthreads();
      if (valid) {
        const int pos = s_pre[wave][d] + rank;
        keys_out[pos] = key;
        vals_out[pos] = val;
      }
    }
  }
}

struct SortGeometry {
  int iters;
  int32_t tiles;
  int64_t count_elems;
  int64_t chunks;
};

SortGeometry sort_geometry(int64_t n_max) {
  SortGeometry g;
  const int64_t sub = std::max<int64_t>(1, (n_max + kSortTile - 1) / kSortTile);
  g.iters = (int)((sub + kSortMaxTiles - 1) / kSortMaxTiles);
  g.tiles = (int32_t)std::max<int64_t>(1, (sub + g.iters - 1) / g.iters);
  g.count_elems = 256 * (int64_t)g.tiles;
  g.chunks = (g.count_elems + kScanChunk - 1) / kScanChunk;
  return g;
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

}  // namespace

size_t scan_temp_bytes(int64_t n_max) {
  return align256(sizeof(int32_t) * (size_t)((std::max<int64_t>(n_max, 1) + kScanChunk - 1) /
                                             kScanChunk));
}

hipError_t exclusive_scan_i32(int32_t* data, int64_t n_max, const int64_t* enable, void* temp,
                              hipStream_t s) {
  const int64_t chunks = (std::max<int64_t>(n_max, 1) + kScanChunk - 1) / kScanChunk;
  if (chunks > kScanTopMax) return hipErrorInvalidValue;
  int32_t* sums = static_cast<int32_t*>(temp);
  hipLaunchKernelGGL(scan_reduce_kernel, dim3((unsigned)chunks), dim3(kSortThreads), 0, s, data,
                     n_max, enable, sums);
  hipLaunchKernelGGL(scan_top_kernel, dim3(1), dim3(1024), 0, s, sums, (int32_t)chunks, enable);
  hipLaunchKernelGGL(scan_down_kernel, dim3((unsigned)chunks), dim3(kSortThreads), 0, s, data,
                     n_max, enable, sums);
  return hipGetLastError();
}

size_t radix_sort_temp_bytes(int64_t n_max) {
  const SortGeometry g = sort_geometry(n_max);
  return align256(sizeof(int32_t) * (size_t)g.count_elems) +
         align256(sizeof(int32_t) * (size_t)g.chunks);
}

hipError_t radix_sort_pairs(int32_t* keys0, const int32_t* vals_in, int32_t* vals0,
                            int32_t* keys1, int32_t* vals1, void* temp, int64_t n_max,
                            const int64_t* n_dev, const int64_t* enable, int bits, hipStream_t s,
                            int* result) {
  const SortGeometry g = sort_geometry(n_max);
  if (g.chunks > kScanTopMax) return hipErrorInvalidValue;
  int32_t* counts = static_cast<int32_t*>(temp);
  int32_t* sums = reinterpret_cast<int32_t*>(static_cast<char*>(temp) +
                                             align256(sizeof(int32_t) * (size_t)g.count_elems));
  const int passes = std::max(1, (bits + 7) / 8);
  int32_t* k[2] = {keys0, keys1};
  int32_t* v[2] = {vals0, vals1};
  int cur = 0;
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = 8 * pass;
    hipLaunchKernelGGL(radix_count_kernel, dim3(g.tiles), dim3(kSortThreads), 0, s, k[cur],
                       n_max, n_dev, enable, shift, g.iters, g.tiles, counts);
    hipLaunchKernelGGL(scan_reduce_kernel, dim3((unsigned)g.chunks), dim3(kSortThreads), 0, s,
                       counts, g.count_elems, enable, sums);
    hipLaunchKernelGGL(scan_top_kernel, dim3(1), dim3(1024), 0, s, sums, (int32_t)g.chunks,
                       enable);
    hipLaunchKernelGGL(scan_down_kernel, dim3((unsigned)g.chunks), dim3(kSortThreads), 0, s,
                       counts, g.count_elems, enable, sums);
    // the first pass of an index sort takes the positions as its values
    hipLaunchKernelGGL(radix_scatter_kernel, dim3(g.tiles), dim3(kSortThreads), 0, s, k[cur],
                       pass == 0 ? vals_in : v[cur], n_max, n_dev, enable, shift, g.iters, g.tiles,
                       counts, k[1 - cur], v[1 - cur]);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    cur = 1 - cur;
  }
  *result = cur;
  return hipSuccess;
}

}  // namespace spmv
