// Host-side launch interface between the C ABI (api.hip) and the kernels
// (plan_kernels.hip, merge_kernels.hip, binned_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

namespace spmv {

// Launch a kernel; with timing events, the dispatch itself records them at
// the kernel's start and end (AMD's extended launch), so they bracket the
// kernel alone, as a kernel trace does. Without events, a plain launch.
template <typename... Args, typename F = void (*)(Args...)>
inline void launch_timed(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s,
                         hipEvent_t ev0, hipEvent_t ev1, Args... args) {
  if (ev0 || ev1)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, ev0, ev1, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

constexpr int kWave = 64;             // CDNA4 wavefront
constexpr int kBlock = 256;           // threads per workgroup (4 waves)
constexpr int kLdsBytes = 160 * 1024;  // LDS of one CU, the most one workgroup may take
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kXcds = 8;              // MI355X: 8 accelerator complex dies
constexpr int64_t kXcdL2Bytes = int64_t(4) << 20;   // L2 of one XCD
constexpr int kMaxBins = 8;
constexpr int kBinRowsPerBlock = 1024;   // rows one binning workgroup owns
constexpr int kWinIntervals = 3;         // column intervals of one x window
constexpr int kWinTable = 8;             // int32 per window: {lo, len} x 3, total, flags

// Waves per SIMD the stream kernel's register budget allows: 8 (at most 64
// VGPRs) up to T = 448; larger partitions, and fp64 with the x window, need
// more registers than that, and spilling would cost more than the waves
// given up.
constexpr int stream_min_waves(int vbytes, int ipt, bool win) {
  return ipt >= 16 ? (vbytes == 8 && win ? 3 : 4) : ipt < 8 ? 8 : vbytes == 4 ? 7 : win ? 5 : 8;
}

// LDS of the stream kernel. Its staging buffer per wave holds the T + T/8
// units of one partition (+16 for quad alignment). The x window of a
// workgroup of wpb waves takes what is left of the workgroup's share of the
// CU's 160 KiB at the occupancy the registers allow, minus 512 bytes of
// allocation slack; below 2 KiB it is not worth a barrier and is 0.
constexpr int stream_buf_elems(int ipt) { return kWave * ipt + kWave * ipt / 8 + 16; }
constexpr int stream_window_raw(int ipt, int vbytes, int wpb) {
  return (163840 * wpb / (4 * stream_min_waves(vbytes, ipt, true)) - 512 -
          wpb * stream_buf_elems(ipt) * vbytes) / 16 * 16;
}
constexpr int stream_window_bytes(int ipt, int vbytes, int wpb) {
  return stream_window_raw(ipt, vbytes, wpb) >= 2048 ? stream_window_raw(ipt, vbytes, wpb) : 0;
}

// Layout of the statistics block the plan copies back to the host (int64).
enum StatSlot : int {
  kStatMaxLen = 0,
  kStatEmpty = 1,
  kStatError = 2,          // bit 0: row_ptr malformed, bit 1: column out of range
  kStatNonEmptyBins = 3,
  kStatWindowFits = 4,     // stream workgroups whose columns fit one x interval
  kStatWindowSamples = 5,  // stream workgroups examined
  kStatWindowFitsMulti = 6,  // ... that fit kWinIntervals intervals
  kStatBinOffset = 7,      // kMaxBins + 1 entries
  kStatInterior = kStatBinOffset + kMaxBins + 1,  // partitions inside one row
  kStatIpt = kStatInterior + 1,      // merge-path items per lane the plan chose
  kStatParts = kStatIpt + 1,         // P at that partition size
  kStatResplit = kStatParts + 1,     // 1: the second split pass runs (T = 256)
  kStatOrder = kStatResplit + 1,     // 1: walk partitions dealt in column order
  kStatTileOk = kStatOrder + 1,      // 1: the plan may tile long rows (walk, x > one block)
  kStatTileRows = kStatTileOk + 1,   // tile rows found (0: no tiles)
  kStatWalkParts = kStatTileRows + 1,  // partitions the walk kernel still runs, with tiles
  kStatTileEntries = kStatWalkParts + 1,  // nonzeros in the tile rows' interior runs
  kStatSlabOk = kStatTileEntries + 1,     // 1: the plan builds x slabs (auto: unless runs stray)
  kStatSlabStray = kStatSlabOk + 1,       // slab runs whose middle entry strays (rows not sorted)
  kStatSlabSegs = kStatSlabStray + 1,     // (row, slab) segments with at least one entry
  kStatSlabChunks = kStatSlabSegs + 1,    // workgroups of the copy into the slab-major order
  kStatCount = kStatSlabChunks + 1
};

// ---- column-blocked tiles of long rows (tile_kernels.hip) ------------------------
constexpr int kTileBytes = 16384;   // x block of one tile in LDS: 4096 fp32 / 2048 fp64
constexpr int kTileRows = 64;       // tile rows one workgroup takes per column block
constexpr int kTileBatch = 4;      // tile rows whose quads a wave requests together
constexpr int kTileSub = 4;        // segment bounds per column block (quarter blocks)
constexpr int kTileRowInts = 8;     // per tile row: row, first / end nonzero, first / end partition
constexpr int kTileMinPerBlock = 64;  // a row is tiled when its interior run holds this many
                                      // nonzeros per column block on average

// Plan-time buffers of the tiles (all in the plan's workspace).
struct TilePlan {
  int32_t cap;            // tile rows the buffers hold
  int32_t nb;             // column blocks
  int32_t bc;             // columns per block
  int64_t min_entries;    // kTileMinPerBlock * nb
  int32_t* rows;          // cap x kTileRowInts
  int32_t* seg;           // cap x (nb kTileSub + 1): bounds at every quarter block
  int32_t* skip;          // p_max: 1 where the walk kernel skips the partition
  int32_t* scan;          // p_max: flags, then their prefix sums
  int32_t* list;          // p_max: the walk kernel's dispatch list
  int32_t* mask_end;      // p_max: the walk kernel ignores nonzeros below this
  int32_t* mask_start;    // p_max: ... and from this one on (tile rows' ends)
  const int32_t* row_ptr;
  void* scan_temp;        // scan_temp_bytes(p_max)
};
// Tile rows (whole rows: their interior partitions skipped with zero
// carries, their nonzeros in the first and last partition masked off for
// the walk kernel), segments and the walk dispatch list, every launch gated
// by the statistics (kStatTileOk, then kStatTileRows). Tiles are kept only
// when their rows hold at least half of the nnz nonzeros.
hipError_t launch_tile_plan(const TilePlan& tp, const int32_t* split_row, const int32_t* split_nz,
                            const int32_t* col_idx, int64_t M, int64_t nnz, int64_t p_max,
                            int64_t* stats, int32_t* carry_row, void* carry_val, int vbytes,
                            hipStream_t s);

template <typename V>
struct TileArgs {
  const int32_t* rows;    // kTileRowInts per tile row
  const int32_t* seg;     // n_rows x (nb kTileSub + 1), quarter-block bounds
  const int32_t* col_idx;
  const V* val;
  const V* x;
  V* y;
  V* partial;             // n_rows x nb
  const int32_t* skip;    // per partition: 1 where the walk skips it (P entries)
  V alpha;
  int32_t n_rows;
  int32_t nb;
  int32_t ngroups;        // ceil(n_rows / kTileRows)
  int32_t N;
  int32_t nnz;
  int32_t x_aligned;      // x is 16-byte aligned (direct-to-LDS staging)
};

// Error bits of stats[kStatError].
constexpr int64_t kErrRowPtr = 1;     // row_ptr is not a CSR row pointer array
constexpr int64_t kErrColumn = 2;     // a column index outside [0, N) (validated)
constexpr int64_t kErrCooRows = 4;    // COO row indices out of range or order

// What the planning kernels decide on the device from the counted rows
// (host-known inputs of those decisions).
struct PlanCtl {
  int64_t M, N, nnz;
  int32_t vbytes;       // 4 or 8
  int32_t forced_ipt;   // items per lane given by the caller (0: chosen here)
  int32_t wide_x;       // x is larger than one XCD's L2
  int32_t reduce_req;   // 0 auto, 1 walk, 2 stream
  int32_t order_req;    // 0 auto, 1 partition order, 2 column order
  int32_t tiles_req;    // 0 auto, 1 off
  int32_t slabs_req;    // 0 auto, 1 off, 2 on
  int32_t mid_x;        // x of 1..4 MiB with mean row length x x bytes >= 1e8
  int32_t slab_room;    // the workspace holds the x slabs' row tables
};

struct BinEdges {
  int32_t n_bins;
  int32_t pad;
  int64_t max_len[kMaxBins];   // inclusive upper row length of bins 0..n_bins-2
};

// ---- plan kernels -----------------------------------------------------------
hipError_t launch_bin_count(const int32_t* row_ptr, int64_t M, int64_t nnz,
                            const BinEdges& edges, int32_t* counts, int32_t* wg_max,
                            int32_t* wg_empty, int64_t* stats, hipStream_t s);
hipError_t launch_bin_scan(int64_t M, const BinEdges& edges, int32_t* counts,
                           const int32_t* wg_max, const int32_t* wg_empty,
                           int64_t* stats, hipStream_t s);
hipError_t launch_bin_scatter(const int32_t* row_ptr, int64_t M, const BinEdges& edges,
                              const int32_t* offsets, const int64_t* stats,
                              int32_t* bins, hipStream_t s);
// Planning decisions on the device, one thread (stage 0: items per lane
// from the row lengths; 1: whether to split again at T = 256; 2: whether
// the walk partitions take the column dispatch order). See plan_kernels.hip.
hipError_t launch_plan_choose(const PlanCtl& c, int64_t* stats, int stage, hipStream_t s);
// Merge-path split at the partition size in stats[kStatIpt] (pass 1 runs
// only when stats[kStatResplit] is set); p_max bounds the partitions of any
// size the plan may choose. Also counts, into stats[kStatInterior], the
// partitions no row ends in (every item a nonzero of one row).
hipError_t launch_split_search(const int32_t* row_ptr, int64_t M, int64_t nnz, int64_t p_max,
                               int pass, int32_t* split_row, int32_t* split_nz,
                               int32_t* row_bounds, int64_t* stats, hipStream_t s);
hipError_t launch_check_columns(const int32_t* col_idx, int64_t nnz, int64_t N,
                                int64_t* stats, hipStream_t s);
hipError_t launch_clear_stats(int64_t* stats, hipStream_t s);
// row_ptr[0..M] from row indices sorted by row (COO); stats[kStatError]
// gets kErrCooRows when an index is outside [0, M) or out of order.
hipError_t launch_coo_row_ptr(const int32_t* row_idx, int64_t nnz, int64_t M, int32_t* row_ptr,
                              int64_t* stats, hipStream_t s);
// *flag |= 1 unless row_ptr is a valid CSR row pointer array for nnz entries.
hipError_t launch_csr_check(const int32_t* row_ptr, int64_t M, int64_t nnz, int32_t* flag,
                            hipStream_t s);
// col_t[t] = row of A holding entry perm[t]; val_t[t] = values[perm[t]].
hipError_t launch_transpose_gather(const int32_t* row_ptr, int64_t M, const int32_t* perm,
                                   const void* values, int vbytes, int64_t nnz, int32_t* col_t,
                                   void* val_t, hipStream_t s);
// Stable LSD radix sort (8-bit digits) of (key, value) pairs by the keys'
// low `bits` bits (keys >= 0). Pass 0 reads keys0 and vals_in (nullptr: the
// value of key i is i) and writes keys1 / vals1; later passes ping-pong;
// *result = 0 when the sorted pairs end in keys0 / vals0, 1 in keys1 /
// vals1. The element count is n_dev[0] when n_dev is set (at most n_max),
// else n_max; with `enable` set, every launch does nothing while *enable is
// 0. temp holds radix_sort_temp_bytes(n_max) bytes.
size_t radix_sort_temp_bytes(int64_t n_max);
// Exclusive prefix sum, in place, of n_max int32 (sum < 2^31); nothing while
// *enable is 0 (enable may be null). n_max <= 8192 * 4096. temp holds
// scan_temp_bytes(n_max) bytes.
size_t scan_temp_bytes(int64_t n_max);
hipError_t exclusive_scan_i32(int32_t* data, int64_t n_max, const int64_t* enable, void* temp,
                              hipStream_t s);
hipError_t radix_sort_pairs(int32_t* keys0, const int32_t* vals_in, int32_t* vals0,
                            int32_t* keys1, int32_t* vals1, void* temp, int64_t n_max,
                            const int64_t* n_dev, const int64_t* enable, int bits, hipStream_t s,
                            int* result);
// Per group of kWavesPerBlock consecutive stream partitions at the plan's
// chosen partition size: up to kWinIntervals chunk-aligned column intervals
// covering the group's quads within the stream kernel's window for that
// size (kWinTable int32 per group; win_span holds the groups of p_max
// partitions); counts groups and fitting groups in stats. Nothing for walk
// plans or a malformed row_ptr.
hipError_t launch_window_spans(const PlanCtl& c, const int32_t* row_ptr, const int32_t* col_idx,
                               const int32_t* split_row, int64_t p_max, int32_t* win_span,
                               int64_t* stats, hipStream_t s);
// stats[kError] |= bits when *flag != 0
hipError_t launch_fold_flag(const int32_t* flag, int64_t bits, int64_t* stats, hipStream_t s);

// ---- x slabs: one column slab of x per XCD (slab_kernels.hip) -----------------------
// A walk plan whose x is larger than one XCD's L2 gathers most x entries from
// beyond that L2. With x slabs the plan keeps a copy A' of A whose entries are
// ordered slab-major: slab s (columns [ceil(s N / 8), ceil((s + 1) N / 8)))
// holds, row after row, the run of each row's entries in those columns -- a
// segment, one row of the CSR matrix A' (M' segments, nnz entries). The walk
// over A' hands each XCD a contiguous eighth of its partitions, so XCD s
// gathers from slab s of x; a combine kernel then adds each row's segment
// sums, in slab order, into y with alpha and beta. Requires columns sorted
// within each row (checked while the tables are built; otherwise no slabs).
constexpr int kSlabs = kXcds;                    // one column slab per XCD
constexpr int kSlabTileRows = kBlock / kSlabs;   // rows per planning workgroup (8 lanes a row)

// Tables filled before the plan's read-back (inside its one workspace). Every
// launch does nothing unless stats[kStatSlabOk] is set.
constexpr int kSlabChunk = 4096;   // entries one workgroup copies into A'
struct SlabRows {
  uint8_t* mask;     // M: bit s set when the row has an entry in slab s
  int32_t* tile_e;   // kSlabs x n_tiles + 1, slab-major: entries of (slab, row tile), then prefix
  int32_t* tile_g;   // kSlabs x n_tiles + 1: segments of (slab, row tile), then prefix
  int32_t* tile_c;   // n_tiles + 1: copy chunks of each tile, then prefix
  void* scan_temp;   // scan_temp_bytes(slab_scan_max(M))
  int64_t n_tiles;   // ceil(M / kSlabTileRows)
};
constexpr int64_t kScanMaxElems = int64_t(8192) * 4096;   // exclusive_scan_i32's limit
inline int64_t slab_tiles(int64_t M) { return (M + kSlabTileRows - 1) / kSlabTileRows; }
inline int64_t slab_scan_max(int64_t M) { return kSlabs * slab_tiles(M) + 1; }
// Slab masks of the rows, the (slab, tile) counts and the tiles' copy
// chunks, their prefix sums; runs whose middle entry strays from the slab
// into stats[kStatSlabStray]; stats[kStatSlabSegs] = M', [kStatSlabChunks].
hipError_t launch_slab_rows(const SlabRows& t, const int32_t* row_ptr, const int32_t* col_idx,
                            int64_t M, int64_t N, int64_t nnz, int64_t* stats, hipStream_t s);

// A' (after the read-back, in the plan's second allocation).
struct SlabMatrix {
  int32_t* seg_ptr;   // M' + 1: A' row offsets
  int32_t* col;       // nnz
  void* val;          // nnz of the plan's dtype
  int64_t n_seg;      // M'
  int64_t n_chunks;   // workgroups of the copy
};
// Copies col_idx / values into A' and writes seg_ptr (also the values
// refresh of spmv_plan_update_values).
hipError_t launch_slab_emit(const SlabRows& t, const SlabMatrix& m, const int32_t* row_ptr,
                            const int32_t* col_idx, const void* values, int vbytes, int64_t M,
                            int64_t N, int64_t nnz, hipStream_t s);
// A statistics block for A's merge-path split: all zero but the items per
// lane and the partition count.
hipError_t launch_slab_stats(int64_t* stats, int ipt, int64_t P, hipStream_t s);
// y[r] = alpha * (sum over the slabs of row r of yp[segment]) + beta * y[r];
// a segment's id follows from the row's mask and the tile prefix sums.
template <typename V>
hipError_t launch_slab_combine(const SlabRows& t, const V* yp, V* y, V alpha, V beta,
                               int beta_nonzero, int64_t M, hipStream_t s);

// ---- merge-path exec ----------------------------------------------------------
template <typename V>
struct MergeArgs {
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const V* val;
  const V* x;
  V* y;
  const int32_t* split_row;
  const int32_t* split_nz;
  const int32_t* row_bounds;  // per boundary p: {split_row[p], row_ptr[split_row[p]]}
  int32_t* carry_row;
  V* carry_val;
  V alpha;
  V beta;
  int32_t beta_nonzero;
  int32_t P;
  int32_t M;
  int32_t nnz;
  int32_t xcd_remap;
  int32_t stream;        // 1: rows never cross partitions (all rows <= T/8)
  int32_t stream_lanes;  // lanes per row in the stream reduction
  int32_t x_window;      // stream kernel's x window: 0 none, 1 one interval, 3 up to three
  const int32_t* win_span;  // per stream workgroup: kWinTable int32 (window intervals)
  const int32_t* part_order;  // walk kernel: dispatch slot -> partition (null: identity)
  int32_t n_dispatch;    // walk kernel: dispatch slots (0: P)
  // walk kernel with long-row tiles: per partition, the nonzeros it leaves
  // to the tiles ([n0, mask_end) and [mask_start, n1)); null without tiles
  const int32_t* mask_end;
  const int32_t* mask_start;
};

// Streaming read of `bytes` (multiple of 16) at data; the xor of each 4 KiB
// block is stored to the 4-byte sink only when it equals key.
hipError_t launch_read_probe(const void* data, int64_t bytes, int32_t key, int32_t* sink,
                             hipStream_t s);

// Sort key of each walk partition for the column dispatch order: the column
// of its middle nonzero (0 for a partition without nonzeros); P from stats,
// nothing unless stats[kStatOrder] is set. p_max bounds P.
hipError_t launch_partition_keys(const int32_t* split_nz, const int32_t* col_idx, int64_t p_max,
                                 const int64_t* stats, int32_t* keys, hipStream_t s);
// Measurement aids (probe_kernels.hip).
hipError_t launch_gather_probe(const int32_t* col_idx, int64_t nnz, const void* x, int64_t n_x,
                               int vbytes, int32_t key, int32_t* sink, hipStream_t s);
hipError_t launch_gather_rows_probe(const int32_t* col_idx, int64_t nnz, const void* X,
                                    int64_t n_rows, int row_bytes, int32_t key, int32_t* sink,
                                    hipStream_t s);
hipError_t launch_stream_probe(const int32_t* row_ptr, const int32_t* col_idx, const void* values,
                               int64_t M, int64_t nnz, int vbytes, int ipt, void* y,
                               hipStream_t s);

// The walk or stream kernel (with tiles, for plans that have long-row
// tiles: the walk over the partitions they leave and the tiles, one grid),
// then the walk's carry fix-up (with tiles, in one grid with the tiles'
// reduction into y). ev0 / ev1 (may be null) are recorded by the
// main kernel's dispatch at its start and end.
template <typename V>
hipError_t launch_merge(const MergeArgs<V>& a, int ipt, hipStream_t s, hipEvent_t ev0,
                        hipEvent_t ev1, const TileArgs<V>* tiles = nullptr);

// ---- multi-vector exec (SpMM) -------------------------------------------------------
// Y = alpha * A X + beta * Y, X N x k and Y M x k row-major (k <= 64 per
// launch), over the plan's merge-path partitions.
template <typename V>
struct SpmmArgs {
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const V* val;
  const V* X;
  V* Y;
  int64_t ldx, ldy;          // row strides of X and Y, elements
  const int32_t* split_row;
  const int32_t* split_nz;
  const int32_t* row_bounds;
  int32_t* carry_row;        // P (not stream)
  V* carry_vec;              // P x k (not stream)
  V alpha;
  V beta;
  int32_t beta_nonzero;
  int32_t k;
  int32_t P;
  int32_t M;
  int32_t N;
  int32_t nnz;
  int32_t T;
  int32_t cap;               // staged entries per array and wave
  int32_t stream;            // 1: partitions end at row ends (no carries)
  int32_t xcd_remap;
  const int32_t* part_order;  // walk plans: dispatch slot -> partition (null: identity)
  // plans with long-row tiles, when the tiles run for this k (else null / 0):
  // the first n_dispatch slots of part_order are the partitions the tiles
  // leave (the tiles zero the others' carries), and the masks of the
  // partitions a tile row starts or ends in (entries outside
  // [mask_end[p], mask_start[p]) belong to the tiles)
  int32_t n_dispatch;
  const int32_t* mask_end;
  const int32_t* mask_start;
};

// Long-row tiles of a multi-vector product: a tile is one sub-block of
// bck X rows (k-wide, staged in LDS, at most kSpmmTileBytes) and the
// segments of up to kSpmmTileWaves x 32 tile rows in it (8, 16 or 32 a
// wave: the most that leaves kSpmmTileMinGrid tiles). Sub-blocks split the plan's
// SpMV column blocks (bc columns) in m equal parts, m dividing kTileSub, so
// their bounds are among the plan's quarter-block bounds.
constexpr int kSpmmTileBytes = 65536;
constexpr int kSpmmTileWaves = 8;       // waves of one SpMM tile workgroup (two fit a CU)
constexpr int kSpmmTileMinGrid = 1024;  // tiles wanted before a tile takes more rows
template <typename V>
struct SpmmTileArgs {
  const int32_t* rows;        // plan: kTileRowInts per tile row
  const int32_t* seg;         // plan: n_rows x (nb kTileSub + 1) quarter-block bounds
  const int32_t* col_idx;
  const V* val;
  const V* X;
  V* Y;
  V* partial;                 // workspace: n_rows x nb m x k
  V* carry_vec;               // the merge kernel's carries (P x k): the tiles zero
                              // those of the partitions they cover
  const int32_t* skip;        // plan: per partition, 1 where the walk skips it
  int64_t ldx, ldy;
  V alpha;
  int32_t k;
  int32_t n_rows;
  int32_t nb, m, bc, bck;     // SpMV blocks, sub-blocks per block, their widths (columns)
  int32_t ngroups;            // row groups of one tile (set by launch_spmm_tiles)
  int32_t N;
  int32_t nnz;
  int32_t x_dma;              // X rows contiguous (ldx == k) and 16-byte aligned
};
// Sub-blocks per SpMV block for k columns of vbytes each: the power of two m
// with bc / m X rows in kSpmmTileBytes; 0 when the tiles do not apply (k
// not a multiple of a 16-byte lane, or X rows wider than 32 bytes).
int spmm_tile_split(int k, int vbytes, int bc);
template <typename V>
size_t spmm_tile_workspace(int n_rows, int nb, int m, int k);
// The tiles (before the merge kernel, whose fix-up reads the carries they
// zero), and, after the merge kernel (launched without its fix-up), the
// fix-up and the reduction of the partials into Y in one launch.
template <typename V>
hipError_t launch_spmm_tiles(const SpmmTileArgs<V>& t, hipStream_t s);
template <typename V>
hipError_t launch_spmm_fixup_tile_reduce(const SpmmArgs<V>& a, const SpmmTileArgs<V>& t,
                                         hipStream_t s);

// Staging room per array for partitions of T units (at most T + T/8 rows or
// nonzeros, plus quad alignment).
constexpr int spmm_stage_cap(int T) { return T + T / 8 + 8; }

// ev0/ev1 (either may be null) are recorded by the main kernel's dispatch;
// fixup false leaves the carry fix-up to launch_spmm_fixup_tile_reduce
template <typename V>
hipError_t launch_spmm(const SpmmArgs<V>& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1,
                       bool fixup = true);

// ---- group-mapped exec ----------------------------------------------------------------
constexpr int kGroupRowsPerWave = 256;  // rows (tiles) a group may take, per wavefront
constexpr int kGroupChunkPerWave = 512; // nonzeros per LDS chunk, per wavefront
template <typename V>
struct GroupArgs {
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const V* val;
  const V* x;
  V* y;
  V alpha;
  V beta;
  int32_t beta_nonzero;
  int32_t M;
  int32_t rows_per_group;   // 1..kGroupRowsPerWave * wavefronts per group
};
template <typename V>
hipError_t launch_group(const GroupArgs<V>& a, int group_waves, hipStream_t s, hipEvent_t ev0,
                        hipEvent_t ev1);

// ---- row-grouped CSR --------------------------------------------------------------
template <typename V>
struct RgArgs {
  const int32_t* rl;       // entries per row
  const int64_t* base;     // first slot of each group
  const int32_t* col;      // column-interleaved column indices
  const V* val;            // and values
  const V* x;
  V* y;
  V alpha;
  V beta;
  int32_t beta_nonzero;
  int32_t M;
  int32_t G;               // rows per group
};
// group widths gw[ceil(M/G)], group bases base[ngroups + 1] (the last the
// total slots) and *stored += sum of width x rows over groups
hipError_t launch_rg_widths(const int32_t* row_ptr, int64_t M, int32_t G, int32_t* gw,
                            int64_t* base, unsigned long long* stored, hipStream_t s);
// row lengths and the column-interleaved copy of col_idx / values
hipError_t launch_rg_build(const int32_t* row_ptr, const int32_t* col_idx, const void* values,
                           int vbytes, int64_t M, int32_t G, int32_t* gw, int64_t* base,
                           int32_t* rl, int32_t* col_rg, void* val_rg, hipStream_t s);
template <typename V>
hipError_t launch_rg_spmv(const RgArgs<V>& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);

// ---- binned exec ----------------------------------------------------------------
struct BinLaunch {
  int32_t block_begin;   // first workgroup of this bin in the fused grid
  int32_t n_blocks;
  int32_t row_begin;     // first entry of this bin in the row-id array
  int32_t n_rows;
  int32_t lanes;         // lanes per row: 1..64 (power of two) or 256
  int32_t pad[3];
};

template <typename V>
struct BinnedArgs {
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const V* val;
  const V* x;
  V* y;
  const int32_t* bins;   // row ids grouped by bin; unused when identity
  V alpha;
  V beta;
  int32_t beta_nonzero;
  int32_t identity;
  int32_t n_launch;
  int32_t xcd_remap;
  int32_t nnz;           // the arrays' length (their last quad may be partial)
  BinLaunch bin[kMaxBins];
};

template <typename V>
hipError_t launch_binned(const BinnedArgs<V>& a, int total_blocks, hipStream_t s,
                         hipEvent_t ev0, hipEvent_t ev1);

}  // namespace spmv
