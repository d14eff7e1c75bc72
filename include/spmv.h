/*
 * spmv.h -- C ABI of libspmv.so: load-balanced CSR sparse matrix-vector
 * multiplication y = alpha*A*x + beta*y on one AMD Instinct MI355X (gfx950).
 *
 * Sources of the operation (the pages this library is written from):
 *  - CSR storage: "New Row-grouped CSR format for storing the sparse matrices
 *    on GPU with implementation in CUDA" (arXiv 1012.2270), Section 3 and its
 *    Fig. 1: row pointers with M+1 entries whose last entry is nnz; values and
 *    column indices with nnz entries each, stored row after row; 32-bit
 *    integer indices (its peak-performance estimate, Table 1).
 *  - The product itself: the same page, Section 3 (sequential CSR loop), and
 *    "A Programming Model for GPU Load Balancing" (Osama, Porumbescu, Owens,
 *    PPoPP'23), Section 4.3, Listing 3 (sum of a row's atoms, then y[row]).
 *  - The alpha/beta form: "Accelerating Sparse Approximate Matrix
 *    Multiplication on GPUs" (arXiv 2103.13042), background section, which
 *    states its product in the BLAS form C = alpha*A*B + beta*C.
 *  - Load balance: the PPoPP'23 page, Section 5.2.1 (merge-path: every row
 *    and every nonzero is one unit of work; the units are split evenly and
 *    each worker finds its start by a 2-D binary search) and Sidebar 1 (the
 *    segmented fix-up of rows split between workers); Sections 5.2.2 and 4.2
 *    (warp/block-mapped and thread-mapped schedules); and "OpSparse: a Highly
 *    Optimized Framework for Sparse General Matrix Multiplication on GPUs"
 *    (arXiv 2206.07244), Section 5.1 (two-pass binning with shared-memory
 *    counters, exclusive sum, and the all-rows-in-one-bin fast path) and its
 *    advice to allocate all metadata with one allocation.
 *
 * Conventions shared by every entry point:
 *  - Every pointer named "device" is a device (HBM) pointer owned by the
 *    caller; every pointer named "host" is ordinary host memory.
 *  - Indices are 0-based int32. Values and vectors are fp32 or fp64
 *    (all of one plan use the same dtype).
 *  - No function throws; each returns an spmv_status_t. On failure nothing
 *    stays allocated and *out handles are set to NULL. spmv_last_error()
 *    gives a thread-local text with the detail of the last failure.
 *  - beta == 0 means y is write-only: it is never read, so it may hold NaN.
 *  - Nothing here allocates device memory after a plan is built; the
 *    spmv_plan_copy_* calls copy to host memory the caller provides.
 *  - Where no page defines a point (error codes, introspection), the
 *    declaration says "library convention".
 *
 * Environment (read at plan time; an explicit option wins; for tuning and
 * tests, never needed for correct results):
 *   SPMV_STRATEGY=merge|binned|group   schedule when options leave it AUTO
 *   SPMV_ITEMS_PER_THREAD=4|7|8|16     merge-path items per lane
 *   SPMV_MERGE_REDUCE=walk|stream      merge-path reduction
 *   SPMV_STREAM_LANES=G                lanes per row in the stream reduction
 *   SPMV_X_WINDOW=0|1                  stream kernel's x window off / on
 *   SPMV_DISPATCH_ORDER=partition|column   walk kernel's partition order
 *   SPMV_BIN_STREAMS=n                 binned schedule: launches per bin
 *   SPMV_XCD_REMAP=0                   plain workgroup order (default 1:
 *                                      each XCD takes a contiguous run)
 *   SPMV_VALIDATE=1                    check 0 <= col_idx < N at plan time
 *   SPMV_LOG=1                         one line per plan on stderr
 *   SPMV_TEST_FAIL_ALLOC=1             make the workspace allocation fail
 *                                      (tests of the error path)
 *   SPMV_TEST_FAIL_ALLOC=2             make the x-slab copy's allocation
 *                                      fail (the plan is made without it)
 */
#ifndef SPMV_H_
#define SPMV_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPMV_API __attribute__((visibility("default")))

typedef enum spmv_status {
  SPMV_SUCCESS = 0,
  SPMV_ERR_INVALID_ARG = 1,    /* null/aliased pointer, negative size, nnz
                                  beyond int32 indices, bad enum */
  SPMV_ERR_UNSUPPORTED = 2,    /* M or N beyond int32 indices, or M + nnz
                                  beyond the int32 item model (spmv_plan) */
  SPMV_ERR_ALLOC = 3,          /* a plan-time device allocation failed (the
                                  workspace, or a copy a plan_* call owns) */
  SPMV_ERR_HIP = 4,            /* a HIP launch or runtime call failed */
  SPMV_ERR_INVALID_PLAN = 5,   /* NULL, destroyed or foreign handle */
  SPMV_ERR_INVALID_MATRIX = 6  /* row_ptr (or, when validated, col_idx) malformed */
} spmv_status_t;

typedef enum spmv_dtype { SPMV_F32 = 0, SPMV_F64 = 1 } spmv_dtype_t;

/* Execution schedules.
 *  MERGE : merge-path over the M + nnz work items (PPoPP'23 page, Sec. 5.2.1),
 *          one partition of T items per 64-lane wavefront, plus a carry fix-up.
 *  BINNED: rows grouped into row-length bins (OpSparse, Sec. 5.1); each bin
 *          runs a thread-, lane-group-, wavefront- or workgroup-per-row variant
 *          (PPoPP'23 page, Secs. 4.2 and 5.2.2), longest bins dispatched first.
 *  AUTO  : the planner picks MERGE or BINNED from the matrix size and row
 *          lengths (a switch fitted on MI355X: BINNED below 3,000,000
 *          nonzeros when some row is longer than T/8, below 2,000,000 when
 *          none is and T = 1024; MERGE above, and whenever every row fits
 *          T/8 with T = 256). */
typedef enum spmv_strategy {
  SPMV_STRATEGY_AUTO = 0,
  SPMV_STRATEGY_MERGE = 1,
  SPMV_STRATEGY_BINNED = 2,
  SPMV_STRATEGY_RGCSR = 3,    /* row-grouped CSR copy (spmv_plan_rgcsr only) */
  SPMV_STRATEGY_GROUP = 4     /* group-mapped (PPoPP'23 page, Sec. 5.2.3): a
                                 workgroup of 1, 2 or 4 wavefronts takes an
                                 equal share of rows; its threads take the
                                 share's nonzeros in turn, each finding its
                                 row by a binary search in the rows' prefix
                                 sum (spmv_plan_set_group) */
} spmv_strategy_t;

#define SPMV_MAX_BINS 8

typedef struct spmv_plan_st* spmv_plan_t;

/* Optional planning parameters (spmv_plan_ex). Zero-initialise and set only
 * what you need; a zero field means "library default". Results never depend
 * on these values, only speed does. */
typedef struct spmv_plan_options {
  int32_t strategy;           /* spmv_strategy_t; 0 = AUTO (env SPMV_STRATEGY
                                 = auto|merge|binned overrides AUTO) */
  int32_t items_per_thread;   /* merge-path items per lane: 4, 7, 8 or 16;
                                 T = 64 * items_per_thread items per wavefront.
                                 0: env SPMV_ITEMS_PER_THREAD, else chosen from
                                 the row lengths: 4 when every row has <= 32
                                 entries and the mean is < 12, otherwise 16
                                 (fp32) or 8 (fp64) -- but 4 again when rows
                                 cross those partitions, x is larger than
                                 4 MiB (one XCD's L2) and fewer than half the
                                 partitions lie inside one row */
  int32_t n_bins;             /* 1..SPMV_MAX_BINS; 0 = default bins */
  int32_t validate_columns;   /* 1: also check 0 <= col_idx < N at plan time
                                 (one pass over col_idx); env SPMV_VALIDATE=1 */
  int32_t merge_reduce;       /* how a merge-path partition sums its rows:
                                 0 auto, 1 walk (exact merge-path split, per-lane
                                 walk, carries + fix-up), 2 stream (only when every
                                 row has <= T/8 entries: partitions end at row
                                 starts, no carries) */
  int32_t stream_lanes;       /* stream reduction: lanes per row, 1..64 power
                                 of two; 0 = from the mean row length */
  int32_t x_window;           /* stream reduction: 0 auto, 1 off, 2 on. On, each
                                 workgroup of 4 partitions copies the x entries
                                 its quads use into LDS, as one column interval
                                 or, when the columns form separate bands (a
                                 stencil), up to three, when they fit the LDS
                                 the staging buffers leave at full occupancy
                                 (none for fp64 with items_per_thread >= 8),
                                 and gathers from there; a wave with a column
                                 outside them gathers from global x. Auto: on
                                 when at least half the workgroups fit. Needs a
                                 16-byte aligned x at exec time (else off) */
  int32_t bin_streams;        /* binned schedule: 0 = all bins in one grid,
                                 longest rows first (default; env
                                 SPMV_BIN_STREAMS). n in 1..SPMV_MAX_BINS: one
                                 launch per bin, longest first, dealt round
                                 robin over the caller's stream and n - 1
                                 streams the plan creates (OpSparse page,
                                 Sec. 5.1, runs its bins on concurrent
                                 streams); spmv_exec forks them from the
                                 caller's stream and joins them back with
                                 events, so the call stays asynchronous and
                                 capturable. Same per-row arithmetic, so y is
                                 bitwise equal to the single-grid result. */
  int64_t bin_max_len[SPMV_MAX_BINS];
                              /* inclusive upper row length of bins 0..n_bins-2,
                                 strictly increasing; the last bin is unbounded */
  int32_t bin_lanes[SPMV_MAX_BINS];
                              /* lanes per row of each bin: 1,2,4,...,64, or 256
                                 (one 256-thread workgroup per row) */
  int32_t dispatch_order;     /* merge-path with the walk reduction: the order
                                 in which partitions are dealt to wavefronts.
                                 0 auto (env SPMV_DISPATCH_ORDER =
                                 partition|column; else column order when at
                                 least 1/8 of the partitions lie inside one
                                 row and every row has < N/4 entries),
                                 1 partition order, 2 column
                                 order: partitions sorted by the column of
                                 their middle nonzero, so the four waves of a
                                 workgroup gather over the same columns (long
                                 rows: parts of different rows) and each XCD,
                                 which takes a contiguous run of workgroups,
                                 from a narrow part of x. Same partitions,
                                 carries and fix-up: y is bitwise equal
                                 either way. */
  int32_t long_row_tiles;     /* merge-path walk plans: 0 auto, 1 off (env
                                 SPMV_TILES=0). Auto: the interior nonzeros
                                 of rows long enough to hold, on average,
                                 >= 64 nonzeros per block of 16 KiB of x
                                 (4096 fp32 / 2048 fp64 columns) are summed
                                 by column-blocked tiles (x staged in LDS)
                                 instead of the walk kernel; needs x larger
                                 than one block and the partition order */
  int32_t x_slabs;            /* merge-path: 0 auto, 1 off, 2 on (env
                                 SPMV_X_SLABS = 0 / 1). The columns are cut
                                 into 8 slabs, one per XCD, and the plan keeps
                                 a copy of A ordered slab-major (each row's run
                                 of entries in slab 0, for every row, then
                                 slab 1, ...): the walk over that copy hands
                                 each XCD the partitions of one slab, so its
                                 gathers stay within an eighth of x, and a
                                 final kernel adds each row's slab sums in slab
                                 order. Auto (only with static_matrix below,
                                 as the copy holds A's columns and values of
                                 plan time): plans whose gathers spread over
                                 an x larger than 4 MiB (one XCD's L2) -- walk
                                 plans split again at T = 256 (their
                                 partitions mostly hold row ends), stream
                                 plans whose workgroups' columns fit no x
                                 window (x_window above) -- or over an x of
                                 1..4 MiB whose rows average at least
                                 1e8 / (x bytes) entries (walk plans with
                                 partitions mostly holding row ends, the same
                                 stream plans); on:
                                 every plan. Either way only MERGE plans that
                                 keep no long-row tiles (those win where both
                                 apply). Each row's entries are
                                 cut into slab runs by binary search over its
                                 columns: results are right in any column
                                 order, but the x locality needs the columns
                                 sorted within rows, so auto keeps no slabs
                                 when a run's middle entry lies outside its
                                 slab or below the entry before it. Costs a
                                 second allocation
                                 the size of A. The
                                 copy holds A's values as they were at plan
                                 time: call spmv_plan_update_values after
                                 changing them (spmv_plan_info.x_slabs tells
                                 whether the plan took slabs). */
  int32_t static_matrix;      /* 0 (default): the plan borrows row_ptr,
                                 col_idx and values, and the contents of
                                 col_idx and values may change between
                                 spmv_exec calls (row_ptr may not). 1: the
                                 caller keeps col_idx and values as they are
                                 at plan time, or changes values only through
                                 spmv_plan_update_values; the plan may then
                                 hold a copy of A in another layout (x slabs,
                                 auto). */
} spmv_plan_options_t;

typedef struct spmv_plan_info {
  int64_t M, N, nnz;
  int32_t dtype;              /* spmv_dtype_t */
  int32_t strategy;           /* the schedule spmv_exec runs (never AUTO) */
  int32_t items_per_thread;
  int32_t items_per_wave;     /* T */
  int64_t n_partitions;       /* P = ceil((M + nnz) / T) */
  int32_t merge_reduce;       /* 1 walk, 2 stream */
  int32_t stream_lanes;
  int32_t x_window;           /* stream kernel's LDS x window: 0 none, 1 one
                                 column interval, 3 up to three */
  int32_t bin_streams;        /* binned exec: streams its per-bin launches use
                                 (0: one grid for all bins) */
  int32_t n_bins;
  int32_t bin_identity;       /* 1: every row fell in one bin, no row-id array */
  int64_t bin_max_len[SPMV_MAX_BINS];
  int32_t bin_lanes[SPMV_MAX_BINS];
  int64_t bin_count[SPMV_MAX_BINS];
  int64_t max_row_len;
  int64_t n_empty_rows;
  int64_t workspace_bytes;    /* size of the plan's single device allocation */
  int32_t rgcsr_group;        /* rows per group of the row-grouped copy (0: none) */
  int32_t pad1;
  int64_t rgcsr_stored;       /* entries that copy stores for existing rows
                                 (group width x rows, summed): nnz + padding */
  int32_t group_waves;        /* group-mapped schedule: wavefronts per group */
  int32_t group_rows;         /* ... and rows per group */
  int32_t dispatch_order;     /* walk kernel's partition order: 1 partition,
                                 2 column (spmv_exec_multi follows it when at
                                 least half the partitions are interior) */
  int32_t interior_partitions;  /* partitions no row ends in */
  int32_t plan_allocs;        /* device allocations the plan's construction
                                 made (1 for spmv_plan / _ex / _coo) */
  int32_t plan_syncs;         /* host synchronisations it made (1 for
                                 spmv_plan / _ex / _coo) */
  int32_t tile_rows;          /* long rows summed by column-blocked tiles */
  int32_t tile_blocks;        /* column blocks of those tiles */
  int32_t walk_partitions;    /* partitions the walk kernel runs (P without
                                 tiles; those the tiles leave with them) */
  int32_t x_slabs;            /* 1: spmv_exec walks the plan's slab-major copy
                                 of A (options.x_slabs) */
  int64_t slab_segments;      /* that copy's (row, slab) runs: its rows */
  int64_t slab_bytes;         /* size of the copy's allocation (0: none) */
} spmv_plan_info_t;

/* Build a plan for the CSR matrix A (M x N, nnz stored entries).
 * Sources: CSR as the RgCSR page, Section 3 and Fig. 1, defines it (row
 * pointers ending in nnz, 32-bit indices); the plan's steps are the PPoPP'23
 * page's Section 5.2.1 (merge-path split of rows + nonzeros, one binary
 * search per partition) and the OpSparse page's Section 5.1 (row-length bins
 * counted in shared memory, exclusive sum, scatter; one allocation for all
 * metadata, no synchronisation mid-pipeline).
 *
 * row_ptr  device int32[M+1]; row_ptr[0] == 0, non-decreasing,
 *          row_ptr[M] == nnz (RgCSR page, Sec. 3). Checked on the device;
 *          a violation returns SPMV_ERR_INVALID_MATRIX.
 * col_idx  device int32[nnz], each in [0, N). Any order within a row;
 *          repeated columns add up. Checked only with validate_columns.
 * values   device fp32[nnz] or fp64[nnz] per dtype.
 * stream   the HIP stream the planning kernels run on (0 = null stream).
 *
 * Ownership: the plan borrows row_ptr, col_idx and values; they must stay
 * allocated until spmv_destroy, and row_ptr must stay unchanged (the plan's
 * partition and bins are derived from it). col_idx and values may change
 * between spmv_exec calls (the plan samples col_idx once to choose a kernel
 * variant; results never depend on that choice). row_ptr, col_idx and values
 * must be 16-byte aligned (any hipMalloc allocation is), else
 * SPMV_ERR_INVALID_ARG. The plan owns one device workspace (all of its
 * metadata, the column dispatch order included), plus the streams and events
 * of per-bin launches when asked for; all are made here and freed by
 * spmv_destroy.
 *
 * Work, all enqueued on `stream` back to back: row-length statistics and
 * per-workgroup bin counts kept in LDS, an exclusive scan of the bin counts,
 * a stable scatter of row ids into bins, the partition size chosen on the
 * device from the counted rows, one merge-path binary search per wavefront
 * partition (a second pass at T = 256 when the device decides so), the
 * stream workgroups' x windows, and for walk plans that take the column
 * dispatch order the partitions' keys and a radix sort of them. Then one
 * device-to-host copy of a small statistics block and one stream
 * synchronisation: exactly one allocation and one synchronisation
 * (spmv_plan_info reports both). Errors: SPMV_ERR_INVALID_ARG for a NULL
 * out, a NULL or misaligned array, a negative size or nnz > 2^31 - 1;
 * SPMV_ERR_UNSUPPORTED for M >= 2^31 - 1, N > 2^31 - 1 or
 * M + nnz > 2^31 - 65 (the kernels keep 64 units of int32 headroom past the
 * last one); SPMV_ERR_ALLOC when the workspace allocation fails;
 * SPMV_ERR_INVALID_MATRIX as above. M == 0 or nnz == 0 is allowed. */
SPMV_API spmv_status_t spmv_plan(spmv_plan_t* out, int64_t M, int64_t N, int64_t nnz,
                        const int32_t* row_ptr, const int32_t* col_idx,
                        const void* values, spmv_dtype_t dtype,
                        hipStream_t stream);

/* spmv_plan with explicit options (NULL = defaults). */
SPMV_API spmv_status_t spmv_plan_ex(spmv_plan_t* out, int64_t M, int64_t N, int64_t nnz,
                           const int32_t* row_ptr, const int32_t* col_idx,
                           const void* values, spmv_dtype_t dtype,
                           const spmv_plan_options_t* options,
                           hipStream_t stream);

/* Build a plan for A given in COO form: entry e is (row_idx[e], col_idx[e],
 * values[e]), e < nnz, sorted by row (non-decreasing row_idx; any order
 * within a row, repeated positions add up). "A Programming Model for GPU
 * Load Balancing" (PPoPP'23), Section 3.1: the same atoms (nonzeros) and
 * tiles (rows) as CSR, named by a row index per atom. The plan derives the
 * CSR row offsets on the device (row r starts at the first entry whose row
 * index is >= r), keeps them in an allocation of its own, and then plans and
 * executes exactly as spmv_plan_ex would; spmv_exec and spmv_exec_multi
 * apply unchanged.
 *
 * row_idx  device int32[nnz], each in [0, M), sorted; read only during this
 *          call (it may be freed afterwards). Out of range or out of order
 *          gives SPMV_ERR_INVALID_MATRIX (checked on the device).
 * col_idx, values, dtype, options, stream: as for spmv_plan_ex (borrowed).
 * The row offsets live in the plan's one workspace; the order check joins
 * the plan's statistics, so this too makes one allocation and one
 * synchronisation. */
SPMV_API spmv_status_t spmv_plan_coo(spmv_plan_t* out, int64_t M, int64_t N, int64_t nnz,
                                     const int32_t* row_idx, const int32_t* col_idx,
                                     const void* values, spmv_dtype_t dtype,
                                     const spmv_plan_options_t* options, hipStream_t stream);

/* Build a plan whose spmv_exec computes y = alpha * A^T * x + beta * y for
 * the CSR matrix A (M x N): x has M entries, y has N; the plan's shape is
 * N x M. The transpose is built once here: a stable device radix sort of
 * the column indices with their entry positions, then A^T's column indices
 * (A's rows) and values gathered in that order, which is CSR of A^T with
 * each row's entries in ascending column order; its row offsets are
 * derived as for spmv_plan_coo. "A Programming Model for GPU Load
 * Balancing" (PPoPP'23), Section 3.1 (atoms and tiles of a CSC layout).
 * Then it plans and executes as spmv_plan_ex would (spmv_exec_multi too).
 *
 * row_ptr, col_idx, values, dtype, options, stream: A as for spmv_plan_ex;
 * all three are read only during this call. The plan keeps its own copy of
 * A^T's indices and values (nnz * (4 + value size) bytes plus the offsets,
 * in its one workspace), so later changes to A's values do not reach it.
 * SPMV_ERR_INVALID_MATRIX when row_ptr is malformed or a column index is
 * outside [0, N). The sort's scratch (about 16 * nnz bytes) is a second
 * allocation, freed before the call returns, after one more stream
 * synchronisation (two allocations and two synchronisations in all). The
 * sort is the library's own (sort_kernels.hip: LSD radix, 8-bit digits,
 * stable). */
SPMV_API spmv_status_t spmv_plan_transpose(spmv_plan_t* out, int64_t M, int64_t N,
                                           int64_t nnz, const int32_t* row_ptr,
                                           const int32_t* col_idx, const void* values,
                                           spmv_dtype_t dtype,
                                           const spmv_plan_options_t* options,
                                           hipStream_t stream);

/* Build a plan for y = alpha * A * x + beta * y with A (M x N) given in CSC:
 * col_ptr int32[N+1], row_idx int32[nnz] (each in [0, M)), values[nnz]. The
 * CSC arrays of A are the CSR arrays of A^T, so this is
 * spmv_plan_transpose of that N x M matrix; the same copies, checks and
 * errors apply. */
SPMV_API spmv_status_t spmv_plan_csc(spmv_plan_t* out, int64_t M, int64_t N, int64_t nnz,
                                     const int32_t* col_ptr, const int32_t* row_idx,
                                     const void* values, spmv_dtype_t dtype,
                                     const spmv_plan_options_t* options, hipStream_t stream);

/* spmv_plan_ex, then a row-grouped CSR copy of A that spmv_exec uses
 * ("New Row-grouped CSR format for storing the sparse matrices on GPU with
 * implementation in CUDA", arXiv 1012.2270, Section 4): rows in groups of
 * group_rows consecutive rows; inside a group, entry k of the group's row i
 * is stored at groupPointers[group] + k * group_rows + i, to the width of
 * the group's longest row (shorter rows padded with value 0), with the row
 * lengths beside. One lane per row, the group's lanes reading consecutive
 * addresses.
 *
 * group_rows  1..1024; 0 = 64 (one wavefront).
 * The copy is taken here: later changes to values do not reach spmv_exec
 * while the plan's strategy is SPMV_STRATEGY_RGCSR (spmv_plan_set_strategy
 * may switch it to MERGE or BINNED, which read the borrowed arrays, and
 * back). It is kept in one more device allocation of about
 * rgcsr_stored * (4 + value size) bytes (spmv_plan_info), freed by
 * spmv_destroy. spmv_exec_multi uses the merge-path partitions as always. */
SPMV_API spmv_status_t spmv_plan_rgcsr(spmv_plan_t* out, int64_t M, int64_t N, int64_t nnz,
                                       const int32_t* row_ptr, const int32_t* col_idx,
                                       const void* values, spmv_dtype_t dtype,
                                       int32_t group_rows, hipStream_t stream);

/* y = alpha * A * x + beta * y.
 * Sources: the product of the RgCSR page, Section 3 (sequential CSR loop,
 * 2 flops per stored entry) and the PPoPP'23 page, Section 4.3, Listing 3
 * (each row's atoms summed, then y[row] written), load-balanced as its
 * Section 5.2.1 and Sidebar 1 describe (merge-path partitions, segmented
 * fix-up of rows cut between them); the alpha/beta form is the SpAMM page's
 * background section (C = alpha A B + beta C).
 *
 * x  device array of N elements of the plan's dtype.
 * y  device array of M elements; read only when beta != 0. The byte ranges
 *    of x and y must not overlap (SPMV_ERR_INVALID_ARG).
 * alpha, beta are converted once to the plan's dtype.
 *
 * Asynchronous: only enqueues work on stream (with per-bin launches, event
 * records and waits that fork the plan's streams from it and join them back);
 * never allocates, frees or synchronises, so it can be captured in a HIP
 * graph. Rows with no entries give exactly beta*y (0 when beta == 0). For a
 * fixed plan the result is bitwise reproducible (no float atomics). One plan
 * must not run concurrently on two streams (its carry buffer, its x slabs'
 * segment sums and its events are per plan); distinct plans are
 * independent. A plan with x slabs (options.x_slabs) runs the walk over its
 * slab-major copy, its fix-up and a combine of each row's slab sums: three
 * launches, all on stream. */
SPMV_API spmv_status_t spmv_exec(spmv_plan_t plan, const void* x, void* y,
                        double alpha, double beta, hipStream_t stream);

/* Library convention (measurement): spmv_exec that also has the dispatch of
 * the dominant kernel (the
 * merge-path main kernel, the fused binned kernel, the group-mapped or the
 * row-grouped kernel) record ev_begin at its start and ev_end at its end, on
 * the same stream, so a caller can time that kernel alone. With bins on
 * several streams they bracket the fork and the join instead. Either event
 * may be NULL; a call with M = 0 launches nothing and records neither. */
SPMV_API spmv_status_t spmv_exec_events(spmv_plan_t plan, const void* x, void* y,
                               double alpha, double beta, hipStream_t stream,
                               hipEvent_t ev_begin, hipEvent_t ev_end);

/* Multi-vector SpMV (SpMM) over the same plan: Y = alpha * A * X + beta * Y
 * for k right-hand sides. "A Programming Model for GPU Load Balancing"
 * (PPoPP'23), Section 5.3, Listing 4: the SpMV with a loop over the dense
 * matrix's columns, column c of Y from column c of X.
 *
 * X  device array, N x k row-major of the plan's dtype: X[j*ldx + c]; ldx >= k.
 * Y  device array, M x k row-major: Y[i*ldy + c]; ldy >= k; read only when
 *    beta != 0. X and Y must not overlap; both aligned to the element size.
 * workspace, workspace_bytes: device memory of at least
 *    spmv_spmm_workspace_size(plan, k) bytes for the k-wide carries of rows
 *    cut between partitions (0 bytes, NULL allowed, when the plan's
 *    partitions end at row ends: merge_reduce = stream), plus, on a plan
 *    with long-row tiles and X rows of 16 or 32 bytes, the tiles' partial
 *    sums per row, X sub-block and column. Owned by the caller; its
 *    contents need no initialisation and are scratch after the call.
 *    (The tiles run when X and Y are 16-byte aligned and ldx, ldy and k
 *    are whole 16-byte lanes; otherwise the merge-path walk takes every
 *    row. Results differ by rounding order only.)
 * k = 0 or M = 0 does nothing. k > 64 runs in column blocks of 64. k = 1
 * with ldx = ldy = 1 is an SpMV and runs as spmv_exec (the plan's strategy,
 * tiles and x slabs; the workspace is then not touched).
 *
 * Otherwise uses the plan's merge-path partitions whatever its SpMV
 * strategy.
 * Asynchronous like spmv_exec (no allocation, no synchronisation);
 * bitwise reproducible for a fixed plan and k; the plan's carry-row array
 * is shared with spmv_exec, so one plan must not run either call
 * concurrently on two streams. SPMV_ERR_INVALID_ARG on a bad size, pointer,
 * overlap or short workspace. */
SPMV_API spmv_status_t spmv_spmm_workspace_size(spmv_plan_t plan, int64_t k, size_t* bytes);
SPMV_API spmv_status_t spmv_exec_multi(spmv_plan_t plan, int64_t k, const void* X,
                                       int64_t ldx, void* Y, int64_t ldy, double alpha,
                                       double beta, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/* spmv_exec_multi that also records ev_begin and ev_end on the same stream:
 * for k <= 64 the main kernel's dispatch records them at its start and end
 * (the carry fix-up that follows is outside); for k > 64, and when the
 * long-row tiles run, they bracket every launch of the call. Either event may be NULL; a call with k = 0 or M = 0
 * launches nothing and records neither. */
SPMV_API spmv_status_t spmv_exec_multi_events(spmv_plan_t plan, int64_t k, const void* X,
                                              int64_t ldx, void* Y, int64_t ldy, double alpha,
                                              double beta, void* workspace,
                                              size_t workspace_bytes, hipStream_t stream,
                                              hipEvent_t ev_begin, hipEvent_t ev_end);

/* Release the plan's workspace (hipFree, which synchronises the device).
 * The OpSparse page, Section 5.1, frees its metadata only at the end of the
 * pipeline, since a free synchronises; the plan's memory is freed here and
 * nowhere else. NULL is a no-op; a destroyed or foreign handle gives
 * SPMV_ERR_INVALID_PLAN (library convention: live handles are tracked, so a
 * stale one is never dereferenced). */
SPMV_API spmv_status_t spmv_destroy(spmv_plan_t plan);

/* Library convention (the inspector-executor pattern: a plan may hold a
 * copy of A made in its own layout): make the plan use `values` (device,
 * fp32 or fp64 per the plan's dtype, nnz entries in the layout of the values
 * given to spmv_plan / _ex / _coo, 16-byte aligned; the same array after its
 * contents changed, or another one, which the plan then borrows) from the
 * next spmv_exec on. Plans with x slabs (spmv_plan_info.x_slabs) rewrite
 * their slab-major copy on `stream`, asynchronously; an exec of the plan on
 * another stream must not overlap it. Other plans read values at every exec
 * and only store the pointer. Errors: INVALID_PLAN; INVALID_ARG for a NULL
 * (nnz > 0) or misaligned pointer; UNSUPPORTED for transposed, CSC and
 * row-grouped plans (their copies are in another layout: plan again). */
SPMV_API spmv_status_t spmv_plan_update_values(spmv_plan_t plan, const void* values,
                                               hipStream_t stream);

/* Switch a live plan between MERGE (PPoPP'23 page, Sec. 5.2.1) and BINNED
 * (OpSparse page, Sec. 5.1; PPoPP'23 page, Secs. 4.2 and 5.2.2) -- both are
 * always built -- or to RGCSR when the plan has the row-grouped copy (RgCSR
 * page, Sec. 4). Library convention: SPMV_ERR_INVALID_ARG for an unknown
 * strategy or RGCSR without the copy. */
SPMV_API spmv_status_t spmv_plan_set_strategy(spmv_plan_t plan, spmv_strategy_t strategy);

/* Select the group-mapped schedule (SPMV_STRATEGY_GROUP) for a live plan:
 * group_waves 1, 2 or 4 wavefronts per group (0 = 4), rows_per_group
 * 1..256 * group_waves (0 = 512 * group_waves nonzeros' worth of rows at the
 * mean row length). Results do not depend on either. SPMV_ERR_INVALID_ARG
 * outside those ranges. */
SPMV_API spmv_status_t spmv_plan_set_group(spmv_plan_t plan, int32_t group_waves,
                                           int32_t rows_per_group);

/* Library convention (introspection for tests and reports): fill *info
 * (host struct) with the plan's choices, sizes and bin counts.
 * SPMV_ERR_INVALID_PLAN for a dead handle, SPMV_ERR_INVALID_ARG for NULL. */
SPMV_API spmv_status_t spmv_plan_info(spmv_plan_t plan, spmv_plan_info_t* info);

/* Copy the merge-path split coordinates to host arrays of cap >= P+1 entries
 * (PPoPP'23 page, Sec. 5.2.1: the coordinates of each worker's start on the
 * merge path): rows_host[p] = rows whose end item precedes diagonal
 * min(p*T, M+nnz), nnz_host[p] = nonzeros before it. Synchronous
 * (stream-ordered on the null stream after the plan's work). Library
 * convention: SPMV_ERR_INVALID_ARG for NULL buffers or cap < P + 1. */
SPMV_API spmv_status_t spmv_plan_copy_splits(spmv_plan_t plan, int32_t* rows_host,
                                    int32_t* nnz_host, int64_t cap);

/* Copy the binning result to host (OpSparse page, Sec. 5.1: the row ids
 * grouped by bin and the bins' offsets from the exclusive sum):
 * bins_host[M] (ascending within a bin; the identity when bin_identity is
 * set) and offsets_host[n_bins+1]. Synchronous. Library convention:
 * SPMV_ERR_INVALID_ARG for NULL buffers or bins_cap < M. */
SPMV_API spmv_status_t spmv_plan_copy_bins(spmv_plan_t plan, int32_t* bins_host,
                                  int64_t bins_cap, int64_t* offsets_host);

/* Measurement aid, not part of the SpMV: enqueue one streaming read of
 * `bytes` bytes at device pointer `data` (16-byte aligned, bytes a multiple
 * of 16, at most 2^31 - 1 workgroups' worth) on `stream`, with each 64-lane
 * wavefront loading one 4 KiB block once. Timed by the caller, it gives the
 * device's achievable read bandwidth for the same kind of access the SpMV
 * kernels make. `sink` is a device int32 that keeps the loads live: the
 * xor of a 4 KiB block is written there only if it equals 0x5bd1e995 (never,
 * for buffers of equal words). Asynchronous; SPMV_ERR_INVALID_ARG on a bad
 * pointer or size. */
SPMV_API spmv_status_t spmv_read_probe(const void* data, int64_t bytes, void* sink,
                                       hipStream_t stream);

/* Measurement aid, not part of the SpMV: read col_idx[0..nnz) once, in
 * storage order (16-byte loads, 1,024 indices per wavefront), and gather
 * x[col_idx[k]] for every k, nothing else; the x-gather cost of an SpMV of
 * that matrix, with its own column locality (the RgCSR page, Section 3,
 * counts an x element per nonzero in its bandwidth estimate; caching x is
 * what its results improve). col_idx 16-byte aligned; x of n_x elements
 * (0 < n_x < 2^32) of `dtype`; columns are clamped to [0, n_x), so any
 * col_idx is safe. `sink` (device int32) keeps the loads live. Asynchronous. */
SPMV_API spmv_status_t spmv_gather_probe(const int32_t* col_idx, int64_t nnz, const void* x,
                                         int64_t n_x, spmv_dtype_t dtype, void* sink,
                                         hipStream_t stream);

/* Measurement aid, not part of the SpMV: the X-row gathers of a
 * multi-vector product (the PPoPP'23 page, Section 5.3, Listing 4: a row of
 * the dense operand per nonzero), nothing else. Reads col_idx[0..nnz) once
 * and, for every k, the row col_idx[k] of X, a dense array of n_rows rows of
 * row_bytes bytes each (16, 32, 64, 128 or 256; rows contiguous), with
 * 16-byte lanes grouped as the SpMM kernels group them (row_bytes / 16 lanes
 * per row, 8 rows per lane group in flight). Rows are clamped to
 * [0, n_rows), so any col_idx is safe. X 16-byte aligned, 0 < n_rows < 2^32;
 * `sink` (device int32) keeps the loads live. Asynchronous;
 * SPMV_ERR_INVALID_ARG on a bad size or pointer. */
SPMV_API spmv_status_t spmv_gather_rows_probe(const int32_t* col_idx, int64_t nnz, const void* X,
                                              int64_t n_rows, int32_t row_bytes, void* sink,
                                              hipStream_t stream);

/* Measurement aid, not part of the SpMV: the merge-path kernels' access
 * pattern without x. The M + nnz units are cut into P = ceil((M + nnz) / T)
 * equal partitions, T = 64 * items_per_thread (4, 8 or 16); each 64-lane
 * wavefront streams its partition's share of row_ptr, col_idx and values
 * (16-byte non-temporal loads, all issued first, clamped to the arrays) and
 * writes its share of y (M elements of `dtype`) with a value folded from the
 * loads. Timed, it gives what plain streaming of the CSR arrays and y
 * reaches on this device. Arrays 16-byte aligned; M > 0, M + nnz < 2^31.
 * Asynchronous. */
SPMV_API spmv_status_t spmv_stream_probe(const int32_t* row_ptr, const int32_t* col_idx,
                                         const void* values, int64_t M, int64_t nnz,
                                         spmv_dtype_t dtype, int32_t items_per_thread, void* y,
                                         hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): one
 * y = alpha * A * x + beta * y with A given directly in CSR (no plan), as
 * spmv_plan_ex + spmv_exec compute it for a merge-path walk plan with
 * items_per_thread 16 (fp32) or 8 (fp64) in partition order and without
 * long-row tiles -- the same partitions, kernels and fix-up, so the same y
 * bit for bit. The split
 * coordinates and carries live in a 32 MiB device array of the library,
 * one per GPU, held until the process ends: nothing is allocated, freed or
 * synchronised, and every step is enqueued on `stream`.
 *
 * Arguments and conventions as for spmv_plan_ex and spmv_exec (row_ptr,
 * col_idx, values 16-byte aligned; x and y must not overlap; beta == 0
 * means y is not read). row_ptr is not validated (that needs a read-back);
 * a malformed row_ptr gives an undefined y but no access outside the
 * arrays' declared sizes. SPMV_ERR_UNSUPPORTED when M + nnz needs more
 * partitions than the scratch holds (about 1.19M: M + nnz up to ~1.2e9 for
 * fp32, ~0.6e9 for fp64). Calls that overlap on one GPU (two streams, or
 * two host threads) share that scratch and race: serialise them. */
SPMV_API spmv_status_t spmv_exec_noalloc(int64_t M, int64_t N, int64_t nnz,
                                         const int32_t* row_ptr, const int32_t* col_idx,
                                         const void* values, spmv_dtype_t dtype, const void* x,
                                         void* y, double alpha, double beta, hipStream_t stream);

/* Library convention: a fixed text for each status. */
SPMV_API const char* spmv_status_string(spmv_status_t status);
/* Library convention: the calling thread's text of its last failure. */
SPMV_API const char* spmv_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SPMV_H_ */
