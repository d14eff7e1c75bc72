// C ABI of libspmv.so (declared in include/spmv.h): argument checks, the
// plan's single workspace allocation, planning launches, strategy choice and
// the exec launches. No computation of the SpMV happens on the host.
#include "spmv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>
#include <new>
#include <string>
#include <unordered_set>

#include "internal.hpp"

using namespace spmv;

namespace {

constexpr uint64_t kMagic = 0x53504d5650414e31ull;  // "SPMVPAN1"
constexpr int64_t kInt32Max = 2147483647ll;
// M + nnz at most 2^31 - 65: the kernels index the quads and partition ends
// past the last unit in int32 (a quad's last entry, a lane's clamped
// start), so 64 units of headroom stay below 2^31.
constexpr int64_t kMaxUnits = kInt32Max - 64;

thread_local std::string g_last_error;

spmv_status_t fail(spmv_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
spmv_status_t fail(spmv_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

spmv_status_t hip_fail(hipError_t e, const char* where) {
  return fail(SPMV_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  return (v && *v) ? std::atoi(v) : dflt;
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Default row-length bins: inclusive upper lengths and lanes per row.
const int64_t kDefaultMaxLen[kMaxBins - 1] = {2, 8, 16, 32, 128, 512, 4096};
// measured with the quad-load row sums (laplacian, power-law, bimodal,
// banded): rows of 17..32 on 4 lanes and 33..128 on 8 beat 8 and 16
const int32_t kDefaultLanes[kMaxBins] = {1, 2, 4, 4, 8, 32, 64, 256};

}  // namespace

namespace spmv {
// other sources of the library report their failures through the same text
void set_last_error(const char* text) { g_last_error = text; }
}  // namespace spmv

struct spmv_plan_st {
  uint64_t magic;
  int64_t M, N, nnz;
  spmv_dtype_t dtype;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const void* values;

  int32_t strategy;
  int32_t ipt, T;
  int64_t P;
  int32_t xcd_remap;
  int32_t xcd_remap_stream;  // the stream kernel's workgroup order (default: plain)
  int32_t merge_reduce;     // 1 walk, 2 stream
  int32_t stream_lanes;
  int32_t x_window;

  BinEdges edges;
  int32_t lanes[kMaxBins];
  int64_t bin_offset[kMaxBins + 1];
  int32_t identity;
  int64_t max_len, n_empty;
  int32_t n_launch;
  BinLaunch launch[kMaxBins];
  int32_t binned_blocks;

  void* ws;
  size_t ws_bytes;
  int64_t* stats;
  int32_t* counts;
  int32_t* wg_max;
  int32_t* wg_empty;
  int32_t* split_row;
  int32_t* split_nz;
  int32_t* row_bounds;
  int32_t* carry_row;
  void* carry_val;
  int32_t* bins;
  int32_t* win_span;
  // row-grouped copy (spmv_plan_rgcsr): metadata and entries, own allocations
  void* owned_rg_meta;
  void* owned_rg_data;
  int32_t rg_group;
  int64_t rg_stored;
  const int32_t* rg_rl;
  const int64_t* rg_base;
  const int32_t* rg_col;
  const void* rg_val;
  int32_t group_waves;    // group-mapped schedule
  int32_t group_rows;
  // walk kernel's dispatch order (options.dispatch_order): 1 partition
  // order, 2 column order through part_order (in the workspace)
  int32_t dispatch_order;
  int64_t interior;       // partitions no row ends in
  const int32_t* part_order;
  // device allocations and host synchronisations the plan's construction made
  int32_t plan_allocs;
  int32_t plan_syncs;
  // column-blocked tiles of long rows (walk plans): tile rows, their segment
  // bounds and block partials, and the walk kernel's list of the partitions
  // the tiles leave (part_order, n_dispatch entries)
  int32_t n_tile_rows;
  int32_t tile_nb;
  int32_t n_dispatch;
  const int32_t* tile_list;
  const int32_t* tile_skip;   // per partition: 1 where the walk skips it (in win_span's room)
  const int32_t* tile_mask_end;
  const int32_t* tile_mask_start;
  const int32_t* tile_rows;
  const int32_t* tile_seg;
  void* tile_partial;
  // per-bin launches (options.bin_streams): bins dealt over the caller's
  // stream and n_side streams of the plan, forked and joined by events
  int32_t bin_streams;
  int32_t n_side;
  hipStream_t side[kMaxBins];
  hipEvent_t fork_ev;
  hipEvent_t join_ev[kMaxBins];
  // x slabs (walk plans whose x is wider than one XCD's L2): the row tables
  // (in the workspace), and in a second allocation the slab-major copy A',
  // its merge-path split and carries, and y' (one sum per segment)
  int32_t x_slabs;          // 1: spmv_exec walks A' and combines
  int32_t slab_ipt;
  int64_t slab_P;
  SlabRows slab_rows;
  SlabMatrix slab_m;
  void* owned_slab;
  size_t slab_bytes;
  int64_t* slab_stats;
  int32_t* slab_split_row;
  int32_t* slab_split_nz;
  int32_t* slab_row_bounds;
  int32_t* slab_carry_row;
  void* slab_carry_val;
  void* slab_y;
  // values held as a copy made at plan time in another layout (transposed,
  // CSC and row-grouped plans); spmv_plan_update_values refuses those
  int32_t values_copied;
};

namespace {

// Live plans. A handle is only dereferenced after it is found here, so a
// destroyed or foreign handle is rejected without touching its memory.
std::mutex g_plans_mu;
std::unordered_set<const spmv_plan_st*> g_plans;

spmv_status_t check_plan(spmv_plan_t p) {
  if (!p) return fail(SPMV_ERR_INVALID_PLAN, "plan is NULL");
  {
    std::lock_guard<std::mutex> lk(g_plans_mu);
    if (!g_plans.count(p)) return fail(SPMV_ERR_INVALID_PLAN, "not a live plan handle");
  }
  if (p->magic != kMagic) return fail(SPMV_ERR_INVALID_PLAN, "corrupted plan handle");
  return SPMV_SUCCESS;
}

spmv_status_t check_options(const spmv_plan_options_t* o) {
  if (!o) return SPMV_SUCCESS;
  if (o->strategy < 0 || o->strategy > SPMV_STRATEGY_GROUP || o->strategy == SPMV_STRATEGY_RGCSR)
    return fail(SPMV_ERR_INVALID_ARG, "options.strategy %d unknown here", o->strategy);
  if (o->items_per_thread != 0 && o->items_per_thread != 4 && o->items_per_thread != 7 &&
      o->items_per_thread != 8 && o->items_per_thread != 16)
    return fail(SPMV_ERR_INVALID_ARG, "options.items_per_thread must be 4, 7, 8 or 16");
  if (o->x_window < 0 || o->x_window > 2)
    return fail(SPMV_ERR_INVALID_ARG, "options.x_window %d unknown", o->x_window);
  if (o->merge_reduce < 0 || o->merge_reduce > 2)
    return fail(SPMV_ERR_INVALID_ARG, "options.merge_reduce %d unknown", o->merge_reduce);
  if (o->stream_lanes != 0 && (o->stream_lanes < 1 || o->stream_lanes > 64 ||
                               (o->stream_lanes & (o->stream_lanes - 1))))
    return fail(SPMV_ERR_INVALID_ARG, "options.stream_lanes must be a power of two <= 64");
  if (o->dispatch_order < 0 || o->dispatch_order > 2)
    return fail(SPMV_ERR_INVALID_ARG, "options.dispatch_order %d unknown", o->dispatch_order);
  if (o->long_row_tiles < 0 || o->long_row_tiles > 1)
    return fail(SPMV_ERR_INVALID_ARG, "options.long_row_tiles %d unknown", o->long_row_tiles);
  if (o->x_slabs < 0 || o->x_slabs > 2)
    return fail(SPMV_ERR_INVALID_ARG, "options.x_slabs %d unknown", o->x_slabs);
  if (o->static_matrix < 0 || o->static_matrix > 1)
    return fail(SPMV_ERR_INVALID_ARG, "options.static_matrix %d unknown", o->static_matrix);
  if (o->bin_streams < 0 || o->bin_streams > SPMV_MAX_BINS)
    return fail(SPMV_ERR_INVALID_ARG, "options.bin_streams must be in [0, %d]", SPMV_MAX_BINS);
  if (o->n_bins < 0 || o->n_bins > SPMV_MAX_BINS)
    return fail(SPMV_ERR_INVALID_ARG, "options.n_bins must be in [0, %d]", SPMV_MAX_BINS);
  if (o->n_bins > 0) {
    for (int b = 0; b < o->n_bins; ++b) {
      const int g = o->bin_lanes[b];
      if (!(g == 1 || g == 2 || g == 4 || g == 8 || g == 16 || g == 32 || g == 64 || g == 256))
        return fail(SPMV_ERR_INVALID_ARG, "options.bin_lanes[%d] = %d not allowed", b, g);
    }
    for (int b = 0; b + 1 < o->n_bins; ++b) {
      if (o->bin_max_len[b] < 0 || (b > 0 && o->bin_max_len[b] <= o->bin_max_len[b - 1]))
        return fail(SPMV_ERR_INVALID_ARG, "options.bin_max_len must increase strictly");
    }
  }
  return SPMV_SUCCESS;
}

// Lay out the binned grid: bins with the longest rows first.
void build_binned_launch(spmv_plan_st* p) {
  p->n_launch = 0;
  int32_t next = 0;
  for (int b = p->edges.n_bins - 1; b >= 0; --b) {
    const int64_t rows = p->bin_offset[b + 1] - p->bin_offset[b];
    if (rows == 0) continue;
    BinLaunch& L = p->launch[p->n_launch++];
    L.lanes = p->lanes[b];
    L.row_begin = (int32_t)p->bin_offset[b];
    L.n_rows = (int32_t)rows;
    const int64_t per = L.lanes >= kBlock ? 1 : kBlock / L.lanes;
    L.n_blocks = (int32_t)((rows + per - 1) / per);
    L.block_begin = next;
    next += L.n_blocks;
  }
  p->binned_blocks = next;
}

// Streams and events of the per-bin launches (none when the bins share one
// grid or there is one bin).
void release_bin_streams(spmv_plan_st* p) {
  for (int i = 0; i < p->n_side; ++i) {
    if (p->join_ev[i]) (void)hipEventDestroy(p->join_ev[i]);
    if (p->side[i]) (void)hipStreamDestroy(p->side[i]);
    p->join_ev[i] = nullptr;
    p->side[i] = nullptr;
  }
  if (p->fork_ev) (void)hipEventDestroy(p->fork_ev);
  p->fork_ev = nullptr;
  p->n_side = 0;
}

hipError_t create_bin_streams(spmv_plan_st* p) {
  const int want = std::min<int>(p->bin_streams, p->n_launch) - 1;
  if (want <= 0) return hipSuccess;
  hipError_t err = hipEventCreateWithFlags(&p->fork_ev, hipEventDisableTiming);
  for (int i = 0; err == hipSuccess && i < want; ++i) {
    // default priority, like every stream of this library
    err = hipStreamCreateWithFlags(&p->side[i], hipStreamNonBlocking);
    if (err == hipSuccess) err = hipEventCreateWithFlags(&p->join_ev[i], hipEventDisableTiming);
    p->n_side = i + 1;
  }
  return err;
}

// Rows per group of the group-mapped schedule: one LDS chunk of nonzeros
// (512 per wavefront) at the mean row length, between 1 and the group's cap.
int32_t default_group_rows(const spmv_plan_st* p, int waves) {
  const double avg = p->M > 0 ? (double)p->nnz / (double)p->M : 0.0;
  const double r = kGroupChunkPerWave * waves / (avg + 1.0);
  return (int32_t)std::max(1.0, std::min((double)(kGroupRowsPerWave * waves), r));
}

// The schedule used when none is forced: the analogue, measured on MI355X,
// of the PPoPP'23 page's size switch (Section 6.2), which leaves merge-path
// for small matrices. Small matrices are launch-bound, and the binned
// schedule is one launch while merge-path with the walk reduction is two
// (main kernel and carry fix-up): binned below kBinnedMaxNnzWalk nonzeros
// when rows cross partitions, below kBinnedMaxNnzStream when they do not,
// merge-path above (a sweep of 42 synthetic matrices, 167 to 29M nonzeros,
// uniform and skewed rows; the group-mapped schedule was never the fastest;
// re-run when the binned rows went to 16-byte quad loads, which moved the
// stream cap from 200,000 to 2,000,000: 479,464 nonzeros 9.6 against
// 12.7 us, 1.9M 18.8 against 19.0, 9.6M 65.2 against 59.6).
constexpr int64_t kBinnedMaxNnzWalk = 3000000;
constexpr int64_t kBinnedMaxNnzStream = 2000000;

int32_t choose_strategy(const spmv_plan_st* p) {
  const char* env = std::getenv("SPMV_STRATEGY");
  if (env && !std::strcmp(env, "merge")) return SPMV_STRATEGY_MERGE;
  if (env && !std::strcmp(env, "binned")) return SPMV_STRATEGY_BINNED;
  if (env && !std::strcmp(env, "group")) return SPMV_STRATEGY_GROUP;
  // short rows (T = 256) give small stream plans enough partitions to fill
  // the launch, and merge-path wins or ties there (tiny workload: 7.5 against
  // 8.2 us); with T = 1024 a small plan is a few long-lived waves
  if (p->merge_reduce == 2 && p->ipt == 4) return SPMV_STRATEGY_MERGE;
  const int64_t cap = p->merge_reduce == 2 ? kBinnedMaxNnzStream : kBinnedMaxNnzWalk;
  return p->nnz < cap ? SPMV_STRATEGY_BINNED : SPMV_STRATEGY_MERGE;
}

// One launch per bin, longest rows first, dealt round robin over the
// caller's stream and the plan's side streams; the side streams wait for
// the work queued before the call (fork) and the caller's stream waits for
// them (join), so the call orders like one launch on the caller's stream.
template <typename V>
hipError_t launch_binned_per_bin(const spmv_plan_st* p, const BinnedArgs<V>& all,
                                 hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  hipError_t err;
  if (ev0 && (err = hipEventRecord(ev0, stream)) != hipSuccess) return err;
  const int ns = p->n_side + 1;
  if (p->n_side > 0) {
    if ((err = hipEventRecord(p->fork_ev, stream)) != hipSuccess) return err;
    for (int i = 0; i < p->n_side; ++i)
      if ((err = hipStreamWaitEvent(p->side[i], p->fork_ev, 0)) != hipSuccess) return err;
  }
  for (int d = 0; d < p->n_launch; ++d) {
    BinnedArgs<V> one = all;
    one.n_launch = 1;
    one.bin[0] = p->launch[d];
    one.bin[0].block_begin = 0;
    const hipStream_t s = d % ns == 0 ? stream : p->side[d % ns - 1];
    if ((err = launch_binned<V>(one, one.bin[0].n_blocks, s, nullptr, nullptr)) != hipSuccess)
      return err;
  }
  for (int i = 0; i < p->n_side; ++i) {
    if ((err = hipEventRecord(p->join_ev[i], p->side[i])) != hipSuccess) return err;
    if ((err = hipStreamWaitEvent(stream, p->join_ev[i], 0)) != hipSuccess) return err;
  }
  if (ev1 && (err = hipEventRecord(ev1, stream)) != hipSuccess) return err;
  return hipSuccess;
}

template <typename V>
spmv_status_t exec_typed(spmv_plan_t p, const void* x, void* y, double alpha, double beta,
                         hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  hipError_t err = hipSuccess;
  if (p->strategy == SPMV_STRATEGY_GROUP) {
    GroupArgs<V> a;
    std::memset(&a, 0, sizeof a);
    a.row_ptr = p->row_ptr;
    a.col_idx = p->col_idx;
    a.val = static_cast<const V*>(p->values);
    a.x = static_cast<const V*>(x);
    a.y = static_cast<V*>(y);
    a.alpha = (V)alpha;
    a.beta = (V)beta;
    a.beta_nonzero = beta != 0.0;
    a.M = (int32_t)p->M;
    a.rows_per_group = p->group_rows;
    err = launch_group<V>(a, p->group_waves, stream, ev0, ev1);
  } else if (p->strategy == SPMV_STRATEGY_RGCSR) {
    RgArgs<V> a;
    std::memset(&a, 0, sizeof a);
    a.rl = p->rg_rl;
    a.base = p->rg_base;
    a.col = p->rg_col;
    a.val = static_cast<const V*>(p->rg_val);
    a.x = static_cast<const V*>(x);
    a.y = static_cast<V*>(y);
    a.alpha = (V)alpha;
    a.beta = (V)beta;
    a.beta_nonzero = beta != 0.0;
    a.M = (int32_t)p->M;
    a.G = p->rg_group;
    err = launch_rg_spmv<V>(a, stream, ev0, ev1);
  } else if (p->strategy == SPMV_STRATEGY_MERGE && p->x_slabs) {
    // the walk over A' (partitions in contiguous eighths per XCD, so XCD s
    // gathers from slab s of x) into one sum per segment, its fix-up, then
    // the combine of each row's segment sums into y
    MergeArgs<V> a;
    std::memset(&a, 0, sizeof a);
    a.row_ptr = p->slab_m.seg_ptr;
    a.col_idx = p->slab_m.col;
    a.val = static_cast<const V*>(p->slab_m.val);
    a.x = static_cast<const V*>(x);
    a.y = static_cast<V*>(p->slab_y);
    a.split_row = p->slab_split_row;
    a.split_nz = p->slab_split_nz;
    a.row_bounds = p->slab_row_bounds;
    a.carry_row = p->slab_carry_row;
    a.carry_val = static_cast<V*>(p->slab_carry_val);
    a.alpha = V(1);
    a.beta = V(0);
    a.beta_nonzero = 0;
    a.P = (int32_t)p->slab_P;
    a.M = (int32_t)p->slab_m.n_seg;
    a.nnz = (int32_t)p->nnz;
    a.xcd_remap = 1;
    a.stream = 0;
    err = launch_merge<V>(a, p->slab_ipt, stream, ev0, ev1);
    if (err == hipSuccess)
      err = launch_slab_combine<V>(p->slab_rows, static_cast<const V*>(p->slab_y),
                                   static_cast<V*>(y), (V)alpha, (V)beta, beta != 0.0, p->M,
                                   stream);
  } else if (p->strategy == SPMV_STRATEGY_MERGE) {
    MergeArgs<V> a;
    a.row_ptr = p->row_ptr;
    a.col_idx = p->col_idx;
    a.val = static_cast<const V*>(p->values);
    a.x = static_cast<const V*>(x);
    a.y = static_cast<V*>(y);
    a.split_row = p->split_row;
    a.split_nz = p->split_nz;
    a.row_bounds = p->row_bounds;
    a.carry_row = p->carry_row;
    a.carry_val = static_cast<V*>(p->carry_val);
    a.alpha = (V)alpha;
    a.beta = (V)beta;
    a.beta_nonzero = beta != 0.0;
    a.P = (int32_t)p->P;
    a.M = (int32_t)p->M;
    a.nnz = (int32_t)p->nnz;
    a.xcd_remap = p->xcd_remap;
    a.stream = p->merge_reduce == 2;
    a.stream_lanes = p->stream_lanes;
    // the window's 16-byte direct-to-LDS loads need a 16-byte aligned x
    a.x_window = (reinterpret_cast<uintptr_t>(x) & 15) == 0 ? p->x_window : 0;
    a.win_span = p->win_span;
    // with long-row tiles the walk kernel runs the partitions they leave,
    // in partition order, with their masks; else all, in the plan's order
    const bool tiles = p->n_tile_rows > 0;
    a.part_order = tiles ? p->tile_list : p->dispatch_order == 2 ? p->part_order : nullptr;
    a.n_dispatch = tiles ? p->n_dispatch : 0;
    a.mask_end = tiles ? p->tile_mask_end : nullptr;
    a.mask_start = tiles ? p->tile_mask_start : nullptr;
    // workgroup order: the stream kernel reads best in plain order (each
    // XCD then streams interleaved parts of the arrays: banded 1.466 ->
    // 1.377 ms, laplacian 66.5 -> 64.2 us); the walk kernel's column order
    // needs each XCD to take a contiguous run
    a.xcd_remap = a.stream ? p->xcd_remap_stream : p->xcd_remap;
    if (!tiles) {
      err = launch_merge<V>(a, p->ipt, stream, ev0, ev1);
    } else {
      // one grid for the walk over the partitions the tiles leave and the
      // tiles (ev0 / ev1 bracket it), then one for the walk's fix-up and the
      // reduction that adds each tile row's block partials into y
      TileArgs<V> t;
      std::memset(&t, 0, sizeof t);
      t.rows = p->tile_rows;
      t.seg = p->tile_seg;
      t.col_idx = p->col_idx;
      t.val = static_cast<const V*>(p->values);
      t.x = static_cast<const V*>(x);
      t.y = static_cast<V*>(y);
      t.partial = static_cast<V*>(p->tile_partial);
      t.skip = p->tile_skip;
      t.alpha = (V)alpha;
      t.n_rows = p->n_tile_rows;
      t.nb = p->tile_nb;
      t.ngroups = (p->n_tile_rows + kTileRows - 1) / kTileRows;
      t.N = (int32_t)p->N;
      t.nnz = (int32_t)p->nnz;
      t.x_aligned = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
      err = launch_merge<V>(a, p->ipt, stream, ev0, ev1, &t);
    }
  } else {
    BinnedArgs<V> a;
    std::memset(&a, 0, sizeof a);
    a.row_ptr = p->row_ptr;
    a.col_idx = p->col_idx;
    a.val = static_cast<const V*>(p->values);
    a.x = static_cast<const V*>(x);
    a.y = static_cast<V*>(y);
    a.bins = p->bins;
    a.alpha = (V)alpha;
    a.beta = (V)beta;
    a.beta_nonzero = beta != 0.0;
    a.identity = p->identity;
    a.n_launch = p->n_launch;
    a.xcd_remap = p->xcd_remap;
    a.nnz = (int32_t)p->nnz;
    for (int i = 0; i < p->n_launch; ++i) a.bin[i] = p->launch[i];
    if (p->bin_streams > 0 && p->n_launch > 1)
      err = launch_binned_per_bin<V>(p, a, stream, ev0, ev1);
    else
      err = launch_binned<V>(a, p->binned_blocks, stream, ev0, ev1);
  }
  if (err != hipSuccess) return hip_fail(err, "spmv_exec launch");
  return SPMV_SUCCESS;
}

// Sub-blocks per SpMV tile block when a k-column product runs the plan's
// long-row tiles, else 0 (no tiles in the plan, or X rows too wide).
int spmm_tile_m(const spmv_plan_st* p, int64_t k) {
  if (p->n_tile_rows <= 0 || k <= 0 || k > kWave) return 0;
  const int vs = p->dtype == SPMV_F32 ? 4 : 8;
  return spmm_tile_split((int)k, vs, kTileBytes / vs);
}

size_t spmm_workspace(const spmv_plan_st* p, int64_t k) {
  if (p->merge_reduce == 2 || p->P <= 0 || k <= 0) return 0;
  const size_t vs = p->dtype == SPMV_F32 ? 4 : 8;
  size_t bytes = align256((size_t)p->P * (size_t)std::min<int64_t>(k, kWave) * vs);
  const int m = spmm_tile_m(p, k);
  if (m > 0)
    bytes += p->dtype == SPMV_F32
                 ? spmm_tile_workspace<float>(p->n_tile_rows, p->tile_nb, m, (int)k)
                 : spmm_tile_workspace<double>(p->n_tile_rows, p->tile_nb, m, (int)k);
  return bytes;
}

template <typename V>
spmv_status_t exec_multi_typed(spmv_plan_t p, int64_t k, const void* X, int64_t ldx, void* Y,
                               int64_t ldy, double alpha, double beta, void* workspace,
                               hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  SpmmArgs<V> a;
  std::memset(&a, 0, sizeof a);
  a.row_ptr = p->row_ptr;
  a.col_idx = p->col_idx;
  a.val = static_cast<const V*>(p->values);
  a.ldx = ldx;
  a.ldy = ldy;
  a.split_row = p->split_row;
  a.split_nz = p->split_nz;
  a.row_bounds = p->row_bounds;
  a.carry_row = p->carry_row;
  a.carry_vec = static_cast<V*>(workspace);
  a.alpha = (V)alpha;
  a.beta = (V)beta;
  a.beta_nonzero = beta != 0.0;
  a.P = (int32_t)p->P;
  a.M = (int32_t)p->M;
  a.N = (int32_t)p->N;
  a.nnz = (int32_t)p->nnz;
  a.T = p->T;
  a.cap = spmm_stage_cap(p->T);
  a.stream = p->merge_reduce == 2;
  a.xcd_remap = p->xcd_remap;
  // the column order pays for SpMM only where most partitions lie inside
  // long rows (measured: -37% on the bimodal matrix at k = 8, +9% on the
  // power-law one, where a fifth do)
  a.part_order = !a.stream && p->dispatch_order == 2 && 2 * p->interior >= p->P ? p->part_order
                                                                                : nullptr;
  // long-row tiles, when the plan has them and X rows are narrow enough:
  // the merge kernel leaves the tiled rows' entries to them
  // (16-byte lanes: X and Y aligned, row strides whole lanes, as the vector
  // path of the merge kernel needs too)
  constexpr int VE = 16 / (int)sizeof(V);
  const bool vec = k % VE == 0 && ldx % VE == 0 && ldy % VE == 0 &&
                   ((reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(Y)) & 15) == 0;
  const int tm = vec ? spmm_tile_m(p, k) : 0;
  SpmmTileArgs<V> t;
  std::memset(&t, 0, sizeof t);
  if (tm > 0) {
    const int vs = (int)sizeof(V);
    a.part_order = p->tile_list;   // the partitions the tiles leave, in order
    a.n_dispatch = p->n_dispatch;
    a.mask_end = p->tile_mask_end;
    a.mask_start = p->tile_mask_start;
    char* ws = static_cast<char*>(workspace) + align256((size_t)p->P * (size_t)k * vs);
    t.rows = p->tile_rows;
    t.seg = p->tile_seg;
    t.partial = reinterpret_cast<V*>(ws);
    t.carry_vec = static_cast<V*>(workspace);
    t.skip = p->tile_skip;
    t.col_idx = p->col_idx;
    t.val = static_cast<const V*>(p->values);
    t.X = static_cast<const V*>(X);
    t.Y = static_cast<V*>(Y);
    t.ldx = ldx;
    t.ldy = ldy;
    t.alpha = (V)alpha;
    t.k = (int32_t)k;
    t.n_rows = p->n_tile_rows;
    t.nb = p->tile_nb;
    t.m = tm;
    t.bc = kTileBytes / vs;
    t.bck = t.bc / tm;
    t.ngroups = 0;   // chosen by launch_spmm_tiles
    t.N = (int32_t)p->N;
    t.nnz = (int32_t)p->nnz;
    t.x_dma = ldx == k && (reinterpret_cast<uintptr_t>(X) & 15) == 0 && (k * vs) % 16 == 0;
  }
  // one column block without tiles: the main kernel's dispatch records the
  // events; otherwise they bracket the whole call
  const bool one = k <= kWave && tm == 0;
  hipError_t err = hipSuccess;
  if (!one && ev0 && (err = hipEventRecord(ev0, stream)) != hipSuccess)
    return hip_fail(err, "spmv_exec_multi event");
  // the tiles first: they zero the carries of the partitions they cover,
  // which the merge kernel's fix-up reads
  if (tm > 0 && (err = launch_spmm_tiles<V>(t, stream)) != hipSuccess)
    return hip_fail(err, "spmv_exec_multi tiles");
  for (int64_t kb = 0; kb < k; kb += kWave) {
    a.k = (int32_t)std::min<int64_t>(kWave, k - kb);
    a.X = static_cast<const V*>(X) + kb;
    a.Y = static_cast<V*>(Y) + kb;
    if ((err = launch_spmm<V>(a, stream, one ? ev0 : nullptr, one ? ev1 : nullptr, tm == 0)) !=
        hipSuccess)
      return hip_fail(err, "spmv_exec_multi launch");
  }
  // with tiles (k <= 64: one column block, a as launched): the merge
  // kernel's fix-up and the tiles' partials into Y, one launch
  if (tm > 0 && (err = launch_spmm_fixup_tile_reduce<V>(a, t, stream)) != hipSuccess)
    return hip_fail(err, "spmv_exec_multi tiles");
  if (!one && ev1 && (err = hipEventRecord(ev1, stream)) != hipSuccess)
    return hip_fail(err, "spmv_exec_multi event");
  return SPMV_SUCCESS;
}

}  // namespace

extern "C" {

spmv_status_t spmv_spmm_workspace_size(spmv_plan_t p, int64_t k, size_t* bytes) {
  spmv_status_t st = check_plan(p);
  if (st != SPMV_SUCCESS) return st;
  if (!bytes) return fail(SPMV_ERR_INVALID_ARG, "bytes is NULL");
  if (k < 0) return fail(SPMV_ERR_INVALID_ARG, "k = %lld < 0", (long long)k);
  *bytes = spmm_workspace(p, k);
  return SPMV_SUCCESS;
}

spmv_status_t spmv_exec_multi_events(spmv_plan_t p, int64_t k, const void* X, int64_t ldx,
                                     void* Y, int64_t ldy, double alpha, double beta,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream,
                                     hipEvent_t ev_begin, hipEvent_t ev_end) {
  spmv_status_t st = check_plan(p);
  if (st != SPMV_SUCCESS) return st;
  if (k < 0) return fail(SPMV_ERR_INVALID_ARG, "k = %lld < 0", (long long)k);
  if (k == 0 || p->M == 0) return SPMV_SUCCESS;
  if (ldx < k || ldy < k)
    return fail(SPMV_ERR_INVALID_ARG, "ldx = %lld and ldy = %lld must be >= k = %lld",
                (long long)ldx, (long long)ldy, (long long)k);
  if (!Y) return fail(SPMV_ERR_INVALID_ARG, "Y is NULL");
  if (p->nnz > 0 && !X) return fail(SPMV_ERR_INVALID_ARG, "X is NULL");
  const size_t vs = p->dtype == SPMV_F32 ? 4 : 8;
  if ((reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(Y)) % vs)
    return fail(SPMV_ERR_INVALID_ARG, "X and Y must be aligned to the element size");
  // byte ranges [X, X + ((N-1) ldx + k) vs) and [Y, Y + ((M-1) ldy + k) vs)
  if (X && p->N > 0 && p->nnz > 0) {
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(X);
    const uintptr_t x1 = x0 + (uintptr_t)(((p->N - 1) * ldx + k) * (int64_t)vs);
    const uintptr_t y0 = reinterpret_cast<uintptr_t>(Y);
    const uintptr_t y1 = y0 + (uintptr_t)(((p->M - 1) * ldy + k) * (int64_t)vs);
    if (x0 < y1 && y0 < x1) return fail(SPMV_ERR_INVALID_ARG, "X and Y overlap");
  }
  const size_t need = spmm_workspace(p, k);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(SPMV_ERR_INVALID_ARG, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  // one contiguous column is an SpMV: run it as one, with every schedule
  // the plan has for that (stream or walk, tiles, x slabs)
  if (k == 1 && ldx == 1 && ldy == 1)
    return p->dtype == SPMV_F32
               ? exec_typed<float>(p, X, Y, alpha, beta, stream, ev_begin, ev_end)
               : exec_typed<double>(p, X, Y, alpha, beta, stream, ev_begin, ev_end);
  return p->dtype == SPMV_F32
             ? exec_multi_typed<float>(p, k, X, ldx, Y, ldy, alpha, beta, workspace, stream,
                                       ev_begin, ev_end)
             : exec_multi_typed<double>(p, k, X, ldx, Y, ldy, alpha, beta, workspace, stream,
                                        ev_begin, ev_end);
}

spmv_status_t spmv_exec_multi(spmv_plan_t p, int64_t k, const void* X, int64_t ldx, void* Y,
                              int64_t ldy, double alpha, double beta, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  return spmv_exec_multi_events(p, k, X, ldx, Y, ldy, alpha, beta, workspace, workspace_bytes,
                                stream, nullptr, nullptr);
}

}  // extern "C"

namespace {

// ---- plan construction ----------------------------------------------------------
// Every plan is built by one routine: one workspace allocation, the planning
// kernels enqueued back to back (the decisions that depend on the counted
// rows are taken on the device, see plan_choose_kernel), one read-back of the
// statistics block and one stream synchronisation. The OpSparse page,
// Section 5.1, keeps all metadata in one allocation and avoids frees and
// synchronisations in the middle of its pipeline; this follows it.

// What one build starts from: CSR (row_ptr) or row-sorted COO (row_idx),
// plus an optional region of the workspace the caller fills in `prologue`
// (launched on the stream after the statistics block is cleared and before
// any kernel reads the matrix).
struct PlanSource {
  int64_t M = 0, N = 0, nnz = 0;
  const int32_t* row_ptr = nullptr;
  bool coo = false;                  // derive row_ptr from row_idx (read by this call only)
  const int32_t* row_idx = nullptr;  // may be null when nnz = 0
  const int32_t* col_idx = nullptr;
  const void* values = nullptr;
  spmv_dtype_t dtype = SPMV_F32;
  size_t extra_bytes = 0;
  std::function<hipError_t(spmv_plan_st*, void* extra, hipStream_t)> prologue;
  int32_t allocs_before = 0;   // allocations the caller made for this plan
};

// The x slabs' copy A' of the matrix (slab_kernels.hip), after the plan's
// read-back gave its segment count: one more allocation (A', y', the split
// and carries of its merge-path walk), then its kernels, enqueued without a
// further synchronisation. A' takes partitions of T = 1024 units (fp32) or
// 512 (fp64): its gathers stay in L2, so the walk favours fewer, longer
// waves (power-law, fp32: 0.217 / 0.186 / 0.170 ms at T = 256 / 512 / 1024).
// A failed allocation leaves the plan without slabs.
spmv_status_t build_slabs(spmv_plan_st* p, int64_t n_seg, int64_t n_chunks, hipStream_t stream) {
  const int64_t nnz = p->nnz;
  const size_t vs = p->dtype == SPMV_F32 ? 4 : 8;
  const int ipt = vs == 4 ? 16 : 8;
  const int64_t T = (int64_t)kWave * ipt;
  if (n_seg <= 0 || n_seg > nnz || n_seg + nnz > kMaxUnits || n_chunks <= 0 ||
      n_chunks > 0x7fffffffll)
    return SPMV_SUCCESS;
  const int64_t P = (n_seg + nnz + T - 1) / T;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  const size_t o_stats = take(sizeof(int64_t) * kStatCount);
  const size_t o_segp = take(sizeof(int32_t) * (n_seg + 1));
  const size_t o_col = take(sizeof(int32_t) * nnz);
  const size_t o_val = take(vs * nnz);
  const size_t o_y = take(vs * n_seg);
  const size_t o_srow = take(sizeof(int32_t) * (P + 1));
  const size_t o_snz = take(sizeof(int32_t) * (P + 1));
  const size_t o_rb = take(sizeof(int32_t) * 2 * (P + 1));
  const size_t o_crow = take(sizeof(int32_t) * P);
  const size_t o_cval = take(vs * P);
  // a failed allocation leaves the plan without slabs (it stays valid)
  if (env_int("SPMV_TEST_FAIL_ALLOC", 0) == 2) return SPMV_SUCCESS;
  void* mem = nullptr;
  hipError_t err = hipMalloc(&mem, off);
  if (err != hipSuccess) {
    (void)hipGetLastError();
    return SPMV_SUCCESS;
  }
  ++p->plan_allocs;
  char* b = static_cast<char*>(mem);
  p->owned_slab = mem;
  p->slab_bytes = off;
  p->slab_stats = reinterpret_cast<int64_t*>(b + o_stats);
  p->slab_m.seg_ptr = reinterpret_cast<int32_t*>(b + o_segp);
  p->slab_m.col = reinterpret_cast<int32_t*>(b + o_col);
  p->slab_m.val = b + o_val;
  p->slab_m.n_seg = n_seg;
  p->slab_m.n_chunks = n_chunks;
  p->slab_y = b + o_y;
  p->slab_split_row = reinterpret_cast<int32_t*>(b + o_srow);
  p->slab_split_nz = reinterpret_cast<int32_t*>(b + o_snz);
  p->slab_row_bounds = reinterpret_cast<int32_t*>(b + o_rb);
  p->slab_carry_row = reinterpret_cast<int32_t*>(b + o_crow);
  p->slab_carry_val = b + o_cval;
  p->slab_ipt = ipt;
  p->slab_P = P;
  if ((err = launch_slab_emit(p->slab_rows, p->slab_m, p->row_ptr, p->col_idx, p->values,
                              (int)vs, p->M, p->N, nnz, stream)) != hipSuccess ||
      (err = launch_slab_stats(p->slab_stats, ipt, P, stream)) != hipSuccess ||
      (err = launch_split_search(p->slab_m.seg_ptr, n_seg, nnz, P, 0, p->slab_split_row,
                                 p->slab_split_nz, p->slab_row_bounds, p->slab_stats,
                                 stream)) != hipSuccess)
    return hip_fail(err, "plan: x slabs");
  p->x_slabs = 1;
  return SPMV_SUCCESS;
}

spmv_status_t plan_build(spmv_plan_t* out, const PlanSource& src,
                         const spmv_plan_options_t* options, hipStream_t stream,
                         void** extra_out) {
  const int64_t M = src.M, N = src.N, nnz = src.nnz;
  const spmv_dtype_t dtype = src.dtype;
  spmv_status_t st = check_options(options);
  if (st != SPMV_SUCCESS) return st;

  spmv_plan_st* p = new (std::nothrow) spmv_plan_st;
  if (!p) return fail(SPMV_ERR_ALLOC, "host allocation of the plan failed");
  std::memset(p, 0, sizeof *p);
  p->M = M;
  p->N = N;
  p->nnz = nnz;
  p->dtype = dtype;
  p->row_ptr = src.row_ptr;
  p->col_idx = src.col_idx;
  p->values = src.values;
  p->xcd_remap = env_int("SPMV_XCD_REMAP", 1) != 0;
  p->xcd_remap_stream = env_int("SPMV_XCD_REMAP", 0) != 0;
  p->plan_allocs = src.allocs_before;

  // items per lane: given (options, then environment), else chosen on the
  // device from the row lengths; the partition arrays are sized for the
  // smallest partition the plan may choose (T = 256 unless forced)
  int forced_ipt = options && options->items_per_thread ? options->items_per_thread
                                                         : env_int("SPMV_ITEMS_PER_THREAD", 0);
  if (forced_ipt != 4 && forced_ipt != 7 && forced_ipt != 8 && forced_ipt != 16) forced_ipt = 0;
  const int64_t W = M + nnz;
  const int64_t t_min = (int64_t)kWave * (forced_ipt ? forced_ipt : 4);
  const int64_t p_max = (W + t_min - 1) / t_min;

  if (options && options->n_bins > 0) {
    p->edges.n_bins = options->n_bins;
    for (int b = 0; b + 1 < options->n_bins; ++b) p->edges.max_len[b] = options->bin_max_len[b];
    for (int b = 0; b < options->n_bins; ++b) p->lanes[b] = options->bin_lanes[b];
  } else {
    p->edges.n_bins = kMaxBins;
    for (int b = 0; b + 1 < kMaxBins; ++b) p->edges.max_len[b] = kDefaultMaxLen[b];
    for (int b = 0; b < kMaxBins; ++b) p->lanes[b] = kDefaultLanes[b];
  }
  const bool validate_cols =
      (options && options->validate_columns) || env_int("SPMV_VALIDATE", 0) != 0;
  int reduce_req = options ? options->merge_reduce : 0;
  if (reduce_req == 0) {
    const char* e = std::getenv("SPMV_MERGE_REDUCE");
    if (e && !std::strcmp(e, "walk")) reduce_req = 1;
    else if (e && !std::strcmp(e, "stream")) reduce_req = 2;
  }
  int order_req = options ? options->dispatch_order : 0;
  if (order_req == 0) {
    const char* e = std::getenv("SPMV_DISPATCH_ORDER");
    if (e && !std::strcmp(e, "partition")) order_req = 1;
    else if (e && !std::strcmp(e, "column")) order_req = 2;
  }
  const size_t vs = dtype == SPMV_F32 ? 4 : 8;
  PlanCtl ctl;
  std::memset(&ctl, 0, sizeof ctl);
  ctl.M = M;
  ctl.N = N;
  ctl.nnz = nnz;
  ctl.vbytes = (int32_t)vs;
  ctl.forced_ipt = forced_ipt;
  ctl.wide_x = N * (int64_t)vs > kXcdL2Bytes;
  ctl.reduce_req = reduce_req;
  ctl.order_req = order_req;
  ctl.tiles_req = (options && options->long_row_tiles) ? options->long_row_tiles
                  : env_int("SPMV_TILES", -1) == 0 ? 1 : 0;
  // column-blocked tiles of long rows: blocks of kTileBytes of x; at most
  // one tile row per kTileMinPerBlock * nb nonzeros (and one per partition)
  const int32_t tile_bc = kTileBytes / (int32_t)vs;
  const int64_t tile_nb = (N + tile_bc - 1) / tile_bc;
  const int64_t tile_cap =
      (ctl.tiles_req == 1 || tile_nb < 2 || nnz == 0)
          ? 0
          : std::min<int64_t>(p_max, nnz / (kTileMinPerBlock * tile_nb) + 1);
  int key_bits = 1;
  while (key_bits < 31 && (int64_t(1) << key_bits) < N) ++key_bits;
  // x slabs: 0 auto, 1 off, 2 on (options, then env SPMV_X_SLABS = 0 / 1);
  // auto only for a static matrix (the copy holds A's columns and values of
  // plan time); the workspace reserves their row tables when they may be
  // taken
  ctl.slabs_req = options && options->x_slabs ? options->x_slabs
                  : env_int("SPMV_X_SLABS", -1) == 0 ? 1
                  : env_int("SPMV_X_SLABS", -1) == 1 ? 2 : 0;
  if (ctl.slabs_req == 0 && !(options && options->static_matrix)) ctl.slabs_req = 1;
  // an x of 1..4 MiB takes slabs only when rows are long: measured, they pay
  // where mean row length x x bytes >= 1e8 (uniform rows of 32 over 4 MB,
  // of 90 over 2 MB; not rows of 32 over 2 MB nor of 18 over 4 MB)
  {
    const int64_t xb = N * (int64_t)vs;
    ctl.mid_x = !ctl.wide_x && xb > (int64_t(1) << 20) && M > 0 &&
                (double)nnz / (double)M * (double)xb >= 1e8;
  }
  ctl.slab_room = M > 0 && nnz > 0 && ctl.slabs_req != 1 &&
                  (ctl.slabs_req == 2 || ctl.wide_x || ctl.mid_x) &&
                  slab_scan_max(M) <= kScanMaxElems && 2 * nnz <= kMaxUnits;

  // ---- the one workspace allocation -------------------------------------------
  const int64_t n_wg = (M + kBinRowsPerBlock - 1) / kBinRowsPerBlock;
  const int64_t groups_max = (p_max + kWavesPerBlock - 1) / kWavesPerBlock;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  const size_t o_stats = take(sizeof(int64_t) * kStatCount);
  const size_t o_counts = take(sizeof(int32_t) * kMaxBins * n_wg);
  const size_t o_wgmax = take(sizeof(int32_t) * n_wg);
  const size_t o_wgemp = take(sizeof(int32_t) * n_wg);
  const size_t o_srow = take(sizeof(int32_t) * (p_max + 1));
  const size_t o_snz = take(sizeof(int32_t) * (p_max + 1));
  const size_t o_rb = take(sizeof(int32_t) * 2 * (p_max + 1));
  const size_t o_crow = take(sizeof(int32_t) * std::max<int64_t>(p_max, 1));
  const size_t o_cval = take(vs * std::max<int64_t>(p_max, 1));
  const size_t o_bins = take(sizeof(int32_t) * M);
  const size_t o_wins = take(sizeof(int32_t) * kWinTable * groups_max);
  const size_t o_order = take(sizeof(int32_t) * std::max<int64_t>(p_max, 1));
  const size_t o_order2 = take(sizeof(int32_t) * std::max<int64_t>(p_max, 1));
  const size_t o_sort = take(std::max(radix_sort_temp_bytes(std::max<int64_t>(p_max, 1)),
                                      scan_temp_bytes(p_max)));
  // tiles: their rows, segment bounds and partials, the walk kernel's list
  // of the partitions they leave and its masks; their plan-time skip marks
  // reuse the x-window table, which walk plans never use
  const size_t o_trows = take(sizeof(int32_t) * kTileRowInts * std::max<int64_t>(tile_cap, 1));
  const size_t o_tseg =
      take(sizeof(int32_t) * std::max<int64_t>(tile_cap, 1) * (tile_nb * kTileSub + 1));
  const size_t o_tpart = take(vs * std::max<int64_t>(tile_cap, 1) * std::max<int64_t>(tile_nb, 1));
  const int64_t tile_p = tile_cap > 0 ? std::max<int64_t>(p_max, 1) : 1;
  const size_t o_tscan = take(sizeof(int32_t) * tile_p);
  const size_t o_tlist = take(sizeof(int32_t) * tile_p);
  const size_t o_tmend = take(sizeof(int32_t) * tile_p);
  const size_t o_tmstart = take(sizeof(int32_t) * tile_p);
  // x slabs' row tables
  const int64_t slab_nt = ctl.slab_room ? slab_tiles(M) : 0;
  const size_t o_smask = ctl.slab_room ? take((size_t)M) : 0;
  const size_t o_stile_e = ctl.slab_room ? take(sizeof(int32_t) * (kSlabs * slab_nt + 1)) : 0;
  const size_t o_stile_g = ctl.slab_room ? take(sizeof(int32_t) * (kSlabs * slab_nt + 1)) : 0;
  const size_t o_stile_c = ctl.slab_room ? take(sizeof(int32_t) * (slab_nt + 1)) : 0;
  const size_t o_sscan = ctl.slab_room ? take(scan_temp_bytes(slab_scan_max(M))) : 0;
  const size_t o_rowptr = src.coo ? take(sizeof(int32_t) * (M + 1)) : 0;
  const size_t o_extra = src.extra_bytes ? take(src.extra_bytes) : 0;
  p->ws_bytes = off;
  if (env_int("SPMV_TEST_FAIL_ALLOC", 0) == 1) {
    delete p;
    return fail(SPMV_ERR_ALLOC, "workspace allocation failed (forced by SPMV_TEST_FAIL_ALLOC)");
  }
  hipError_t err = hipMalloc(&p->ws, p->ws_bytes);
  ++p->plan_allocs;
  if (err != hipSuccess) {
    delete p;
    (void)hipGetLastError();
    return fail(SPMV_ERR_ALLOC, "hipMalloc(%zu) failed: %s", off, hipGetErrorString(err));
  }
  char* base = static_cast<char*>(p->ws);
  p->stats = reinterpret_cast<int64_t*>(base + o_stats);
  p->counts = reinterpret_cast<int32_t*>(base + o_counts);
  p->wg_max = reinterpret_cast<int32_t*>(base + o_wgmax);
  p->wg_empty = reinterpret_cast<int32_t*>(base + o_wgemp);
  p->split_row = reinterpret_cast<int32_t*>(base + o_srow);
  p->split_nz = reinterpret_cast<int32_t*>(base + o_snz);
  p->row_bounds = reinterpret_cast<int32_t*>(base + o_rb);
  p->carry_row = reinterpret_cast<int32_t*>(base + o_crow);
  p->carry_val = base + o_cval;
  p->bins = reinterpret_cast<int32_t*>(base + o_bins);
  p->win_span = reinterpret_cast<int32_t*>(base + o_wins);
  int32_t* order0 = reinterpret_cast<int32_t*>(base + o_order);
  int32_t* order1 = reinterpret_cast<int32_t*>(base + o_order2);
  TilePlan tp;
  std::memset(&tp, 0, sizeof tp);
  tp.cap = (int32_t)tile_cap;
  tp.nb = (int32_t)tile_nb;
  tp.bc = tile_bc;
  tp.min_entries = (int64_t)kTileMinPerBlock * tile_nb;
  tp.rows = reinterpret_cast<int32_t*>(base + o_trows);
  tp.seg = reinterpret_cast<int32_t*>(base + o_tseg);
  tp.skip = p->win_span;          // 8 ints per 4 partitions: room for p_max
  tp.scan = reinterpret_cast<int32_t*>(base + o_tscan);
  tp.list = reinterpret_cast<int32_t*>(base + o_tlist);
  tp.mask_end = reinterpret_cast<int32_t*>(base + o_tmend);
  tp.mask_start = reinterpret_cast<int32_t*>(base + o_tmstart);
  tp.scan_temp = base + o_sort;
  p->tile_rows = tp.rows;
  p->tile_skip = tp.skip;
  p->tile_list = tp.list;
  p->tile_mask_end = tp.mask_end;
  p->tile_mask_start = tp.mask_start;
  p->tile_seg = tp.seg;
  p->tile_partial = base + o_tpart;
  p->tile_nb = tp.nb;
  if (ctl.slab_room) {
    p->slab_rows.mask = reinterpret_cast<uint8_t*>(base + o_smask);
    p->slab_rows.tile_e = reinterpret_cast<int32_t*>(base + o_stile_e);
    p->slab_rows.tile_g = reinterpret_cast<int32_t*>(base + o_stile_g);
    p->slab_rows.tile_c = reinterpret_cast<int32_t*>(base + o_stile_c);
    p->slab_rows.scan_temp = base + o_sscan;
    p->slab_rows.n_tiles = slab_nt;
  }
  void* extra = src.extra_bytes ? base + o_extra : nullptr;
  int32_t* coo_row_ptr = src.coo ? reinterpret_cast<int32_t*>(base + o_rowptr) : nullptr;
  if (src.coo) p->row_ptr = coo_row_ptr;
  const int32_t* row_ptr = p->row_ptr;

  auto bail = [&](spmv_status_t s) {
    (void)hipStreamSynchronize(stream);
    (void)hipFree(p->ws);
    if (p->owned_slab) (void)hipFree(p->owned_slab);
    release_bin_streams(p);
    delete p;
    return s;
  };

  // ---- planning kernels, back to back --------------------------------------------
  int sort_result = 0;
  if ((err = launch_clear_stats(p->stats, stream)) != hipSuccess)
    return bail(hip_fail(err, "plan: clear"));
  if (src.prologue && (err = src.prologue(p, extra, stream)) != hipSuccess)
    return bail(hip_fail(err, "plan: prologue"));
  if (src.coo &&
      (err = launch_coo_row_ptr(src.row_idx, nnz, M, coo_row_ptr, p->stats, stream)) != hipSuccess)
    return bail(hip_fail(err, "plan: COO row offsets"));
  if ((err = launch_bin_count(row_ptr, M, nnz, p->edges, p->counts, p->wg_max, p->wg_empty,
                              p->stats, stream)) != hipSuccess ||
      (err = launch_bin_scan(M, p->edges, p->counts, p->wg_max, p->wg_empty, p->stats,
                             stream)) != hipSuccess ||
      (err = launch_bin_scatter(row_ptr, M, p->edges, p->counts, p->stats, p->bins, stream)) !=
          hipSuccess)
    return bail(hip_fail(err, "plan: bins"));
  if (validate_cols &&
      (err = launch_check_columns(p->col_idx, nnz, N, p->stats, stream)) != hipSuccess)
    return bail(hip_fail(err, "plan: column check"));
  if ((err = launch_plan_choose(ctl, p->stats, 0, stream)) != hipSuccess ||
      (err = launch_split_search(row_ptr, M, nnz, p_max, 0, p->split_row, p->split_nz,
                                 p->row_bounds, p->stats, stream)) != hipSuccess ||
      (err = launch_plan_choose(ctl, p->stats, 1, stream)) != hipSuccess ||
      (err = launch_split_search(row_ptr, M, nnz, p_max, 1, p->split_row, p->split_nz,
                                 p->row_bounds, p->stats, stream)) != hipSuccess ||
      (err = launch_plan_choose(ctl, p->stats, 2, stream)) != hipSuccess)
    return bail(hip_fail(err, "plan: merge-path split"));
  if ((err = launch_window_spans(ctl, row_ptr, p->col_idx, p->split_row, p_max, p->win_span,
                                 p->stats, stream)) != hipSuccess)
    return bail(hip_fail(err, "plan: x windows"));

  // column dispatch order (walk plans that chose it; every launch checks
  // the flag): keys in the carry-row array, sorted with their partition ids
  // (ping-pong through the carry-value array, which has room for P ints)
  if (p_max > 0 &&
      ((err = launch_partition_keys(p->split_nz, p->col_idx, p_max, p->stats, p->carry_row,
                                    stream)) != hipSuccess ||
       (err = radix_sort_pairs(p->carry_row, nullptr, order0,
                               reinterpret_cast<int32_t*>(p->carry_val), order1, base + o_sort,
                               p_max, p->stats + kStatParts, p->stats + kStatOrder, key_bits,
                               stream, &sort_result)) != hipSuccess))
    return bail(hip_fail(err, "plan: column dispatch order"));
  // tiles of long rows (walk plans; gated on the device); after the sort,
  // which borrows the carry arrays that the tiles' zero carries live in
  tp.row_ptr = row_ptr;
  if ((err = launch_tile_plan(tp, p->split_row, p->split_nz, p->col_idx, M, nnz, p_max,
                              p->stats, p->carry_row, p->carry_val, (int)vs, stream)) !=
      hipSuccess)
    return bail(hip_fail(err, "plan: long-row tiles"));
  // x slabs' row tables (when stage 3 takes them)
  if ((err = launch_plan_choose(ctl, p->stats, 3, stream)) != hipSuccess ||
      (ctl.slab_room && (err = launch_slab_rows(p->slab_rows, row_ptr, p->col_idx, M, N, nnz,
                                                p->stats, stream)) != hipSuccess))
    return bail(hip_fail(err, "plan: x slab tables"));

  // ---- the one read-back and synchronisation -----------------------------------------
  int64_t host_stats[kStatCount] = {0};
  if ((err = hipMemcpyAsync(host_stats, p->stats, sizeof host_stats, hipMemcpyDeviceToHost,
                            stream)) != hipSuccess ||
      (err = hipStreamSynchronize(stream)) != hipSuccess)
    return bail(hip_fail(err, "plan: statistics read-back"));
  ++p->plan_syncs;

  if (host_stats[kStatError] & kErrCooRows)
    return bail(fail(SPMV_ERR_INVALID_MATRIX,
                     "COO row indices must lie in [0, M) and be sorted in non-decreasing order"));
  if (host_stats[kStatError] & kErrRowPtr)
    return bail(fail(SPMV_ERR_INVALID_MATRIX,
                     "row_ptr is not a CSR row pointer array (row_ptr[0] = 0, "
                     "non-decreasing, row_ptr[M] = nnz)"));
  if (host_stats[kStatError] & kErrColumn)
    return bail(fail(SPMV_ERR_INVALID_MATRIX, "a column index is outside [0, N)"));

  p->ipt = (int32_t)host_stats[kStatIpt];
  p->T = kWave * p->ipt;
  p->P = host_stats[kStatParts];
  p->max_len = host_stats[kStatMaxLen];
  p->n_empty = host_stats[kStatEmpty];
  p->interior = host_stats[kStatInterior];
  for (int b = 0; b <= p->edges.n_bins; ++b)
    p->bin_offset[b] = M > 0 ? host_stats[kStatBinOffset + b] : 0;
  p->identity = M == 0 || host_stats[kStatNonEmptyBins] <= 1;
  build_binned_launch(p);
  if ((int64_t)p->binned_blocks * kBlock > 0xffffffffll)
    return bail(fail(SPMV_ERR_UNSUPPORTED, "binned grid exceeds 2^32 work-items"));
  p->bin_streams = options && options->bin_streams ? options->bin_streams
                                                   : env_int("SPMV_BIN_STREAMS", 0);
  if (p->bin_streams < 0 || p->bin_streams > kMaxBins) p->bin_streams = 0;
  if ((err = create_bin_streams(p)) != hipSuccess)
    return bail(hip_fail(err, "plan: bin streams"));

  // merge-path reduction: stream when every row fits an eighth of a partition
  {
    const bool eligible = p->max_len <= p->T / 8;
    if (reduce_req == 2 && !eligible)
      return bail(fail(SPMV_ERR_INVALID_ARG,
                       "stream reduction needs every row <= T/8 = %d entries (longest: %lld)",
                       p->T / 8, (long long)p->max_len));
    p->merge_reduce = reduce_req ? reduce_req : (eligible ? 2 : 1);
    int g = options ? options->stream_lanes : 0;
    if (g == 0) g = env_int("SPMV_STREAM_LANES", 0);
    if (g == 0) {
      const double avg = M > 0 ? (double)nnz / (double)M : 0.0;
      // about four or more products per lane of a row's group
      g = 1;
      while (g < 64 && 2.0 * g <= avg / 8.0) g *= 2;
    }
    if (g < 1 || g > 64 || (g & (g - 1))) g = 1;
    p->stream_lanes = g;
    int xw = options ? options->x_window : 0;
    if (xw == 0) {
      const int e = env_int("SPMV_X_WINDOW", -1);
      if (e == 0) xw = 1;
      else if (e == 1) xw = 2;
    }
    // x window: one interval where at least half of the stream workgroups'
    // columns fit one, else up to three where at least half fit those (no
    // nonzeros: nothing to gather, and the span table is not computed)
    const int64_t S = host_stats[kStatWindowSamples];
    const int64_t F1 = host_stats[kStatWindowFits], FM = host_stats[kStatWindowFitsMulti];
    const bool room = p->merge_reduce == 2 && nnz > 0 &&
                      stream_window_bytes(p->ipt, (int)vs, kWavesPerBlock) > 0 && S > 0;
    p->x_window = 0;
    if (room && xw == 2) p->x_window = FM > F1 ? kWinIntervals : 1;
    else if (room && xw == 0 && 2 * F1 >= S) p->x_window = 1;
    else if (room && xw == 0 && 2 * FM >= S) p->x_window = kWinIntervals;
  }
  // walk kernel's dispatch order, as chosen and sorted on the device
  p->dispatch_order = host_stats[kStatOrder] ? 2 : 1;
  p->part_order = p->dispatch_order == 2 ? (sort_result ? order1 : order0) : nullptr;
  p->n_tile_rows = p->merge_reduce == 1 ? (int32_t)host_stats[kStatTileRows] : 0;
  // every tile row leaves its row-end partition to the walk kernel, so the
  // list is never empty; were it, the plain walk (all partitions, which
  // rewrites every carry) stays correct
  if (host_stats[kStatWalkParts] <= 0) p->n_tile_rows = 0;
  if (p->n_tile_rows > 0) p->n_dispatch = (int32_t)host_stats[kStatWalkParts];
  p->group_waves = 4;
  p->group_rows = default_group_rows(p, 4);
  p->strategy = options && options->strategy ? options->strategy : choose_strategy(p);
  // x slabs: taken on the device; kept when the plan runs merge-path and,
  // unless asked for, when every slab run's end columns lie in its slab
  if (ctl.slab_room && host_stats[kStatSlabOk] &&
      (ctl.slabs_req == 2 || host_stats[kStatSlabStray] == 0) &&
      p->strategy == SPMV_STRATEGY_MERGE) {
    st = build_slabs(p, host_stats[kStatSlabSegs], host_stats[kStatSlabChunks], stream);
    if (st != SPMV_SUCCESS) return bail(st);
  }
  if (env_int("SPMV_LOG", 0))
    std::fprintf(stderr,
                 "[spmv] plan M=%lld N=%lld nnz=%lld dtype=%s strategy=%s reduce=%s G=%d xwin=%d T=%d "
                 "P=%lld max_len=%lld empty=%lld bins=%d identity=%d ws=%zu order=%s allocs=%d "
                 "syncs=%d slabs=%d segs=%lld\n",
                 (long long)M, (long long)N, (long long)nnz, dtype == SPMV_F32 ? "f32" : "f64",
                 p->strategy == SPMV_STRATEGY_MERGE ? "merge" : p->strategy == SPMV_STRATEGY_GROUP ? "group" : "binned",
                 p->merge_reduce == 2 ? "stream" : "walk", p->stream_lanes, p->x_window, p->T,
                 (long long)p->P, (long long)p->max_len, (long long)p->n_empty,
                 p->edges.n_bins, p->identity, p->ws_bytes,
                 p->dispatch_order == 2 ? "column" : "partition", p->plan_allocs, p->plan_syncs,
                 p->x_slabs, (long long)p->slab_m.n_seg);
  p->magic = kMagic;
  {
    std::lock_guard<std::mutex> lk(g_plans_mu);
    g_plans.insert(p);
  }
  if (extra_out) *extra_out = extra;
  *out = p;
  return SPMV_SUCCESS;
}

// Argument checks shared by the CSR, COO and transposed entry points.
spmv_status_t check_sizes(int64_t M, int64_t N, int64_t nnz, spmv_dtype_t dtype) {
  if (M < 0 || N < 0 || nnz < 0)
    return fail(SPMV_ERR_INVALID_ARG, "negative size (M=%lld N=%lld nnz=%lld)", (long long)M,
                (long long)N, (long long)nnz);
  if (dtype != SPMV_F32 && dtype != SPMV_F64)
    return fail(SPMV_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if ((M == 0 || N == 0) && nnz != 0)
    return fail(SPMV_ERR_INVALID_ARG, "M = 0 or N = 0 needs nnz = 0");
  if (nnz > kInt32Max)
    return fail(SPMV_ERR_INVALID_ARG, "nnz = %lld exceeds the int32 index range",
                (long long)nnz);
  if (M >= kInt32Max || N > kInt32Max)
    return fail(SPMV_ERR_UNSUPPORTED, "M = %lld or N = %lld beyond int32 indices",
                (long long)M, (long long)N);
  if (M + nnz > kMaxUnits)
    return fail(SPMV_ERR_UNSUPPORTED, "M + nnz = %lld exceeds 2^31 - 65 work units",
                (long long)(M + nnz));
  return SPMV_SUCCESS;
}

bool aligned16(const void* a) { return (reinterpret_cast<uintptr_t>(a) & 15) == 0; }

}  // namespace

extern "C" {

spmv_status_t spmv_plan_ex(spmv_plan_t* out, int64_t M, int64_t N, int64_t nnz,
                           const int32_t* row_ptr, const int32_t* col_idx, const void* values,
                           spmv_dtype_t dtype, const spmv_plan_options_t* options,
                           hipStream_t stream) {
  if (!out) return fail(SPMV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  spmv_status_t st = check_sizes(M, N, nnz, dtype);
  if (st != SPMV_SUCCESS) return st;
  if (M > 0 && !row_ptr) return fail(SPMV_ERR_INVALID_ARG, "row_ptr is NULL");
  if (nnz > 0 && (!col_idx || !values))
    return fail(SPMV_ERR_INVALID_ARG, "col_idx or values is NULL");
  if (!aligned16(row_ptr) || !aligned16(col_idx) || !aligned16(values))
    return fail(SPMV_ERR_INVALID_ARG, "row_ptr, col_idx and values must be 16-byte aligned");
  PlanSource src;
  src.M = M;
  src.N = N;
  src.nnz = nnz;
  src.row_ptr = row_ptr;
  src.col_idx = col_idx;
  src.values = values;
  src.dtype = dtype;
  return plan_build(out, src, options, stream, nullptr);
}

spmv_status_t spmv_plan(spmv_plan_t* out, int64_t M, int64_t N, int64_t nnz,
                        const int32_t* row_ptr, const int32_t* col_idx, const void* values,
                        spmv_dtype_t dtype, hipStream_t stream) {
  return spmv_plan_ex(out, M, N, nnz, row_ptr, col_idx, values, dtype, nullptr, stream);
}

spmv_status_t spmv_plan_coo(spmv_plan_t* out, int64_t M, int64_t N, int64_t nnz,
                            const int32_t* row_idx, const int32_t* col_idx, const void* values,
                            spmv_dtype_t dtype, const spmv_plan_options_t* options,
                            hipStream_t stream) {
  if (!out) return fail(SPMV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  spmv_status_t st = check_sizes(M, N, nnz, dtype);
  if (st != SPMV_SUCCESS) return st;
  if (nnz > 0 && (!row_idx || !col_idx || !values))
    return fail(SPMV_ERR_INVALID_ARG, "row_idx, col_idx or values is NULL");
  if (!aligned16(col_idx) || !aligned16(values))
    return fail(SPMV_ERR_INVALID_ARG, "col_idx and values must be 16-byte aligned");
  // the row offsets are derived into the plan's workspace; row_idx is read
  // only by this call's kernels (not at all when nnz = 0: every offset is 0)
  PlanSource src;
  src.M = M;
  src.N = N;
  src.nnz = nnz;
  src.coo = true;
  src.row_idx = row_idx;
  src.col_idx = col_idx;
  src.values = values;
  src.dtype = dtype;
  return plan_build(out, src, options, stream, nullptr);
}

spmv_status_t spmv_plan_transpose(spmv_plan_t* out, int64_t M, int64_t N, int64_t nnz,
                                  const int32_t* row_ptr, const int32_t* col_idx,
                                  const void* values, spmv_dtype_t dtype,
                                  const spmv_plan_options_t* options, hipStream_t stream) {
  if (!out) return fail(SPMV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  spmv_status_t st = check_sizes(N, M, nnz, dtype);
  if (st != SPMV_SUCCESS) return st;
  if (M > 0 && !row_ptr) return fail(SPMV_ERR_INVALID_ARG, "row_ptr is NULL");
  if (nnz > 0 && (!col_idx || !values))
    return fail(SPMV_ERR_INVALID_ARG, "col_idx or values is NULL");
  if (M >= kInt32Max) return fail(SPMV_ERR_UNSUPPORTED, "M beyond int32 indices");
  const size_t vs = dtype == SPMV_F32 ? 4 : 8;
  int bits = 1;
  while (bits < 31 && (int64_t(1) << bits) < N) ++bits;
  // scratch for this call (freed before it returns): the sort's keys and
  // positions in two ping-pong pairs, its counts, and a flag for A's row_ptr
  const size_t n1 = std::max<int64_t>(nnz, 1);
  const size_t o_k1 = align256(sizeof(int32_t) * n1);
  const size_t o_v0 = o_k1 + align256(sizeof(int32_t) * n1);
  const size_t o_v1 = o_v0 + align256(sizeof(int32_t) * n1);
  const size_t o_flag = o_v1 + align256(sizeof(int32_t) * n1);
  const size_t o_temp = o_flag + 256;
  void* scratch = nullptr;
  hipError_t err = hipMalloc(&scratch, o_temp + radix_sort_temp_bytes((int64_t)n1));
  if (err != hipSuccess) {
    (void)hipGetLastError();
    return fail(SPMV_ERR_ALLOC, "hipMalloc for the transpose scratch failed: %s",
                hipGetErrorString(err));
  }
  char* sb = static_cast<char*>(scratch);
  int32_t* k0 = reinterpret_cast<int32_t*>(sb);
  int32_t* k1 = reinterpret_cast<int32_t*>(sb + o_k1);
  int32_t* v0 = reinterpret_cast<int32_t*>(sb + o_v0);
  int32_t* v1 = reinterpret_cast<int32_t*>(sb + o_v1);
  int32_t* flag = reinterpret_cast<int32_t*>(sb + o_flag);
  int which = 0;
  auto release = [&](spmv_status_t s2) {
    (void)hipStreamSynchronize(stream);
    (void)hipFree(scratch);
    return s2;
  };
  // A's row_ptr check, and the stable sort of (column, position)
  if ((err = hipMemsetAsync(flag, 0, sizeof(int32_t), stream)) != hipSuccess ||
      (M > 0 && (err = launch_csr_check(row_ptr, M, nnz, flag, stream)) != hipSuccess) ||
      (nnz > 0 && (err = hipMemcpyAsync(k0, col_idx, sizeof(int32_t) * nnz,
                                        hipMemcpyDeviceToDevice, stream)) != hipSuccess) ||
      (nnz > 0 && (err = radix_sort_pairs(k0, nullptr, v0, k1, v1, sb + o_temp, nnz, nullptr,
                                          nullptr, bits, stream, &which)) != hipSuccess))
    return release(hip_fail(err, "spmv_plan_transpose: sort"));
  const int32_t* keys_t = which ? k1 : k0;
  const int32_t* perm = which ? v1 : v0;
  // A^T as COO sorted by its rows (A's columns); its column indices and
  // values live in the plan's workspace. Out-of-range columns of A show up
  // as out-of-range or unsorted rows of A^T.
  const size_t o_val = align256(sizeof(int32_t) * n1);
  PlanSource src;
  src.M = N;
  src.N = M;
  src.nnz = nnz;
  src.coo = true;
  src.row_idx = keys_t;
  src.dtype = dtype;
  src.extra_bytes = o_val + align256(vs * n1);
  src.allocs_before = 1;
  src.prologue = [&](spmv_plan_st* p, void* extra, hipStream_t s) -> hipError_t {
    int32_t* col_t = static_cast<int32_t*>(extra);
    void* val_t = static_cast<char*>(extra) + o_val;
    p->col_idx = col_t;
    p->values = val_t;
    p->values_copied = 1;
    hipError_t e = launch_fold_flag(flag, kErrRowPtr, p->stats, s);
    if (e == hipSuccess && nnz > 0)
      e = launch_transpose_gather(row_ptr, M, perm, values, (int)vs, nnz, col_t, val_t, s);
    return e;
  };
  st = plan_build(out, src, options, stream, nullptr);
  st = release(st);
  if (st == SPMV_SUCCESS) ++(*out)->plan_syncs;   // the wait before the scratch is freed
  return st;
}

spmv_status_t spmv_plan_csc(spmv_plan_t* out, int64_t M, int64_t N, int64_t nnz,
                            const int32_t* col_ptr, const int32_t* row_idx, const void* values,
                            spmv_dtype_t dtype, const spmv_plan_options_t* options,
                            hipStream_t stream) {
  // the CSC arrays of A (M x N) are the CSR arrays of A^T (N x M)
  return spmv_plan_transpose(out, N, M, nnz, col_ptr, row_idx, values, dtype, options, stream);
}

spmv_status_t spmv_plan_rgcsr(spmv_plan_t* out, int64_t M, int64_t N, int64_t nnz,
                              const int32_t* row_ptr, const int32_t* col_idx, const void* values,
                              spmv_dtype_t dtype, int32_t group_rows, hipStream_t stream) {
  if (!out) return fail(SPMV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (group_rows < 0 || group_rows > 1024)
    return fail(SPMV_ERR_INVALID_ARG, "group_rows = %d outside 0..1024", group_rows);
  const int32_t G = group_rows ? group_rows : kWave;
  spmv_status_t st = spmv_plan_ex(out, M, N, nnz, row_ptr, col_idx, values, dtype, nullptr,
                                  stream);
  if (st != SPMV_SUCCESS) return st;
  spmv_plan_st* p = *out;
  p->values_copied = 1;
  auto undo = [&](spmv_status_t s2) {
    (void)hipStreamSynchronize(stream);
    (void)spmv_destroy(p);
    *out = nullptr;
    return s2;
  };
  const int64_t ngroups = (M + G - 1) / G;
  // metadata: group widths, group bases (+1), row lengths, the stored count
  const size_t o_base = align256(sizeof(int32_t) * (size_t)ngroups);
  const size_t o_rl = o_base + align256(sizeof(int64_t) * (size_t)(ngroups + 1));
  const size_t o_cnt = o_rl + align256(sizeof(int32_t) * (size_t)M);
  hipError_t err = hipMalloc(&p->owned_rg_meta, o_cnt + 256);
  ++p->plan_allocs;
  if (err != hipSuccess) {
    (void)hipGetLastError();
    p->owned_rg_meta = nullptr;
    return undo(fail(SPMV_ERR_ALLOC, "hipMalloc for the row-grouped metadata failed"));
  }
  char* meta = static_cast<char*>(p->owned_rg_meta);
  int32_t* gw = reinterpret_cast<int32_t*>(meta);
  int64_t* base = reinterpret_cast<int64_t*>(meta + o_base);
  int32_t* rl = reinterpret_cast<int32_t*>(meta + o_rl);
  unsigned long long* cnt = reinterpret_cast<unsigned long long*>(meta + o_cnt);
  int64_t host[2] = {0, 0};   // total slots, stored entries
  if (M > 0 &&
      ((err = hipMemsetAsync(cnt, 0, sizeof *cnt, stream)) != hipSuccess ||
       (err = launch_rg_widths(row_ptr, M, G, gw, base, cnt, stream)) != hipSuccess ||
       (err = hipMemcpyAsync(&host[0], base + ngroups, sizeof(int64_t), hipMemcpyDeviceToHost,
                             stream)) != hipSuccess ||
       (err = hipMemcpyAsync(&host[1], cnt, sizeof(int64_t), hipMemcpyDeviceToHost, stream)) !=
           hipSuccess ||
       (err = hipStreamSynchronize(stream)) != hipSuccess))
    return undo(hip_fail(err, "spmv_plan_rgcsr: widths"));
  ++p->plan_syncs;
  const size_t vs = dtype == SPMV_F32 ? 4 : 8;
  const size_t o_val = align256(sizeof(int32_t) * (size_t)host[0]);
  err = hipMalloc(&p->owned_rg_data, o_val + align256(vs * (size_t)host[0]) + 256);
  ++p->plan_allocs;
  if (err != hipSuccess) {
    (void)hipGetLastError();
    p->owned_rg_data = nullptr;
    return undo(fail(SPMV_ERR_ALLOC, "hipMalloc of %lld row-grouped slots failed",
                     (long long)host[0]));
  }
  int32_t* col_rg = static_cast<int32_t*>(p->owned_rg_data);
  void* val_rg = static_cast<char*>(p->owned_rg_data) + o_val;
  if ((err = launch_rg_build(row_ptr, col_idx, values, (int)vs, M, G, gw, base, rl, col_rg,
                             val_rg, stream)) != hipSuccess ||
      (err = hipStreamSynchronize(stream)) != hipSuccess)
    return undo(hip_fail(err, "spmv_plan_rgcsr: copy"));
  ++p->plan_syncs;
  p->rg_group = G;
  p->rg_stored = host[1];
  p->rg_rl = rl;
  p->rg_base = base;
  p->rg_col = col_rg;
  p->rg_val = val_rg;
  p->strategy = SPMV_STRATEGY_RGCSR;
  return SPMV_SUCCESS;
}

spmv_status_t spmv_read_probe(const void* data, int64_t bytes, void* sink, hipStream_t stream) {
  if (!data || !sink || bytes < 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(data) & 15) ||
      (reinterpret_cast<uintptr_t>(sink) & 3))
    return fail(SPMV_ERR_INVALID_ARG, "read probe: data must be 16-byte aligned, bytes a "
                                      "multiple of 16, sink 4-byte aligned");
  // a key no 4 KiB block of the callers' buffers (ones, zeros) folds to
  const hipError_t err =
      launch_read_probe(data, bytes, 0x5bd1e995, static_cast<int32_t*>(sink), stream);
  if (err != hipSuccess) return hip_fail(err, "read probe launch");
  return SPMV_SUCCESS;
}

spmv_status_t spmv_gather_probe(const int32_t* col_idx, int64_t nnz, const void* x, int64_t n_x,
                                spmv_dtype_t dtype, void* sink, hipStream_t stream) {
  if (dtype != SPMV_F32 && dtype != SPMV_F64)
    return fail(SPMV_ERR_INVALID_ARG, "gather probe: unknown dtype %d", (int)dtype);
  if (nnz < 0 || n_x <= 0 || n_x > 0xffffffffll || (nnz > 0 && (!col_idx || !x)) || !sink ||
      (reinterpret_cast<uintptr_t>(col_idx) & 15) || (reinterpret_cast<uintptr_t>(sink) & 3))
    return fail(SPMV_ERR_INVALID_ARG, "gather probe: col_idx 16-byte aligned, 0 < n_x < 2^32, "
                                      "sink 4-byte aligned");
  const hipError_t err = launch_gather_probe(col_idx, nnz, x, n_x, dtype == SPMV_F32 ? 4 : 8,
                                             0x5bd1e995, static_cast<int32_t*>(sink), stream);
  if (err != hipSuccess) return hip_fail(err, "gather probe launch");
  return SPMV_SUCCESS;
}

spmv_status_t spmv_gather_rows_probe(const int32_t* col_idx, int64_t nnz, const void* X,
                                     int64_t n_rows, int32_t row_bytes, void* sink,
                                     hipStream_t stream) {
  const bool rb_ok = row_bytes == 16 || row_bytes == 32 || row_bytes == 64 || row_bytes == 128 ||
                     row_bytes == 256;
  if (!rb_ok || nnz < 0 || n_rows <= 0 || n_rows > 0xffffffffll ||
      (nnz > 0 && (!col_idx || !X)) || !sink || (reinterpret_cast<uintptr_t>(X) & 15) ||
      (reinterpret_cast<uintptr_t>(sink) & 3))
    return fail(SPMV_ERR_INVALID_ARG, "gather rows probe: row_bytes 16/32/64/128/256, X 16-byte "
                                      "aligned, 0 < n_rows < 2^32, sink 4-byte aligned");
  const hipError_t err = launch_gather_rows_probe(col_idx, nnz, X, n_rows, row_bytes, 0x5bd1e995,
                                                  static_cast<int32_t*>(sink), stream);
  if (err != hipSuccess) return hip_fail(err, "gather rows probe launch");
  return SPMV_SUCCESS;
}

spmv_status_t spmv_stream_probe(const int32_t* row_ptr, const int32_t* col_idx,
                                const void* values, int64_t M, int64_t nnz, spmv_dtype_t dtype,
                                int32_t items_per_thread, void* y, hipStream_t stream) {
  if (dtype != SPMV_F32 && dtype != SPMV_F64)
    return fail(SPMV_ERR_INVALID_ARG, "stream probe: unknown dtype %d", (int)dtype);
  if (items_per_thread != 4 && items_per_thread != 8 && items_per_thread != 16)
    return fail(SPMV_ERR_INVALID_ARG, "stream probe: items_per_thread must be 4, 8 or 16");
  if (M <= 0 || nnz < 0 || M + nnz > kInt32Max || !row_ptr || !y ||
      (nnz > 0 && (!col_idx || !values)) ||
      ((reinterpret_cast<uintptr_t>(row_ptr) | reinterpret_cast<uintptr_t>(col_idx) |
        reinterpret_cast<uintptr_t>(values)) & 15))
    return fail(SPMV_ERR_INVALID_ARG, "stream probe: M > 0, M + nnz < 2^31, arrays 16-byte "
                                      "aligned");
  const hipError_t err = launch_stream_probe(row_ptr, col_idx, values, M, nnz,
                                             dtype == SPMV_F32 ? 4 : 8, items_per_thread, y,
                                             stream);
  if (err != hipSuccess) return hip_fail(err, "stream probe launch");
  return SPMV_SUCCESS;
}

spmv_status_t spmv_exec_events(spmv_plan_t p, const void* x, void* y, double alpha,
                               double beta, hipStream_t stream, hipEvent_t ev_begin,
                               hipEvent_t ev_end) {
  spmv_status_t st = check_plan(p);
  if (st != SPMV_SUCCESS) return st;
  if (p->M > 0 && !y) return fail(SPMV_ERR_INVALID_ARG, "y is NULL");
  if (p->N > 0 && p->nnz > 0 && !x) return fail(SPMV_ERR_INVALID_ARG, "x is NULL");
  if (x && y && p->N > 0 && p->M > 0) {
    // byte ranges [x, x + N vs) and [y, y + M vs) must be disjoint
    const uintptr_t vs = p->dtype == SPMV_F32 ? 4 : 8;
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(x), x1 = x0 + (uintptr_t)p->N * vs;
    const uintptr_t y0 = reinterpret_cast<uintptr_t>(y), y1 = y0 + (uintptr_t)p->M * vs;
    if (x0 < y1 && y0 < x1) return fail(SPMV_ERR_INVALID_ARG, "x and y overlap");
  }
  if (p->M == 0) return SPMV_SUCCESS;
  return p->dtype == SPMV_F32
             ? exec_typed<float>(p, x, y, alpha, beta, stream, ev_begin, ev_end)
             : exec_typed<double>(p, x, y, alpha, beta, stream, ev_begin, ev_end);
}

spmv_status_t spmv_exec(spmv_plan_t p, const void* x, void* y, double alpha, double beta,
                        hipStream_t stream) {
  return spmv_exec_events(p, x, y, alpha, beta, stream, nullptr, nullptr);
}

spmv_status_t spmv_plan_update_values(spmv_plan_t p, const void* values, hipStream_t stream) {
  spmv_status_t st = check_plan(p);
  if (st != SPMV_SUCCESS) return st;
  if (p->values_copied)
    return fail(SPMV_ERR_UNSUPPORTED,
                "transposed, CSC and row-grouped plans keep values in their own layout");
  if (p->nnz > 0 && !values) return fail(SPMV_ERR_INVALID_ARG, "values is NULL");
  if (!aligned16(values)) return fail(SPMV_ERR_INVALID_ARG, "values must be 16-byte aligned");
  p->values = values;
  if (p->x_slabs) {
    const hipError_t err =
        launch_slab_emit(p->slab_rows, p->slab_m, p->row_ptr, p->col_idx, values,
                         p->dtype == SPMV_F32 ? 4 : 8, p->M, p->N, p->nnz, stream);
    if (err != hipSuccess) return hip_fail(err, "spmv_plan_update_values");
  }
  return SPMV_SUCCESS;
}

spmv_status_t spmv_destroy(spmv_plan_t p) {
  if (!p) return SPMV_SUCCESS;
  {
    std::lock_guard<std::mutex> lk(g_plans_mu);
    if (!g_plans.erase(p)) return fail(SPMV_ERR_INVALID_PLAN, "not a live plan handle");
  }
  p->magic = 0;
  release_bin_streams(p);
  hipError_t err = hipFree(p->ws);
  for (void* q : {p->owned_rg_meta, p->owned_rg_data, p->owned_slab}) {
    if (!q) continue;
    const hipError_t e2 = hipFree(q);
    if (err == hipSuccess) err = e2;
  }
  delete p;
  if (err != hipSuccess) return hip_fail(err, "spmv_destroy: hipFree");
  return SPMV_SUCCESS;
}

spmv_status_t spmv_plan_set_strategy(spmv_plan_t p, spmv_strategy_t strategy) {
  spmv_status_t st = check_plan(p);
  if (st != SPMV_SUCCESS) return st;
  if (strategy == SPMV_STRATEGY_AUTO) p->strategy = choose_strategy(p);
  else if (strategy == SPMV_STRATEGY_MERGE || strategy == SPMV_STRATEGY_BINNED)
    p->strategy = strategy;
  else if (strategy == SPMV_STRATEGY_RGCSR && p->rg_group > 0)
    p->strategy = strategy;
  else if (strategy == SPMV_STRATEGY_RGCSR)
    return fail(SPMV_ERR_INVALID_ARG, "the plan has no row-grouped copy (spmv_plan_rgcsr)");
  else if (strategy == SPMV_STRATEGY_GROUP)
    p->strategy = strategy;
  else return fail(SPMV_ERR_INVALID_ARG, "unknown strategy %d", (int)strategy);
  return SPMV_SUCCESS;
}

spmv_status_t spmv_plan_info(spmv_plan_t p, spmv_plan_info_t* info) {
  spmv_status_t st = check_plan(p);
  if (st != SPMV_SUCCESS) return st;
  if (!info) return fail(SPMV_ERR_INVALID_ARG, "info is NULL");
  std::memset(info, 0, sizeof *info);
  info->M = p->M;
  info->N = p->N;
  info->nnz = p->nnz;
  info->dtype = p->dtype;
  info->strategy = p->strategy;
  info->items_per_thread = p->ipt;
  info->items_per_wave = p->T;
  info->n_partitions = p->P;
  info->merge_reduce = p->merge_reduce;
  info->rgcsr_group = p->rg_group;
  info->rgcsr_stored = p->rg_stored;
  info->group_waves = p->group_waves;
  info->group_rows = p->group_rows;
  info->stream_lanes = p->stream_lanes;
  info->x_window = p->x_window;
  info->bin_streams = p->bin_streams;
  info->dispatch_order = p->n_tile_rows > 0 ? 1 : p->dispatch_order;
  info->interior_partitions = (int32_t)p->interior;
  info->n_bins = p->edges.n_bins;
  info->bin_identity = p->identity;
  for (int b = 0; b < p->edges.n_bins; ++b) {
    info->bin_max_len[b] = b + 1 < p->edges.n_bins ? p->edges.max_len[b] : -1;
    info->bin_lanes[b] = p->lanes[b];
    info->bin_count[b] = p->bin_offset[b + 1] - p->bin_offset[b];
  }
  info->max_row_len = p->max_len;
  info->n_empty_rows = p->n_empty;
  info->workspace_bytes = (int64_t)p->ws_bytes;
  info->plan_allocs = p->plan_allocs;
  info->plan_syncs = p->plan_syncs;
  info->tile_rows = p->n_tile_rows;
  info->tile_blocks = p->n_tile_rows > 0 ? p->tile_nb : 0;
  info->walk_partitions = p->n_tile_rows > 0 ? p->n_dispatch : (int32_t)p->P;
  info->x_slabs = p->x_slabs;
  info->slab_segments = p->x_slabs ? p->slab_m.n_seg : 0;
  info->slab_bytes = p->x_slabs ? (int64_t)p->slab_bytes : 0;
  return SPMV_SUCCESS;
}

spmv_status_t spmv_plan_set_group(spmv_plan_t p, int32_t group_waves, int32_t rows_per_group) {
  spmv_status_t st = check_plan(p);
  if (st != SPMV_SUCCESS) return st;
  if (group_waves != 0 && group_waves != 1 && group_waves != 2 && group_waves != 4)
    return fail(SPMV_ERR_INVALID_ARG, "group_waves = %d (1, 2 or 4)", group_waves);
  const int waves = group_waves ? group_waves : 4;
  if (rows_per_group < 0 || rows_per_group > kGroupRowsPerWave * waves)
    return fail(SPMV_ERR_INVALID_ARG, "rows_per_group = %d outside 0..%d", rows_per_group,
                kGroupRowsPerWave * waves);
  p->group_waves = waves;
  p->group_rows = rows_per_group ? rows_per_group : default_group_rows(p, waves);
  p->strategy = SPMV_STRATEGY_GROUP;
  return SPMV_SUCCESS;
}

spmv_status_t spmv_plan_copy_splits(spmv_plan_t p, int32_t* rows_host, int32_t* nnz_host,
                                    int64_t cap) {
  spmv_status_t st = check_plan(p);
  if (st != SPMV_SUCCESS) return st;
  if (!rows_host || !nnz_host) return fail(SPMV_ERR_INVALID_ARG, "host buffer is NULL");
  if (cap < p->P + 1) return fail(SPMV_ERR_INVALID_ARG, "cap < P + 1");
  if (p->P == 0) {
    rows_host[0] = 0;
    nnz_host[0] = 0;
    return SPMV_SUCCESS;
  }
  hipError_t err = hipMemcpy(rows_host, p->split_row, sizeof(int32_t) * (p->P + 1),
                             hipMemcpyDeviceToHost);
  if (err == hipSuccess)
    err = hipMemcpy(nnz_host, p->split_nz, sizeof(int32_t) * (p->P + 1), hipMemcpyDeviceToHost);
  if (err != hipSuccess) return hip_fail(err, "spmv_plan_copy_splits");
  return SPMV_SUCCESS;
}

spmv_status_t spmv_plan_copy_bins(spmv_plan_t p, int32_t* bins_host, int64_t bins_cap,
                                  int64_t* offsets_host) {
  spmv_status_t st = check_plan(p);
  if (st != SPMV_SUCCESS) return st;
  if ((!bins_host && p->M > 0) || !offsets_host)
    return fail(SPMV_ERR_INVALID_ARG, "host buffer is NULL");
  if (bins_cap < p->M) return fail(SPMV_ERR_INVALID_ARG, "bins_cap < M");
  for (int b = 0; b <= p->edges.n_bins; ++b) offsets_host[b] = p->bin_offset[b];
  if (p->M == 0) return SPMV_SUCCESS;
  if (p->identity) {
    for (int64_t i = 0; i < p->M; ++i) bins_host[i] = (int32_t)i;
    return SPMV_SUCCESS;
  }
  hipError_t err = hipMemcpy(bins_host, p->bins, sizeof(int32_t) * p->M, hipMemcpyDeviceToHost);
  if (err != hipSuccess) return hip_fail(err, "spmv_plan_copy_bins");
  return SPMV_SUCCESS;
}

const char* spmv_status_string(spmv_status_t s) {
  switch (s) {
    case SPMV_SUCCESS: return "success";
    case SPMV_ERR_INVALID_ARG: return "invalid argument";
    case SPMV_ERR_UNSUPPORTED: return "unsupported size";
    case SPMV_ERR_ALLOC: return "device allocation failed";
    case SPMV_ERR_HIP: return "HIP runtime error";
    case SPMV_ERR_INVALID_PLAN: return "invalid plan handle";
    case SPMV_ERR_INVALID_MATRIX: return "malformed CSR matrix";
  }
  return "unknown status";
}

const char* spmv_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
