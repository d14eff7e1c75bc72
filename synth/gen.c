/*
 * gen.c -- seeded synthetic CSR workloads.
 *
 * Input generation only: no part of the SpMV, its partition or its binning is
 * computed here. Both the GPU path (through tests and bench.py) and the CPU
 * oracle receive the arrays this file writes, as data.
 *
 * Random numbers: every draw is a pure function of (seed, stream, a, b)
 * through the SplitMix64 output function (Steele, Lea, Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014), so the arrays
 * are identical for any thread count.
 *
 * Distinct sorted column sets use Floyd's sampling without replacement
 * (Bentley and Floyd, "A sample of brilliance", CACM 1987) followed by a
 * sort; the draw for candidate j is keyed by j.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

static inline uint64_t mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t key3(uint64_t seed, uint64_t stream, uint64_t a) {
  return mix64(mix64(mix64(seed) ^ stream) ^ a);
}

uint64_t synth_hash(uint64_t seed, uint64_t stream, uint64_t a, uint64_t b) {
  return mix64(key3(seed, stream, a) ^ b);
}

/* integer in [0, n) from a 64-bit draw (multiply-high) */
static inline uint64_t below(uint64_t h, uint64_t n) {
  return (uint64_t)(((unsigned __int128)h * n) >> 64);
}

/* U[-1, 1) with 24 significant bits: exact in fp32 */
static inline float unif_f32(uint64_t h) {
  return (float)((double)((int64_t)(h >> 40) - (1ll << 23)) * 0x1p-23);
}
/* U[-1, 1) with 53 significant bits: exact in fp64 */
static inline double unif_f64(uint64_t h) {
  return (double)((int64_t)(h >> 11) - (1ll << 52)) * 0x1p-52;
}

void synth_uniform_f32(int64_t n, uint64_t seed, uint64_t stream, float* out) {
  uint64_t k = key3(seed, stream, 0);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = unif_f32(mix64(k ^ (uint64_t)i));
}

void synth_uniform_f64(int64_t n, uint64_t seed, uint64_t stream, double* out) {
  uint64_t k = key3(seed, stream, 0);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = unif_f64(mix64(k ^ (uint64_t)i));
}

/* L[i] uniform integer in [lo, hi] */
void synth_rowlen_uniform(int64_t M, int32_t lo, int32_t hi, uint64_t seed,
                          uint64_t stream, int32_t* L) {
  uint64_t k = key3(seed, stream, 0);
  uint64_t span = (uint64_t)(hi - lo + 1);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; ++i)
    L[i] = lo + (int32_t)below(mix64(k ^ (uint64_t)i), span);
}

/* Discrete power law with tail exponent 1 + a (a = 1.1 for exponent 2.1):
 * L = min(max_len, floor(u^(-1/a) + 1/2)), u uniform on (0, 1], so that
 * P(L >= k) = (k - 1/2)^(-a) for 2 <= k <= max_len and L >= 1. */
void synth_rowlen_powerlaw(int64_t M, double a, int32_t max_len, uint64_t seed,
                           uint64_t stream, int32_t* L) {
  uint64_t k = key3(seed, stream, 0);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; ++i) {
    double u = (double)((mix64(k ^ (uint64_t)i) >> 11) + 1) * 0x1p-53;
    double v = floor(pow(u, -1.0 / a) + 0.5);
    L[i] = v >= (double)max_len ? max_len : (int32_t)v;
  }
}

/* ---- distinct sampling (Floyd) ----------------------------------------- */

typedef struct {
  int64_t* slot;   /* open addressing, -1 = empty */
  int64_t cap;     /* slots in use, a power of two */
  int64_t alloc;   /* slots allocated */
} hset;

static int hset_reserve(hset* s, int64_t n) {
  int64_t cap = 64;
  while (cap < 2 * n) cap <<= 1;
  if (cap > s->alloc) {
    free(s->slot);
    s->slot = (int64_t*)malloc((size_t)cap * sizeof(int64_t));
    s->alloc = s->slot ? cap : 0;
    if (!s->slot) return -1;
  }
  for (int64_t i = 0; i < cap; ++i) s->slot[i] = -1;
  s->cap = cap;
  return 0;
}

/* inserts v; returns 1 if it was already present */
static int hset_insert(hset* s, int64_t v) {
  uint64_t m = (uint64_t)s->cap - 1;
  uint64_t h = mix64((uint64_t)v) & m;
  while (s->slot[h] != -1) {
    if (s->slot[h] == v) return 1;
    h = (h + 1) & m;
  }
  s->slot[h] = v;
  return 0;
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* L distinct values from [0, R), written sorted to out[0..L). */
static int floyd_sorted(int64_t R, int64_t L, uint64_t rowkey, hset* hs,
                        int32_t* out) {
  if (L == 0) return 0;
  if (L > R) return -1;
  int64_t n = 0;
  if (L <= 48) {                         /* small: linear membership test */
    for (int64_t j = R - L; j < R; ++j) {
      int64_t t = (int64_t)below(mix64(rowkey ^ (uint64_t)j), (uint64_t)j + 1);
      int dup = 0;
      for (int64_t q = 0; q < n; ++q) if (out[q] == t) { dup = 1; break; }
      out[n++] = (int32_t)(dup ? j : t);
    }
    /* insertion sort */
    for (int64_t a = 1; a < n; ++a) {
      int32_t v = out[a];
      int64_t b = a - 1;
      while (b >= 0 && out[b] > v) { out[b + 1] = out[b]; --b; }
      out[b + 1] = v;
    }
    return 0;
  }
  if (hset_reserve(hs, L)) return -1;
  for (int64_t j = R - L; j < R; ++j) {
    int64_t t = (int64_t)below(mix64(rowkey ^ (uint64_t)j), (uint64_t)j + 1);
    if (hset_insert(hs, t)) { hset_insert(hs, j); out[n++] = (int32_t)j; }
    else out[n++] = (int32_t)t;
  }
  qsort(out, (size_t)n, sizeof(int32_t), cmp_i32);
  return 0;
}

/* Exclusive sum of row lengths into row_ptr[M+1]; returns nnz or -1 when it
 * would not fit in int32. */
int64_t synth_row_ptr(int64_t M, const int32_t* L, int32_t* row_ptr) {
  int64_t acc = 0;
  row_ptr[0] = 0;
  for (int64_t i = 0; i < M; ++i) {
    acc += L[i];
    if (acc > 2147483647ll) return -1;
    row_ptr[i + 1] = (int32_t)acc;
  }
  return acc;
}

/* Distinct sorted columns for every row. half_window < 0: uniform over
 * [0, N); otherwise uniform over [max(0, i-w), min(N-1, i+w)]. Returns 0, or
 * -1 if a row asks for more columns than its range holds. */
int synth_cols_distinct(int64_t M, int64_t N, const int32_t* row_ptr,
                        int64_t half_window, uint64_t seed, uint64_t stream,
                        int32_t* col_idx) {
  int bad = 0;
#pragma omp parallel reduction(| : bad)
  {
    hset hs = {NULL, 0, 0};
#pragma omp for schedule(dynamic, 4096)
    for (int64_t i = 0; i < M; ++i) {
      int64_t lo = 0, hi = N - 1;
      if (half_window >= 0) {
        lo = i - half_window < 0 ? 0 : i - half_window;
        hi = i + half_window > N - 1 ? N - 1 : i + half_window;
      }
      int64_t s = row_ptr[i], e = row_ptr[i + 1];
      uint64_t rk = key3(seed, stream, (uint64_t)i);
      if (floyd_sorted(hi - lo + 1, e - s, rk, &hs, col_idx + s)) { bad = 1; continue; }
      if (lo) for (int64_t k = s; k < e; ++k) col_idx[k] += (int32_t)lo;
    }
    free(hs.slot);
  }
  return bad ? -1 : 0;
}

/* Two-length imbalance: n_long rows (uniform, without replacement) of length
 * long_len, then n_empty rows drawn from the remaining ones left empty, the
 * rest of length short_len. Returns 0 or -1. */
int synth_rowlen_bimodal(int64_t M, int64_t n_long, int32_t long_len,
                         int64_t n_empty, int32_t short_len, uint64_t seed,
                         uint64_t stream, int32_t* L) {
  if (n_long < 0 || n_empty < 0 || n_long + n_empty > M) return -1;
  int rc = -1;
  hset hs = {NULL, 0, 0};
  int64_t np = (n_long > n_empty ? n_long : n_empty) + 1;
  int32_t* pick = (int32_t*)malloc((size_t)np * sizeof(int32_t));
  int32_t* rest = (int32_t*)malloc((size_t)(M - n_long + 1) * sizeof(int32_t));
  if (!pick || !rest) goto done;
  for (int64_t i = 0; i < M; ++i) L[i] = short_len;
  /* long rows: n_long distinct ids from [0, M), sorted */
  if (floyd_sorted(M, n_long, key3(seed, stream, 1), &hs, pick)) goto done;
  for (int64_t q = 0; q < n_long; ++q) L[pick[q]] = long_len;
  /* the ids that are not long, ascending */
  int64_t nr = 0, q = 0;
  for (int64_t i = 0; i < M; ++i) {
    if (q < n_long && pick[q] == i) { ++q; continue; }
    rest[nr++] = (int32_t)i;
  }
  /* empty rows: n_empty distinct positions in rest */
  if (floyd_sorted(nr, n_empty, key3(seed, stream, 2), &hs, pick)) goto done;
  for (int64_t e = 0; e < n_empty; ++e) L[rest[pick[e]]] = 0;
  rc = 0;
done:
  free(hs.slot); free(pick); free(rest);
  return rc;
}

/* Exponential decay values sigma * fl32(lambda^|i-j|) * c, sigma = +-1 from
 * one random bit per entry (the decay-matrix definition |A_ij| < c
 * lambda^|i-j| taken at equality). */
void synth_values_decay_f32(int64_t M, const int32_t* row_ptr,
                            const int32_t* col_idx, double lambda, double c,
                            uint64_t seed, uint64_t stream, float* values) {
#pragma omp parallel for schedule(dynamic, 4096)
  for (int64_t i = 0; i < M; ++i) {
    uint64_t rk = key3(seed, stream, (uint64_t)i);
    for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) {
      int64_t d = col_idx[k] > i ? col_idx[k] - i : i - col_idx[k];
      float mag = (float)(c * pow(lambda, (double)d));
      values[k] = (mix64(rk ^ (uint64_t)k) & 1) ? -mag : mag;
    }
  }
}

/* 5-point 2-D Laplacian on an n x n grid, row i = (r, c) = (i / n, i % n);
 * neighbours outside the grid are dropped; columns in increasing order:
 * i-n, i-1, i, i+1, i+n; diagonal 4, neighbours -1. row_ptr[n*n+1],
 * col_idx/values of 5n^2 - 4n entries. Returns nnz. */
int64_t synth_laplacian_2d(int64_t n, int32_t* row_ptr, int32_t* col_idx,
                           double* values) {
  int64_t M = n * n, k = 0;
  row_ptr[0] = 0;
  for (int64_t i = 0; i < M; ++i) {
    int64_t r = i / n, c = i % n;
    if (r > 0)     { col_idx[k] = (int32_t)(i - n); values[k++] = -1.0; }
    if (c > 0)     { col_idx[k] = (int32_t)(i - 1); values[k++] = -1.0; }
    col_idx[k] = (int32_t)i; values[k++] = 4.0;
    if (c < n - 1) { col_idx[k] = (int32_t)(i + 1); values[k++] = -1.0; }
    if (r < n - 1) { col_idx[k] = (int32_t)(i + n); values[k++] = -1.0; }
    row_ptr[i + 1] = (int32_t)k;
  }
  return k;
}
