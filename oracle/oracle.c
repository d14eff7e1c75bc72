/*
 * oracle.c -- plain, sequential CPU reference for the CSR SpMV path.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this code. The product library
 * (libspmv.so) shares no code, header, table or helper with it.
 *
 * Every function is the plain definition written out, in the order the pages
 * state it, with no blocking, fusion or reordering:
 *
 *  oracle_spmv_f32 / _f64 / _rows_*:
 *      CSR SpMV, "New Row-grouped CSR format for storing the sparse matrices
 *      on GPU with implementation in CUDA" (arXiv 1012.2270), Section 3: rows
 *      stored one after another, row r's entries between rowPointers[r] and
 *      rowPointers[r+1], each entry one multiply and one add into the row's
 *      sum; "A Programming Model for GPU Load Balancing" (PPoPP'23),
 *      Section 4.3 Listing 3: sum over the row's atoms, then write y[row].
 *      The alpha/beta update follows the BLAS form C = alpha*A*B + beta*C
 *      stated in "Accelerating Sparse Approximate Matrix Multiplication on
 *      GPUs" (arXiv 2103.13042), background section. The sum runs in fp64,
 *      sequentially in storage order; fp32 products are exact in fp64.
 *      Also returned: scale[i] = sum_k |a_ik * x_k|, the magnitude the
 *      acceptance bound is measured against.
 *      Pinned by tests/test_oracle.py: dense brute force on tiny matrices,
 *      identity, diagonal, integer row sums, the 2-D Laplacian closed forms,
 *      power-of-two linearity, empty rows, and the worked CSR example.
 *
 *  oracle_spmm_f32 / _f64:
 *      multi-vector SpMV (SpMM), PPoPP'23 page, Section 5.3, Listing 4: the
 *      SpMV of Listing 3 with one more loop over the columns of the dense
 *      matrix, each output column the sum over a row's atoms of the value
 *      times the dense entry in the atom's column index row and that output
 *      column (the extracted listing garbles that index; reading in the
 *      design notes). The dense matrices are row-major with leading
 *      dimensions ldx / ldy; the same fp64 sum in storage order per column,
 *      the same alpha/beta update and the same scale as the SpMV above.
 *      Pinned by tests/pins.py: numpy's dense product on tiny non-square
 *      inputs, identity, 2-D Laplacian closed forms per column, and exact
 *      alpha/beta arithmetic.
 *
 *  oracle_spmv_coo_f32 / _f64:
 *      the same product for a matrix given as COO entries (row, column,
 *      value), PPoPP'23 page, Section 3.1 (atoms named by their row): each
 *      entry, in storage order, adds its product to its row's fp64 sum;
 *      then the same alpha/beta update and scale. Rows with no entry give
 *      beta * y_old. No ordering of the entries is assumed. Pinned by
 *      tests/pins.py: dense brute force, integer sums of shuffled entries,
 *      empty rows, out-of-order entries.
 *
 *  oracle_spmv_t_f32 / _f64:
 *      the transposed product y = alpha * A^T x + beta * y_old for A in
 *      CSR (M x N; x has M entries, y has N), PPoPP'23 page, Section 3.1
 *      read with rows and columns exchanged: entry (i, j) adds a_ij * x_i
 *      to column j's fp64 sum; entries are taken in storage order (rows
 *      ascending), then the same alpha/beta update and scale. Pinned by
 *      tests/pins.py: dense brute force of A^T x, the adjoint identity
 *      z . (A x) = x . (A^T z) on small integers, a symmetric matrix.
 *
 *  oracle_rgcsr_stored:
 *      entries the row-grouped CSR layout stores (arXiv 1012.2270,
 *      Section 4): rows in groups of G consecutive rows, each group as wide
 *      as its longest row, so width x (rows in the group), summed. Pinned by
 *      the page's worked example (7 artificial zeros with groups of four;
 *      11 for ELLPACK, one group of all rows) and brute force.
 *
 *  oracle_merge_splits:
 *      merge-path partition, PPoPP'23 page, Section 5.2.1: every nonzero and
 *      every row counts as one unit of work; units are split evenly. Written
 *      as a walk over the units in order (row r's nonzeros, then row r's
 *      end), recording how many row ends and nonzeros precede each multiple
 *      of T. Pinned by a hand-worked table on the worked CSR example and by
 *      invariants that hold for any correct split.
 *
 *  oracle_bins:
 *      two-pass binning, "OpSparse" (arXiv 2206.07244), Section 5.1: count
 *      rows per bin, exclusive sum of the counts, then place row ids. Written
 *      sequentially (so the order within a bin is ascending). Pinned by
 *      histogram, permutation and ordering checks against numpy.
 */
#include <stdint.h>
#include <stddef.h>
#include <math.h>

/* ---- SpMV: y_ref = alpha * (A x) + beta * y_old, fp64 ------------------- */

static double row_sum_f32(const int32_t* row_ptr, const int32_t* col_idx,
                          const float* values, const float* x, int64_t i,
                          double* scale) {
  double t = 0.0, s = 0.0;
  for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) {
    double p = (double)values[k] * (double)x[col_idx[k]];
    t = t + p;
    s = s + fabs(p);
  }
  *scale = s;
  return t;
}

static double row_sum_f64(const int32_t* row_ptr, const int32_t* col_idx,
                          const double* values, const double* x, int64_t i,
                          double* scale) {
  double t = 0.0, s = 0.0;
  for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) {
    double p = values[k] * x[col_idx[k]];
    t = t + p;
    s = s + fabs(p);
  }
  *scale = s;
  return t;
}

/* beta == 0 means y_old is not read (it may be NULL). */
int oracle_spmv_f32(int64_t M, const int32_t* row_ptr, const int32_t* col_idx,
                    const float* values, const float* x, double alpha,
                    double beta, const float* y_old, double* ref,
                    double* scale) {
  if (beta != 0.0 && y_old == NULL) return -1;
  for (int64_t i = 0; i < M; ++i) {
    double t = row_sum_f32(row_ptr, col_idx, values, x, i, &scale[i]);
    ref[i] = alpha * t + (beta != 0.0 ? beta * (double)y_old[i] : 0.0);
  }
  return 0;
}

int oracle_spmv_f64(int64_t M, const int32_t* row_ptr, const int32_t* col_idx,
                    const double* values, const double* x, double alpha,
                    double beta, const double* y_old, double* ref,
                    double* scale) {
  if (beta != 0.0 && y_old == NULL) return -1;
  for (int64_t i = 0; i < M; ++i) {
    double t = row_sum_f64(row_ptr, col_idx, values, x, i, &scale[i]);
    ref[i] = alpha * t + (beta != 0.0 ? beta * y_old[i] : 0.0);
  }
  return 0;
}

/* ---- SpMM: Y_ref = alpha * (A X) + beta * Y_old, k columns, fp64 --------- */

/* ref and scale are M x k, row-major with leading dimension k. */
int oracle_spmm_f32(int64_t M, const int32_t* row_ptr, const int32_t* col_idx,
                    const float* values, int64_t k, const float* X, int64_t ldx,
                    double alpha, double beta, const float* Y_old, int64_t ldy,
                    double* ref, double* scale) {
  if (beta != 0.0 && Y_old == NULL) return -1;
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t c = 0; c < k; ++c) {
      double t = 0.0, s = 0.0;
      for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
        double p = (double)values[e] * (double)X[(int64_t)col_idx[e] * ldx + c];
        t = t + p;
        s = s + fabs(p);
      }
      ref[i * k + c] = alpha * t + (beta != 0.0 ? beta * (double)Y_old[i * ldy + c] : 0.0);
      scale[i * k + c] = s;
    }
  }
  return 0;
}

int oracle_spmm_f64(int64_t M, const int32_t* row_ptr, const int32_t* col_idx,
                    const double* values, int64_t k, const double* X, int64_t ldx,
                    double alpha, double beta, const double* Y_old, int64_t ldy,
                    double* ref, double* scale) {
  if (beta != 0.0 && Y_old == NULL) return -1;
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t c = 0; c < k; ++c) {
      double t = 0.0, s = 0.0;
      for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
        double p = values[e] * X[(int64_t)col_idx[e] * ldx + c];
        t = t + p;
        s = s + fabs(p);
      }
      ref[i * k + c] = alpha * t + (beta != 0.0 ? beta * Y_old[i * ldy + c] : 0.0);
      scale[i * k + c] = s;
    }
  }
  return 0;
}

/* ---- COO SpMV: y_ref = alpha * (A x) + beta * y_old, fp64 ---------------- */

int oracle_spmv_coo_f32(int64_t M, int64_t nnz, const int32_t* row_idx,
                        const int32_t* col_idx, const float* values, const float* x,
                        double alpha, double beta, const float* y_old, double* ref,
                        double* scale) {
  if (beta != 0.0 && y_old == NULL) return -1;
  for (int64_t i = 0; i < M; ++i) {
    ref[i] = 0.0;
    scale[i] = 0.0;
  }
  for (int64_t e = 0; e < nnz; ++e) {
    int64_t i = row_idx[e];
    if (i < 0 || i >= M) return -2;
    double p = (double)values[e] * (double)x[col_idx[e]];
    ref[i] = ref[i] + p;
    scale[i] = scale[i] + fabs(p);
  }
  for (int64_t i = 0; i < M; ++i)
    ref[i] = alpha * ref[i] + (beta != 0.0 ? beta * (double)y_old[i] : 0.0);
  return 0;
}

int oracle_spmv_coo_f64(int64_t M, int64_t nnz, const int32_t* row_idx,
                        const int32_t* col_idx, const double* values, const double* x,
                        double alpha, double beta, const double* y_old, double* ref,
                        double* scale) {
  if (beta != 0.0 && y_old == NULL) return -1;
  for (int64_t i = 0; i < M; ++i) {
    ref[i] = 0.0;
    scale[i] = 0.0;
  }
  for (int64_t e = 0; e < nnz; ++e) {
    int64_t i = row_idx[e];
    if (i < 0 || i >= M) return -2;
    double p = values[e] * x[col_idx[e]];
    ref[i] = ref[i] + p;
    scale[i] = scale[i] + fabs(p);
  }
  for (int64_t i = 0; i < M; ++i)
    ref[i] = alpha * ref[i] + (beta != 0.0 ? beta * y_old[i] : 0.0);
  return 0;
}

/* ---- transposed SpMV: y_ref = alpha * (A^T x) + beta * y_old, fp64 ------- */

int oracle_spmv_t_f32(int64_t M, int64_t N, const int32_t* row_ptr, const int32_t* col_idx,
                      const float* values, const float* x, double alpha, double beta,
                      const float* y_old, double* ref, double* scale) {
  if (beta != 0.0 && y_old == NULL) return -1;
  for (int64_t j = 0; j < N; ++j) {
    ref[j] = 0.0;
    scale[j] = 0.0;
  }
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
      int64_t j = col_idx[e];
      double p = (double)values[e] * (double)x[i];
      ref[j] = ref[j] + p;
      scale[j] = scale[j] + fabs(p);
    }
  }
  for (int64_t j = 0; j < N; ++j)
    ref[j] = alpha * ref[j] + (beta != 0.0 ? beta * (double)y_old[j] : 0.0);
  return 0;
}

int oracle_spmv_t_f64(int64_t M, int64_t N, const int32_t* row_ptr, const int32_t* col_idx,
                      const double* values, const double* x, double alpha, double beta,
                      const double* y_old, double* ref, double* scale) {
  if (beta != 0.0 && y_old == NULL) return -1;
  for (int64_t j = 0; j < N; ++j) {
    ref[j] = 0.0;
    scale[j] = 0.0;
  }
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
      int64_t j = col_idx[e];
      double p = values[e] * x[i];
      ref[j] = ref[j] + p;
      scale[j] = scale[j] + fabs(p);
    }
  }
  for (int64_t j = 0; j < N; ++j)
    ref[j] = alpha * ref[j] + (beta != 0.0 ? beta * y_old[j] : 0.0);
  return 0;
}

/* ---- row-grouped CSR: stored entries ---------------------------------------- */

int64_t oracle_rgcsr_stored(int64_t M, const int32_t* row_ptr, int64_t G) {
  int64_t stored = 0;
  for (int64_t g0 = 0; g0 < M; g0 += G) {
    int64_t g1 = g0 + G < M ? g0 + G : M;
    int64_t width = 0;
    for (int64_t i = g0; i < g1; ++i) {
      int64_t L = row_ptr[i + 1] - row_ptr[i];
      if (L > width) width = L;
    }
    stored += width * (g1 - g0);
  }
  return stored;
}

/* The same definition evaluated only on the rows listed in rows[0..n). */
int oracle_spmv_rows_f32(const int32_t* row_ptr, const int32_t* col_idx,
                         const float* values, const float* x, double alpha,
                         double beta, const float* y_old, const int64_t* rows,
                         int64_t n, double* ref, double* scale) {
  if (beta != 0.0 && y_old == NULL) return -1;
  for (int64_t q = 0; q < n; ++q) {
    int64_t i = rows[q];
    double t = row_sum_f32(row_ptr, col_idx, values, x, i, &scale[q]);
    ref[q] = alpha * t + (beta != 0.0 ? beta * (double)y_old[i] : 0.0);
  }
  return 0;
}

int oracle_spmv_rows_f64(const int32_t* row_ptr, const int32_t* col_idx,
                         const double* values, const double* x, double alpha,
                         double beta, const double* y_old, const int64_t* rows,
                         int64_t n, double* ref, double* scale) {
  if (beta != 0.0 && y_old == NULL) return -1;
  for (int64_t q = 0; q < n; ++q) {
    int64_t i = rows[q];
    double t = row_sum_f64(row_ptr, col_idx, values, x, i, &scale[q]);
    ref[q] = alpha * t + (beta != 0.0 ? beta * y_old[i] : 0.0);
  }
  return 0;
}

/* ---- merge-path split coordinates by walking the work units ------------- */

/* Writes P+1 entries, P = ceil((M + nnz) / T). Entry p holds the number of
 * row ends (split_row) and nonzeros (split_nz) among the first min(p*T, W)
 * units, W = M + nnz. Returns P, or -1 on bad arguments. */
int64_t oracle_merge_splits(int64_t M, int64_t nnz, const int32_t* row_ptr,
                            int64_t T, int32_t* split_row, int32_t* split_nz) {
  if (T <= 0 || M < 0 || nnz < 0) return -1;
  int64_t W = M + nnz;
  int64_t P = (W + T - 1) / T;
  int64_t rows_done = 0, nz_done = 0, units = 0, p = 0;
  split_row[0] = 0;
  split_nz[0] = 0;
  p = 1;
  for (int64_t r = 0; r < M; ++r) {
    for (int64_t k = row_ptr[r]; k < row_ptr[r + 1]; ++k) {
      nz_done += 1;                       /* unit: nonzero k of row r */
      units += 1;
      if (units == p * T) {
        split_row[p] = (int32_t)rows_done;
        split_nz[p] = (int32_t)nz_done;
        p += 1;
      }
    }
    rows_done += 1;                       /* unit: end of row r */
    units += 1;
    if (units == p * T) {
      split_row[p] = (int32_t)rows_done;
      split_nz[p] = (int32_t)nz_done;
      p += 1;
    }
  }
  if (p == P) {                           /* short last partition */
    split_row[P] = (int32_t)rows_done;
    split_nz[P] = (int32_t)nz_done;
  }
  return P;
}

/* ---- two-pass binning by row length ------------------------------------ */

/* Bin of a row of length L: the first b < n_bins-1 with L <= max_len[b],
 * otherwise the last bin. counts[n_bins], offsets[n_bins+1], bins[M]. */
int oracle_bins(int64_t M, const int32_t* row_ptr, int32_t n_bins,
                const int64_t* max_len, int64_t* counts, int64_t* offsets,
                int32_t* bins) {
  if (n_bins < 1 || n_bins > 64) return -1;
  for (int32_t b = 0; b < n_bins; ++b) counts[b] = 0;
  /* pass 1: count rows per bin */
  for (int64_t r = 0; r < M; ++r) {
    int64_t L = (int64_t)row_ptr[r + 1] - row_ptr[r];
    int32_t b = 0;
    while (b < n_bins - 1 && L > max_len[b]) ++b;
    counts[b] += 1;
  }
  /* exclusive sum of the counts */
  offsets[0] = 0;
  for (int32_t b = 0; b < n_bins; ++b) offsets[b + 1] = offsets[b] + counts[b];
  /* pass 2: place row ids */
  int64_t fill[64];
  for (int32_t b = 0; b < n_bins; ++b) fill[b] = offsets[b];
  for (int64_t r = 0; r < M; ++r) {
    int64_t L = (int64_t)row_ptr[r + 1] - row_ptr[r];
    int32_t b = 0;
    while (b < n_bins - 1 && L > max_len[b]) ++b;
    bins[fill[b]] = (int32_t)r;
    fill[b] += 1;
  }
  return 0;
}
