"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one of them."""
import os

import pytest

import oracle
import pins

# (name, exact text in oracle.c, replacement)
MUTANTS = [
    ("x indexed by row", "double p = (double)values[k] * (double)x[col_idx[k]];",
     "double p = (double)values[k] * (double)x[i % 2];"),
    ("x indexed by row f64", "double p = values[k] * x[col_idx[k]];",
     "double p = values[k] * x[i % 2];"),
    ("sign flip", "    t = t + p;\n    s = s + fabs(p);\n  }\n  *scale = s;\n  return t;\n}\n\nstatic double row_sum_f64",
     "    t = t - p;\n    s = s + fabs(p);\n  }\n  *scale = s;\n  return t;\n}\n\nstatic double row_sum_f64"),
    ("first entry skipped", "for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) {\n    double p = (double)",
     "for (int64_t k = row_ptr[i] + (row_ptr[i] < row_ptr[i + 1]); k < row_ptr[i + 1]; ++k) {\n    double p = (double)"),
    ("beta term dropped", "ref[i] = alpha * t + (beta != 0.0 ? beta * (double)y_old[i] : 0.0);",
     "ref[i] = alpha * t;"),
    ("alpha dropped", "ref[i] = alpha * t + (beta != 0.0 ? beta * y_old[i] : 0.0);",
     "ref[i] = t + (beta != 0.0 ? beta * y_old[i] : 0.0);"),
    ("scale not absolute", "    s = s + fabs(p);\n  }\n  *scale = s;\n  return t;\n}\n\n/* beta",
     "    s = s + p;\n  }\n  *scale = s;\n  return t;\n}\n\n/* beta"),
    ("row end counted before its nonzeros",
     "      units += 1;\n      if (units == p * T) {\n        split_row[p] = (int32_t)rows_done;",
     "      units += 1;\n      if (units == p * T) {\n        split_row[p] = (int32_t)(rows_done + 1);"),
    ("split diagonal off by one", "      if (units == p * T) {\n        split_row[p] = (int32_t)rows_done;\n        split_nz[p] = (int32_t)nz_done;\n        p += 1;\n      }\n    }\n    rows_done",
     "      if (units == p * T + 1) {\n        split_row[p] = (int32_t)rows_done;\n        split_nz[p] = (int32_t)nz_done;\n        p += 1;\n      }\n    }\n    rows_done"),
    ("bin edge exclusive", "while (b < n_bins - 1 && L > max_len[b]) ++b;\n    counts[b] += 1;",
     "while (b < n_bins - 1 && L >= max_len[b]) ++b;\n    counts[b] += 1;"),
    ("spmm X read column-major", "double p = (double)values[e] * (double)X[(int64_t)col_idx[e] * ldx + c];",
     "double p = (double)values[e] * (double)X[c * ldx + col_idx[e]];"),
    ("spmm first column only", "double p = values[e] * X[(int64_t)col_idx[e] * ldx + c];",
     "double p = values[e] * X[(int64_t)col_idx[e] * ldx];"),
    ("spmm beta row stride", "ref[i * k + c] = alpha * t + (beta != 0.0 ? beta * (double)Y_old[i * ldy + c] : 0.0);",
     "ref[i * k + c] = alpha * t + (beta != 0.0 ? beta * (double)Y_old[i + c] : 0.0);"),
    ("spmm alpha dropped", "ref[i * k + c] = alpha * t + (beta != 0.0 ? beta * Y_old[i * ldy + c] : 0.0);",
     "ref[i * k + c] = t + (beta != 0.0 ? beta * Y_old[i * ldy + c] : 0.0);"),
    ("coo value of the next entry", "    double p = (double)values[e] * (double)x[col_idx[e]];\n    ref[i] = ref[i] + p;",
     "    double p = (double)values[e + (e + 1 < nnz)] * (double)x[col_idx[e]];\n    ref[i] = ref[i] + p;"),
    ("coo beta dropped", "    ref[i] = alpha * ref[i] + (beta != 0.0 ? beta * y_old[i] : 0.0);",
     "    ref[i] = alpha * ref[i];"),
    ("transposed: x indexed by column", "double p = (double)values[e] * (double)x[i];",
     "double p = (double)values[e] * (double)x[j];"),
    ("transposed: sum into the row", "      double p = values[e] * x[i];\n      ref[j] = ref[j] + p;",
     "      double p = values[e] * x[i];\n      ref[i % N] = ref[i % N] + p;"),
    ("rgcsr width from the first row", "      if (L > width) width = L;", "      if (i == g0) width = L;"),
    ("rgcsr full groups only", "    stored += width * (g1 - g0);", "    stored += width * G;"),
    ("bins reversed order", "bins[fill[b]] = (int32_t)r;", "bins[offsets[b + 1] - 1 - (fill[b] - offsets[b])] = (int32_t)r;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = oracle.source_text()
    assert src.count(old) == 1, "mutation anchor must match exactly once: " + name
    lib = oracle.compile_variant(src.replace(old, new), str(tmp_path / "mut.so"))
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake: " + name
