"""Checks that pin the CPU oracle to facts that do not come from the oracle.

Each ``pin_*`` function takes an ``OracleLib``-like object ``o`` and raises
AssertionError when the oracle disagrees with the fact it checks. The same
functions run against the real oracle (tests/test_oracle.py) and against
copies with a planted mistake (tests/test_oracle_mutants.py), which must each
fail at least one pin.
"""
import numpy as np

from conftest import read_golden

F32, F64 = np.float32, np.float64


def _csr_from_dense(A):
    """CSR of a dense matrix by numpy (row-major scan, columns ascending)."""
    rows, cols = np.nonzero(A)
    rp = np.zeros(A.shape[0] + 1, dtype=np.int32)
    np.add.at(rp, rows + 1, 1)
    rp = np.cumsum(rp).astype(np.int32)
    return rp, cols.astype(np.int32), A[rows, cols]


def _dense_matvec_ascending(A, x):
    """y_i = sum over j = 0..N-1 (ascending) of A_ij * x_j in fp64, by hand."""
    M, N = A.shape
    y = np.empty(M, dtype=np.float64)
    s = np.empty(M, dtype=np.float64)
    for i in range(M):
        t = 0.0
        a = 0.0
        for j in range(N):
            p = float(A[i, j]) * float(x[j])
            t = t + p
            a = a + abs(p)
        y[i] = t
        s[i] = a
    return y, s


def pin_dense_bruteforce(o):
    """CSR SpMV equals the dense matrix-vector product, bit for bit, on tiny
    random matrices with empty rows and columns, M != N, fp32 and fp64."""
    rng = np.random.default_rng(7)
    for trial in range(24):
        M = int(rng.integers(1, 40))
        N = int(rng.integers(1, 40))
        if M == N:
            N += 1
        dens = [0.0, 0.05, 0.3, 0.7, 1.0][trial % 5]
        dt = F32 if trial % 2 == 0 else F64
        A = np.where(rng.random((M, N)) < dens, rng.uniform(-1, 1, (M, N)), 0.0).astype(dt)
        A[rng.random(M) < 0.2, :] = 0          # empty rows
        A[:, rng.random(N) < 0.2] = 0          # empty columns
        x = rng.uniform(-1, 1, N).astype(dt)
        rp, col, val = _csr_from_dense(A)
        ref, scale = o.spmv(rp, col, val, x)
        want, wscale = _dense_matvec_ascending(A, x)
        assert np.array_equal(ref, want), ("dense brute force", trial)
        assert np.array_equal(scale, wscale), ("dense scale", trial)


def pin_identity(o):
    """A = I gives y = x exactly."""
    for dt in (F32, F64):
        n = 257
        rp = np.arange(n + 1, dtype=np.int32)
        col = np.arange(n, dtype=np.int32)
        val = np.ones(n, dtype=dt)
        x = np.random.default_rng(1).uniform(-1, 1, n).astype(dt)
        ref, _ = o.spmv(rp, col, val, x)
        assert np.array_equal(ref, x.astype(np.float64)), "identity"


def pin_diagonal(o):
    """A = diag(d) gives y_i = d_i * x_i (one exact product for fp32 inputs,
    one rounding for fp64)."""
    rng = np.random.default_rng(2)
    for dt in (F32, F64):
        n = 300
        d = rng.uniform(-4, 4, n).astype(dt)
        x = rng.uniform(-1, 1, n).astype(dt)
        rp = np.arange(n + 1, dtype=np.int32)
        ref, _ = o.spmv(rp, np.arange(n, dtype=np.int32), d, x)
        want = np.array([float(a) * float(b) for a, b in zip(d, x)])
        assert np.array_equal(ref, want), "diagonal"


def pin_integer_row_sums(o):
    """Small-integer values with x = 1 give the integer row sums (exact in
    any order); x = 1 with values = 1 gives the row lengths."""
    rng = np.random.default_rng(3)
    M, N = 500, 700
    L = rng.integers(0, 40, M)
    rp = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    col = np.concatenate([np.sort(rng.choice(N, l, replace=False)) for l in L]).astype(np.int32)
    ints = rng.choice(np.array([-1, 1, 2, 4]), rp[-1])
    for dt in (F32, F64):
        ref, _ = o.spmv(rp, col, ints.astype(dt), np.ones(N, dtype=dt))
        want = np.array([ints[rp[i]:rp[i + 1]].sum() for i in range(M)], dtype=np.float64)
        assert np.array_equal(ref, want), "integer row sums"
        ref, _ = o.spmv(rp, col, np.ones(rp[-1], dtype=dt), np.ones(N, dtype=dt))
        assert np.array_equal(ref, L.astype(np.float64)), "row lengths"


def _laplacian(n):
    """5-point Laplacian on an n x n grid built directly from the stencil."""
    rp, col, val = [0], [], []
    for r in range(n):
        for c in range(n):
            i = r * n + c
            for (rr, cc, v) in ((r - 1, c, -1.0), (r, c - 1, -1.0), (r, c, 4.0),
                                (r, c + 1, -1.0), (r + 1, c, -1.0)):
                if 0 <= rr < n and 0 <= cc < n:
                    col.append(rr * n + cc)
                    val.append(v)
            rp.append(len(col))
    return (np.array(rp, dtype=np.int32), np.array(col, dtype=np.int32),
            np.array(val, dtype=np.float64))


def pin_laplacian_closed_forms(o):
    """For the 5-point Laplacian: x = 1 gives 0 inside, 1 on edges, 2 at the
    corners; x = grid row index gives 0 inside; x = r^2 + c^2 gives -4 inside."""
    n = 24
    rp, col, val = _laplacian(n)
    r, c = np.divmod(np.arange(n * n), n)
    inner = (r > 0) & (r < n - 1) & (c > 0) & (c < n - 1)
    nbrs = 4 - (r == 0) - (r == n - 1) - (c == 0) - (c == n - 1)
    ref, _ = o.spmv(rp, col, val, np.ones(n * n))
    assert np.array_equal(ref, (4 - nbrs).astype(np.float64)), "laplacian x=1"
    ref, _ = o.spmv(rp, col, val, r.astype(np.float64))
    assert np.all(ref[inner] == 0.0), "laplacian x=r"
    ref, _ = o.spmv(rp, col, val, (r * r + c * c).astype(np.float64))
    assert np.all(ref[inner] == -4.0), "laplacian x=r^2+c^2"


def _small_random(seed, M=60, N=45, dt=F32):
    rng = np.random.default_rng(seed)
    L = rng.integers(0, 12, M)
    L[::7] = 0
    rp = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    col = np.concatenate([np.sort(rng.choice(N, l, replace=False)) for l in L]).astype(np.int32)
    val = rng.uniform(-1, 1, rp[-1]).astype(dt)
    x = rng.uniform(-1, 1, N).astype(dt)
    y0 = rng.uniform(-1, 1, M).astype(dt)
    return rp, col, val, x, y0


def pin_alpha_beta(o):
    """Power-of-two alpha scales the result exactly; beta = 0 ignores y_old
    (NaN there is harmless); empty rows give exactly beta * y_old; with
    beta != 0 the result changes by beta * y_old."""
    for dt in (F32, F64):
        rp, col, val, x, y0 = _small_random(4, dt=dt)
        base, s1 = o.spmv(rp, col, val, x, 1.0, 0.0)
        for a in (2.0, 0.5, -4.0):
            ra, sa = o.spmv(rp, col, val, x, a, 0.0)
            assert np.array_equal(ra, a * base), ("alpha scaling", a)
            assert np.array_equal(sa, s1), "scale independent of alpha"
        nan_y = np.full(y0.shape, np.nan, dtype=dt)
        r0, _ = o.spmv(rp, col, val, x, 1.0, 0.0, nan_y)
        assert np.array_equal(r0, base), "beta=0 must not read y"
        rb, _ = o.spmv(rp, col, val, x, 1.5, -0.5, y0)
        empty = np.diff(rp) == 0
        assert np.array_equal(rb[empty], -0.5 * y0[empty].astype(np.float64)), "empty rows"
        # away from empty rows: rb - 1.5*base equals -0.5*y0 up to one rounding
        yb = -0.5 * y0.astype(np.float64)
        d = rb - 1.5 * base - yb
        assert np.all(np.abs(d) <= 4e-16 * (np.abs(1.5 * base) + np.abs(yb) + 1.0)), "beta term"
        assert not np.array_equal(rb, 1.5 * base), "beta term present"


def pin_scale(o):
    """scale_i = sum |a_ik x_k|: equals the row sum when all products are
    non-negative and bounds |A x| otherwise."""
    rp, col, val, x, _ = _small_random(5, dt=F64)
    ref, scale = o.spmv(rp, col, np.abs(val), np.abs(x))
    assert np.array_equal(ref, scale), "scale = sum for non-negative"
    ref, scale = o.spmv(rp, col, val, x)
    assert np.all(scale >= np.abs(ref)), "scale bounds |y|"
    assert np.any(scale > np.abs(ref)), "scale uses absolute values"


def pin_rows_subset(o):
    """The row-subset evaluation equals the full evaluation on those rows."""
    for dt in (F32, F64):
        rp, col, val, x, y0 = _small_random(6, dt=dt)
        full, fs = o.spmv(rp, col, val, x, 1.5, 0.5, y0)
        rows = np.array([0, 3, 7, 59, 14, 14])
        sub, ss = o.spmv_rows(rows, rp, col, val, x, 1.5, 0.5, y0)
        assert np.array_equal(sub, full[rows]) and np.array_equal(ss, fs[rows]), "rows subset"


def split_invariants(rp, T, sr, sn):
    """Properties every correct merge-path split has."""
    M = rp.size - 1
    nnz = int(rp[-1])
    W = M + nnz
    P = (W + T - 1) // T
    assert sr.size == P + 1 and sn.size == P + 1
    assert sr[0] == 0 and sn[0] == 0 and sr[-1] == M and sn[-1] == nnz
    d = np.minimum(np.arange(P + 1, dtype=np.int64) * T, W)
    assert np.array_equal(sr.astype(np.int64) + sn, d), "i + j = diagonal"
    assert np.all(np.diff(sr) >= 0) and np.all(np.diff(sn) >= 0), "monotone"
    inner = sr < M
    assert np.all(rp[sr[inner]] <= sn[inner]) and np.all(sn[inner] <= rp[sr[inner] + 1]), \
        "nonzero coordinate inside the current row"
    assert np.all(sn[sr == M] == nnz)


def split_closed_form(rp, T):
    """i(d) = max{i : row_ptr[i] + i <= d}: the row ends that precede
    diagonal d, computed by sorted search instead of a walk."""
    M = rp.size - 1
    W = M + int(rp[-1])
    P = (W + T - 1) // T
    d = np.minimum(np.arange(P + 1, dtype=np.int64) * T, W)
    key = rp.astype(np.int64) + np.arange(M + 1)
    i = np.searchsorted(key, d, side="right") - 1
    return i.astype(np.int32), (d - i).astype(np.int32)


def pin_merge_splits(o):
    """The walk reproduces the hand-worked table of the worked example, the
    sorted-search closed form, and the split invariants, on edge cases."""
    g = read_golden("merge_splits_worked_T4.txt")
    rp = np.array(read_golden("rgcsr_worked_example.txt")["row_ptr"], dtype=np.int32)
    sr, sn = o.merge_splits(rp, g["T"][0])
    assert list(sr) == g["split_row"] and list(sn) == g["split_nz"], "worked split table"
    cases = [rp,
             np.array(read_golden("loadbalance_fig1_tiles.txt")["row_ptr"], dtype=np.int32),
             np.zeros(1, dtype=np.int32),                   # M = 0
             np.zeros(9, dtype=np.int32),                   # all rows empty
             np.array([0, 1000], dtype=np.int32)]           # one dense row
    rng = np.random.default_rng(8)
    for _ in range(6):
        L = rng.integers(0, 30, rng.integers(1, 400))
        L[rng.random(L.size) < 0.2] = 0
        cases.append(np.concatenate([[0], np.cumsum(L)]).astype(np.int32))
    for c in cases:
        for T in (1, 2, 3, 4, 7, 64, 1024):
            sr, sn = o.merge_splits(c, T)
            split_invariants(c, T, sr, sn)
            cr, cn = split_closed_form(c, T)
            assert np.array_equal(sr, cr) and np.array_equal(sn, cn), ("closed form", T)


def pin_bins(o):
    """Binning groups every row by length: a permutation, counts equal a
    histogram, each row in its bin's range, ascending within a bin."""
    rp = np.array(read_golden("rgcsr_worked_example.txt")["row_ptr"], dtype=np.int32)
    b, off, cnt = o.bins(rp, [1, 2])
    assert list(cnt) == [4, 3, 1] and list(b) == [1, 2, 3, 4, 0, 5, 7, 6], "worked bins"
    rng = np.random.default_rng(9)
    for edges in ([0], [0, 4, 32, 256], [3, 5, 9], [10 ** 6]):
        L = rng.integers(0, 400, 5000) * (rng.random(5000) < 0.9)
        rp = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
        b, off, cnt = o.bins(rp, edges)
        which = np.searchsorted(np.array(edges), L, side="left")
        assert np.array_equal(cnt, np.bincount(which, minlength=len(edges) + 1)), "counts"
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(cnt)])), "offsets"
        assert np.array_equal(np.sort(b), np.arange(L.size)), "permutation"
        for k in range(len(edges) + 1):
            seg = b[off[k]:off[k + 1]]
            assert np.all(which[seg] == k), "row in its bin"
            assert np.all(np.diff(seg) > 0), "ascending within a bin"


def _dense_matmat_ascending(A, X):
    """Y[i, c] = sum over j ascending of A_ij * X_jc in fp64, by hand, and the
    matching sums of |A_ij * X_jc|."""
    M, N = A.shape
    k = X.shape[1]
    Y = np.empty((M, k), dtype=np.float64)
    S = np.empty((M, k), dtype=np.float64)
    for c in range(k):
        Y[:, c], S[:, c] = _dense_matvec_ascending(A, X[:, c])
    return Y, S


def pin_spmm_dense(o):
    """CSR times a dense N x k matrix equals the dense product bit for bit
    (ascending sums) on tiny random non-square inputs with M, N, k distinct,
    and numpy's matrix product within fp64 rounding."""
    rng = np.random.default_rng(17)
    for trial in range(12):
        M, N, k = int(rng.integers(1, 30)), int(rng.integers(1, 30)), int(rng.integers(1, 9))
        while len({M, N, k}) < 3:
            N += 1
            k = k + 1 if k == M or k == N else k
        dt = F32 if trial % 2 == 0 else F64
        A = np.where(rng.random((M, N)) < 0.3, rng.uniform(-1, 1, (M, N)), 0.0).astype(dt)
        A[rng.random(M) < 0.2, :] = 0
        X = rng.uniform(-1, 1, (N, k)).astype(dt)
        rp, col, val = _csr_from_dense(A)
        ref, scale = o.spmm(rp, col, val, X)
        want, wscale = _dense_matmat_ascending(A, X)
        assert np.array_equal(ref, want), ("spmm dense", trial)
        assert np.array_equal(scale, wscale), ("spmm scale", trial)
        mm = A.astype(np.float64) @ X.astype(np.float64)
        assert np.allclose(ref, mm, rtol=0, atol=1e-12 * max(1, N)), ("spmm vs matmul", trial)


def pin_spmm_identity_and_laplacian(o):
    """A = I gives Y = alpha X + beta Y_old (dyadic alpha, beta: exact); for
    the 5-point Laplacian, column c of X equal to (c + 1) everywhere gives
    column c of Y equal to (c + 1) * (4 - neighbours)."""
    rng = np.random.default_rng(18)
    for dt in (F32, F64):
        n, k = 97, 5
        rp = np.arange(n + 1, dtype=np.int32)
        X = rng.uniform(-1, 1, (n, k)).astype(dt)
        Y0 = rng.uniform(-1, 1, (n, k)).astype(dt)
        ref, _ = o.spmm(rp, np.arange(n, dtype=np.int32), np.ones(n, dtype=dt), X, 2.0, -0.5, Y0)
        want = 2.0 * X.astype(np.float64) - 0.5 * Y0.astype(np.float64)
        assert np.array_equal(ref, want), "spmm identity"
    g = 12
    rp, col, val = _laplacian(g)
    r, c = np.divmod(np.arange(g * g), g)
    nbrs = 4 - (r == 0) - (r == g - 1) - (c == 0) - (c == g - 1)
    k = 6
    X = np.tile(np.arange(1, k + 1, dtype=np.float64), (g * g, 1))
    ref, _ = o.spmm(rp, col, val, X)
    want = (4 - nbrs)[:, None].astype(np.float64) * np.arange(1, k + 1)[None, :]
    assert np.array_equal(ref, want), "spmm laplacian"


def pin_spmm_alpha_beta(o):
    """alpha = -2 scales exactly; beta = 0 does not read Y_old (NaN there is
    harmless); empty rows give exactly beta * Y_old in every column."""
    for dt in (F32, F64):
        rp, col, val, x, _ = _small_random(19, dt=dt)
        rng = np.random.default_rng(20)
        X = rng.uniform(-1, 1, (x.size, 3)).astype(dt)
        Y0 = rng.uniform(-1, 1, (rp.size - 1, 3)).astype(dt)
        base, _ = o.spmm(rp, col, val, X)
        r2, _ = o.spmm(rp, col, val, X, -2.0, 0.0, np.full(Y0.shape, np.nan, dtype=dt))
        assert np.array_equal(r2, -2.0 * base), "spmm alpha / beta = 0"
        rb, _ = o.spmm(rp, col, val, X, 1.0, 0.5, Y0)
        empty = np.diff(rp) == 0
        assert np.array_equal(rb[empty], 0.5 * Y0[empty].astype(np.float64)), "spmm empty rows"
        assert not np.array_equal(rb, base), "spmm beta term present"


def pin_coo(o):
    """COO entries of a dense matrix (row-major scan) give the dense product
    bit for bit; shuffled entries with small-integer values give the exact
    integer row sums; rows without entries give beta * y_old exactly."""
    rng = np.random.default_rng(21)
    for trial in range(8):
        M, N = int(rng.integers(1, 30)), int(rng.integers(1, 30))
        dt = F32 if trial % 2 == 0 else F64
        A = np.where(rng.random((M, N)) < 0.3, rng.uniform(-1, 1, (M, N)), 0.0).astype(dt)
        A[rng.random(M) < 0.3, :] = 0
        x = rng.uniform(-1, 1, N).astype(dt)
        rows, cols = np.nonzero(A)
        ref, scale = o.spmv_coo(M, rows, cols, A[rows, cols], x)
        want, wscale = _dense_matvec_ascending(A, x)
        assert np.array_equal(ref, want) and np.array_equal(scale, wscale), ("coo dense", trial)
    M, N, nnz = 400, 300, 5000
    rows = rng.integers(0, M, nnz)
    rows[rows % 7 == 0] = 1                       # rows that are multiples of 7 stay empty
    cols = rng.integers(0, N, nnz)
    perm = rng.permutation(nnz)
    for dt in (F32, F64):
        ints = rng.choice(np.array([-1, 1, 2, 4]), nnz).astype(dt)
        y0 = rng.uniform(-1, 1, M).astype(dt)
        ref, _ = o.spmv_coo(M, rows[perm], cols[perm], ints[perm], np.ones(N, dt), 1.0, 0.5, y0)
        want = np.zeros(M)
        np.add.at(want, rows, ints.astype(np.float64))
        want = want + 0.5 * y0.astype(np.float64)
        assert np.array_equal(ref, want), "coo integer sums, shuffled"
        empty = np.setdiff1d(np.arange(M), rows)
        assert empty.size > 0 and np.array_equal(ref[empty], 0.5 * y0[empty].astype(np.float64))


def pin_transposed(o):
    """A^T x equals the hand-written dense product with A transposed, bit for
    bit (rows ascending), on non-square matrices; z . (A x) = x . (A^T z)
    exactly for small integers; the 5-point Laplacian (symmetric, columns of
    a row in the order its rows reach a column) gives A^T x = A x bit for bit."""
    rng = np.random.default_rng(22)
    for trial in range(10):
        M, N = int(rng.integers(1, 30)), int(rng.integers(1, 30))
        if M == N:
            N += 3
        dt = F32 if trial % 2 == 0 else F64
        A = np.where(rng.random((M, N)) < 0.3, rng.uniform(-1, 1, (M, N)), 0.0).astype(dt)
        A[:, rng.random(N) < 0.3] = 0                 # empty columns of A: rows of A^T
        x = rng.uniform(-1, 1, M).astype(dt)
        rp, col, val = _csr_from_dense(A)
        ref, scale = o.spmv_t(N, rp, col, val, x)
        want, wscale = _dense_matvec_ascending(np.ascontiguousarray(A.T), x)
        assert np.array_equal(ref, want) and np.array_equal(scale, wscale), ("A^T x", trial)
    M, N = 300, 200
    L = rng.integers(0, 15, M)
    rp = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    col = np.concatenate([np.sort(rng.choice(N, l, replace=False)) for l in L]).astype(np.int32)
    ints = rng.choice(np.array([-2, -1, 1, 3]), rp[-1]).astype(F64)
    x = rng.integers(-3, 4, N).astype(F64)
    z = rng.integers(-3, 4, M).astype(F64)
    ax, _ = o.spmv(rp, col, ints, x)
    atz, _ = o.spmv_t(N, rp, col, ints, z)
    assert float(np.dot(z, ax)) == float(np.dot(x, atz)), "adjoint identity"
    rp, col, val = _laplacian(9)
    xx = rng.uniform(-1, 1, 81)
    assert np.array_equal(o.spmv_t(81, rp, col, val, xx)[0], o.spmv(rp, col, val, xx)[0])


def pin_rgcsr_stored(o):
    """The worked example: groups of four rows store 7 artificial zeros
    beside the 13 entries, one group of all eight rows (ELLPACK) 11; random
    row lengths against a numpy reshape-and-max."""
    g = read_golden("rgcsr_worked_example.txt")
    rp = np.array(g["row_ptr"], dtype=np.int32)
    nnz = int(g["nnz"][0])
    assert o.rgcsr_stored(rp, int(g["rgcsr_group_size"][0])) - nnz == int(g["rgcsr_artificial_zeros"][0])
    assert o.rgcsr_stored(rp, 8) - nnz == int(g["ellpack_artificial_zeros"][0])
    rng = np.random.default_rng(23)
    for G in (1, 3, 4, 64, 100):
        L = rng.integers(0, 50, 1000)
        rp = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
        pad = (-L.size) % G
        Lp = np.concatenate([L, np.full(pad, -1)]).reshape(-1, G)
        rows = np.concatenate([np.full(Lp.shape[0] - 1, G), [G - pad]])
        assert o.rgcsr_stored(rp, G) == int((Lp.max(1) * rows).sum()), ("rgcsr stored", G)


ALL_PINS = [pin_dense_bruteforce, pin_identity, pin_diagonal, pin_integer_row_sums,
            pin_laplacian_closed_forms, pin_alpha_beta, pin_scale, pin_rows_subset,
            pin_merge_splits, pin_bins, pin_spmm_dense, pin_spmm_identity_and_laplacian,
            pin_spmm_alpha_beta, pin_coo, pin_transposed, pin_rgcsr_stored]
