"""Pins of the CSR SpMV oracle against facts that do not go through it.

* identity matrix: y = x exactly;
* 5-point Laplacian times all-ones: 4 minus the number of grid neighbours;
* Laplacian sine modes: A v = lambda v in closed form (bounded by the fp32
  rounding of the input vector, computed from the rounding error itself);
* dense brute force at n <= 256 with NumPy fp64 matmul (a different summation
  order), covering empty rows, unsorted and duplicate columns, beta != 0.
"""
import numpy as np
import pytest

import gen
import oracle


def test_identity_exact():
    n = 1000
    rp = np.arange(n + 1, dtype=np.int32)
    ci = np.arange(n, dtype=np.int32)
    v = np.ones(n, np.float32)
    x = np.random.default_rng(7).uniform(-1, 1, n).astype(np.float32)
    y, s = oracle.csr_spmv(rp, ci, v, x)
    assert np.array_equal(y, x.astype(np.float64))
    assert np.array_equal(s, np.abs(x).astype(np.float64))


@pytest.mark.parametrize("N", [7, 64, 1000])
def test_laplacian_times_ones(N):
    L = gen.laplacian_2d(N, with_x=False)
    y, _ = oracle.csr_spmv(L.row_ptr, L.col_idx, L.vals, np.ones(L.n_cols, np.float32))
    iy, ix = np.divmod(np.arange(N * N), N)
    neighbours = (ix > 0).astype(int) + (ix < N - 1) + (iy > 0) + (iy < N - 1)
    assert np.array_equal(y, (4 - neighbours).astype(np.float64))
    if N == 1000:
        vals, counts = np.unique(y, return_counts=True)
        assert dict(zip(vals.tolist(), counts.tolist())) == {0.0: 996004, 1.0: 3992, 2.0: 4}


@pytest.mark.parametrize("N,p,q", [(1000, 1, 1), (1000, 500, 500), (200, 3, 17), (64, 64, 1)])
def test_laplacian_sine_modes(N, p, q):
    L = gen.laplacian_2d(N, with_x=False)
    v, lam = gen.sine_mode(N, p, q)
    x32 = v.astype(np.float32)
    err = x32.astype(np.float64) - v              # exact rounding error of the input
    y, _ = oracle.csr_spmv(L.row_ptr, L.col_idx, L.vals, x32)
    # |A x32 - lam v| <= |A (x32 - v)| <= sum_j |a_ij| |err_j|, plus fp64 noise
    absA = np.abs(L.vals.astype(np.float64))
    rows = np.repeat(np.arange(L.n_rows), np.diff(L.row_ptr))
    bound = np.zeros(L.n_rows)
    np.add.at(bound, rows, absA * np.abs(err[L.col_idx]))
    resid = np.abs(y - lam * v)
    assert np.all(resid <= bound + 1e-12 * np.max(np.abs(v)))
    # the mode is not trivially reproduced by a wrong operator: a dropped
    # neighbour or a sign flip moves y far off lambda v
    assert np.max(np.abs(v)) > 0.9


def _dense_ref(n_rows, n_cols, rp, ci, v, x, alpha, beta, y_in):
    D = np.zeros((n_rows, n_cols))
    rows = np.repeat(np.arange(n_rows), np.diff(rp))
    np.add.at(D, (rows, ci), v.astype(np.float64))
    out = alpha * (D @ x.astype(np.float64))
    if beta != 0:
        out += beta * y_in.astype(np.float64)
    return out


@pytest.mark.parametrize("seed", range(6))
def test_dense_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    n_rows = int(rng.integers(1, 257))
    n_cols = int(rng.integers(1, 257))
    lens = rng.integers(0, min(n_cols, 40) + 1, n_rows)
    lens[rng.random(n_rows) < 0.2] = 0                     # empty rows
    A = gen.random_csr(n_rows, n_cols, lens, seed=seed, sorted_cols=(seed % 2 == 0))
    ci = A.col_idx.copy()
    if seed % 3 == 0 and A.nnz > 1:                         # duplicate columns
        for i in range(n_rows):
            a, b = A.row_ptr[i], A.row_ptr[i + 1]
            if b - a >= 2:
                ci[b - 1] = ci[a]
    alpha = float(rng.uniform(-2, 2))
    beta = 0.0 if seed % 2 else float(rng.uniform(-2, 2))
    y_in = rng.uniform(-1, 1, n_rows).astype(np.float32)
    y, s = oracle.csr_spmv(A.row_ptr, ci, A.vals, A.x, alpha, beta, y_in)
    ref = _dense_ref(n_rows, n_cols, A.row_ptr, ci, A.vals, A.x, alpha, beta, y_in)
    assert np.all(np.abs(y - ref) <= 1e-13 * s + 1e-300)
    # the scale is the absolute-value product
    rows = np.repeat(np.arange(n_rows), np.diff(A.row_ptr))
    sc = np.zeros(n_rows)
    np.add.at(sc, rows, np.abs(A.vals.astype(np.float64) * A.x[ci].astype(np.float64)))
    sc = abs(alpha) * sc + (abs(beta * y_in.astype(np.float64)) if beta else 0)
    assert np.allclose(s, sc, rtol=1e-13, atol=0)


def test_beta_zero_ignores_y_nan():
    """y is not read when beta == 0 (BLAS convention): NaN in y_in is harmless."""
    A = gen.random_csr(10, 10, [3] * 10, seed=1)
    y_in = np.full(10, np.nan, np.float32)
    y, _ = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x, 1.0, 0.0, y_in)
    assert np.all(np.isfinite(y))


def test_row_stats_against_numpy():
    A = gen.powerlaw_csr(n=20000, seed=9)
    lens = np.diff(A.row_ptr).astype(np.int64)
    assert oracle.row_stats(A.row_ptr) == (int(lens.max()), int(lens.sum()), int((lens * lens).sum()))
    assert oracle.row_stats(np.zeros(1, np.int32)) == (0, 0, 0)


def test_f64_valued_csr_matches_dense():
    rng = np.random.default_rng(3)
    A = gen.random_csr(50, 40, rng.integers(0, 10, 50), seed=3)
    v64 = A.vals.astype(np.float64) / 3.0
    y, s = oracle.csr_spmv_f64(A.row_ptr, A.col_idx, v64, A.x, 1.5, 0.0)
    D = np.zeros((50, 40))
    rows = np.repeat(np.arange(50), np.diff(A.row_ptr))
    np.add.at(D, (rows, A.col_idx), v64)
    assert np.all(np.abs(y - 1.5 * D @ A.x.astype(np.float64)) <= 1e-13 * s + 1e-300)


@pytest.mark.parametrize("seed", range(4))
def test_f64_vector_csr_matches_dense(seed):
    """y = A x with fp64 values and an fp64 x (the fp64 solver's matvec):
    NumPy dense brute force with duplicate columns and empty rows, and an
    exact closed form: the 1-D Laplacian (2, -1) applied to i^2 gives -2
    inside (second difference), exactly in fp64 for these small integers."""
    rng = np.random.default_rng(200 + seed)
    n_rows, n_cols = int(rng.integers(1, 200)), int(rng.integers(1, 200))
    lens = rng.integers(0, 12, n_rows)
    A = gen.random_csr(n_rows, n_cols, lens, seed=seed, sorted_cols=bool(seed % 2))
    ci = A.col_idx.copy()
    if A.nnz > 2:
        ci[-1] = ci[0]
    v64 = rng.standard_normal(A.nnz)
    x64 = rng.standard_normal(n_cols)
    y = oracle.csr_spmv_f64v(A.row_ptr, ci, v64, x64)
    D = np.zeros((n_rows, n_cols))
    rows = np.repeat(np.arange(n_rows), np.diff(A.row_ptr))
    np.add.at(D, (rows, ci), v64)
    scale = np.abs(D) @ np.abs(x64)
    assert np.all(np.abs(y - D @ x64) <= 1e-13 * scale + 1e-300)
    n = 50
    rp = np.arange(0, 3 * n + 1, 3, dtype=np.int32)
    cols = np.stack([np.arange(n) - 1, np.arange(n), np.arange(n) + 1], 1).clip(0, n - 1).astype(np.int32).ravel()
    vals = np.tile([-1.0, 2.0, -1.0], n)
    vals[0] = 0.0
    vals[-1] = 0.0
    y = oracle.csr_spmv_f64v(rp, cols, vals, np.arange(n, dtype=np.float64) ** 2)
    assert np.array_equal(y[1:-1], np.full(n - 2, -2.0))
