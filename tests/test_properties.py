"""Property tests of the oracle on small random CSR matrices (Hypothesis,
derandomised): no rows, empty rows, unsorted and repeated columns, one row of
8,192-12,000 entries.  Each property is checked against something outside the
oracle: NumPy dense products and sorts, or closed-form counts.

* CSR: y = alpha A x + beta y_in within 1e-13 of NumPy's dense fp64 product
  (relative to the absolute-value scale), and the scale is sum |a x|;
* row grouping: perm is a permutation, groups are contiguous and in order,
  rows ascend inside a group, group sizes are NumPy's counts;
* ELL (width = longest row) and HYB (any width) give the CSR oracle's
  result bit for bit, and HYB's tail sizes are NumPy's counts;
* MACKO (sorted distinct columns, nonzero fp16 values): decoding returns the
  input entries, pads only add zero values, and the entry count is the
  closed form sum(ceil(gap / 2^b)) rounded up to 1024 / b per row.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from strategies import csr_matrices

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


def _dense(A, ci=None):
    D = np.zeros((A.n_rows, A.n_cols))
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr))
    np.add.at(D, (rows, A.col_idx if ci is None else ci), A.vals.astype(np.float64))
    return D


@SETTINGS
@given(csr_matrices(), st.floats(-2, 2), st.sampled_from([0.0, 1.0, -0.5]))
def test_csr_matches_numpy(A, alpha, beta):
    y_in = np.linspace(-1, 1, A.n_rows).astype(np.float32)
    y, s = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x, alpha, beta, y_in)
    D = _dense(A)
    ref = alpha * (D @ A.x.astype(np.float64)) + (beta * y_in.astype(np.float64) if beta else 0.0)
    rows = np.repeat(np.arange(A.n_rows), np.diff(A.row_ptr))
    sc = np.zeros(A.n_rows)
    np.add.at(sc, rows, np.abs(A.vals.astype(np.float64) * A.x[A.col_idx].astype(np.float64)))
    sc = abs(alpha) * sc + (np.abs(beta * y_in.astype(np.float64)) if beta else 0.0)
    assert np.allclose(s, sc, rtol=1e-12, atol=0)
    assert np.all(np.abs(y - ref) <= 1e-13 * sc + 1e-300)


@SETTINGS
@given(csr_matrices(), st.sampled_from([(32, 512, 8192), (128, 512, 8192), (2, 5, 9), (1, 2, 3)]))
def test_row_grouping_invariants(A, thr):
    off, perm = oracle.bins(A.row_ptr, thr)
    lens = np.diff(A.row_ptr)
    grp = np.digitize(lens, thr)
    assert np.array_equal(np.sort(perm), np.arange(A.n_rows))
    assert off[0] == 0 and off[-1] == A.n_rows
    for g in range(4):
        seg = perm[off[g]:off[g + 1]]
        assert off[g + 1] - off[g] == int((grp == g).sum())
        assert np.all(grp[seg] == g) and np.all(np.diff(seg) > 0)


@SETTINGS
@given(csr_matrices(), st.integers(0, 14))
def test_ell_and_hyb_equal_csr(A, w):
    y, _ = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x)
    W = int(np.diff(A.row_ptr).max()) if A.n_rows else 0
    if A.n_rows and W * A.n_rows <= 4_000_000:
        ec, ev = oracle.ell_from_csr(A.row_ptr, A.col_idx, A.vals, W)
        ye, _ = oracle.ell_spmv(A.n_rows, W, ec, ev, A.x)
        assert np.array_equal(ye, y)
    lens = np.diff(A.row_ptr).astype(np.int64)
    assert oracle.hyb_tail_size(A.row_ptr, w) == (int((lens > w).sum()), int(np.maximum(lens - w, 0).sum()))
    parts = oracle.hyb_from_csr(A.row_ptr, A.col_idx, A.vals, w)
    yh, _ = oracle.hyb_spmv(A.n_rows, w, *parts, A.x)
    assert np.array_equal(yh, y)


@SETTINGS
@given(csr_matrices(max_cols=3000, sorted_distinct=True), st.sampled_from([1, 2, 4, 8]))
def test_macko_round_trip_and_size(A, b):
    v16 = A.vals.astype(np.float16)
    v16[v16 == 0] = np.float16(0.5)
    vb = v16.view(np.uint16)
    mrp, codes, mv = oracle.macko_encode(A.n_cols, A.row_ptr, A.col_idx, vb, bdelta=b)
    cols = oracle.macko_decode(mrp, codes, bdelta=b)
    span, align = 1 << b, 1024 // b
    for i in range(A.n_rows):
        c = A.col_idx[A.row_ptr[i]:A.row_ptr[i + 1]].astype(np.int64)
        gaps = np.diff(np.concatenate([[-1], c]))
        n = int(np.sum(-(-gaps // span)))
        assert mrp[i + 1] - mrp[i] == -(-n // align) * align
        seg_c, seg_v = cols[mrp[i]:mrp[i + 1]], mv[mrp[i]:mrp[i + 1]]
        real = seg_v != 0
        assert np.array_equal(seg_c[real], c) and np.array_equal(seg_v[real], vb[A.row_ptr[i]:A.row_ptr[i + 1]])
        assert np.all(seg_v[~real] == 0)
