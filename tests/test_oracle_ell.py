"""Pins of the ELL conversion and ELL SpMV oracle.

* Laplacian: width 5 and exactly 4N padding slots (closed form);
* round trip ELL -> CSR rebuilt with NumPy equals the input;
* ELL SpMV equals the (independently pinned) CSR oracle bit for bit, since
  the pages' ELL computes the same sum in the same order;
* padding slots never read x (NaN in x at an unused column stays out).
"""
import numpy as np
import pytest

import gen
import oracle


@pytest.mark.parametrize("N", [5, 33, 1000])
def test_laplacian_padding_closed_form(N):
    L = gen.laplacian_2d(N)
    W = oracle.row_stats(L.row_ptr)[0]
    assert W == 5
    ec, ev = oracle.ell_from_csr(L.row_ptr, L.col_idx, L.vals, W)
    assert int((ec < 0).sum()) == 4 * N
    assert np.all(ev[ec < 0] == 0) and not np.any(np.signbit(ev[ec < 0]))


def _ell_to_csr(n, W, ec, ev):
    E = ec.reshape(W, n).T
    V = ev.reshape(W, n).T
    lens = (E >= 0).sum(axis=1)
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return rp, E[E >= 0], V[E >= 0]


@pytest.mark.parametrize("seed", range(3))
def test_round_trip_and_spmv(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 500))
    lens = rng.integers(0, 12, n)
    A = gen.random_csr(n, n, lens, seed=seed)
    W = int(lens.max()) + int(seed)            # also wider than needed
    ec, ev = oracle.ell_from_csr(A.row_ptr, A.col_idx, A.vals, W)
    rp, ci, v = _ell_to_csr(n, W, ec, ev)
    assert np.array_equal(rp, A.row_ptr) and np.array_equal(ci, A.col_idx) and np.array_equal(v, A.vals)
    y_in = rng.uniform(-1, 1, n).astype(np.float32)
    for alpha, beta in [(1.0, 0.0), (-0.5, 2.0)]:
        y1, s1 = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x, alpha, beta, y_in)
        y2, s2 = oracle.ell_spmv(n, W, ec, ev, A.x, alpha, beta, y_in)
        assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


def test_width_too_small_rejected():
    A = gen.random_csr(4, 8, [1, 5, 2, 0], seed=0)
    with pytest.raises(ValueError):
        oracle.ell_from_csr(A.row_ptr, A.col_idx, A.vals, 4)


def test_padding_does_not_touch_x():
    A = gen.random_csr(3, 4, [1, 2, 0], seed=1)
    x = A.x.copy()
    unused = sorted(set(range(4)) - set(A.col_idx.tolist()))
    x[unused] = np.nan
    ec, ev = oracle.ell_from_csr(A.row_ptr, A.col_idx, A.vals, 3)
    y, _ = oracle.ell_spmv(3, 3, ec, ev, x)
    assert np.all(np.isfinite(y))
