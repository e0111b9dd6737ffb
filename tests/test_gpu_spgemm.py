"""GPU parity of the hash-based multi-phase SpGEMM (C = A*B) against the
oracle, through the C ABI.

* row pointers and column indices of C bit-exact with the oracle's (each
  row's distinct columns in increasing order, cancelled sums kept); values
  |c - c_ref| <= 1e-5 * sum |a_ik b_kj| (fp32 products and atomic sums);
* random rectangular products with empty rows, repeated columns in A's rows
  and rows of B of many lengths, so that every IP group (0-31, 32-511,
  512-8191, >= 8192) is exercised, with the group sizes equal to the
  oracle's intermediate-product counts;
* the square of the 2-D Laplacian (1000 x 1000 grid) in full, and the square
  of the 916k-row power-law matrix on every row of the global-table group
  plus sampled rows of the others;
* recomputation after the values change, empty products, and rejection of
  out-of-range columns.
"""
import numpy as np
import pytest
import scipy.sparse as sp

import gen
import oracle
from helpers import TAU_F32, dev, host

torch = pytest.importorskip("torch")
S = pytest.importorskip("sparse_matrix_vector_amd")

pytestmark = pytest.mark.gpu


def _run(m, k, n, A, B):
    """A, B: (rp, ci, v) host arrays.  Returns the GPU (rp, ci, v) and the handle's info."""
    arrs = [dev(np.asarray(x)) for x in (*A, *B)]
    G = S.SpGEMM(m, k, n, *arrs)
    rp, ci, v = G.compute()
    torch.cuda.synchronize()
    info = (G.nnz, G.intermediate_products, G.group_rows)
    G.close()
    return host(rp), host(ci), host(v), info


def _check(n, A, B, got, rows=None):
    rp, ci, v, info = got
    if rows is None:
        orp, oci, ov, osc = oracle.spgemm(n, *A, *B)
        assert np.array_equal(rp, orp), "row pointers"
        assert np.array_equal(ci, oci), "columns"
        err = np.abs(v.astype(np.float64) - ov)
        assert np.all(err <= TAU_F32 * osc), float(np.max(err / np.maximum(osc, 1e-300)))
        return
    # rows of C depend only on the same rows of A
    rpa, cia, va = A
    sub_rp = np.concatenate([[0], np.cumsum(rpa[rows + 1] - rpa[rows])]).astype(np.int32)
    sub_ci = np.concatenate([cia[rpa[r]:rpa[r + 1]] for r in rows]).astype(np.int32)
    sub_v = np.concatenate([va[rpa[r]:rpa[r + 1]] for r in rows]).astype(np.float32)
    orp, oci, ov, osc = oracle.spgemm(n, sub_rp, sub_ci, sub_v, *B)
    for q, r in enumerate(rows):
        a, b = rp[r], rp[r + 1]
        oa, ob = orp[q], orp[q + 1]
        assert b - a == ob - oa, r
        assert np.array_equal(ci[a:b], oci[oa:ob]), r
        assert np.all(np.abs(v[a:b].astype(np.float64) - ov[oa:ob]) <= TAU_F32 * osc[oa:ob]), r


def _csr(M):
    M = sp.csr_matrix(M)
    return M.indptr.astype(np.int32), M.indices.astype(np.int32), M.data.astype(np.float32)


def _mixed(seed):
    """A (m x k) with repeated columns and empty rows; B (k x n) whose row
    lengths span 0..3000, so that A's rows fall in all four IP groups."""
    rng = np.random.default_rng(seed)
    k, n, m = 3000, 5000, 1200
    blens = np.where(rng.random(k) < 0.02, rng.integers(500, 3000, k), rng.integers(0, 12, k))
    B = gen.random_csr(k, n, blens, seed)
    alens = np.where(rng.random(m) < 0.1, rng.integers(20, 60, m), rng.integers(0, 5, m))
    alens[::37] = 0
    heavy = np.flatnonzero(blens >= 500)
    alens[[5, 600]] = 40                                   # rows that reach only long rows of B (group 3)
    rows = np.repeat(np.arange(m), alens)
    cols = rng.integers(0, k, len(rows)).astype(np.int32)
    cols[1::50] = cols[0::50][:len(cols[1::50])]           # some repeated (row, column) pairs
    rp0 = np.concatenate([[0], np.cumsum(alens)])
    for r in (5, 600):
        cols[rp0[r]:rp0[r + 1]] = rng.choice(heavy, 40)
    order = np.lexsort((cols, rows))
    rp = np.concatenate([[0], np.cumsum(alens)]).astype(np.int32)
    A = (rp, cols[order], rng.uniform(-1, 1, len(rows)).astype(np.float32))
    return m, k, n, A, (B.row_ptr, B.col_idx, B.vals)


@pytest.mark.parametrize("seed", [0, 1])
def test_mixed_groups(seed):
    m, k, n, A, B = _mixed(seed)
    got = _run(m, k, n, A, B)
    ip = oracle.spgemm_ip(A[0], A[1], B[0])
    groups = np.bincount(np.digitize(ip, [32, 512, 8192]), minlength=4).tolist()
    print(f"[spgemm] mixed seed={seed} groups={got[3][2]} nnz={got[3][0]}", flush=True)
    assert got[3][2] == groups and got[3][1] == int(ip.sum())
    assert all(g > 0 for g in groups)
    _check(n, A, B, got)


def test_global_rows_many_sorted_runs():
    """Global-table rows whose C row has more than 16,384 entries (sorted in
    LDS runs, then merged): one of 47,455 entries (three runs, two merge
    passes, an uneven last run), one of 19,806 (two runs) and one of 16,592
    (a 208-entry second run), next to small rows."""
    rng = np.random.default_rng(41)
    k, n = 6000, 400_000
    B = gen.random_csr(k, n, rng.integers(8, 17, k), seed=42)
    alens = np.array([4200, 0, 3, 1700, 1, 1400, 7], dtype=np.int64)
    rows = np.repeat(np.arange(len(alens)), alens)
    cols = np.concatenate([np.sort(rng.choice(k, L, replace=False)) for L in alens]).astype(np.int32)
    rp = np.concatenate([[0], np.cumsum(alens)]).astype(np.int32)
    A = (rp, cols, rng.uniform(-1, 1, len(rows)).astype(np.float32))
    Bt = (B.row_ptr, B.col_idx, B.vals)
    got = _run(len(alens), k, n, A, Bt)
    lens = np.diff(got[0])
    print(f"[spgemm] long rows nnz per row={lens.tolist()} groups={got[3][2]}", flush=True)
    assert lens[0] > 2 * 16384 and 16384 < lens[3] <= 2 * 16384 and lens[5] > 16384 and got[3][2][3] == 3
    _check(n, A, Bt, got)


@pytest.mark.parametrize("shape", [(30, 40, 20), (1, 1, 1), (200, 50, 300)])
def test_small_random(shape):
    m, k, n = shape
    rng = np.random.default_rng(sum(shape))
    A = _csr(sp.random(m, k, density=0.2, random_state=rng, format="csr"))
    B = _csr(sp.random(k, n, density=0.2, random_state=rng, format="csr"))
    _check(n, A, B, _run(m, k, n, A, B))


def test_laplacian_squared_full():
    L = gen.laplacian_2d(1000, with_x=False)
    A = (L.row_ptr, L.col_idx, L.vals)
    got = _run(L.n_rows, L.n_cols, L.n_cols, A, A)
    print(f"[spgemm] laplacian^2 nnz={got[3][0]}", flush=True)
    _check(L.n_cols, A, A, got)


def test_powerlaw_squared_sampled():
    P = gen.powerlaw_csr()
    A = (P.row_ptr, P.col_idx, P.vals)
    got = _run(P.n_rows, P.n_cols, P.n_cols, A, A)
    ip = oracle.spgemm_ip(P.row_ptr, P.col_idx, P.row_ptr)
    g = np.digitize(ip, [32, 512, 8192])
    rng = np.random.default_rng(7)
    rows = np.concatenate([np.flatnonzero(g == 3)] +
                          [rng.choice(np.flatnonzero(g == q), 1500, replace=False) for q in range(3)])
    print(f"[spgemm] powerlaw^2 nnz={got[3][0]} ip={got[3][1]} groups={got[3][2]}", flush=True)
    assert got[3][2] == np.bincount(g, minlength=4).tolist()
    assert got[0][-1] == got[3][0]
    _check(P.n_cols, A, A, got, rows=np.sort(rows))


def test_recompute_after_value_change_and_empty():
    m, k, n, A, B = _mixed(3)
    arrs = [dev(np.asarray(x)) for x in (*A, *B)]
    G = S.SpGEMM(m, k, n, *arrs)
    out = G.compute()
    arrs[2].mul_(-2.0)                                   # new values of A, same pattern
    G.compute(out)
    torch.cuda.synchronize()
    A2 = (A[0], A[1], (A[2] * np.float32(-2.0)).astype(np.float32))
    _check(n, A2, B, (host(out[0]), host(out[1]), host(out[2]), None))
    G.close()
    # a product with no entries
    Z = (np.zeros(5, np.int32), np.zeros(0, np.int32), np.zeros(0, np.float32))
    rp, ci, v, info = _run(4, 3, 6, Z, (np.zeros(4, np.int32), np.zeros(0, np.int32), np.zeros(0, np.float32)))
    assert info[0] == 0 and np.array_equal(rp, np.zeros(5, np.int32))


def test_rejects_bad_columns():
    rp = np.array([0, 2], np.int32)
    ci = np.array([0, 3], np.int32)                      # column 3 outside k = 3
    v = np.ones(2, np.float32)
    B = (np.array([0, 1, 1, 2], np.int32), np.array([0, 1], np.int32), np.ones(2, np.float32))
    with pytest.raises(S.SpmvError) as e:
        _run(1, 3, 2, (rp, ci, v), B)
    assert e.value.status == 2
