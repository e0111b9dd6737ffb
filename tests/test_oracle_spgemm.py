"""Pins of the SpGEMM oracle (C = A*B, Gustavson rows with a dense fp64
accumulator; the hash-based multi-phase SpGEMM page, sections 1.1 and 2.1).

* the pattern equals SciPy's boolean product of the patterns (nonnegative
  values cannot cancel), and the values SciPy's product, on random
  rectangular matrices with empty rows and columns;
* NumPy dense brute force on small matrices (values and, with exact zeros
  kept, the column sets);
* closed forms: the square of the 1-D Laplacian (pentadiagonal 1 -4 6 -4 1,
  boundary rows 5 -4 1) and of the 2-D 5-point Laplacian (13-point stencil
  20 / -8 / 2 / 1) in exact integers; permutation times permutation is the
  composed permutation;
* intermediate products: sum over k in row i of nnz(B row k), checked by
  NumPy, and the identity's IP = row lengths of B; the row groups of
  section 2.1.1 (0-31, 32-511, 512-8191, >= 8192) by NumPy digitize.
"""
import numpy as np
import pytest
import scipy.sparse as sp

import gen
import oracle


def _csr(M):
    M = sp.csr_matrix(M)
    M.sort_indices()
    return M.indptr.astype(np.int32), M.indices.astype(np.int32), M.data.astype(np.float32)


def _rand(m, n, density, seed, positive=False):
    rng = np.random.default_rng(seed)
    M = sp.random(m, n, density=density, format="csr", random_state=rng, dtype=np.float64)
    if not positive:
        M.data = rng.uniform(-1, 1, M.nnz)
    M.data = M.data.astype(np.float32).astype(np.float64)
    if m > 3:
        M = sp.csr_matrix(M.toarray() * (np.arange(m) % 7 != 3)[:, None])   # some empty rows
    return M


@pytest.mark.parametrize("shape,seed", [((40, 30, 50), 0), ((200, 150, 120), 1), ((1, 5, 1), 2), ((64, 64, 64), 3)])
def test_pattern_and_values_vs_scipy(shape, seed):
    m, k, n = shape
    A, B = _rand(m, k, 0.08, seed), _rand(k, n, 0.1, seed + 10)
    rpc, cic, vc, sc = oracle.spgemm(n, *_csr(A), *_csr(B))
    P = (abs(A) @ abs(B)).tocsr()          # nonnegative: the structural pattern
    P.sort_indices()
    assert np.array_equal(rpc, P.indptr) and np.array_equal(cic, P.indices)
    C = (A @ B).toarray()
    assert np.allclose(vc, C[np.repeat(np.arange(m), np.diff(rpc)), cic], rtol=1e-12, atol=1e-12)
    assert np.allclose(sc, P.data, rtol=1e-12)
    for i in range(m):                       # increasing columns in each row
        assert np.all(np.diff(cic[rpc[i]:rpc[i + 1]]) > 0)


def test_dense_brute_force_with_cancellation():
    A = np.array([[1, -1, 0], [0, 0, 0], [2, 0, 1]], np.float64)
    B = np.array([[1, 0, 3], [1, 0, 3], [0, 4, 0]], np.float64)
    rpc, cic, vc, sc = oracle.spgemm(3, *_csr(A), *_csr(B))
    # row 0: columns 0 and 2 are reached but cancel to exactly 0, and stay
    assert rpc.tolist() == [0, 2, 2, 5]
    assert cic.tolist() == [0, 2, 0, 1, 2]
    assert vc.tolist() == [0.0, 0.0, 2.0, 4.0, 6.0]
    assert sc.tolist() == [2.0, 6.0, 2.0, 4.0, 6.0]


def _lap1d(n):
    return sp.diags([-np.ones(n - 1), 2 * np.ones(n), -np.ones(n - 1)], [-1, 0, 1], format="csr")


def test_laplacian_1d_squared_closed_form():
    n = 9
    rpc, cic, vc, _ = oracle.spgemm(n, *_csr(_lap1d(n)), *_csr(_lap1d(n)))
    for i in range(n):
        row = dict(zip(cic[rpc[i]:rpc[i + 1]].tolist(), vc[rpc[i]:rpc[i + 1]].tolist()))
        want = {i - 2: 1.0, i - 1: -4.0, i: 6.0, i + 1: -4.0, i + 2: 1.0}
        if i == 0 or i == n - 1:
            want[i] = 5.0
        want = {c: v for c, v in want.items() if 0 <= c < n}
        assert row == want, (i, row)


def test_laplacian_2d_squared_stencil():
    N = 7
    L = gen.laplacian_2d(N, with_x=False)
    rpc, cic, vc, _ = oracle.spgemm(L.n_cols, L.row_ptr, L.col_idx, L.vals, L.row_ptr, L.col_idx, L.vals)
    i0 = 3 * N + 3                                   # interior node (3, 3)
    row = dict(zip(cic[rpc[i0]:rpc[i0 + 1]].tolist(), vc[rpc[i0]:rpc[i0 + 1]].tolist()))
    want = {i0: 20.0}
    for d in (1, -1, N, -N):
        want[i0 + d] = -8.0
        want[i0 + 2 * d] = 1.0
    for d in (N + 1, N - 1, -N + 1, -N - 1):
        want[i0 + d] = 2.0
    assert row == want
    assert np.diff(rpc).max() == 13


def test_permutations_compose():
    n = 50
    rng = np.random.default_rng(4)
    p, q = rng.permutation(n), rng.permutation(n)
    P = sp.csr_matrix((np.ones(n), (np.arange(n), p)), shape=(n, n))
    Q = sp.csr_matrix((np.ones(n), (np.arange(n), q)), shape=(n, n))
    rpc, cic, vc, _ = oracle.spgemm(n, *_csr(P), *_csr(Q))
    assert rpc.tolist() == list(range(n + 1)) and np.array_equal(cic, q[p]) and np.all(vc == 1.0)


def test_intermediate_products_and_groups():
    A = gen.powerlaw_csr(20000, seed=5)
    ip = oracle.spgemm_ip(A.row_ptr, A.col_idx, A.row_ptr)
    deg = np.diff(A.row_ptr).astype(np.int64)
    want = np.array([deg[A.col_idx[A.row_ptr[i]:A.row_ptr[i + 1]]].sum() for i in range(A.n_rows)])
    assert np.array_equal(ip, want)
    eye = np.arange(A.n_rows + 1, dtype=np.int32)
    assert np.array_equal(oracle.spgemm_ip(eye, np.arange(A.n_rows, dtype=np.int32), A.row_ptr), deg)
    g = np.array([oracle.row_bin(int(min(x, 2 ** 31 - 1))) for x in ip])
    assert np.array_equal(g, np.digitize(ip, [32, 512, 8192]))
