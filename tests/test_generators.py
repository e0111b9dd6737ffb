"""Statistics of the seeded input generators (inputs only; no method arithmetic)."""
import numpy as np

import gen


def test_tiny_shape_and_determinism():
    a = gen.tiny_csr()
    b = gen.tiny_csr()
    assert a.nnz == 32768 and a.n_rows == 4096
    assert np.array_equal(a.col_idx, b.col_idx) and np.array_equal(a.vals, b.vals)
    c = a.col_idx.reshape(4096, 8)
    assert np.all(np.diff(c, axis=1) > 0)
    assert a.vals.dtype == np.float32 and np.all(np.abs(a.vals) <= 1)


def test_laplacian_counts():
    L = gen.laplacian_2d(1000)
    assert L.nnz == 5 * 1000 ** 2 - 4 * 1000 == 4_996_000
    assert np.all(np.diff(L.row_ptr) >= 3) and np.max(np.diff(L.row_ptr)) == 5
    diag = L.vals[L.col_idx == np.repeat(np.arange(L.n_rows), np.diff(L.row_ptr))]
    assert np.all(diag == 4.0)


def test_powerlaw_statistics():
    P = gen.powerlaw_csr()
    lens = np.diff(P.row_ptr)
    assert P.n_rows == 916_428
    assert lens.min() >= 1 and lens.max() <= 4334
    # calibrated mean 5.5703, standard error of the total about 9e4
    assert abs(P.nnz - 5_104_804) < 5 * 9.0e4
    # distinct sorted columns per row
    rows = np.repeat(np.arange(P.n_rows), lens)
    key = rows.astype(np.int64) * P.n_cols + P.col_idx
    assert np.all(np.diff(key) > 0)
    assert P.vals.min() >= 0 and P.vals.max() < 1


def test_pruned_exact_k_and_no_zero_values():
    for s, k in [(0.5, 6144), (0.7, 3686), (0.9, 1229)]:
        W = gen.pruned_weight(s, n_rows=8, n_cols=12288)
        assert np.all(np.diff(W.row_ptr) == k)
        assert np.all(W.vals_f16 & 0x7FFF != 0)
        for i in range(8):
            c = W.col_idx[W.row_ptr[i]:W.row_ptr[i + 1]]
            assert np.all(np.diff(c) > 0) and c[0] >= 0 and c[-1] < 12288
        std = W.vals_f16.view(np.float16).astype(np.float64).std()
        assert abs(std - 0.02) < 0.002


def test_fe_mesh_structure():
    M = gen.fe_mesh(3, 2, 2, clamp_x0=False)
    assert M.n_dof == 3 * 4 * 3 * 3
    # every element has 8 distinct nodes; DOFs of one node are consecutive
    for e in range(M.n_elem):
        d = M.edof[e].reshape(8, 3)
        assert np.all(d[:, 1] == d[:, 0] + 1) and np.all(d[:, 2] == d[:, 0] + 2)
        assert len(set(d[:, 0].tolist())) == 8
    assert np.allclose(M.Ke, M.Ke.T)
    assert np.linalg.eigvalsh(M.Ke.astype(np.float64)).min() >= 1.0 - 1e-5


def test_stencil_structure():
    offs = (-5, 0, 3)
    A = gen.stencil_csr(20, offs, seed=1)
    rows = [A.col_idx[A.row_ptr[i]:A.row_ptr[i + 1]].tolist() for i in range(20)]
    for i, r in enumerate(rows):
        assert r == [i + d for d in sorted(offs) if 0 <= i + d < 20]
    assert A.vals.dtype == np.float32 and len(A.vals) == A.nnz
    B = gen.stencil_csr(20, offs, seed=1)
    assert np.array_equal(A.vals, B.vals) and np.array_equal(A.x, B.x)
