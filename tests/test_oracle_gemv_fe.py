"""Pins of the dense fp16 GEMV oracle and of the finite-element operator oracle.

Dense GEMV:
* equals a NumPy fp64 product and the MACKO oracle on the densified matrix.

FE operator (element loop and assembled CSR):
* assembled nonzero count equals the closed form 9 (3nx-2)(3ny+1)(3nz+1)
  with the x = 0 face clamped, and 9 (3nx+1)(3ny+1)(3nz+1) without;
* a single unconstrained element assembles to rho^3 Ke exactly;
* a 2x2x2 mesh against a dense NumPy assembly (brute force);
* with a translation-free element matrix the unconstrained operator maps each
  rigid translation to (numerically) zero, which any edof error would break;
* symmetry x^T K y = y^T K x and positivity x^T K x > 0 with an SPD Ke;
* the element loop equals the assembled CSR applied by the pinned CSR oracle.
"""
import numpy as np
import pytest

import gen
import oracle


def test_gemv_against_numpy_and_macko():
    W = gen.pruned_weight(0.5, n_rows=40, n_cols=300, seed=5)
    D = W.dense_f16()
    y_in = np.linspace(-1, 1, 40).astype(np.float32)
    y, s = oracle.gemv_f16(D, W.x_f16, 0.75, 0.5, y_in)
    ref = 0.75 * D.view(np.float16).astype(np.float64) @ W.x_f16.view(np.float16).astype(np.float64) \
        + 0.5 * y_in.astype(np.float64)
    assert np.all(np.abs(y - ref) <= 1e-13 * s)
    mrp, codes, mv = oracle.macko_encode(300, W.row_ptr, W.col_idx, W.vals_f16)
    y2, _ = oracle.macko_spmv(300, mrp, codes, mv, W.x_f16, 0.75, 0.5, y_in)
    assert np.all(np.abs(y - y2) <= 1e-13 * s)


def _closed_form_nnz(nx, ny, nz, clamp):
    return 9 * ((3 * nx - 2) if clamp else (3 * nx + 1)) * (3 * ny + 1) * (3 * nz + 1)


@pytest.mark.parametrize("dims,clamp", [((1, 1, 1), False), ((2, 2, 2), True), ((4, 3, 2), True),
                                        ((6, 3, 3), False), ((12, 6, 3), True)])
def test_assembled_nnz_closed_form(dims, clamp):
    M = gen.fe_mesh(*dims, clamp_x0=clamp)
    rp, ci, v = oracle.fe_assemble(M.edof, M.rho, M.Ke, M.n_dof)
    assert len(ci) == _closed_form_nnz(*dims, clamp)
    assert rp[-1] == len(ci)
    # full-size values of the closed form (the 120x60x30 cantilever)
    assert _closed_form_nnz(120, 60, 30, True) == 53_069_562
    assert _closed_form_nnz(120, 60, 30, False) == 53_514_279


def test_single_element_is_scaled_ke():
    M = gen.fe_mesh(1, 1, 1, clamp_x0=False)
    rp, ci, v = oracle.fe_assemble(M.edof, M.rho, M.Ke, M.n_dof)
    K = np.zeros((24, 24))
    rows = np.repeat(np.arange(24), np.diff(rp))
    K[rows, ci] = v
    perm = M.edof[0]                          # local DOF a -> global DOF
    s = float(M.rho[0]) ** 3
    assert np.array_equal(K[np.ix_(perm, perm)], s * M.Ke.astype(np.float64))


def _dense_fe(M, Ke=None):
    Ke = M.Ke if Ke is None else Ke
    K = np.zeros((M.n_dof, M.n_dof))
    for e in range(M.n_elem):
        d = M.edof[e]
        keep = d >= 0
        s = float(M.rho[e]) ** M.penalty
        K[np.ix_(d[keep], d[keep])] += s * Ke.astype(np.float64)[np.ix_(keep, keep)]
    return K


@pytest.mark.parametrize("clamp", [True, False])
def test_small_mesh_brute_force(clamp):
    M = gen.fe_mesh(2, 2, 2, clamp_x0=clamp, seed=8)
    K = _dense_fe(M)
    rng = np.random.default_rng(2)
    y_in = rng.uniform(-1, 1, M.n_dof).astype(np.float32)
    for alpha, beta in [(1.0, 0.0), (-2.0, 0.5)]:
        y, s = oracle.fe_matvec(M.edof, M.rho, M.Ke, M.x, M.n_dof, 3, alpha, beta, y_in)
        ref = alpha * K @ M.x.astype(np.float64) + (beta * y_in.astype(np.float64) if beta else 0)
        assert np.all(np.abs(y - ref) <= 1e-13 * s + 1e-300)


def test_translation_null_space():
    Kt = gen.fe_ke_translation_free(seed=5)
    M = gen.fe_mesh(5, 4, 3, clamp_x0=False, seed=6)
    for c in range(3):
        t = np.zeros(M.n_dof, np.float32)
        t[c::3] = 1.0                               # unconstrained: DOF = 3*node + c
        y, s = oracle.fe_matvec(M.edof, M.rho, Kt.astype(np.float32), t, M.n_dof, 3)
        # fp32 rounding of Kt is the only error source: |Kt32 - Kt| row sums
        err = np.abs(Kt.astype(np.float32).astype(np.float64) - Kt).sum(axis=1).max()
        assert np.max(np.abs(y)) <= 8 * err * 1.0001 + 1e-12
        assert np.max(s) > 1.0                      # the scale is far from zero
    # the clamped mesh has no such null space
    Mc = gen.fe_mesh(5, 4, 3, clamp_x0=True, seed=6)
    t = np.zeros(Mc.n_dof, np.float32)
    t[0::3] = 1.0
    y, _ = oracle.fe_matvec(Mc.edof, Mc.rho, Kt.astype(np.float32), t, Mc.n_dof, 3)
    assert np.max(np.abs(y)) > 1e-3


def test_symmetry_positivity_and_assembled_equals_element_loop():
    M = gen.fe_mesh(6, 5, 4, seed=10)
    rng = np.random.default_rng(1)
    a = rng.uniform(-1, 1, M.n_dof).astype(np.float32)
    b = rng.uniform(-1, 1, M.n_dof).astype(np.float32)
    Ka, _ = oracle.fe_matvec(M.edof, M.rho, M.Ke, a, M.n_dof)
    Kb, _ = oracle.fe_matvec(M.edof, M.rho, M.Ke, b, M.n_dof)
    lhs = float(b.astype(np.float64) @ Ka)
    rhs = float(a.astype(np.float64) @ Kb)
    assert abs(lhs - rhs) <= 1e-12 * (abs(lhs) + 1)
    assert float(a.astype(np.float64) @ Ka) > 0
    rp, ci, v = oracle.fe_assemble(M.edof, M.rho, M.Ke, M.n_dof)
    y1, s1 = oracle.fe_matvec(M.edof, M.rho, M.Ke, M.x, M.n_dof, 3, 0.5, 0.0)
    y2, s2 = oracle.csr_spmv_f64(rp, ci, v, M.x, 0.5, 0.0)
    assert np.all(np.abs(y1 - y2) <= 1e-12 * s1 + 1e-300)
    # element-wise scale bounds the assembled one
    assert np.all(s2 <= s1 * (1 + 1e-12))


def test_full_mesh_sizes():
    M = gen.fe_mesh()
    assert M.n_elem == 216_000 and M.n_dof == 680_760
    assert int((M.edof < 0).sum()) == 60 * 30 * 4 * 3
    assert M.edof.max() == M.n_dof - 1
