"""Pins of the FE solver oracle (oracle/solver.py) and of the elasticity
element matrix it is run on.

* hex8 elasticity Ke (generator input): symmetric; exactly six zero
  eigenvalues whose null space holds the three translations and three
  rotations; the patch test -- for each of the six unit strain states the
  nodal energy u^T Ke u equals eps^T D eps of the unit cube exactly;
* Jacobi diagonal: equals the diagonal of the assembled operator (the C
  oracle's assembly, separate code) and, for one element, rho^p diag(Ke);
* PCG: one iteration on a diagonal matrix; termination within the number of
  distinct eigenvalues on a constant-diagonal (circulant) matrix; agreement
  with a direct solve on random SPD and FE systems; the iteration cap;
* power / inverse iteration: the closed-form extreme eigenvalues
  2 - 2 cos(k pi / (n + 1)) of the 1-D Dirichlet Laplacian, and LAPACK's
  eigenvalues of small assembled cantilevers.
"""
import numpy as np
import pytest
import scipy.sparse as sp
import scipy.sparse.linalg as sla

import gen
import oracle


def _D(E=1.0, nu=0.3):
    lam, mu = E * nu / ((1 + nu) * (1 - 2 * nu)), E / (2 * (1 + nu))
    D = np.zeros((6, 6))
    D[:3, :3] = lam
    D[range(3), range(3)] = lam + 2 * mu
    D[range(3, 6), range(3, 6)] = mu
    return D


def _nodal(field):
    X = gen.HEX8_LOCAL_NODES.astype(np.float64)
    return np.array([field(p) for p in X]).reshape(-1)


@pytest.mark.parametrize("nu", [0.3, 0.0, 0.45])
def test_elasticity_ke(nu):
    K = gen.hex8_elasticity_ke(2.0, nu)
    assert np.array_equal(K, K.T)
    w = np.linalg.eigvalsh(K)
    assert np.all(np.abs(w[:6]) < 1e-12 * w[-1]) and w[6] > 1e-3 * w[-1]
    rigid = [_nodal(lambda p, c=c: np.eye(3)[c]) for c in range(3)]
    rigid += [_nodal(lambda p, a=a: np.cross(np.eye(3)[a], p)) for a in range(3)]
    for u in rigid:
        assert np.max(np.abs(K @ u)) < 1e-12
    D = _D(2.0, nu)
    for k in range(6):
        eps = np.zeros(6)
        eps[k] = 1.0
        E3 = np.array([[eps[0], eps[3] / 2, eps[5] / 2], [eps[3] / 2, eps[1], eps[4] / 2],
                       [eps[5] / 2, eps[4] / 2, eps[2]]])
        u = _nodal(lambda p: E3 @ p)
        assert abs(u @ K @ u - eps @ D @ eps) < 1e-12


def _fe_K(m):
    rp, ci, v = oracle.fe_assemble(m.edof, m.rho, m.Ke, m.n_dof, m.penalty)
    return sp.csr_matrix((v, ci, rp), shape=(m.n_dof, m.n_dof))


def test_diagonal_matches_assembly_and_one_element():
    m = gen.fe_mesh(7, 5, 3, seed=8)
    d = oracle.fe_diagonal(m.edof, m.rho, m.Ke, m.n_dof, m.penalty)
    assert np.allclose(d, _fe_K(m).diagonal(), rtol=1e-14, atol=0)   # summation order differs
    one = gen.fe_mesh(1, 1, 1, seed=9, clamp_x0=False)
    d1 = oracle.fe_diagonal(one.edof, one.rho, one.Ke, one.n_dof, 3)
    assert np.allclose(d1[one.edof[0]], float(one.rho[0]) ** 3 * np.diag(one.Ke.astype(np.float64)), rtol=1e-15)


def test_pcg_diagonal_system_one_iteration():
    d = np.linspace(1.0, 50.0, 40)
    f = np.random.default_rng(0).standard_normal(40)
    u, it, rr = oracle.pcg_jacobi(lambda x: d * x, d, f, rtol=1e-14)
    assert it == 1 and np.allclose(u, f / d, rtol=1e-15)


def test_pcg_terminates_within_distinct_eigenvalues():
    # symmetric circulant, constant diagonal 4: eigenvalues 4 - 2 cos(2 pi k / 8),
    # five distinct values, and Jacobi only rescales
    n = 8
    c = np.zeros(n)
    c[0], c[1], c[-1] = 4.0, -1.0, -1.0
    A = np.array([[c[(j - i) % n] for j in range(n)] for i in range(n)])
    assert len(np.unique(np.round(np.linalg.eigvalsh(A), 12))) == 5
    f = np.random.default_rng(1).standard_normal(n)
    u, it, rr = oracle.pcg_jacobi(lambda x: A @ x, np.diag(A), f, rtol=1e-13, max_iter=50)
    assert it <= 5 and np.allclose(u, np.linalg.solve(A, f), rtol=1e-11, atol=1e-12)


def test_pcg_random_spd_and_cap():
    rng = np.random.default_rng(2)
    G = rng.standard_normal((60, 60))
    A = G @ G.T + 60 * np.eye(60)
    f = rng.standard_normal(60)
    u, it, rr = oracle.pcg_jacobi(lambda x: A @ x, np.diag(A), f, rtol=1e-12, max_iter=200)
    assert rr <= 1e-12 and np.allclose(u, np.linalg.solve(A, f), rtol=1e-9)
    u3, it3, rr3 = oracle.pcg_jacobi(lambda x: A @ x, np.diag(A), f, rtol=1e-12, max_iter=3)
    assert it3 == 3 and rr3 > 1e-12


@pytest.mark.parametrize("dims", [(4, 2, 2), (10, 4, 3)])
def test_pcg_fe_matches_direct_solve(dims):
    m = gen.fe_cantilever(*dims)
    K = _fe_K(m)
    d = oracle.fe_diagonal(m.edof, m.rho, m.Ke, m.n_dof, m.penalty)
    u, it, rr = oracle.pcg_jacobi(lambda x: K @ x, d, m.f, rtol=1e-11, max_iter=5000)
    ud = sla.spsolve(K.tocsc(), m.f.astype(np.float64))
    assert rr <= 1e-11
    assert np.linalg.norm(u - ud) <= 1e-6 * np.linalg.norm(ud)


def test_power_and_inverse_closed_form():
    n = 20
    A = 2 * np.eye(n) - np.eye(n, k=1) - np.eye(n, k=-1)
    lmax = 2 - 2 * np.cos(n * np.pi / (n + 1))
    lmin = 2 - 2 * np.cos(np.pi / (n + 1))
    v0 = np.random.default_rng(3).standard_normal(n)
    lam = oracle.power_lambda_max(lambda x: A @ x, v0, 1500)
    assert abs(lam[-1] - lmax) < 1e-9 and np.all(np.diff(lam) >= -1e-12)   # Rayleigh quotients rise
    mu = oracle.inverse_lambda_min(lambda x: A @ x, lambda b: np.linalg.solve(A, b), v0, 40)
    assert abs(mu[-1] - lmin) < 1e-12


@pytest.mark.parametrize("dims", [(4, 2, 2), (12, 6, 3)])
def test_cantilever_extreme_eigenvalues(dims):
    m = gen.fe_cantilever(*dims)
    K = _fe_K(m)
    w = np.linalg.eigvalsh(K.toarray())
    v0 = np.random.default_rng(4).standard_normal(m.n_dof)
    lam = oracle.power_lambda_max(lambda x: K @ x, v0, 3000)
    lu = sla.splu(K.tocsc())
    mu = oracle.inverse_lambda_min(lambda x: K @ x, lu.solve, v0, 30)
    assert abs(lam[-1] - w[-1]) <= 2e-3 * w[-1]
    assert abs(mu[-1] - w[0]) <= 1e-10 * w[0]
