"""Oracle of the FE solver step -- TEST INFRASTRUCTURE ONLY.

Plain fp64 NumPy, one statement per step of the textbook algorithms, so that
each function can be read against its definition:

* ``fe_diagonal``: the diagonal of the assembled stiffness operator,
  K_dd = sum over elements e and local DOFs a with edof[e, a] = d of
  rho_e^p Ke[a, a] -- the Jacobi preconditioner the fused-FE page's solver
  uses ("Fused GPU SpMV kernel optimisation", section 6.1);
* ``pcg_jacobi``: conjugate gradients preconditioned by that diagonal
  (section 6.1: Jacobi-PCG around the matvec, with an iteration cap);
* ``power_lambda_max`` / ``inverse_lambda_min``: the power iteration the
  page's section 4.1 uses to estimate the condition number of K, for the
  largest eigenvalue, and the same iteration on K^-1 (each step a solve) for
  the smallest; kappa = lambda_max / lambda_min.

The operator is passed in as a function (``matvec``), e.g. the assembled fp64
CSR of ``oracle.fe_assemble`` through SciPy, so the steps here do not depend
on how K is stored.  Only the tests, the smoke check and the bench's CPU leg
may import this module.
"""
from __future__ import annotations

import numpy as np


def fe_diagonal(edof, rho, Ke, n_dof, penalty=3):
    """fp64 diagonal of sum_e rho_e^p P_e^T Ke P_e (constrained entries of
    edof, i.e. outside [0, n_dof), are skipped)."""
    ed = np.asarray(edof, np.int64).reshape(-1, 24)
    w = np.asarray(rho, np.float64) ** penalty
    kd = np.diag(np.asarray(Ke, np.float64).reshape(24, 24))
    d = np.zeros(n_dof)
    contrib = w[:, None] * kd[None, :]
    ok = (ed >= 0) & (ed < n_dof)
    np.add.at(d, ed[ok], contrib[ok])
    return d


def pcg_jacobi(matvec, diag, f, u0=None, rtol=1e-6, max_iter=1000):
    """Solves K u = f.  Stops when ||r|| <= rtol ||f|| (r the recursively
    updated residual) or after max_iter iterations.
    Returns (u, iterations, ||r|| / ||f||)."""
    f = np.asarray(f, np.float64)
    dinv = 1.0 / np.asarray(diag, np.float64)
    u = np.zeros_like(f) if u0 is None else np.array(u0, np.float64)
    r = f - matvec(u)
    z = dinv * r
    p = z.copy()
    rz = r @ z
    ff = f @ f
    it = 0
    while it < max_iter and r @ r > rtol * rtol * ff:
        q = matvec(p)
        alpha = rz / (p @ q)
        u = u + alpha * p
        r = r - alpha * q
        it += 1
        if r @ r <= rtol * rtol * ff:
            break
        z = dinv * r
        rz_new = r @ z
        beta = rz_new / rz
        rz = rz_new
        p = z + beta * p
    return u, it, float(np.sqrt((r @ r) / ff)) if ff > 0 else 0.0


def power_lambda_max(matvec, v0, iters):
    """Power iteration: v <- K v / ||K v|| from v0; returns the Rayleigh
    quotients v^T K v of the normalised iterates (the last one is the
    estimate of the largest eigenvalue)."""
    v = np.asarray(v0, np.float64)
    v = v / np.linalg.norm(v)
    lam = []
    for _ in range(iters):
        w = matvec(v)
        lam.append(float(v @ w))
        v = w / np.linalg.norm(w)
    return np.array(lam)


def inverse_lambda_min(matvec, solve, v0, iters):
    """Power iteration on K^-1: v <- w / ||w|| with K w = v (``solve``);
    returns the Rayleigh quotients v^T K v of the normalised iterates (the
    last one estimates the smallest eigenvalue)."""
    v = np.asarray(v0, np.float64)
    v = v / np.linalg.norm(v)
    lam = []
    for _ in range(iters):
        w = solve(v)
        v = w / np.linalg.norm(w)
        lam.append(float(v @ matvec(v)))
    return np.array(lam)
