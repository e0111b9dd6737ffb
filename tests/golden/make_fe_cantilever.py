"""Writes tests/golden/fe_cantilever.json from the CPU oracle alone.

The cantilever of gen.fe_cantilever at 80 x 40 x 20 (64k elements) and
120 x 60 x 30 (216k elements), assembled in fp64 by oracle.fe_assemble and
applied by the oracle's fp64 CSR product: the fp64 Jacobi-PCG iteration count at rtol 1e-6, the
compliance f.u of a tight solve (rtol 1e-10), and the extreme eigenvalues by
the oracle's power iteration (400 steps) and inverse iteration (4 steps,
inner PCG at rtol 1e-9), all from the start vector the GPU tests use
(standard normal, default_rng(5), rounded to fp32).

Run from the repository root: python tests/golden/make_fe_cantilever.py
(about 15 minutes on one core).
"""
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import gen  # noqa: E402
import oracle  # noqa: E402


def main():
    out = {"source": "fused-FE page, sections 4.1 (kappa by power iteration at 64k / 216k / 512k elements: "
                     "6.1e5 / 1.3e6 / 2.3e6, rho = 0.5) and 6.1 (Jacobi-PCG); values computed by this script "
                     "with the fp64 oracle", "cases": {}}
    for dims in [(80, 40, 20), (120, 60, 30)]:
        t0 = time.time()
        m = gen.fe_cantilever(*dims)
        rp, ci, v = oracle.fe_assemble(m.edof, m.rho, m.Ke, m.n_dof, m.penalty)
        mv = lambda x: oracle.csr_spmv_f64v(rp, ci, v, x)  # noqa: E731
        d = oracle.fe_diagonal(m.edof, m.rho, m.Ke, m.n_dof, m.penalty)
        f = m.f.astype(np.float64)
        _, it6, _ = oracle.pcg_jacobi(mv, d, f, rtol=1e-6, max_iter=20000)
        u, it10, rr10 = oracle.pcg_jacobi(mv, d, f, rtol=1e-10, max_iter=50000)
        v0 = np.random.default_rng(5).standard_normal(m.n_dof).astype(np.float32).astype(np.float64)
        lam = oracle.power_lambda_max(mv, v0, 400)
        solve = lambda b: oracle.pcg_jacobi(mv, d, b, rtol=1e-9, max_iter=50000)[0]  # noqa: E731
        mu = oracle.inverse_lambda_min(mv, solve, v0, 4)
        key = "x".join(map(str, dims))
        out["cases"][key] = {
            "n_elem": m.n_elem, "n_dof": m.n_dof, "pcg_iterations_rtol_1e-6": it6,
            "pcg_iterations_rtol_1e-10": it10, "compliance": float(f @ u),
            "lambda_max_power_400": float(lam[-1]), "lambda_max_power_100": float(lam[99]),
            "lambda_min_inverse": [float(x) for x in mu], "kappa": float(lam[-1] / mu[-1])}
        print(key, out["cases"][key], f"{time.time() - t0:.0f}s", flush=True)
    with open(os.path.join(ROOT, "tests", "golden", "fe_cantilever.json"), "w") as fh:
        json.dump(out, fh, indent=1)


if __name__ == "__main__":
    main()
