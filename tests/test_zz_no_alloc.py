"""GPU check of fem_matvec_threestage_noalloc, the FE three-stage matvec whose
per-element vectors live in the library's static device scratch (no
workspace, no allocation), called through the C ABI with ctypes.

Two calls in a row, the second on a smaller mesh: each result is compared
with fem_matvec_threestage (the workspace form) on the same inputs and with
the oracle's element loop, |y - y_ref| <= 1e-5 * scale for the oracle (the
required bound) and 2e-5 * scale between the two GPU forms (each within
1e-5 of the exact sum).  The first mesh (216,000 elements) runs as four
chunks of the 65,536-element scratch; the second (455 elements) as one
partial chunk over what the first left in the scratch.
"""
import ctypes

import numpy as np
import pytest

import gen
import oracle
from helpers import TAU_F32, assert_close, dev, host

torch = pytest.importorskip("torch")
S = pytest.importorskip("sparse_matrix_vector_amd")

pytestmark = pytest.mark.gpu


def _noalloc(M, x, alpha, beta, y):
    L = S.lib()
    edof, rho, Ke = dev(M.edof.reshape(-1)), dev(M.rho), dev(M.Ke.reshape(-1))
    stream = torch.cuda.current_stream().cuda_stream
    st = L.fem_matvec_threestage_noalloc(M.n_elem, M.n_dof, edof.data_ptr(), rho.data_ptr(), M.penalty,
                                         Ke.data_ptr(), ctypes.c_float(alpha), x.data_ptr(), ctypes.c_float(beta),
                                         y.data_ptr(), stream)
    assert st == 0, L.spmv_last_error()
    torch.cuda.synchronize()
    return host(y)


def _workspace_form(M, x, alpha, beta, y):
    ws = torch.empty(S.fem_threestage_size(M.n_elem), dtype=torch.uint8, device="cuda")
    S.fem_matvec_threestage(M.n_elem, M.n_dof, dev(M.edof.reshape(-1)), dev(M.rho), M.penalty,
                            dev(M.Ke.reshape(-1)), alpha, x, beta, y, ws)
    torch.cuda.synchronize()
    return host(y)


def test_noalloc_matches_workspace_form_two_calls():
    rng = np.random.default_rng(21)
    for dims, alpha, beta in [((120, 60, 30), 1.0, 0.0), ((13, 7, 5), -0.5, 1.5)]:
        M = gen.fe_mesh(*dims, seed=4)
        print(f"[noalloc] mesh {dims}: {M.n_elem} elements, alpha={alpha} beta={beta}", flush=True)
        y_in = rng.uniform(-1, 1, M.n_dof).astype(np.float32)
        x = dev(M.x)
        a = _noalloc(M, x, alpha, beta, dev(y_in))
        b = _workspace_form(M, x, alpha, beta, dev(y_in))
        yr, sc = oracle.fe_matvec(M.edof, M.rho, M.Ke, M.x, M.n_dof, M.penalty, alpha, beta, y_in)
        assert_close(a, yr, sc, TAU_F32, f"noalloc {dims} vs oracle")
        assert_close(a, b.astype(np.float64), sc, 2 * TAU_F32, f"noalloc {dims} vs workspace form")


def test_noalloc_validation_and_empty():
    L = S.lib()
    # host-side validation before any launch
    assert L.fem_matvec_threestage_noalloc(-1, 4, None, None, 3, None, ctypes.c_float(1.0), None,
                                           ctypes.c_float(0.0), None, None) == 1
    assert L.fem_matvec_threestage_noalloc(4, 10, 16, 16, 9, 16, ctypes.c_float(1.0), 16, ctypes.c_float(0.0),
                                           16, None) == 1            # penalty > 8
    # no elements: y = beta * y
    y = torch.tensor([1.0, -2.0, 4.0], device="cuda")
    S.fem_matvec_threestage_noalloc(0, 3, torch.zeros(0, dtype=torch.int32, device="cuda"),
                                    torch.zeros(0, device="cuda"), 3, torch.zeros(576, device="cuda"), 1.0,
                                    torch.zeros(3, device="cuda"), 0.5, y)
    torch.cuda.synchronize()
    assert host(y).tolist() == [0.5, -1.0, 2.0]
