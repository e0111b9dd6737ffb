"""Property tests of the GPU CSR paths against the oracle (Hypothesis,
derandomised, bounded example counts), through the C ABI.

Small random CSR matrices with no rows, empty rows, unsorted and repeated
columns, and one row of 8,192-12,000 entries (split into chunk tasks by the
binned planner): every variant (scalar, vector, binned) meets
|y - y_ref| <= 1e-5 * scale with random alpha and beta (y not read when
beta = 0: it starts as NaN), the binned plan's row grouping is the oracle's
bit for bit, and the ELL conversion at the longest row's width is the
oracle's bit for bit.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from helpers import TAU_F32, assert_close, dev, host
from strategies import csr_matrices

torch = pytest.importorskip("torch")
S = pytest.importorskip("sparse_matrix_vector_amd")

pytestmark = pytest.mark.gpu

SETTINGS = settings(max_examples=80, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large,
                                           HealthCheck.function_scoped_fixture])


# alpha is an fp32 argument of the C ABI: drawn as fp32 values, 0 or of
# normal magnitude (the oracle applies it in fp64)
ALPHA = st.floats(-2, 2, width=32).filter(lambda a: a == 0.0 or abs(a) >= 1e-3)


@SETTINGS
@given(csr_matrices(), st.sampled_from(["scalar", "vector", "binned"]), ALPHA, st.sampled_from([0.0, 1.0, -0.75]))
def test_csr_variants_match_oracle(A, variant, alpha, beta):
    var = {"scalar": S.CSR_SCALAR, "vector": S.CSR_VECTOR, "binned": S.CSR_BINNED}[variant]
    rp, ci, v = dev(A.row_ptr), dev(A.col_idx), dev(A.vals)
    M = S.CSRMatrix(A.n_rows, A.n_cols, rp, ci, v, var)
    y_in = np.linspace(-1, 1, A.n_rows).astype(np.float32)
    y = dev(y_in) if beta else torch.full((A.n_rows,), float("nan"), device="cuda")
    M.apply(dev(A.x), y, alpha, beta)
    torch.cuda.synchronize()
    yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x, alpha, beta, y_in)
    assert_close(host(y), yr, sc, TAU_F32, f"{variant} n={A.n_rows} nnz={len(A.col_idx)}")
    if var == S.CSR_BINNED and A.n_rows:
        thr = (128, 512, 8192)
        perm = torch.empty(A.n_rows, dtype=torch.int32, device="cuda")
        off = M.plan(perm)
        ooff, operm = oracle.bins(A.row_ptr, thr)
        assert list(off) == list(ooff) and np.array_equal(host(perm), operm)
    M.close()


@SETTINGS
@given(csr_matrices())
def test_ell_conversion_matches_oracle(A):
    if A.n_rows == 0:
        return
    W = int(np.diff(A.row_ptr).max())
    if W == 0 or W * A.n_rows > 4_000_000:
        return
    ec = torch.empty(W * A.n_rows, dtype=torch.int32, device="cuda")
    ev = torch.empty(W * A.n_rows, dtype=torch.float32, device="cuda")
    S.spmv_ell_from_csr(A.n_rows, A.n_cols, dev(A.row_ptr), dev(A.col_idx), dev(A.vals), W, ec, ev)
    oec, oev = oracle.ell_from_csr(A.row_ptr, A.col_idx, A.vals, W)
    assert np.array_equal(host(ec), oec) and np.array_equal(host(ev).view(np.uint32), oev.view(np.uint32))
    y = torch.full((A.n_rows,), float("nan"), device="cuda")
    S.spmv_ell_apply(A.n_rows, A.n_cols, W, ec, ev, 1.0, dev(A.x), 0.0, y)
    torch.cuda.synchronize()
    yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x)
    assert_close(host(y), yr, sc, TAU_F32, "ell")
