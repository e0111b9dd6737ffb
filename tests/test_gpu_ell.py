"""GPU parity of the ELL path against the oracle, through the C ABI.

* conversion: ell_col / ell_val bit-exact with the oracle's slot-major
  layout (Laplacian at full size, tiny, ragged shapes with n % 4 != 0);
* apply: |y - y_ref| <= 1e-5 * scale, four-rows-per-lane and one-row paths,
  alpha / beta, width larger than needed, width 0;
* a width shorter than the longest row is rejected.
"""
import numpy as np
import pytest

import gen
import oracle
from helpers import TAU_F32, assert_close, dev, host

torch = pytest.importorskip("torch")
S = pytest.importorskip("sparse_matrix_vector_amd")

pytestmark = pytest.mark.gpu


def _convert(A, width):
    ec = torch.empty(A.n_rows * width, dtype=torch.int32, device="cuda")
    ev = torch.empty(A.n_rows * width, dtype=torch.float32, device="cuda")
    S.spmv_ell_from_csr(A.n_rows, A.n_cols, dev(A.row_ptr), dev(A.col_idx), dev(A.vals), width, ec, ev)
    return ec, ev


CASES = {
    "laplacian": lambda: gen.laplacian_2d(1000),
    "tiny": lambda: gen.tiny_csr(),
    "ragged": lambda: gen.random_csr(1003, 800, np.random.default_rng(1).integers(0, 9, 1003), seed=1),
    "single": lambda: gen.random_csr(1, 10, [4], seed=2),
}


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("extra", [0, 3])
def test_convert_and_apply(case, extra):
    A = CASES[case]()
    W = oracle.row_stats(A.row_ptr)[0] + extra
    print(f"[ell] {case} W={W}", flush=True)
    ec, ev = _convert(A, W)
    oec, oev = oracle.ell_from_csr(A.row_ptr, A.col_idx, A.vals, W)
    assert np.array_equal(host(ec), oec)
    assert np.array_equal(host(ev).view(np.uint32), oev.view(np.uint32))
    rng = np.random.default_rng(7)
    y_in = rng.uniform(-1, 1, A.n_rows).astype(np.float32)
    for alpha, beta in [(1.0, 0.0), (-0.5, 2.0)]:
        y = dev(y_in) if beta else torch.full((A.n_rows,), float("nan"), device="cuda")
        S.spmv_ell_apply(A.n_rows, A.n_cols, W, ec, ev, alpha, dev(A.x), beta, y)
        yr, sc = oracle.ell_spmv(A.n_rows, W, oec, oev, A.x, alpha, beta, y_in)
        assert_close(host(y), yr, sc, TAU_F32, f"{case}/{alpha}/{beta}")


def test_width_too_small_rejected():
    A = gen.random_csr(10, 10, [1, 5, 2, 0, 3, 3, 3, 3, 3, 3], seed=0)
    with pytest.raises(S.SpmvError) as e:
        _convert(A, 4)
    assert e.value.status == 1


def test_width_zero_scales_y():
    y = torch.tensor([1.0, -2.0, 3.0, 4.0], device="cuda")
    S.spmv_ell_apply(4, 4, 0, torch.zeros(0, dtype=torch.int32, device="cuda"),
                     torch.zeros(0, device="cuda"), 1.0, torch.zeros(4, device="cuda"), 0.5, y)
    assert host(y).tolist() == [0.5, -1.0, 1.5, 2.0]


def test_bit_reproducible_and_equal_to_csr_order():
    A = gen.laplacian_2d(300)
    ec, ev = _convert(A, 5)
    x = dev(A.x)
    y1 = torch.empty(A.n_rows, device="cuda")
    y2 = torch.empty(A.n_rows, device="cuda")
    S.spmv_ell_apply(A.n_rows, A.n_cols, 5, ec, ev, 1.0, x, 0.0, y1)
    S.spmv_ell_apply(A.n_rows, A.n_cols, 5, ec, ev, 1.0, x, 0.0, y2)
    assert torch.equal(y1, y2)
