"""GPU assembly of the FE stiffness matrix in CSR (fem_assemble_*) against the
oracle's fp64 assembly (COO sorted, duplicates merged), through the C ABI.

* the pattern (row pointers and columns) is bit-exact with the oracle's on
  small meshes and the 40 x 20 x 10 mesh; every value is the oracle's fp64
  entry rounded to fp32, within one fp32 rounding step (the GPU sums an
  entry's element terms in fp64 in another order than the oracle's merge);
* on the full 120 x 60 x 30 mesh (the oracle's assembly takes about a
  minute there), properties that hold at any size: nnz is the closed form
  9 (3 nx - 2)(3 ny + 1)(3 nz + 1) = 53,069,562, every row's length is 3 x
  the free nodes among the node's grid neighbours (NumPy, from the mesh
  coordinates), columns increase within rows;
* the CSR SpMV on the assembled K agrees with the element-loop oracle within
  1e-5 of the element-wise scale, at every size;
* a row with more than 256 candidates is rejected.
"""
import numpy as np
import pytest

import gen
import oracle
from helpers import TAU_F32, assert_close, dev, host

torch = pytest.importorskip("torch")
S = pytest.importorskip("sparse_matrix_vector_amd")

pytestmark = pytest.mark.gpu


def _assemble(M):
    return S.fem_assemble_csr(M.n_elem, M.n_dof, dev(M.edof.reshape(-1)), dev(M.rho), M.penalty,
                              dev(M.Ke.reshape(-1)))


def _spmv_check(M, rp, ci, v, tag):
    A = S.CSRMatrix(M.n_dof, M.n_dof, rp, ci, v)
    y = torch.full((M.n_dof,), float("nan"), device="cuda")
    A.apply(dev(M.x), y)
    torch.cuda.synchronize()
    yr, sc = oracle.fe_matvec(M.edof, M.rho, M.Ke, M.x, M.n_dof)
    assert_close(host(y), yr, sc, TAU_F32, f"assembled CSR {tag}")


@pytest.mark.parametrize("dims,clamp", [((1, 1, 1), False), ((3, 2, 2), True), ((13, 7, 5), False),
                                        ((40, 20, 10), True)])
def test_assembly_matches_oracle(dims, clamp):
    M = gen.fe_mesh(*dims, clamp_x0=clamp, seed=8)
    print(f"[assemble] {dims}: {M.n_elem} elements, {M.n_dof} DOFs", flush=True)
    rp, ci, v = _assemble(M)
    orp, oci, ov = oracle.fe_assemble(M.edof, M.rho, M.Ke, M.n_dof, M.penalty)
    assert np.array_equal(host(rp), orp)
    assert np.array_equal(host(ci), oci)
    gv = host(v).astype(np.float64)
    ulp = np.spacing(np.abs(ov).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(gv - ov) <= ulp), float(np.max(np.abs(gv - ov) / ulp))
    _spmv_check(M, rp, ci, v, str(dims))


def test_full_mesh_properties():
    nx, ny, nz = 120, 60, 30
    M = gen.fe_mesh(nx, ny, nz, seed=4)
    rp, ci, v = _assemble(M)
    hrp, hci = host(rp), host(ci)
    assert hrp[-1] == 9 * (3 * nx - 2) * (3 * ny + 1) * (3 * nz + 1) == 53_069_562
    # row length of a free DOF at node (ix, iy, iz): 3 x the free nodes (ix' > 0)
    # among its neighbours (ix' - ix, iy' - iy, iz' - iz in {-1, 0, 1}) on the grid
    nnx, nny, nnz_ = nx + 1, ny + 1, nz + 1
    ix, iy, iz = np.meshgrid(np.arange(nnx), np.arange(nny), np.arange(nnz_), indexing="ij")
    ix, iy, iz = (a.transpose(2, 1, 0).reshape(-1) for a in (ix, iy, iz))

    def span(c, n, lo=0):
        return np.minimum(c + 1, n - 1) - np.maximum(c - 1, lo) + 1
    nb = span(ix, nnx, lo=1) * span(iy, nny) * span(iz, nnz_)
    free_nodes = ix > 0
    want = np.repeat(3 * nb[free_nodes], 3)
    assert np.array_equal(np.diff(hrp), want)
    starts = hrp[:-1]
    d = np.diff(hci.astype(np.int64))
    d[starts[1:] - 1] = 1                      # row boundaries
    assert np.all(d > 0)
    _spmv_check(M, rp, ci, v, "120x60x30")


def test_rejects_rows_with_too_many_candidates():
    # 11 elements all reaching DOF 0: 264 candidates in row 0
    n_elem, n_dof = 11, 300
    edof = np.arange(n_elem * 24, dtype=np.int32).reshape(n_elem, 24) % n_dof
    edof[:, 0] = 0
    with pytest.raises(S.SpmvError) as e:
        S.fem_assemble_csr(n_elem, n_dof, dev(edof.reshape(-1)), torch.ones(n_elem, device="cuda"), 3,
                           torch.eye(24, device="cuda").reshape(-1))
    assert e.value.status == 5
