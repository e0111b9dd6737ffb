"""GPU parity at index ranges past the 32-bit buffer offsets, through the C
ABI: the kernels then take their pointer-addressed forms (no buffer
resources), which smaller inputs never reach.

* CSR with 2^30 + 64 columns (x: 4.3 GB): a few thousand rows whose
  columns spread over the whole range, binned (16-byte and scalar stream
  loads), vector and scalar variants, alpha / beta;
* the FE matvec with 540 million DOFs (x and y: 2.2 GB each): a 13 x 7 x 5
  mesh whose DOFs are relabelled across the whole range, so the node-line
  merge still finds its pairs but every gather and add is pointer-addressed.

The oracle runs on a compact renumbering of the columns (DOFs) that occur,
which leaves every sum and its order unchanged; x is built on the GPU from
a closed form of the index, so no multi-gigabyte host array is needed.
"""
import numpy as np
import pytest

import gen
import oracle
from helpers import TAU_F32, assert_close, dev, host

torch = pytest.importorskip("torch")
S = pytest.importorskip("sparse_matrix_vector_amd")

pytestmark = pytest.mark.gpu


def _x_of(idx):
    """x[i] = ((i * 2654435761) mod 2^16) / 2^15 - 1 (exact in fp32), for int64 indices."""
    return (((idx.astype(np.int64) * 2654435761) % 65536).astype(np.float64) / 32768.0 - 1.0).astype(np.float32)


def _x_on_gpu(n, chunk=1 << 26):
    x = torch.empty(n, dtype=torch.float32, device="cuda")
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        i = torch.arange(a, b, dtype=torch.int64, device="cuda")
        x[a:b] = (((i * 2654435761) % 65536).to(torch.float64) / 32768.0 - 1.0).to(torch.float32)
        del i
    return x


def test_x_closed_form_matches_on_gpu():
    n = 1 << 20
    assert np.array_equal(host(_x_on_gpu(n)), _x_of(np.arange(n)))


@pytest.mark.parametrize("variant", ["binned", "binned_unaligned", "vector", "scalar"])
def test_csr_columns_past_4gib(variant):
    n_cols = (1 << 30) + 64
    rng = np.random.default_rng(51)
    lens = rng.integers(0, 300, 3000)
    lens[::50] = 2000                               # some row tasks and chunks too
    rows = [np.unique(rng.integers(0, n_cols, k)) for k in lens]
    rows[7] = np.array([0, n_cols - 1], np.int64)   # both ends of x
    rp = np.zeros(len(rows) + 1, np.int64)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ci = np.concatenate(rows).astype(np.int32)
    v = rng.uniform(-1, 1, len(ci)).astype(np.float32)
    n = len(rows)
    print(f"[large csr] {variant} rows={n} nnz={len(ci)} n_cols={n_cols}", flush=True)
    x = _x_on_gpu(n_cols)
    var = {"binned": S.CSR_BINNED, "binned_unaligned": S.CSR_BINNED, "vector": S.CSR_VECTOR,
           "scalar": S.CSR_SCALAR}[variant]
    if variant == "binned_unaligned":               # streams off 16-byte alignment: scalar stream loads
        cbuf = torch.zeros(len(ci) + 1, dtype=torch.int32, device="cuda")
        vbuf = torch.zeros(len(v) + 1, dtype=torch.float32, device="cuda")
        cbuf[1:] = dev(ci)
        vbuf[1:] = dev(v)
        cd, vd = cbuf[1:], vbuf[1:]
    else:
        cd, vd = dev(ci), dev(v)
    M = S.CSRMatrix(n, n_cols, dev(rp.astype(np.int32)), cd, vd, var)
    y0 = rng.uniform(-1, 1, n).astype(np.float32)
    u, inv = np.unique(ci, return_inverse=True)     # compact columns for the oracle
    for alpha, beta in [(1.0, 0.0), (0.5, -1.5)]:
        y = dev(y0) if beta else torch.full((n,), float("nan"), device="cuda")
        M.apply(x, y, alpha, beta)
        torch.cuda.synchronize()
        yr, sc = oracle.csr_spmv(rp.astype(np.int32), inv.astype(np.int32), v, _x_of(u), alpha, beta,
                                 y0 if beta else None)
        assert_close(host(y), yr, sc, TAU_F32, f"large csr {variant} {alpha} {beta}")
    del x
    torch.cuda.empty_cache()


def test_fe_dofs_past_2gib():
    M = gen.fe_mesh(13, 7, 5, clamp_x0=True, seed=8)
    n_dof = (1 << 29) + 4096                         # 4 * n_dof bytes is past the 2 GiB buffer range
    rng = np.random.default_rng(52)
    # DOF d -> a distinct index spread over [0, n_dof), the largest ones at the top of the range
    q = np.sort(rng.choice(n_dof - 1, M.n_dof - 1, replace=False)).astype(np.int64)
    q = np.append(q, n_dof - 1)[rng.permutation(M.n_dof)]
    ed = np.where(M.edof >= 0, q[np.maximum(M.edof, 0)], -1).astype(np.int32)
    print(f"[large fe] n_dof={n_dof} used={M.n_dof}", flush=True)
    x = _x_on_gpu(n_dof)
    xs = _x_of(q)                                   # x at the used DOFs, in the mesh's own numbering
    y = torch.full((n_dof,), float("nan"), device="cuda")
    y[dev(q)] = dev(np.linspace(-1, 1, M.n_dof).astype(np.float32))
    y_in = host(y[dev(q)])
    S.fem_matvec_apply(M.n_elem, n_dof, dev(ed.reshape(-1)), dev(M.rho), M.penalty, dev(M.Ke.reshape(-1)), 0.75,
                       x, 0.0, y)
    torch.cuda.synchronize()
    yr, sc = oracle.fe_matvec(M.edof, M.rho, M.Ke, xs, M.n_dof, M.penalty, 0.75, 0.0, None)
    assert_close(host(y[dev(q)]), yr, sc, TAU_F32, "large fe")
    # every other entry: beta = 0 writes zeros (sampled)
    probe = rng.integers(0, n_dof, 200_000)
    probe = probe[~np.isin(probe, q)]
    assert np.all(host(y[dev(probe)]) == 0.0)
    # beta != 0 on the used DOFs
    y[dev(q)] = dev(y_in)
    S.fem_matvec_apply(M.n_elem, n_dof, dev(ed.reshape(-1)), dev(M.rho), M.penalty, dev(M.Ke.reshape(-1)), 1.0,
                       x, -0.5, y)
    torch.cuda.synchronize()
    yr, sc = oracle.fe_matvec(M.edof, M.rho, M.Ke, xs, M.n_dof, M.penalty, 1.0, -0.5, y_in)
    assert_close(host(y[dev(q)]), yr, sc, TAU_F32, "large fe beta")
    del x, y
    torch.cuda.empty_cache()
