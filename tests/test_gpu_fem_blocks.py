"""GPU parity of the element-block FE matvec (plan once, two kernels, no
global atomics) against the oracle's element loop, through the C ABI.

Same bound as the fused kernel (|y - y_ref| <= 1e-5 x the element-wise
scale): the full 120 x 60 x 30 cantilever, small meshes with alpha / beta,
other numberings (elements shuffled or y-fastest, DOFs relabelled), a mesh
whose blocks have no free DOF, no elements at all (y = beta y only), a new
rho on the same plan, agreement with fem_matvec_apply, and the assembled
form of the oracle at both scales on 40 x 20 x 10.  Every addition
happens in an order the plan fixes, so a repeated apply must give the same
bits.
"""
import numpy as np
import pytest

import gen
import oracle
from helpers import TAU_F32, assert_close, dev, host

torch = pytest.importorskip("torch")
S = pytest.importorskip("sparse_matrix_vector_amd")

pytestmark = pytest.mark.gpu

_MESH = {}


def _mesh(dims, clamp=True, seed=4):
    key = (dims, clamp, seed)
    if key not in _MESH:
        _MESH[key] = gen.fe_mesh(*dims, clamp_x0=clamp, seed=seed)
    return _MESH[key]


def _run(ed, n_dof, rho, Ke, x, penalty, alpha=1.0, beta=0.0, y_in=None, plan=None, group=0):
    plan = plan or S.FEBlocks(ed.shape[0], n_dof, dev(np.ascontiguousarray(ed).reshape(-1)), group=group)
    y = dev(y_in) if y_in is not None else torch.full((n_dof,), float("nan"), device="cuda")
    plan.apply(dev(rho), penalty, dev(Ke.reshape(-1)), alpha, dev(x), beta, y)
    torch.cuda.synchronize()
    return host(y), plan


@pytest.mark.parametrize("group", [0, 1])
def test_full_mesh(group):
    M = _mesh((120, 60, 30))
    print(f"[blocks] full mesh, group {group}", flush=True)
    y, plan = _run(M.edof.reshape(M.n_elem, 24), M.n_dof, M.rho, M.Ke, M.x, M.penalty, group=group)
    print(f"[blocks] {plan.info()}", flush=True)
    assert plan.info()["group"] == (group or 3)
    yr, sc = oracle.fe_matvec(M.edof, M.rho, M.Ke, M.x, M.n_dof)
    assert_close(y, yr, sc, TAU_F32, "blocks full mesh")
    # the same bits again
    y_again, _ = _run(M.edof.reshape(M.n_elem, 24), M.n_dof, M.rho, M.Ke, M.x, M.penalty, plan=plan)
    assert np.array_equal(y.view(np.uint32), y_again.view(np.uint32)), "repeated apply changed bits"
    # the same operator as the fused kernel
    yf = torch.full((M.n_dof,), float("nan"), device="cuda")
    S.fem_matvec_apply(M.n_elem, M.n_dof, dev(M.edof.reshape(-1)), dev(M.rho), M.penalty, dev(M.Ke.reshape(-1)),
                       1.0, dev(M.x), 0.0, yf)
    torch.cuda.synchronize()
    assert_close(y, host(yf).astype(np.float64), sc, 2 * TAU_F32, "blocks vs fused")
    # a new rho on the same plan
    rho2 = np.random.default_rng(5).uniform(0.001, 1.0, M.n_elem).astype(np.float32)
    y2, _ = _run(M.edof.reshape(M.n_elem, 24), M.n_dof, rho2, M.Ke, M.x, M.penalty, plan=plan)
    yr2, sc2 = oracle.fe_matvec(M.edof, rho2, M.Ke, M.x, M.n_dof)
    assert_close(y2, yr2, sc2, TAU_F32, "blocks, new rho")


@pytest.mark.parametrize("group", [3, 1])
@pytest.mark.parametrize("dims,clamp", [((1, 1, 1), False), ((3, 2, 2), True), ((13, 7, 5), True),
                                        ((16, 16, 1), False), ((40, 20, 10), True)])
def test_small_meshes(dims, clamp, group):
    M = _mesh(dims, clamp, seed=8)
    ed = M.edof.reshape(M.n_elem, 24)
    y_in = np.random.default_rng(3).uniform(-1, 1, M.n_dof).astype(np.float32)
    plan = None
    for alpha, beta in [(1.0, 0.0), (-0.5, 1.0), (2.0, -0.25)]:
        y, plan = _run(ed, M.n_dof, M.rho, M.Ke, M.x, M.penalty, alpha, beta, y_in if beta else None, plan, group)
        yr, sc = oracle.fe_matvec(M.edof, M.rho, M.Ke, M.x, M.n_dof, M.penalty, alpha, beta, y_in)
        assert_close(y, yr, sc, TAU_F32, f"blocks {dims} G={group} {alpha} {beta}")


def test_node_units_with_a_cut_last_node():
    """n_dof one past the mesh's DOFs: the last unit of the node plan holds
    one DOF, touched by no element (y = beta y there)."""
    M = _mesh((13, 7, 5), True, seed=8)
    n = M.n_dof + 1
    x = np.concatenate([M.x, [7.0]]).astype(np.float32)
    y_in = np.random.default_rng(6).uniform(-1, 1, n).astype(np.float32)
    y, plan = _run(M.edof.reshape(M.n_elem, 24), n, M.rho, M.Ke, x, M.penalty, 1.0, 0.5, y_in)
    assert plan.info()["group"] == 3
    yr, sc = oracle.fe_matvec(M.edof, M.rho, M.Ke, x, n, M.penalty, 1.0, 0.5, y_in)
    assert_close(y, yr, sc, TAU_F32, "cut last node")


@pytest.mark.parametrize("how", ["elements_shuffled", "elements_y_fastest", "dofs_relabelled"])
@pytest.mark.parametrize("dims", [(13, 7, 5), (40, 20, 10)])
def test_other_numberings(how, dims):
    M = _mesh(dims, clamp=True)
    rng = np.random.default_rng(21)
    ed, rho, x = M.edof.reshape(M.n_elem, 24), M.rho, M.x
    if how == "elements_shuffled":
        p = rng.permutation(M.n_elem)
        ed, rho = ed[p], rho[p]
    elif how == "elements_y_fastest":
        p = np.arange(M.n_elem).reshape(M.nz, M.ny, M.nx).transpose(0, 2, 1).reshape(-1)
        ed, rho = ed[p], rho[p]
    else:
        q = rng.permutation(M.n_dof)
        ed = np.where(ed >= 0, q[np.maximum(ed, 0)], -1).astype(np.int32)
        xq = np.empty_like(x)
        xq[q] = x
        x = xq
    print(f"[blocks] {dims} {how}", flush=True)
    y_in = np.random.default_rng(5).uniform(-1, 1, M.n_dof).astype(np.float32)
    ed, rho, x = np.ascontiguousarray(ed), np.ascontiguousarray(rho), np.ascontiguousarray(x)
    y, plan = _run(ed, M.n_dof, rho, M.Ke, x, M.penalty, 0.5, -2.0, y_in)
    assert plan.info()["group"] == (1 if how == "dofs_relabelled" else 3)
    yr, sc = oracle.fe_matvec(ed, rho, M.Ke, x, M.n_dof, M.penalty, 0.5, -2.0, y_in)
    assert_close(y, yr, sc, TAU_F32, f"blocks {dims} {how}")
    if how == "dofs_relabelled":   # no node structure left: G = 3 is refused
        with pytest.raises(S.SpmvError):
            S.FEBlocks(M.n_elem, M.n_dof, dev(ed.reshape(-1)), group=3)


def test_no_free_dofs_and_no_elements():
    # every DOF of the one element constrained: y = beta y on all DOFs
    Ke = _mesh((1, 1, 1), False).Ke
    y_in = np.arange(1, 6, dtype=np.float32)
    y, _ = _run(np.full((1, 24), -1, np.int32), 5, np.ones(1, np.float32), Ke, np.ones(5, np.float32), 3, 1.0, 2.0,
                y_in)
    assert y.tolist() == (2 * y_in).tolist()
    # no elements: beta = 0 writes zeros over NaN, beta = 3 scales
    plan = S.FEBlocks(0, 4, torch.zeros(0, dtype=torch.int32, device="cuda"))
    for beta, want in [(0.0, [0.0] * 4), (3.0, [3.0, 6.0, 9.0, 12.0])]:
        y = torch.tensor([1.0, 2.0, 3.0, 4.0], device="cuda") if beta else torch.full((4,), float("nan"), device="cuda")
        plan.apply(torch.zeros(0, device="cuda"), 3, torch.zeros(576, device="cuda"), 1.0,
                   torch.zeros(4, device="cuda"), beta, y)
        torch.cuda.synchronize()
        assert host(y).tolist() == want


def test_rejects_bad_arguments():
    M = _mesh((3, 2, 2), True, seed=8)
    plan = S.FEBlocks(M.n_elem, M.n_dof, dev(M.edof.reshape(-1)))
    y = torch.zeros(M.n_dof, device="cuda")
    with pytest.raises(S.SpmvError):
        plan.apply(dev(M.rho), 9, dev(M.Ke.reshape(-1)), 1.0, dev(M.x), 0.0, y)     # penalty > 8
    small = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(S.SpmvError):
        S.fem_blocks_create(M.n_elem, M.n_dof, dev(M.edof.reshape(-1)), small)
    with pytest.raises(S.SpmvError):
        S.FEBlocks(M.n_elem, M.n_dof, dev(M.edof.reshape(-1)), group=2)


@pytest.mark.parametrize("group", [1, 3])
def test_partial_sums_past_the_rank_planes(group):
    """Every element also lists one extra node, so that node lies in every
    block (more than 8): its partial sums run past the 8 rank planes into the
    overflow list of the second kernel."""
    M = gen.fe_mesh(40, 24, 6, clamp_x0=True, seed=6)
    ed = M.edof.reshape(M.n_elem, 24).copy()
    n = M.n_dof + 3
    ed[:, 0:3] = [M.n_dof, M.n_dof + 1, M.n_dof + 2]
    x = np.random.default_rng(9).uniform(-1, 1, n).astype(np.float32)
    y_in = np.random.default_rng(4).uniform(-1, 1, n).astype(np.float32)
    print(f"[blocks] hub node, group {group}", flush=True)
    y, plan = _run(ed, n, M.rho, M.Ke, x, M.penalty, 0.5, 2.0, y_in, group=group)
    info = plan.info()
    assert info["planes"] == 8 and info["n_blocks"] > 8
    yr, sc = oracle.fe_matvec(ed, M.rho, M.Ke, x, n, M.penalty, 0.5, 2.0, y_in)
    assert_close(y, yr, sc, TAU_F32, f"hub node, G={group}")


@pytest.mark.parametrize("group", [1, 3])
def test_long_blocks_chain(group):
    """Elements in a chain, each sharing one node with the next: ~1,800 nodes
    per block, past what a lane stages from registers, so the apply's
    remainder loops (staging and run sums) carry most of the block."""
    Ke = _mesh((1, 1, 1), False).Ke
    E = 600
    nodes = 7 * np.arange(E)[:, None] + np.arange(8)[None, :]
    ed = (3 * nodes[:, :, None] + np.arange(3)[None, None, :]).reshape(E, 24).astype(np.int32)
    n = 3 * (7 * E + 1)
    rng = np.random.default_rng(11)
    rho = rng.uniform(0.1, 1.0, E).astype(np.float32)
    x = rng.uniform(-1, 1, n).astype(np.float32)
    y_in = rng.uniform(-1, 1, n).astype(np.float32)
    print(f"[blocks] chain, group {group}", flush=True)
    y, plan = _run(ed, n, rho, Ke, x, 3, 1.5, -0.5, y_in, group=group)
    assert plan.info()["Lmax"] > (1792 if group == 1 else 768)
    yr, sc = oracle.fe_matvec(ed, rho, Ke, x, n, 3, 1.5, -0.5, y_in)
    assert_close(y, yr, sc, TAU_F32, f"chain, G={group}")


@pytest.mark.parametrize("group", [3, 1])
@pytest.mark.parametrize("clamp", [True, False])
def test_assembled_form(clamp, group):
    """The element-block apply against K x with K assembled by the oracle in
    fp64 (COO sorted, duplicates merged) and applied by the oracle's CSR
    product, on 40 x 20 x 10 (32 blocks, shared nodes on every block face):
    within 1e-5 of the element-wise scale, and of the smaller assembled
    scale sum_j |K_ij x_j| as well."""
    M = _mesh((40, 20, 10), clamp, seed=12)
    rp, ci, v = oracle.fe_assemble(M.edof, M.rho, M.Ke, M.n_dof)
    ya, sa = oracle.csr_spmv_f64(rp, ci, v, M.x)
    y, _ = _run(M.edof.reshape(M.n_elem, 24), M.n_dof, M.rho, M.Ke, M.x, M.penalty, group=group)
    _, sc = oracle.fe_matvec(M.edof, M.rho, M.Ke, M.x, M.n_dof)
    err = assert_close(y, ya, sc, TAU_F32, f"blocks G={group} vs assembled (element scale)")
    nz = sa > 0
    worst = float(np.max(np.abs(y[nz] - ya[nz]) / sa[nz]))
    print(f"[blocks] clamp={clamp} G={group}: max err / element scale {err:.2e}, "
          f"max err / assembled scale {worst:.2e}", flush=True)
    assert_close(y, ya, sa, TAU_F32, f"blocks G={group} vs assembled (assembled scale)")


@pytest.mark.parametrize("nodewise", [True, False])
def test_random_connectivity(nodewise):
    """1,500 elements on 300 random nodes: every node in ~40 element corners,
    so the runs are long (up to ~20 entries per block) and most nodes are
    shared by all blocks."""
    rng = np.random.default_rng(42)
    E, nodes = 1500, 300
    Ke = _mesh((1, 1, 1), False).Ke
    if nodewise:
        corner = rng.integers(0, nodes, (E, 8))
        ed = (3 * corner[:, :, None] + np.arange(3)[None, None, :]).reshape(E, 24)
    else:
        ed = np.where(rng.random((E, 24)) < 0.1, -1, rng.integers(0, 3 * nodes, (E, 24)))
    ed = ed.astype(np.int32)
    n = 3 * nodes
    rho = rng.uniform(0.05, 1.0, E).astype(np.float32)
    x = rng.uniform(-1, 1, n).astype(np.float32)
    y_in = rng.uniform(-1, 1, n).astype(np.float32)
    for group in ((3, 1) if nodewise else (1,)):
        print(f"[blocks] random connectivity, group {group}", flush=True)
        y, plan = _run(ed, n, rho, Ke, x, 3, 0.75, 0.5, y_in, group=group)
        yr, sc = oracle.fe_matvec(ed, rho, Ke, x, n, 3, 0.75, 0.5, y_in)
        assert_close(y, yr, sc, TAU_F32, f"random connectivity G={group}")
