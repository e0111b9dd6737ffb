"""The applies inside a captured HIP graph: each path's apply is captured once
(torch.cuda.CUDAGraph on a side stream) and replayed several times, with
eager work between the replays that changes x and resets y; every replay
must equal an eager apply on the same inputs (bit for bit on the
deterministic paths, the element-block FE apply included; within the
oracle's bound for the fused FE matvec, whose atomics add in a varying
order, and for SpGEMM, whose values do too).

Nothing in these applies may record a memset or an allocation into the
graph; a path that did would fail here on a replay after the first.
"""
import numpy as np
import pytest

import gen
import oracle
from helpers import TAU_F32, assert_close, dev, host

torch = pytest.importorskip("torch")
S = pytest.importorskip("sparse_matrix_vector_amd")

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_compare(name, fn, x, x_values, y, y0, eager_equal):
    """fn applies with x into y; x_values: host arrays put into x between
    replays; y is reset to y0 each time.  eager_equal(y_graph, x_host) checks
    one replay."""
    g = _capture(fn)
    for i, xv in enumerate(x_values):
        x.copy_(dev(xv))
        y.copy_(dev(y0))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = host(y).copy()
        print(f"[graph] {name} replay {i}", flush=True)
        eager_equal(got, xv)


def _bitwise_vs_eager(fn, x, y, y0):
    def check(got, xv):
        y.copy_(dev(y0))
        fn()
        torch.cuda.synchronize()
        assert np.array_equal(got.view(np.uint32), host(y).view(np.uint32))
    return check


@pytest.mark.parametrize("kind", ["csr-binned", "csr-vector", "ell", "auto-hyb", "auto-hyb-short"])
def test_spmv_paths_replay(kind):
    """auto-hyb: tails up to ~25 entries (ELL kernel, then the binned tail);
    auto-hyb-short: tails of at most 16 (ELL and tail in one kernel)."""
    rng = np.random.default_rng(5)
    if kind == "auto-hyb":
        lens = rng.integers(1, 13, 20_000)
        lens[rng.choice(20_000, 100, replace=False)] = 30
    elif kind == "auto-hyb-short":
        lens = rng.integers(1, 13, 20_000)
    else:
        lens = rng.integers(0, 40, 20_000)
        lens[::997] = 700                       # rows of several chunks
    A = gen.random_csr(len(lens), 20_000, lens, seed=6)
    rp, ci, v = dev(A.row_ptr), dev(A.col_idx), dev(A.vals)
    x = dev(A.x)
    y = torch.zeros(A.n_rows, device="cuda")
    y0 = rng.uniform(-1, 1, A.n_rows).astype(np.float32)
    if kind.startswith("csr"):
        M = S.CSRMatrix(A.n_rows, A.n_cols, rp, ci, v, S.CSR_BINNED if kind == "csr-binned" else S.CSR_VECTOR)
        fn = lambda: M.apply(x, y, 0.5, -1.0)  # noqa: E731
    elif kind == "ell":
        W = int(lens.max())
        ec = torch.empty(W * A.n_rows, dtype=torch.int32, device="cuda")
        ev = torch.empty(W * A.n_rows, dtype=torch.float32, device="cuda")
        S.spmv_ell_from_csr(A.n_rows, A.n_cols, rp, ci, v, W, ec, ev)
        fn = lambda: S.spmv_ell_apply(A.n_rows, A.n_cols, W, ec, ev, 0.5, x, -1.0, y)  # noqa: E731
    else:
        M = S.AutoMatrix(A.n_rows, A.n_cols, rp, ci, v)
        assert M.format == 1
        fn = lambda: M.apply(x, y, 0.5, -1.0)  # noqa: E731
    xs = [rng.uniform(-1, 1, A.n_cols).astype(np.float32) for _ in range(REPLAYS)]
    check = _bitwise_vs_eager(fn, x, y, y0)

    def both(got, xv):
        check(got, xv)
        yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, xv, 0.5, -1.0, y0)
        assert_close(got, yr, sc, TAU_F32, f"graph {kind}")
    _replay_and_compare(kind, fn, x, xs, y, y0, both)


def test_macko_and_dense_replay():
    W = gen.pruned_weight(0.7, n_rows=512, n_cols=3000, seed=8)
    mrp, codes, mv = S.macko_encode(W.n_rows, W.n_cols, W.row_ptr, W.col_idx, W.vals_f16)
    d_mrp, d_codes, d_mv = dev(mrp), dev(codes), dev(mv)
    x = dev(W.x_f16)
    y = torch.zeros(W.n_rows, device="cuda")
    y0 = np.linspace(-1, 1, W.n_rows).astype(np.float32)
    rng = np.random.default_rng(9)
    xs = [rng.uniform(-1, 1, W.n_cols).astype(np.float16).view(np.uint16) for _ in range(REPLAYS)]
    fn = lambda: S.macko_spmv(W.n_rows, W.n_cols, d_mrp, d_codes, d_mv, 1.5, x, 0.25, y)  # noqa: E731
    _replay_and_compare("macko", fn, x, xs, y, y0, _bitwise_vs_eager(fn, x, y, y0))
    Wd = dev(W.dense_f16())
    fd = lambda: S.dense_gemv_f16(W.n_rows, W.n_cols, Wd, x, 1.5, 0.25, y)  # noqa: E731
    _replay_and_compare("dense", fd, x, xs, y, y0, _bitwise_vs_eager(fd, x, y, y0))


@pytest.mark.parametrize("dims", [(12, 6, 5), (40, 20, 10)])
def test_fe_fused_replay(dims):
    """The beta kernel and the fused kernel in one graph, replayed; an eager
    call between the replays must agree with the oracle too."""
    M = gen.fe_mesh(*dims, seed=3)
    ed, rho, Ke = dev(M.edof.reshape(-1)), dev(M.rho), dev(M.Ke.reshape(-1))
    x = dev(M.x)
    y = torch.zeros(M.n_dof, device="cuda")
    y0 = np.random.default_rng(2).uniform(-1, 1, M.n_dof).astype(np.float32)
    rng = np.random.default_rng(10)
    xs = [rng.uniform(-1, 1, M.n_dof).astype(np.float32) for _ in range(REPLAYS)]
    fn = lambda: S.fem_matvec_apply(M.n_elem, M.n_dof, ed, rho, M.penalty, Ke, 2.0, x, -0.5, y)  # noqa: E731

    def check(got, xv):
        yr, sc = oracle.fe_matvec(M.edof, M.rho, M.Ke, xv, M.n_dof, M.penalty, 2.0, -0.5, y0)
        assert_close(got, yr, sc, TAU_F32, "graph fe")
        y.copy_(dev(y0))
        fn()                                   # an eager call between the replays
        torch.cuda.synchronize()
        assert_close(host(y), yr, sc, TAU_F32, "eager fe between replays")
    _replay_and_compare("fe", fn, x, xs, y, y0, check)


@pytest.mark.parametrize("group", [3, 1])
def test_fe_blocks_replay(group):
    """The element-block apply (two kernels, no atomics) in one graph,
    replayed: every replay bit for bit equal to an eager apply, and within the
    oracle's bound."""
    M = gen.fe_mesh(40, 20, 10, seed=3)
    ed, rho, Ke = dev(M.edof.reshape(-1)), dev(M.rho), dev(M.Ke.reshape(-1))
    plan = S.FEBlocks(M.n_elem, M.n_dof, ed, group=group)
    x = dev(M.x)
    y = torch.zeros(M.n_dof, device="cuda")
    y0 = np.random.default_rng(2).uniform(-1, 1, M.n_dof).astype(np.float32)
    rng = np.random.default_rng(10)
    xs = [rng.uniform(-1, 1, M.n_dof).astype(np.float32) for _ in range(REPLAYS)]
    fn = lambda: plan.apply(rho, M.penalty, Ke, 2.0, x, -0.5, y)  # noqa: E731
    bitwise = _bitwise_vs_eager(fn, x, y, y0)

    def check(got, xv):
        yr, sc = oracle.fe_matvec(M.edof, M.rho, M.Ke, xv, M.n_dof, M.penalty, 2.0, -0.5, y0)
        assert_close(got, yr, sc, TAU_F32, "graph fe blocks")
        bitwise(got, xv)
    _replay_and_compare(f"fe-blocks G={group}", fn, x, xs, y, y0, check)


def test_spgemm_compute_replay():
    """The accumulation phase forks its bins to side streams and joins them
    with events; the capture must take them in, and every replay must redo
    the whole row set (values change between replays through A)."""
    rng = np.random.default_rng(12)
    k, n, m = 2000, 3000, 800
    blens = np.where(rng.random(k) < 0.03, rng.integers(300, 1500, k), rng.integers(0, 10, k))
    B = gen.random_csr(k, n, blens, seed=13)
    alens = np.where(rng.random(m) < 0.1, rng.integers(10, 40, m), rng.integers(0, 5, m))
    A = gen.random_csr(m, k, alens, seed=14)
    rpa, cia, va = dev(A.row_ptr), dev(A.col_idx), dev(A.vals)
    rpb, cib, vb = dev(B.row_ptr), dev(B.col_idx), dev(B.vals)
    G = S.SpGEMM(m, k, n, rpa, cia, va, rpb, cib, vb)
    assert sum(g > 0 for g in G.group_rows) >= 3
    out = G.compute()
    torch.cuda.synchronize()
    fn = lambda: G.compute(out)  # noqa: E731
    vals = [rng.uniform(-1, 1, A.nnz).astype(np.float32) for _ in range(REPLAYS)]

    def check(_, av):
        orp, oci, ov, osc = oracle.spgemm(n, A.row_ptr, A.col_idx, av, B.row_ptr, B.col_idx, B.vals)
        assert np.array_equal(host(out[0]), orp) and np.array_equal(host(out[1]), oci)
        err = np.abs(host(out[2]).astype(np.float64) - ov)
        assert np.all(err <= TAU_F32 * osc)
    g = _capture(fn)
    for i, av in enumerate(vals):
        va.copy_(dev(av))
        out[2].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph] spgemm replay {i}", flush=True)
        check(None, av)
    G.close()


def test_two_streams_at_once():
    """Applies of different handles on two streams at the same time (CSR
    plans are read-only during an apply; two SpGEMM handles share the
    device's side streams) give the results each gives alone."""
    rng = np.random.default_rng(21)
    mats = [gen.random_csr(30_000, 30_000, rng.integers(0, 30, 30_000), seed=s) for s in (22, 23)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs, Ms = [], []
    for A in mats:
        M = S.CSRMatrix(A.n_rows, A.n_cols, dev(A.row_ptr), dev(A.col_idx), dev(A.vals), S.CSR_BINNED)
        Ms.append((M, dev(A.x), torch.zeros(A.n_rows, device="cuda")))
    torch.cuda.synchronize()
    for (M, x, y), st in zip(Ms, streams):
        with torch.cuda.stream(st):
            for _ in range(20):
                M.apply(x, y)
    torch.cuda.synchronize()
    for A, (M, x, y) in zip(mats, Ms):
        yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x)
        assert_close(host(y), yr, sc, TAU_F32, "two streams csr")
    # two SpGEMM products at once
    Gs, pairs = [], []
    for s in (24, 25):
        k, n, m = 1500, 2000, 600
        blens = np.where(rng.random(k) < 0.03, rng.integers(300, 1200, k), rng.integers(0, 10, k))
        B = gen.random_csr(k, n, blens, seed=s)
        alens = np.where(rng.random(m) < 0.1, rng.integers(10, 40, m), rng.integers(0, 5, m))
        A = gen.random_csr(m, k, alens, seed=s + 10)
        arrs = [dev(a) for a in (A.row_ptr, A.col_idx, A.vals, B.row_ptr, B.col_idx, B.vals)]
        Gs.append((S.SpGEMM(m, k, n, *arrs), arrs))
        pairs.append((n, A, B))
    torch.cuda.synchronize()
    results = []
    for (G, _), st in zip(Gs, streams):
        with torch.cuda.stream(st):
            results.append(G.compute(stream=st))
    torch.cuda.synchronize()
    print("[streams] csr and spgemm on two streams", flush=True)
    for (n, A, B), out in zip(pairs, results):
        orp, oci, ov, osc = oracle.spgemm(n, A.row_ptr, A.col_idx, A.vals, B.row_ptr, B.col_idx, B.vals)
        assert np.array_equal(host(out[0]), orp) and np.array_equal(host(out[1]), oci)
        assert np.all(np.abs(host(out[2]).astype(np.float64) - ov) <= TAU_F32 * osc)
    for G, _ in Gs:
        G.close()
