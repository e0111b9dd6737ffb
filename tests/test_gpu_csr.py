"""GPU parity of the CSR path (planner, scalar / vector / binned apply) against
the fp64 CPU oracle, through the C ABI.

* grouping plan (bin_offsets, perm): bit-exact with the oracle's counting sort
  on the tiny, Laplacian and power-law configs, custom thresholds, and a
  matrix with rows of 8,192 and 100,000 nonzeros (group 3);
* values: |y - y_ref| <= 1e-5 * scale for every row, every variant, at the
  configs' full sizes and on edge cases (empty rows, n_rows = 0, nnz = 0,
  unsorted and duplicate columns, misaligned arrays, rows around the group
  bounds, alpha / beta);
* every variant is bit-reproducible run to run;
* invalid matrices are rejected by the on-GPU validation.
"""
import numpy as np
import pytest

import gen
import oracle
from helpers import TAU_F32, assert_close, dev, host

torch = pytest.importorskip("torch")
S = pytest.importorskip("sparse_matrix_vector_amd")

pytestmark = pytest.mark.gpu

VARIANTS = {"scalar": S.CSR_SCALAR, "vector": S.CSR_VECTOR, "binned": S.CSR_BINNED}
PAGE_BOUNDS = (32, 512, 8192)          # the grouping page's table
DEFAULT_BOUNDS = (128, 512, 8192)      # the library's default (first bound raised for wave64 tasks)


def _mat(A):
    return dev(A.row_ptr), dev(A.col_idx), dev(A.vals)


def _run(A, variant, alpha=1.0, beta=0.0, y_in=None, thresholds=None, tensors=None):
    rp, ci, v = tensors if tensors is not None else _mat(A)
    M = S.CSRMatrix(A.n_rows, A.n_cols, rp, ci, v, variant, thresholds)
    x = dev(A.x)
    y = dev(y_in) if y_in is not None else torch.full((A.n_rows,), float("nan"), device="cuda")
    M.apply(x, y, alpha, beta)
    torch.cuda.synchronize()
    return M, host(y)


_CACHE = {}


def _config(name):
    if name not in _CACHE:
        _CACHE[name] = {"tiny": gen.tiny_csr, "laplacian": gen.laplacian_2d,
                        "powerlaw": gen.powerlaw_csr}[name]()
    return _CACHE[name]


@pytest.mark.parametrize("name", ["tiny", "laplacian", "powerlaw"])
def test_plan_bit_exact(name):
    A = _config(name)
    print(f"[plan] {name} n={A.n_rows} nnz={A.nnz}", flush=True)
    rp, ci, v = _mat(A)
    for bounds, given in [(PAGE_BOUNDS, PAGE_BOUNDS), (DEFAULT_BOUNDS, None)]:
        M = S.CSRMatrix(A.n_rows, A.n_cols, rp, ci, v, S.CSR_BINNED, given)
        perm = torch.empty(A.n_rows, dtype=torch.int32, device="cuda")
        off = M.plan(perm)
        ooff, operm = oracle.bins(A.row_ptr, bounds)
        assert off == ooff.tolist()
        assert np.array_equal(host(perm), operm)
        if name == "powerlaw" and bounds == PAGE_BOUNDS:
            assert off[4] - off[3] == 0 and off[3] - off[2] > 500 and off[2] - off[1] > 10000
        x = dev(A.x)
        y = torch.empty(A.n_rows, device="cuda")
        M.apply(x, y)
        yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x)
        assert_close(host(y), yr, sc, TAU_F32, f"{name} bounds {bounds}")


@pytest.mark.parametrize("name", ["tiny", "laplacian", "powerlaw"])
@pytest.mark.parametrize("variant", list(VARIANTS))
def test_values_full_configs(name, variant):
    A = _config(name)
    print(f"[apply] {name} {variant}", flush=True)
    M, y = _run(A, VARIANTS[variant])
    yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x)
    assert_close(y, yr, sc, TAU_F32, f"{name}/{variant}")


def _long_rows_matrix():
    lens = np.array([3, 8192, 0, 100_000, 31, 32, 511, 512, 8191, 1, 9000, 0, 5], dtype=np.int64)
    return gen.random_csr(len(lens), 120_000, lens, seed=5)


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_group_bounds_and_long_rows(variant):
    A = _long_rows_matrix()
    M, y = _run(A, VARIANTS[variant], alpha=0.5, beta=-2.0,
                y_in=np.linspace(-1, 1, A.n_rows).astype(np.float32))
    yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x, 0.5, -2.0,
                             np.linspace(-1, 1, A.n_rows).astype(np.float32))
    assert_close(y, yr, sc, TAU_F32, f"long/{variant}")
    if variant == "binned":
        perm = torch.empty(A.n_rows, dtype=torch.int32, device="cuda")
        off = M.plan(perm)
        ooff, operm = oracle.bins(A.row_ptr, DEFAULT_BOUNDS)
        assert off == ooff.tolist() and np.array_equal(host(perm), operm)
        assert off[4] - off[3] == 3


@pytest.mark.parametrize("lo,hi", [(100, 128), (120, 128), (1, 128)])
def test_short_rows_near_the_bound(lo, hi):
    """Short rows up to 127 entries (the default first bound is 128): runs are
    cut at windows of 512 - L - 2 nonzeros, L the longest short row, so every
    block still fits one 512-entry task; empty rows mixed in."""
    rng = np.random.default_rng(lo)
    lens = rng.integers(lo, hi, 6000)
    lens[::97] = 0
    A = gen.random_csr(len(lens), 20_000, lens, seed=lo + 1)
    print(f"[near bound] {lo}..{hi - 1}", flush=True)
    M, y = _run(A, S.CSR_BINNED, alpha=-1.0, beta=0.5, y_in=np.ones(A.n_rows, np.float32))
    yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x, -1.0, 0.5, np.ones(A.n_rows, np.float32))
    assert_close(y, yr, sc, TAU_F32, f"near bound {lo}")
    perm = torch.empty(A.n_rows, dtype=torch.int32, device="cuda")
    off = M.plan(perm)
    assert off[1] == A.n_rows                     # every row is short under the default bounds


@pytest.mark.parametrize("lens_kind", ["fe_like", "mixed", "two_rows"])
def test_blocks_of_few_rows(lens_kind):
    """Short-row blocks of at most 32 rows, summed by a group of lanes per
    row (groups of 2 to 32 lanes): rows of ~78 entries as in an assembled
    stiffness matrix, a mix of lengths 0..127 where blocks hold 2..30 rows,
    and blocks of exactly two long short rows; alpha, beta, bit-reproducible."""
    rng = np.random.default_rng(41)
    if lens_kind == "fe_like":
        lens = rng.integers(72, 82, 20_000)
    elif lens_kind == "mixed":
        lens = rng.choice([0, 1, 5, 17, 33, 64, 100, 127], 20_000)
    else:
        lens = np.full(4000, 126)
        lens[1::2] = 127
    A = gen.random_csr(len(lens), 30_000, lens, seed=42)
    y0 = rng.uniform(-1, 1, A.n_rows).astype(np.float32)
    print(f"[few rows] {lens_kind} n={A.n_rows} nnz={A.nnz}", flush=True)
    for alpha, beta in [(1.0, 0.0), (-0.5, 2.0)]:
        M, y = _run(A, S.CSR_BINNED, alpha=alpha, beta=beta, y_in=y0 if beta else None)
        yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x, alpha, beta, y0 if beta else None)
        assert_close(y, yr, sc, TAU_F32, f"few rows {lens_kind} {alpha} {beta}")
    M2, y2 = _run(A, S.CSR_BINNED, alpha=-0.5, beta=2.0, y_in=y0)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def test_workgroup_rows_and_chunked_rows():
    """Rows of 2-16 chunks (one workgroup each, no second kernel) next to
    rows of 1 chunk and of more than 16 chunks (chunk partials), from
    unaligned starts, among short rows; alpha, beta and run-to-run bits."""
    rng = np.random.default_rng(31)
    longs = [600, 1021, 1024, 1500, 2049, 4334, 8188, 8200, 20000, 509, 510, 513]
    lens = np.concatenate([rng.integers(0, 12, 3000), longs, rng.integers(0, 40, 500), longs[::-1]])
    A = gen.random_csr(len(lens), 50_000, lens, seed=32)
    y0 = rng.uniform(-1, 1, A.n_rows).astype(np.float32)
    print(f"[wgrows] n={A.n_rows} nnz={A.nnz}", flush=True)
    M, y = _run(A, S.CSR_BINNED, alpha=1.5, beta=0.25, y_in=y0)
    yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x, alpha=1.5, beta=0.25, y_in=y0)
    assert_close(y, yr, sc, TAU_F32, "workgroup rows")
    x = dev(A.x)
    y2 = dev(y0)
    M.apply(x, y2, 1.5, 0.25)
    torch.cuda.synchronize()
    assert np.array_equal(host(y2).view(np.uint32), y.view(np.uint32))


@pytest.mark.parametrize("thr", [(4, 8, 16), (2, 3, 4), (256, 1000, 5000), (1, 2, 100000)])
def test_custom_thresholds(thr):
    rng = np.random.default_rng(11)
    lens = rng.choice([0, 1, 2, 3, 5, 9, 17, 40, 300], size=3000)
    A = gen.random_csr(3000, 3000, lens, seed=12)
    M, y = _run(A, S.CSR_BINNED, thresholds=thr)
    perm = torch.empty(A.n_rows, dtype=torch.int32, device="cuda")
    off = M.plan(perm)
    ooff, operm = oracle.bins(A.row_ptr, thr)
    assert off == ooff.tolist() and np.array_equal(host(perm), operm)
    yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x)
    assert_close(y, yr, sc, TAU_F32, f"thr={thr}")


EDGE = {
    "empty_rows": lambda: gen.random_csr(700, 300, np.where(np.arange(700) % 3 == 0, 0, 7), seed=1),
    "all_empty": lambda: gen.random_csr(513, 10, np.zeros(513, np.int64), seed=2),
    "one_row": lambda: gen.random_csr(1, 50, [37], seed=3),
    "ragged_tail": lambda: gen.random_csr(1001, 1001, np.random.default_rng(4).integers(0, 31, 1001), seed=4),
    "unsorted": lambda: gen.random_csr(500, 400, np.random.default_rng(5).integers(0, 60, 500), seed=5,
                                       sorted_cols=False),
    "many_len1": lambda: gen.random_csr(5000, 5000, np.ones(5000, np.int64), seed=6),
    "wide": lambda: gen.random_csr(64, 1_000_000, np.full(64, 700), seed=7),
}


@pytest.mark.parametrize("case", list(EDGE))
@pytest.mark.parametrize("variant", list(VARIANTS))
def test_edge_cases(case, variant):
    A = EDGE[case]()
    print(f"[edge] {case} {variant}", flush=True)
    M, y = _run(A, VARIANTS[variant])
    yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x)
    assert_close(y, yr, sc, TAU_F32, f"{case}/{variant}")


@pytest.mark.parametrize("offsets", [(-2700, -1300, -1, 0, 1, 900, 2650),
                                     (-2900, -2100, -777, -64, -3, 0, 5, 31, 400, 1999, 2500, 2900)])
def test_x_window_sparse_bands(offsets):
    """Rows whose entries fall in a few bands far apart: every block
    workgroup's column window fits in LDS, but most of its segments hold no
    column (the apply stages only the touched ones), with beta != 0."""
    A = gen.stencil_csr(300_000, offsets, seed=21)
    y0 = np.random.default_rng(22).uniform(-1, 1, A.n_rows).astype(np.float32)
    print(f"[window] offsets {offsets}", flush=True)
    M, y = _run(A, S.CSR_BINNED, alpha=0.75, beta=-0.5, y_in=y0)
    yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x, alpha=0.75, beta=-0.5, y_in=y0)
    assert_close(y, yr, sc, TAU_F32, f"bands {offsets}")


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_duplicates_summed(variant):
    A = gen.random_csr(200, 100, np.random.default_rng(9).integers(2, 20, 200), seed=9)
    ci = A.col_idx.copy()
    for i in range(A.n_rows):
        a, b = A.row_ptr[i], A.row_ptr[i + 1]
        ci[b - 1] = ci[a]
    A.col_idx = ci
    M, y = _run(A, VARIANTS[variant])
    yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x)
    assert_close(y, yr, sc, TAU_F32, f"dup/{variant}")


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_misaligned_arrays(variant):
    """Arrays that start 4 bytes past a 16-byte boundary take the 4-byte path."""
    A = gen.random_csr(900, 900, np.random.default_rng(3).integers(0, 40, 900), seed=13)
    ci_pad = torch.zeros(A.nnz + 1, dtype=torch.int32, device="cuda")
    v_pad = torch.zeros(A.nnz + 1, dtype=torch.float32, device="cuda")
    ci_pad[1:] = dev(A.col_idx)
    v_pad[1:] = dev(A.vals)
    M, y = _run(A, VARIANTS[variant], tensors=(dev(A.row_ptr), ci_pad[1:], v_pad[1:]))
    yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x)
    assert_close(y, yr, sc, TAU_F32, f"misaligned/{variant}")


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_alpha_beta_and_nan_y(variant):
    A = gen.random_csr(2000, 1500, np.random.default_rng(2).integers(0, 50, 2000), seed=14)
    y_in = np.random.default_rng(3).uniform(-1, 1, 2000).astype(np.float32)
    for alpha, beta in [(2.5, 0.0), (-1.0, 1.0), (0.0, 0.5), (1.0, -3.0)]:
        M, y = _run(A, VARIANTS[variant], alpha, beta, y_in)
        yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x, alpha, beta, y_in)
        assert_close(y, yr, sc, TAU_F32, f"ab/{variant}/{alpha}/{beta}")
    # beta == 0: y is not read (NaN-filled y gives finite output)
    M, y = _run(A, VARIANTS[variant], 1.0, 0.0, None)
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_bit_reproducible(variant):
    A = _config("powerlaw")
    rp, ci, v = _mat(A)
    M = S.CSRMatrix(A.n_rows, A.n_cols, rp, ci, v, VARIANTS[variant])
    x = dev(A.x)
    ys = []
    for _ in range(3):
        y = torch.empty(A.n_rows, device="cuda")
        M.apply(x, y)
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], ys[2])


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("case", ["short", "long"])
def test_apply_rows_scatter(variant, case):
    """y[map[i]] = alpha (A x)_i + beta y[map[i]]; other entries untouched
    (short rows: blocks; long rows: chunked rows and their finishing pass)."""
    if case == "short":
        A = gen.random_csr(5000, 3000, np.random.default_rng(3).integers(0, 20, 5000), seed=3)
    else:
        A = _long_rows_matrix()
    rng = np.random.default_rng(4)
    n_y = 3 * A.n_rows + 7
    row_map = rng.permutation(n_y)[:A.n_rows].astype(np.int32)
    y_in = rng.uniform(-1, 1, n_y).astype(np.float32)
    rp, ci, v = _mat(A)
    M = S.CSRMatrix(A.n_rows, A.n_cols, rp, ci, v, VARIANTS[variant])
    for alpha, beta in [(1.0, 1.0), (-0.5, 0.0)]:
        y = dev(y_in)
        print(f"[apply_rows] {case} {variant} {alpha} {beta}", flush=True)
        M.apply_rows(dev(A.x), y, dev(row_map), alpha, beta)
        got = host(y)
        yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x, alpha, beta, y_in[row_map])
        assert_close(got[row_map], yr, sc, TAU_F32, f"rows/{case}/{variant}")
        rest = np.ones(n_y, bool)
        rest[row_map] = False
        assert np.array_equal(got[rest].view(np.uint32), y_in[rest].view(np.uint32))


def test_zero_rows_and_zero_nnz():
    rp = torch.zeros(1, dtype=torch.int32, device="cuda")
    e_i = torch.zeros(0, dtype=torch.int32, device="cuda")
    e_f = torch.zeros(0, dtype=torch.float32, device="cuda")
    for var in VARIANTS.values():
        M = S.CSRMatrix(0, 5, rp, e_i, e_f, var)
        M.apply(torch.zeros(5, device="cuda"), torch.zeros(0, device="cuda"))
    rp = torch.zeros(4, dtype=torch.int32, device="cuda")
    for var in VARIANTS.values():
        M = S.CSRMatrix(3, 0, rp, e_i, e_f, var)
        y = torch.tensor([1.0, 2.0, 3.0], device="cuda")
        M.apply(torch.zeros(0, device="cuda"), y, 1.0, 2.0)
        assert host(y).tolist() == [2.0, 4.0, 6.0]


@pytest.mark.parametrize("bad", ["col_high", "col_neg", "rp_decreasing", "rp_last", "rp_first"])
def test_invalid_matrix_rejected(bad):
    A = gen.random_csr(50, 40, np.full(50, 4), seed=1)
    rp, ci = A.row_ptr.copy(), A.col_idx.copy()
    if bad == "col_high":
        ci[17] = 40
    elif bad == "col_neg":
        ci[3] = -1
    elif bad == "rp_decreasing":
        rp[10] = rp[11] + 1
    elif bad == "rp_last":
        rp[-1] -= 1
    elif bad == "rp_first":
        rp[0] = 1
    nnz = len(ci)
    for var in VARIANTS.values():
        ws = torch.empty(S.spmv_csr_plan_size(50, nnz), dtype=torch.uint8, device="cuda")
        with pytest.raises(S.SpmvError) as e:
            S.spmv_csr_create(50, 40, dev(rp), dev(ci), dev(A.vals), var, None, ws)
        assert e.value.status == 2


def test_row_stats_and_recommendation():
    for name, want in [("tiny", 0), ("laplacian", 0), ("powerlaw", 2)]:
        A = _config(name)
        st = S.spmv_csr_row_stats(dev(A.row_ptr))
        assert st == oracle.row_stats(A.row_ptr)
        assert S.spmv_format_recommend(A.n_rows, st[1], st[2]) == want
