"""GPU parity of the HYB path (ELL part + CSR tail) and of the CV-driven
format choice against the oracle, through the C ABI.

* width rule and tail sizes equal the oracle's (golden cases, configs);
* the split is bit-exact with the oracle's (ELL slots, tail rows, tail row
  pointers, tail entries), at the rule's width and at widths 0 and max;
* apply: |y - y_ref| <= 1e-5 * scale with alpha / beta, on tiny, Laplacian,
  power-law and moderate-CV (HYB range) matrices, empty rows, a single row;
* the auto handle picks the CV rule's format (tiny and Laplacian -> ELL,
  moderate CV -> HYB, power-law -> binned CSR) and matches the oracle;
* wrong tail sizes and out-of-range columns are rejected.
"""
import json
import os

import numpy as np
import pytest

import gen
import oracle
from helpers import TAU_F32, assert_close, dev, host

torch = pytest.importorskip("torch")
S = pytest.importorskip("sparse_matrix_vector_amd")

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
SPMV_ERR_OVERFLOW = 4   # include/spmv.h

CASES = {
    "tiny": lambda: gen.tiny_csr(),
    "laplacian": lambda: gen.laplacian_2d(1000),
    "powerlaw": lambda: gen.powerlaw_csr(),
    "varlen": lambda: gen.varlen_banded(),
    "ragged": lambda: gen.random_csr(1003, 800, np.r_[np.random.default_rng(1).integers(0, 30, 1000), 0, 0, 700],
                                     seed=1),
    "single": lambda: gen.random_csr(1, 10, [7], seed=2),
}
_CACHE = {}


def _case(name):
    if name not in _CACHE:
        _CACHE.clear()
        _CACHE[name] = CASES[name]()
    return _CACHE[name]


def test_width_golden():
    for c in json.load(open(os.path.join(HERE, "golden", "hyb_width.json")))["cases"]:
        rp = np.concatenate([[0], np.cumsum(c["lens"])]).astype(np.int32)
        got = S.spmv_hyb_width(len(c["lens"]), dev(rp), c["num"], c["den"])
        assert got == (c["width"], c["tail_rows"], c["tail_nnz"]), c


def _split(A, W=None):
    w, r, t = S.spmv_hyb_width(A.n_rows, dev(A.row_ptr))
    if W is not None and W != w:
        w = W
        r, t = S.spmv_hyb_tail_size(A.n_rows, dev(A.row_ptr), w)
        assert (r, t) == oracle.hyb_tail_size(A.row_ptr, w)
    arrs = dict(ec=torch.empty(w * A.n_rows, dtype=torch.int32, device="cuda"),
                ev=torch.empty(w * A.n_rows, dtype=torch.float32, device="cuda"),
                tr=torch.empty(r, dtype=torch.int32, device="cuda"),
                trp=torch.empty(r + 1, dtype=torch.int32, device="cuda"),
                tc=torch.empty(t, dtype=torch.int32, device="cuda"),
                tv=torch.empty(t, dtype=torch.float32, device="cuda"))
    S.spmv_hyb_from_csr(A.n_rows, A.n_cols, dev(A.row_ptr), dev(A.col_idx), dev(A.vals), w, r, t,
                        arrs["ec"], arrs["ev"], arrs["tr"], arrs["trp"], arrs["tc"], arrs["tv"])
    return w, r, t, arrs


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("which", ["rule", "zero", "max"])
def test_split_and_apply(case, which):
    A = _case(case)
    W = {"rule": None, "zero": 0, "max": oracle.row_stats(A.row_ptr)[0]}[which]
    if which == "max" and W * A.n_rows > 2**31 - 1:
        # power-law: 4,334 slots x 916k rows exceed int32 slot indices; both
        # conversions refuse before anything is read or written
        print(f"[hyb] {case} W={W}: {W * A.n_rows} slots", flush=True)
        L = S.lib()
        sc = torch.empty(S.spmv_scratch_size(A.n_rows), dtype=torch.uint8, device="cuda")
        rp, ci, v = dev(A.row_ptr), dev(A.col_idx), dev(A.vals)
        st = L.spmv_ell_from_csr(A.n_rows, A.n_cols, A.nnz, rp.data_ptr(), ci.data_ptr(), v.data_ptr(), W, None, None,
                                 sc.data_ptr(), sc.numel(), None)
        assert st == SPMV_ERR_OVERFLOW
        st = L.spmv_hyb_from_csr(A.n_rows, A.n_cols, A.nnz, rp.data_ptr(), ci.data_ptr(), v.data_ptr(), W, None, None,
                                 0, 0, None, rp.data_ptr(), None, None, sc.data_ptr(), sc.numel(), None)
        assert st == SPMV_ERR_OVERFLOW
        return
    w, r, t, a = _split(A, W)
    print(f"[hyb] {case} W={w} tail rows={r} entries={t}", flush=True)
    if W is None:
        assert w == oracle.hyb_width(A.row_ptr)
        assert (r, t) == oracle.hyb_tail_size(A.row_ptr, w)
    oec, oev, otr, otrp, otc, otv = oracle.hyb_from_csr(A.row_ptr, A.col_idx, A.vals, w)
    assert np.array_equal(host(a["ec"]), oec)
    assert np.array_equal(host(a["ev"]).view(np.uint32), oev.view(np.uint32))
    assert np.array_equal(host(a["tr"]), otr) and np.array_equal(host(a["trp"]), otrp)
    assert np.array_equal(host(a["tc"]), otc)
    assert np.array_equal(host(a["tv"]).view(np.uint32), otv.view(np.uint32))
    rng = np.random.default_rng(7)
    y_in = rng.uniform(-1, 1, A.n_rows).astype(np.float32)
    for alpha, beta in [(1.0, 0.0), (-0.5, 2.0)]:
        y = dev(y_in) if beta else torch.full((A.n_rows,), float("nan"), device="cuda")
        S.spmv_hyb_apply(A.n_rows, A.n_cols, w, a["ec"], a["ev"], r, t, a["tr"], a["trp"], a["tc"], a["tv"],
                         alpha, dev(A.x), beta, y)
        yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x, alpha, beta, y_in)
        assert_close(host(y), yr, sc, TAU_F32, f"{case}/{which}/{alpha}/{beta}")


@pytest.mark.parametrize("case,expect", [("tiny", 0), ("laplacian", 0), ("varlen", 1), ("powerlaw", 2),
                                         ("ragged", 2)])
def test_auto_choice_and_apply(case, expect):
    A = _case(case)
    M = S.AutoMatrix(A.n_rows, A.n_cols, dev(A.row_ptr), dev(A.col_idx), dev(A.vals))
    lens = np.diff(A.row_ptr).astype(np.int64)
    rule = oracle.format_choice(len(lens), int(lens.sum()), int((lens ** 2).sum()))
    print(f"[auto] {case} format={M.format} rule={rule}", flush=True)
    assert M.format == expect == rule
    rng = np.random.default_rng(9)
    y_in = rng.uniform(-1, 1, A.n_rows).astype(np.float32)
    for alpha, beta in [(1.0, 0.0), (0.25, -1.0)]:
        y = dev(y_in) if beta else torch.full((A.n_rows,), float("nan"), device="cuda")
        M.apply(dev(A.x), y, alpha, beta)
        yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x, alpha, beta, y_in)
        assert_close(host(y), yr, sc, TAU_F32, f"auto {case}")


@pytest.mark.parametrize("n,misaligned_y", [(8192, False), (8190, False), (8192, True), (4 * 1024 * 3 + 4, False)])
def test_auto_hyb_shapes(n, misaligned_y):
    """Moderate-CV matrices (HYB) through the auto handle: the 4-row ELL
    kernel (n % 4 == 0, aligned) or the 1-row one (n % 4 != 0, misaligned y),
    then the binned tail. Rows up to 40 entries, tail rows at ELL-workgroup
    edges, a partial last workgroup; alpha / beta; repeated applies are
    bit-equal."""
    rng = np.random.default_rng(n)
    lens = rng.integers(1, 13, n)
    lens[rng.choice(n, n // 200, replace=False)] = rng.integers(20, 41, n // 200)
    lens[[0, 1023, 1024, 4095, 4096, n - 1]] = 17
    A = gen.random_csr(n, 3000, lens, seed=n + 1)
    s1, s2 = int(lens.sum()), int((lens.astype(np.int64) ** 2).sum())
    assert oracle.format_choice(n, s1, s2) == 1
    M = S.AutoMatrix(A.n_rows, A.n_cols, dev(A.row_ptr), dev(A.col_idx), dev(A.vals))
    assert M.format == 1
    y_in = rng.uniform(-1, 1, n).astype(np.float32)
    buf = torch.zeros(n + 1, device="cuda")
    y = buf[1:] if misaligned_y else buf[:n]
    outs = []
    for _ in range(2):
        y.copy_(dev(y_in))
        M.apply(dev(A.x), y, 0.5, 2.0)
        torch.cuda.synchronize()
        outs.append(host(y).copy())
    print(f"[auto hyb] n={n} misaligned_y={misaligned_y}", flush=True)
    yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x, 0.5, 2.0, y_in)
    assert_close(outs[0], yr, sc, TAU_F32, f"auto hyb n={n}")
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


@pytest.mark.parametrize("n,x_off,y_off,n_cols", [(8192, 0, 0, 3000), (4 * 1024 * 3 + 4, 0, 0, 3000),
                                                  (8190, 0, 0, 3000), (8192, 1, 0, 3000), (8192, 0, 1, 3000),
                                                  (8192, 0, 0, 3001)])
def test_auto_hyb_one_launch(n, x_off, y_off, n_cols):
    """HYB with short tails (every row at most 16 entries past the width):
    with n % 4 == 0 and x, y 16-byte aligned the ELL part and the tail run in
    one kernel, each wave summing its rows' run of tail entries in rounds of
    512; otherwise (n or n_cols not a multiple of 4, x or y misaligned) the
    ELL kernel and then the binned tail.  Rows of 1..12 entries, one wave of 256 rows with 17
    each (a run of several rounds), waves without tail rows, tail rows at
    wave and workgroup edges; alpha / beta against the oracle, and the two
    forms against each other."""
    rng = np.random.default_rng(n + 7 * x_off + 3 * y_off)
    lens = rng.integers(1, 13, n)
    lens[2048:2048 + 256] = 17                      # one wave's rows (ELL rows 4 per lane)
    lens[4096:4096 + 512] = rng.integers(1, 4, 512)  # two waves without tails
    lens[[0, 255, 256, 1023, 1024, 4095, n - 1]] = 16
    A = gen.random_csr(n, n_cols, lens, seed=n + 5)
    s1, s2 = int(lens.sum()), int((lens.astype(np.int64) ** 2).sum())
    assert oracle.format_choice(n, s1, s2) == 1
    M = S.AutoMatrix(A.n_rows, A.n_cols, dev(A.row_ptr), dev(A.col_idx), dev(A.vals))
    assert M.format == 1
    W = int(M.plan.width)
    heavy = int(np.maximum(lens[2048:2048 + 256] - W, 0).sum())
    print(f"[auto hyb 1-launch] n={n} n_cols={n_cols} x_off={x_off} y_off={y_off} W={W} heaviest wave run {heavy}",
          flush=True)
    assert lens.max() - W <= 16 and heavy > 512
    y_in = rng.uniform(-1, 1, n).astype(np.float32)
    xb = torch.zeros(A.n_cols + 4, device="cuda")
    x = xb[x_off:x_off + A.n_cols]
    x.copy_(dev(A.x))
    yb = torch.zeros(n + 4, device="cuda")
    y = yb[y_off:y_off + n]
    for alpha, beta in [(1.0, 0.0), (0.5, 2.0)]:
        y.copy_(dev(y_in) if beta else torch.full((n,), float("nan"), device="cuda"))
        M.apply(x, y, alpha, beta)
        torch.cuda.synchronize()
        yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x, alpha, beta, y_in)
        assert_close(host(y), yr, sc, TAU_F32, f"auto hyb 1-launch n={n} {alpha} {beta}")
    # the same handle with a misaligned x (ELL kernel, then the binned tail)
    xm = torch.zeros(A.n_cols + 4, device="cuda")[1:1 + A.n_cols]
    xm.copy_(dev(A.x))
    y2 = torch.zeros(n, device="cuda")
    y2.copy_(dev(y_in))
    M.apply(xm, y2, 0.5, 2.0)
    torch.cuda.synchronize()
    assert_close(host(y2), host(y).astype(np.float64), sc, 2 * TAU_F32, "one launch vs two")


def test_auto_ell_padding_guard():
    """CV < 0.3 but one long row: padding every row to it would more than
    double the storage, so HYB is used instead of ELL."""
    lens = np.full(5000, 10)
    lens[17] = 100                                # CV 0.13, padding 10x
    A = gen.random_csr(5000, 5000, lens, 13)
    s1, s2 = int(lens.sum()), int((lens.astype(np.int64) ** 2).sum())
    assert oracle.format_choice(5000, s1, s2) == 0
    M = S.AutoMatrix(A.n_rows, A.n_cols, dev(A.row_ptr), dev(A.col_idx), dev(A.vals))
    assert M.format == 1
    y = torch.empty(5000, device="cuda")
    M.apply(dev(A.x), y)
    yr, sc = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x)
    assert_close(host(y), yr, sc, TAU_F32, "guard")


def test_all_rows_empty():
    A = gen.random_csr(100, 50, np.zeros(100, np.int64), 0)
    w, r, t, a = _split(A)
    assert (w, r, t) == (0, 0, 0)
    y_in = np.ones(100, np.float32)
    y = dev(y_in)
    S.spmv_hyb_apply(100, 50, w, a["ec"], a["ev"], r, t, a["tr"], a["trp"], a["tc"], a["tv"], 1.0, dev(A.x), 3.0, y)
    assert np.array_equal(host(y), np.full(100, 3.0, np.float32))


def test_tail_size_matches_oracle():
    """spmv_hyb_tail_size at explicit widths, bit-exact with the oracle's
    count, on the moderate-CV and power-law matrices."""
    for name in ("varlen", "powerlaw"):
        A = _case(name)
        mx = oracle.row_stats(A.row_ptr)[0]
        for W in (0, 1, 3, 7, 33, mx - 1, mx, mx + 5):
            assert S.spmv_hyb_tail_size(A.n_rows, dev(A.row_ptr), W) == oracle.hyb_tail_size(A.row_ptr, W), (name, W)


def test_rejects_wrong_tail_sizes_and_bad_columns():
    A = gen.random_csr(64, 64, np.arange(64) % 7, 3)
    w, r, t = S.spmv_hyb_width(64, dev(A.row_ptr))
    bufs = [torch.full((max(n, 1),), 77, dtype=d, device="cuda") for n, d in
            [(w * 64, torch.int32), (w * 64, torch.float32), (r + 1, torch.int32), (r + 2, torch.int32),
             (t + 1, torch.int32), (t + 1, torch.float32)]]
    with pytest.raises(S.SpmvError) as e:
        S.spmv_hyb_from_csr(64, 64, dev(A.row_ptr), dev(A.col_idx), dev(A.vals), w, r + 1, t, *bufs)
    assert e.value.status == 1
    # sizes are checked before any kernel writes the caller's arrays
    for b in bufs:
        assert bool((b == 77).all())
    bad = A.col_idx.copy()
    bad[-1] = 64                                   # last entry of the last nonempty row
    with pytest.raises(S.SpmvError) as e:
        S.spmv_hyb_from_csr(64, 64, dev(A.row_ptr), dev(bad), dev(A.vals), w, r, t, *bufs)
    assert e.value.status == 2
