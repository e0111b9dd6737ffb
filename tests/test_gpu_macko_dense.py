"""GPU parity of the MACKO path and the dense fp16 GEMV against the oracle,
through the C ABI.

* the host encoder is bit-exact with the oracle encoder (mrow_ptr, codes,
  values) at every shape here, the full 12288 x 12288 ones included, and the
  references below come from the oracle's own encoding;
* on-GPU column decoding is bit-exact with the oracle decoder (12288 x 12288
  at 50 / 70 / 90 % sparsity, and small shapes);
* at 50 / 70 / 90 % the MACKO result also meets the bound against the dense
  fp16 oracle on the densified matrix (no MACKO code on the reference side);
* MACKO SpMV: |y - y_ref| <= 4e-3 * scale (fp16 values and x, fp32
  accumulation) at the full pruned-weight sizes, with alpha / beta, x in LDS
  and x from global memory (n_cols > 32768), trailing pads past the last
  column, empty rows; bit-reproducible run to run;
* dense GEMV: same tolerance at 12288 x 12288 and odd shapes (n % 8 != 0).
"""
import numpy as np
import pytest

import gen
import oracle
from helpers import TAU_F16, assert_close, dev, host

torch = pytest.importorskip("torch")
S = pytest.importorskip("sparse_matrix_vector_amd")

pytestmark = pytest.mark.gpu

_CACHE = {}


def _pruned(s, n_rows=12288, n_cols=None, seed=3):
    key = (s, n_rows, n_cols, seed)
    if key not in _CACHE:
        W = gen.pruned_weight(s, n_rows=n_rows, n_cols=n_cols, seed=seed)
        enc = S.macko_encode(W.n_rows, W.n_cols, W.row_ptr, W.col_idx, W.vals_f16)
        oenc = oracle.macko_encode(W.n_cols, W.row_ptr, W.col_idx, W.vals_f16)
        for name, a, b in zip(("mrow_ptr", "codes", "values"), enc, oenc):
            assert np.array_equal(a, b), f"encoder differs from the oracle in {name} ({key})"
        _CACHE.clear()
        _CACHE[key] = (W, enc, oenc)
    return _CACHE[key]


def _spmv(W, enc, alpha=1.0, beta=0.0, y_in=None):
    mrp, codes, mv = enc
    y = dev(y_in) if y_in is not None else torch.full((W.n_rows,), float("nan"), device="cuda")
    S.macko_spmv(W.n_rows, W.n_cols, dev(mrp), dev(codes), dev(mv), alpha, dev(W.x_f16), beta, y)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("s", [0.5, 0.7, 0.9])
def test_full_size_decode_and_spmv(s):
    W, enc, oenc = _pruned(s)
    mrp, codes, mv = enc
    omrp, ocodes, omv = oenc
    print(f"[macko] s={s} entries={mrp[-1]}", flush=True)
    cols = torch.empty(int(mrp[-1]), dtype=torch.int32, device="cuda")
    S.macko_decode_columns(W.n_rows, dev(mrp), dev(codes), cols)
    torch.cuda.synchronize()
    assert np.array_equal(host(cols), oracle.macko_decode(omrp, ocodes))
    y = _spmv(W, enc)
    yr, sc = oracle.macko_spmv(W.n_cols, omrp, ocodes, omv, W.x_f16)
    err = assert_close(y, yr, sc, TAU_F16, f"macko s={s}")
    assert err < 1e-5      # fp16 products are exact in fp32: far inside the bound
    yd, scd = oracle.gemv_f16(W.dense_f16(), W.x_f16)
    assert_close(y, yd, scd, TAU_F16, f"macko s={s} against the dense oracle")


@pytest.mark.parametrize("shape", [(37, 1000, 0.5), (5, 17, 0.0), (64, 40000, 0.9), (300, 2049, 0.7),
                                   (3, 33000, 0.999)])
def test_small_shapes(shape):
    n_rows, n_cols, s = shape
    W, enc, oenc = _pruned(s, n_rows, n_cols, seed=9)
    mrp, codes, mv = oenc
    cols = torch.empty(max(int(mrp[-1]), 1), dtype=torch.int32, device="cuda")
    S.macko_decode_columns(W.n_rows, dev(mrp), dev(codes), cols)
    torch.cuda.synchronize()
    assert np.array_equal(host(cols)[:int(mrp[-1])], oracle.macko_decode(mrp, codes))
    y_in = np.random.default_rng(1).uniform(-1, 1, n_rows).astype(np.float32)
    for alpha, beta in [(1.0, 0.0), (0.25, -1.5)]:
        y = _spmv(W, enc, alpha, beta, y_in if beta else None)
        yr, sc = oracle.macko_spmv(W.n_cols, mrp, codes, mv, W.x_f16, alpha, beta, y_in)
        assert_close(y, yr, sc, TAU_F16, f"macko {shape} {alpha} {beta}")


def test_trailing_pad_beyond_last_column_and_empty_rows():
    n_cols = 300
    rp = np.array([0, 1, 1, 3, 3], np.int32)
    ci = np.array([299, 0, 299], np.int32)
    v = np.array([1.5, -2.0, 0.25], np.float16).view(np.uint16)
    x = np.linspace(-1, 1, n_cols).astype(np.float16).view(np.uint16)
    enc = S.macko_encode(4, n_cols, rp, ci, v)
    mrp, codes, mv = enc
    y = torch.full((4,), float("nan"), device="cuda")
    S.macko_spmv(4, n_cols, dev(mrp), dev(codes), dev(mv), 1.0, dev(x), 0.0, y)
    yr, sc = oracle.macko_spmv(n_cols, mrp, codes, mv, x)
    assert_close(host(y), yr, sc, TAU_F16, "pads")
    assert host(y)[1] == 0.0 and host(y)[3] == 0.0


def _random_macko(n_rows, n_cols, lens, seed):
    A = gen.random_csr(n_rows, n_cols, lens, seed)
    v16 = A.vals.astype(np.float16)
    v16[v16 == 0] = np.float16(0.5)          # stored entries are nonzero
    x16 = A.x.astype(np.float16).view(np.uint16)
    enc = S.macko_encode(n_rows, n_cols, A.row_ptr, A.col_idx, v16.view(np.uint16))
    return enc, x16


def test_many_rows_per_wave():
    """More than 64 rows per wave (rows are taken in batches of 64), with
    empty rows and rows spanning several groups of 2048 entries."""
    n_rows, n_cols = 450_000, 4096
    rng = np.random.default_rng(11)
    lens = rng.integers(0, 5, n_rows)
    lens[::997] = 3000                     # 3000 entries + pads: 2 groups
    lens[5::13] = 0
    (mrp, codes, mv), x16 = _random_macko(n_rows, n_cols, lens, 12)
    y_in = rng.uniform(-1, 1, n_rows).astype(np.float32)
    for alpha, beta in [(1.0, 0.0), (0.5, 2.0)]:
        y = torch.full((n_rows,), float("nan"), device="cuda") if beta == 0 else dev(y_in)
        print(f"[macko] many rows alpha={alpha} beta={beta}", flush=True)
        S.macko_spmv(n_rows, n_cols, dev(mrp), dev(codes), dev(mv), alpha, dev(x16), beta, y)
        torch.cuda.synchronize()
        yr, sc = oracle.macko_spmv(n_cols, mrp, codes, mv, x16, alpha, beta, y_in)
        assert_close(host(y), yr, sc, TAU_F16, f"many rows {alpha} {beta}")


def test_misaligned_x():
    """x not 16-byte aligned: staged into LDS element by element."""
    n_rows, n_cols = 300, 1001
    lens = np.random.default_rng(5).integers(0, 400, n_rows)
    (mrp, codes, mv), x16 = _random_macko(n_rows, n_cols, lens, 6)
    xbuf = torch.zeros(n_cols + 1, dtype=torch.int16, device="cuda")
    xbuf[1:] = dev(x16.view(np.int16))
    xv = xbuf[1:]
    assert xv.data_ptr() % 16 != 0
    y = torch.full((n_rows,), float("nan"), device="cuda")
    S.macko_spmv(n_rows, n_cols, dev(mrp), dev(codes), dev(mv), 1.0, xv, 0.0, y)
    torch.cuda.synchronize()
    yr, sc = oracle.macko_spmv(n_cols, mrp, codes, mv, x16)
    assert_close(host(y), yr, sc, TAU_F16, "misaligned x")


def test_macko_bit_reproducible():
    W, enc, _ = _pruned(0.7)
    a = _spmv(W, enc)
    b = _spmv(W, enc)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("shape", [(12288, 12288), (100, 1000), (33, 77), (7, 40000)])
def test_dense_gemv(shape):
    m, n = shape
    s = 0.5
    W = gen.pruned_weight(s, n_rows=m, n_cols=n, seed=4)
    D = W.dense_f16()
    print(f"[gemv] {m}x{n}", flush=True)
    y_in = np.random.default_rng(2).uniform(-1, 1, m).astype(np.float32)
    dD = dev(D)
    for alpha, beta in [(1.0, 0.0), (-0.75, 0.5)]:
        y = dev(y_in) if beta else torch.full((m,), float("nan"), device="cuda")
        S.dense_gemv_f16(m, n, dD, dev(W.x_f16), alpha, beta, y)
        torch.cuda.synchronize()
        yr, sc = oracle.gemv_f16(D, W.x_f16, alpha, beta, y_in)
        assert_close(host(y), yr, sc, TAU_F16, f"gemv {shape}")
    if shape == (12288, 12288):
        # the densified matrix gives the MACKO result
        enc = S.macko_encode(m, n, W.row_ptr, W.col_idx, W.vals_f16)
        ym = _spmv(W, enc)
        y = torch.empty(m, device="cuda")
        S.dense_gemv_f16(m, n, dD, dev(W.x_f16), 1.0, 0.0, y)
        yr, sc = oracle.gemv_f16(D, W.x_f16)
        assert_close(ym, yr, sc, TAU_F16, "macko vs dense oracle")
