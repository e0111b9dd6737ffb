"""GPU parity of MACKO with code widths b = 1, 2, 4, 8 and of the 8-bit
value mode against the oracle, through the C ABI.

* on-GPU column decoding is bit-exact with the oracle decoder for every
  width (12288 x 12288 pruned weights and small shapes);
* SpMV with fp16 values and with int8 values (host-quantised, per-row
  scale): |y - y_ref| <= 4e-3 * scale, and in practice within 1e-5 (all
  products are exact in fp32), at the full pruned-weight size, at small and
  ragged shapes with alpha / beta, with x in LDS and x from global memory
  (n_cols > 32768), x not 16-byte aligned, trailing alignment pads far past
  the last column (1023 of them at b = 1), rows shorter than a chunk (b = 8
  aligns rows to 128 entries), empty rows and more than 64 rows per wave.
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


def _encoded(s, b, n_rows=12288, n_cols=None, seed=3):
    key = (s, b, n_rows, n_cols, seed)
    if key not in _CACHE:
        W = gen.pruned_weight(s, n_rows=n_rows, n_cols=n_cols, seed=seed)
        enc = S.macko_encode(W.n_rows, W.n_cols, W.row_ptr, W.col_idx, W.vals_f16, bdelta=b)
        oenc = oracle.macko_encode(W.n_cols, W.row_ptr, W.col_idx, W.vals_f16, bdelta=b)
        for name, x, y in zip(("mrow_ptr", "codes", "values"), enc, oenc):
            assert np.array_equal(x, y), f"encoder differs from the oracle in {name} ({key})"
        _CACHE.clear()
        _CACHE[key] = (W, enc)
    return _CACHE[key]


def _run(n_rows, n_cols, b, enc, x16, i8, alpha=1.0, beta=0.0, y_in=None, xdev=None):
    """GPU result and the oracle's (y, scale).  enc is asserted equal to the
    oracle's encoding where it is built, so the reference uses the same
    arrays; the int8 values are checked against the oracle's quantiser here."""
    mrp, codes, mv = enc
    y = dev(y_in) if beta else torch.full((n_rows,), float("nan"), device="cuda")
    xd = dev(x16) if xdev is None else xdev
    if i8:
        q, sc = S.macko_quantize_i8(n_rows, mrp, mv)
        oq, osc = oracle.macko_quantize_i8(mrp, mv)
        assert np.array_equal(q, oq) and np.array_equal(sc.view(np.uint32), osc.view(np.uint32))
        S.macko_spmv_i8(n_rows, n_cols, dev(mrp), dev(codes), dev(q), dev(sc), alpha, xd, beta, y, bdelta=b)
        torch.cuda.synchronize()
        yr, s = oracle.macko_spmv_i8(n_cols, mrp, codes, oq, osc, x16, alpha, beta, y_in, bdelta=b)
    else:
        S.macko_spmv(n_rows, n_cols, dev(mrp), dev(codes), dev(mv), alpha, xd, beta, y, bdelta=b)
        torch.cuda.synchronize()
        yr, s = oracle.macko_spmv(n_cols, mrp, codes, mv, x16, alpha, beta, y_in, bdelta=b)
    return host(y), yr, s


def _decode_check(n_rows, b, enc):
    mrp, codes, mv = enc
    cols = torch.empty(max(int(mrp[-1]), 1), dtype=torch.int32, device="cuda")
    S.macko_decode_columns(n_rows, dev(mrp), dev(codes), cols, bdelta=b)
    torch.cuda.synchronize()
    assert np.array_equal(host(cols)[:int(mrp[-1])], oracle.macko_decode(mrp, codes, bdelta=b))


@pytest.mark.parametrize("b,s,i8", [(1, 0.5, False), (2, 0.5, False), (2, 0.7, False), (8, 0.9, False),
                                    (4, 0.5, True), (2, 0.7, True), (8, 0.9, True)])
def test_full_size(b, s, i8):
    W, enc = _encoded(s, b)
    print(f"[macko] b={b} s={s} int8={i8} entries={enc[0][-1]}", flush=True)
    if not i8:
        _decode_check(W.n_rows, b, enc)
    y, yr, sc = _run(W.n_rows, W.n_cols, b, enc, W.x_f16, i8)
    err = assert_close(y, yr, sc, TAU_F16, f"macko b={b} s={s} int8={i8}")
    assert err < 1e-5
    if not i8:
        # and against the dense fp16 oracle on the densified matrix
        yd, scd = oracle.gemv_f16(W.dense_f16(), W.x_f16)
        assert_close(y, yd, scd, TAU_F16, f"macko b={b} s={s} against the dense oracle")


SHAPES = [(37, 1000, 0.5), (5, 17, 0.0), (64, 40000, 0.9), (300, 2049, 0.7), (3, 33000, 0.999)]


@pytest.mark.parametrize("b", [1, 2, 8])
@pytest.mark.parametrize("shape", SHAPES)
def test_small_shapes(b, shape):
    n_rows, n_cols, s = shape
    W, enc = _encoded(s, b, n_rows, n_cols, seed=9)
    print(f"[macko] b={b} shape={shape}", flush=True)
    _decode_check(n_rows, b, enc)
    y_in = np.random.default_rng(1).uniform(-1, 1, n_rows).astype(np.float32)
    for i8 in (False, True):
        for alpha, beta in [(1.0, 0.0), (0.25, -1.5)]:
            y, yr, sc = _run(n_rows, n_cols, b, enc, W.x_f16, i8, alpha, beta, y_in if beta else None)
            assert_close(y, yr, sc, TAU_F16, f"b={b} {shape} int8={i8} {alpha} {beta}")


@pytest.mark.parametrize("shape", SHAPES[:3])
def test_int8_width4_small_shapes(shape):
    n_rows, n_cols, s = shape
    W, enc = _encoded(s, 4, n_rows, n_cols, seed=10)
    y, yr, sc = _run(n_rows, n_cols, 4, enc, W.x_f16, True, -2.0, 0.5,
                     np.linspace(-1, 1, n_rows).astype(np.float32))
    assert_close(y, yr, sc, TAU_F16, f"int8 b=4 {shape}")


@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_trailing_pads_and_empty_rows(b):
    n_cols = 300
    rp = np.array([0, 1, 1, 3, 3, 4], np.int32)
    ci = np.array([299, 0, 299, 150], np.int32)
    v = np.array([1.5, -2.0, 0.25, 3.0], np.float16).view(np.uint16)
    x = np.linspace(-1, 1, n_cols).astype(np.float16).view(np.uint16)
    enc = S.macko_encode(5, n_cols, rp, ci, v, bdelta=b)
    for i8 in (False, True):
        y, yr, sc = _run(5, n_cols, b, enc, x, i8)
        assert_close(y, yr, sc, TAU_F16, f"pads b={b} int8={i8}")
        assert y[1] == 0.0 and y[3] == 0.0


@pytest.mark.parametrize("b", [1, 8])
def test_many_rows_per_wave(b):
    n_rows, n_cols = 200_000, 4096
    rng = np.random.default_rng(11)
    lens = rng.integers(0, 5, n_rows)
    lens[::997] = 3000
    lens[5::13] = 0
    A = gen.random_csr(n_rows, n_cols, lens, 12)
    v16 = A.vals.astype(np.float16)
    v16[v16 == 0] = np.float16(0.5)
    x16 = A.x.astype(np.float16).view(np.uint16)
    enc = S.macko_encode(n_rows, n_cols, A.row_ptr, A.col_idx, v16.view(np.uint16), bdelta=b)
    y_in = rng.uniform(-1, 1, n_rows).astype(np.float32)
    for i8 in (False, True):
        print(f"[macko] many rows b={b} int8={i8}", flush=True)
        y, yr, sc = _run(n_rows, n_cols, b, enc, x16, i8, 0.5, 2.0, y_in)
        assert_close(y, yr, sc, TAU_F16, f"many rows b={b} int8={i8}")


@pytest.mark.parametrize("b", [2, 8])
def test_misaligned_x(b):
    n_rows, n_cols = 300, 1001
    lens = np.random.default_rng(5).integers(0, 400, n_rows)
    A = gen.random_csr(n_rows, n_cols, lens, 6)
    v16 = A.vals.astype(np.float16)
    v16[v16 == 0] = np.float16(0.5)
    x16 = A.x.astype(np.float16).view(np.uint16)
    enc = S.macko_encode(n_rows, n_cols, A.row_ptr, A.col_idx, v16.view(np.uint16), bdelta=b)
    xbuf = torch.zeros(n_cols + 1, dtype=torch.int16, device="cuda")
    xbuf[1:] = dev(x16.view(np.int16))
    assert xbuf[1:].data_ptr() % 16 != 0
    for i8 in (False, True):
        y, yr, sc = _run(n_rows, n_cols, b, enc, x16, i8, xdev=xbuf[1:])
        assert_close(y, yr, sc, TAU_F16, f"misaligned x b={b} int8={i8}")


@pytest.mark.parametrize("b,n_cols", [(4, 32448), (4, 32449), (1, 31680), (1, 31681)])
def test_lds_staging_boundary(b, n_cols):
    """x plus its zero padding fills exactly 64 KB of LDS, or one column
    more and x is read from global memory."""
    W, enc = _encoded(0.9, b, 20, n_cols, seed=13)
    for i8 in (False, True):
        y, yr, sc = _run(20, n_cols, b, enc, W.x_f16, i8, 1.0, 0.0)
        assert_close(y, yr, sc, TAU_F16, f"boundary b={b} n_cols={n_cols} int8={i8}")
