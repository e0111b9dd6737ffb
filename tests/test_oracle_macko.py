"""Pins of the MACKO encoder / decoder / SpMV oracle and of the fp16 decoding.

* the page's worked delta example and hand cases (tests/golden);
* fp16 -> fp64 decoding equals NumPy's float16 conversion for all 65,536
  bit patterns;
* round trip: decoded columns of the nonzero-valued entries equal the input
  columns, values equal the input values, pads are +0;
* entry count per row from the gap closed form, sum_k (ceil(g_k/16) - 1),
  plus alignment to 256;
* stored gaps never exceed 16 (the 4-bit span) and every row is a multiple of
  256 entries;
* effective density inside the best/worst bounds and near the expected value
  of the page's section 2.3 formulas (with the density factor restored);
* MACKO SpMV equals the CSR oracle on the same fp16-valued matrix and a NumPy
  dense fp64 product;
* unsorted / duplicate / out-of-range columns are rejected;
* code widths b = 1, 2, 4, 8 (section 3.3): hand-worked codes, packed words,
  pads and decoded columns for each width (tests/golden/macko_widths.json),
  round trip and the entry-count closed form with span 2^b and alignment
  1024/b, effective density against the section 2.3 bounds with z = (1-d)^(2^b),
  the storage ranking of the widths, SpMV equal to the CSR oracle;
* the 8-bit value mode: hand-worked scales and ties-to-even codes
  (tests/golden/macko_int8.json), the rounding bound |s q - v| <= s/2, the
  row maximum mapping to +-127, and SpMV equal to a NumPy dense product of
  the dequantised matrix.
"""
import json
import os

import numpy as np
import pytest

import gen
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _nibbles(codes, E):
    words = np.repeat(codes, 8)[:E]
    shifts = np.tile(np.arange(8, dtype=np.uint32) * 4, len(codes))[:E]
    return ((words >> shifts) & 0xF).astype(np.int64)


def _one_row(cols, n_cols=64):
    cols = np.asarray(cols, np.int32)
    rp = np.array([0, len(cols)], np.int32)
    vals = (np.arange(len(cols)) + 1).astype(np.float16).view(np.uint16)   # nonzero, distinct
    return rp, cols, vals


def test_fp16_decoding_all_patterns():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = allbits.view(np.float16).astype(np.float64)
    L = oracle.lib()
    got = np.array([L.oracle_half_to_double(int(b)) for b in allbits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    assert np.array_equal(np.signbit(got[~np.isnan(got)]), np.signbit(ref[~np.isnan(ref)]))


def test_page_example_and_hand_cases():
    g = json.load(open(os.path.join(GOLD, "macko_examples.json")))
    ex = g["page_example"]
    rp, ci, v = _one_row(ex["columns"])
    mrp, codes, mv = oracle.macko_encode(64, rp, ci, v)
    assert mrp.tolist() == [0, g["alignment_entries"]]
    got = _nibbles(codes, mrp[-1])[:len(ex["codes"])]
    assert got.tolist() == ex["codes"]
    # after the first entry the codes are the page's deltas minus one
    assert (got[1:] + 1).tolist() == ex["page_deltas"][1:]
    for case in g["cases"]:
        rp, ci, v = _one_row(case["columns"])
        mrp, codes, mv = oracle.macko_encode(64, rp, ci, v)
        k = len(case["codes"])
        assert _nibbles(codes, mrp[-1])[:k].tolist() == case["codes"], case
        assert ((mv[:k] == 0) == np.array(case["is_pad"])).all(), case
        assert oracle.macko_decode(mrp, codes)[:k].tolist() == case["decoded"], case
        # trailing alignment entries: code 0, value +0
        assert np.all(_nibbles(codes, mrp[-1])[k:] == 0) and np.all(mv[k:] == 0)


def _gap_count(rp, ci):
    n = len(rp) - 1
    out = np.zeros(n, np.int64)
    for i in range(n):
        c = ci[rp[i]:rp[i + 1]].astype(np.int64)
        if len(c) == 0:
            continue
        gaps = np.diff(np.concatenate([[-1], c]))
        raw = len(c) + int(np.sum((gaps + 15) // 16 - 1))
        out[i] = -(-raw // 256) * 256
    return out


@pytest.mark.parametrize("s,n_cols,n_rows", [(0.5, 2048, 64), (0.7, 3000, 50), (0.9, 12288, 40),
                                             (0.97, 12288, 20), (0.0, 300, 5)])
def test_round_trip_and_counts(s, n_cols, n_rows):
    W = gen.pruned_weight(s, n_rows=n_rows, n_cols=n_cols, seed=21)
    mrp, codes, mv = oracle.macko_encode(n_cols, W.row_ptr, W.col_idx, W.vals_f16)
    E = int(mrp[-1])
    assert E % 256 == 0 and np.all(np.diff(mrp) % 256 == 0)
    assert np.array_equal(np.diff(mrp), _gap_count(W.row_ptr, W.col_idx))
    cols = oracle.macko_decode(mrp, codes)
    real = mv != 0
    assert np.array_equal(cols[real], W.col_idx)
    assert np.array_equal(mv[real], W.vals_f16)
    assert np.all(mv[~real] == 0)              # pads are +0 exactly
    nib = _nibbles(codes, E)
    # every stored gap (code + 1) is within the 4-bit span
    assert nib.max() <= 15
    # columns restart at -1 per row and increase by code + 1
    for i in range(n_rows):
        seg = cols[mrp[i]:mrp[i + 1]].astype(np.int64)
        if len(seg):
            assert seg[0] == nib[mrp[i]]
            assert np.array_equal(np.diff(seg), nib[mrp[i] + 1:mrp[i + 1]] + 1)


def test_effective_density_bounds():
    g = json.load(open(os.path.join(GOLD, "macko_effd.json")))
    for key in ("0.5", "0.3", "0.1"):
        d = float(key)
        n_cols, n_rows = 12288, 48
        W = gen.pruned_weight(1 - d, n_rows=n_rows, n_cols=n_cols, seed=33)
        mrp, codes, mv = oracle.macko_encode(n_cols, W.row_ptr, W.col_idx, W.vals_f16)
        cols = oracle.macko_decode(mrp, codes)
        # entries excluding the trailing alignment of each row
        last_real = np.array([np.max(np.nonzero(mv[mrp[i]:mrp[i + 1]])[0]) + 1 for i in range(n_rows)])
        bits = 20 * last_real.sum()
        effd = bits / (16.0 * n_rows * n_cols)
        assert g["best"][key] <= effd + 1e-12
        assert effd <= g["worst"][key] + 1e-12
        assert abs(effd - g["expected"][key]) / g["expected"][key] < 0.01, (key, effd)
        assert np.all(cols[mv != 0] < n_cols)


@pytest.mark.parametrize("seed", range(3))
def test_spmv_matches_csr_oracle_and_dense(seed):
    rng = np.random.default_rng(seed)
    n_cols = int(rng.integers(17, 700))
    n_rows = int(rng.integers(1, 60))
    s = float(rng.choice([0.3, 0.5, 0.9]))
    W = gen.pruned_weight(s, n_rows=n_rows, n_cols=n_cols, seed=40 + seed)
    mrp, codes, mv = oracle.macko_encode(n_cols, W.row_ptr, W.col_idx, W.vals_f16)
    alpha, beta = 1.25, (0.0 if seed == 0 else -0.5)
    y_in = rng.uniform(-1, 1, n_rows).astype(np.float32)
    y, sc = oracle.macko_spmv(n_cols, mrp, codes, mv, W.x_f16, alpha, beta, y_in)
    v32 = W.vals_f16.view(np.float16).astype(np.float32)
    x32 = W.x_f16.view(np.float16).astype(np.float32)
    y2, sc2 = oracle.csr_spmv(W.row_ptr, W.col_idx, v32, x32, alpha, beta, y_in)
    assert np.all(np.abs(y - y2) <= 1e-13 * sc2 + 1e-300)
    D = W.dense_f16().view(np.float16).astype(np.float64)
    ref = alpha * D @ x32.astype(np.float64) + (beta * y_in.astype(np.float64) if beta else 0)
    assert np.all(np.abs(y - ref) <= 1e-13 * sc + 1e-300)


def test_trailing_pad_past_last_column_is_skipped():
    n_cols = 10
    rp, ci, v = _one_row([9], n_cols)          # trailing pads decode to columns 10, 11, ...
    mrp, codes, mv = oracle.macko_encode(n_cols, rp, ci, v)
    cols = oracle.macko_decode(mrp, codes)
    assert cols[1] == 10
    x = np.ones(n_cols, np.float16).view(np.uint16)
    y, _ = oracle.macko_spmv(n_cols, mrp, codes, mv, x)
    assert y[0] == 1.0


@pytest.mark.parametrize("cols", [[3, 2], [4, 4], [-1, 2], [1, 64]])
def test_invalid_columns_rejected(cols):
    rp = np.array([0, len(cols)], np.int32)
    assert oracle.macko_size(64, rp, np.asarray(cols, np.int32)) == -1


def test_empty_rows():
    rp = np.array([0, 0, 2, 2], np.int32)
    ci = np.array([0, 5], np.int32)
    v = np.array([1.0, 2.0], np.float16).view(np.uint16)
    mrp, codes, mv = oracle.macko_encode(8, rp, ci, v)
    assert mrp.tolist() == [0, 0, 256, 256]


# ---------------------------------------------------------------- code widths

def _fields(codes, E, b):
    per = 32 // b
    words = np.repeat(codes, per)[:E].astype(np.uint64)
    shifts = np.tile(np.arange(per, dtype=np.uint64) * b, len(codes))[:E]
    return ((words >> shifts) & ((1 << b) - 1)).astype(np.int64)


def _gap_count_b(rp, ci, b):
    span, align = 1 << b, 1024 // b
    n = len(rp) - 1
    out = np.zeros(n, np.int64)
    for i in range(n):
        c = ci[rp[i]:rp[i + 1]].astype(np.int64)
        if len(c) == 0:
            continue
        gaps = np.diff(np.concatenate([[-1], c]))
        raw = len(c) + int(np.sum(-(-gaps // span) - 1))
        out[i] = -(-raw // align) * align
    return out


def test_width_hand_cases():
    g = json.load(open(os.path.join(GOLD, "macko_widths.json")))
    for case in g["cases"]:
        b = case["b"]
        rp, ci, v = _one_row(case["columns"], 1024)
        mrp, codes, mv = oracle.macko_encode(1024, rp, ci, v, bdelta=b)
        k = len(case["codes"])
        assert mrp.tolist() == [0, case["align"]] and oracle.macko_align(b) == case["align"], case
        assert len(codes) == case["align"] * b // 32 == 32, case
        assert int(codes[0]) == case["word0"], case
        f = _fields(codes, int(mrp[-1]), b)
        assert f[:k].tolist() == case["codes"], case
        assert np.all(f[k:] == 0) and np.all(mv[k:] == 0), case
        assert ((mv[:k] == 0) == np.array(case["is_pad"])).all(), case
        assert oracle.macko_decode(mrp, codes, bdelta=b)[:k].tolist() == case["decoded"], case


@pytest.mark.parametrize("b", [1, 2, 4, 8])
@pytest.mark.parametrize("s,n_cols,n_rows", [(0.5, 2048, 40), (0.9, 12288, 12), (0.99, 5000, 10)])
def test_round_trip_and_counts_all_widths(b, s, n_cols, n_rows):
    W = gen.pruned_weight(s, n_rows=n_rows, n_cols=n_cols, seed=23)
    mrp, codes, mv = oracle.macko_encode(n_cols, W.row_ptr, W.col_idx, W.vals_f16, bdelta=b)
    E = int(mrp[-1])
    assert np.all(np.diff(mrp) % (1024 // b) == 0) and len(codes) * 32 == E * b
    assert np.array_equal(np.diff(mrp), _gap_count_b(W.row_ptr, W.col_idx, b))
    cols = oracle.macko_decode(mrp, codes, bdelta=b)
    real = mv != 0
    assert np.array_equal(cols[real], W.col_idx)
    assert np.array_equal(mv[real], W.vals_f16)
    f = _fields(codes, E, b)
    for i in range(n_rows):
        seg = cols[mrp[i]:mrp[i + 1]].astype(np.int64)
        assert seg[0] == f[mrp[i]]
        assert np.array_equal(np.diff(seg), f[mrp[i] + 1:mrp[i + 1]] + 1)
        # a pad is only ever followed by a gap that still needs it: pads sit
        # exactly 2^b after their predecessor
        pad = ~real[mrp[i]:mrp[i + 1]]
        last = np.max(np.nonzero(real[mrp[i]:mrp[i + 1]])[0])
        inner = pad[:last]
        assert np.all(f[mrp[i]:mrp[i] + last][inner] == (1 << b) - 1)


def _effd(mrp, mv, n_rows, n_cols, b, bval=16):
    last_real = np.array([np.max(np.nonzero(mv[mrp[i]:mrp[i + 1]])[0]) + 1 for i in range(n_rows)])
    return (bval + b) * last_real.sum() / (16.0 * n_rows * n_cols)


@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_effective_density_all_widths(b):
    span = 1 << b
    for d in (0.5, 0.3, 0.1):
        n_cols, n_rows = 12288, 48
        W = gen.pruned_weight(1 - d, n_rows=n_rows, n_cols=n_cols, seed=35)
        mrp, codes, mv = oracle.macko_encode(n_cols, W.row_ptr, W.col_idx, W.vals_f16, bdelta=b)
        effd = _effd(mrp, mv, n_rows, n_cols, b)
        z = (1 - d) ** span
        f = (16 + b) / 16
        dr = len(W.col_idx) / (n_rows * n_cols)      # the sampled density
        assert dr * f <= effd + 1e-12
        assert effd <= (dr + (1 - dr) / span) * f + 1e-12
        expected = d * (1 + z / (1 - z)) * f
        assert abs(effd - expected) / expected < 0.015, (b, d, effd, expected)


def test_width_storage_ranking():
    """Smallest encoding per density: b = 2 at d = 0.5 and d = 0.7, b = 4 at
    d = 0.3, b = 8 at d = 0.1 -- the span must grow with sparsity, as the
    section 2.3 formulas say (z = (1-d)^(2^b) shrinks with b)."""
    best = {}
    for d in (0.7, 0.5, 0.3, 0.1):
        W = gen.pruned_weight(1 - d, n_rows=32, n_cols=12288, seed=37)
        sizes = {}
        for b in (1, 2, 4, 8):
            mrp, codes, mv = oracle.macko_encode(12288, W.row_ptr, W.col_idx, W.vals_f16, bdelta=b)
            sizes[b] = _effd(mrp, mv, 32, 12288, b)
        best[d] = min(sizes, key=sizes.get)
    assert best == {0.7: 2, 0.5: 2, 0.3: 4, 0.1: 8}


@pytest.mark.parametrize("b", [1, 2, 8])
def test_spmv_all_widths_matches_csr_oracle(b):
    rng = np.random.default_rng(50 + b)
    n_cols, n_rows = 1500, 30
    W = gen.pruned_weight(0.7, n_rows=n_rows, n_cols=n_cols, seed=60 + b)
    mrp, codes, mv = oracle.macko_encode(n_cols, W.row_ptr, W.col_idx, W.vals_f16, bdelta=b)
    y_in = rng.uniform(-1, 1, n_rows).astype(np.float32)
    y, sc = oracle.macko_spmv(n_cols, mrp, codes, mv, W.x_f16, 0.75, 2.0, y_in, bdelta=b)
    D = W.dense_f16().view(np.float16).astype(np.float64)
    x = W.x_f16.view(np.float16).astype(np.float64)
    ref = 0.75 * D @ x + 2.0 * y_in.astype(np.float64)
    assert np.all(np.abs(y - ref) <= 1e-13 * sc + 1e-300)


def test_trailing_pads_past_last_column_all_widths():
    for b in (1, 2, 8):
        rp, ci, v = _one_row([9], 10)
        mrp, codes, mv = oracle.macko_encode(10, rp, ci, v, bdelta=b)
        cols = oracle.macko_decode(mrp, codes, bdelta=b)
        assert cols[-1] == cols[-2] + 1 and cols[-1] >= 10
        y, _ = oracle.macko_spmv(10, mrp, codes, mv, np.ones(10, np.float16).view(np.uint16), bdelta=b)
        assert y[0] == 1.0


@pytest.mark.parametrize("b", [0, 3, 5, 16])
def test_invalid_width_rejected(b):
    assert oracle.macko_size(64, np.array([0, 1], np.int32), np.array([3], np.int32), b) == -2


# ---------------------------------------------------------- 8-bit value mode

def test_int8_hand_cases():
    g = json.load(open(os.path.join(GOLD, "macko_int8.json")))
    rows = g["rows"]
    mrp = np.concatenate([[0], np.cumsum([len(r["values"]) for r in rows])]).astype(np.int32)
    mv = np.concatenate([np.array(r["values"], np.float16) for r in rows]).view(np.uint16)
    q, sc = oracle.macko_quantize_i8(mrp, mv)
    for i, r in enumerate(rows):
        assert float(sc[i]) == r["scale"], r
        assert q[mrp[i]:mrp[i + 1]].tolist() == r["q"], r


@pytest.mark.parametrize("b,s", [(4, 0.5), (2, 0.7), (8, 0.9)])
def test_int8_quantisation_properties(b, s):
    W = gen.pruned_weight(s, n_rows=40, n_cols=3000, seed=70)
    mrp, codes, mv = oracle.macko_encode(3000, W.row_ptr, W.col_idx, W.vals_f16, bdelta=b)
    q, sc = oracle.macko_quantize_i8(mrp, mv)
    v = mv.view(np.float16).astype(np.float64)
    for i in range(40):
        seg = slice(mrp[i], mrp[i + 1])
        m = np.max(np.abs(v[seg]))
        assert sc[i] == np.float32(np.float32(m) / np.float32(127))
        assert np.max(np.abs(q[seg].astype(np.int64))) == 127
        err = np.abs(float(sc[i]) * q[seg].astype(np.float64) - v[seg])
        assert np.all(err <= 0.5 * float(sc[i]) * (1 + 1e-6))
    assert np.all(q[mv == 0] == 0)


def test_int8_spmv_matches_dequantised_dense():
    rng = np.random.default_rng(71)
    n_cols, n_rows, b = 2000, 25, 2
    W = gen.pruned_weight(0.6, n_rows=n_rows, n_cols=n_cols, seed=72)
    mrp, codes, mv = oracle.macko_encode(n_cols, W.row_ptr, W.col_idx, W.vals_f16, bdelta=b)
    q, sc = oracle.macko_quantize_i8(mrp, mv)
    cols = oracle.macko_decode(mrp, codes, bdelta=b)
    D = np.zeros((n_rows, n_cols))
    for i in range(n_rows):
        for e in range(mrp[i], mrp[i + 1]):
            if cols[e] < n_cols:
                D[i, cols[e]] += float(sc[i]) * float(q[e])
    x = W.x_f16.view(np.float16).astype(np.float64)
    y_in = rng.uniform(-1, 1, n_rows).astype(np.float32)
    y, s = oracle.macko_spmv_i8(n_cols, mrp, codes, q, sc, W.x_f16, -1.5, 0.5, y_in, bdelta=b)
    ref = -1.5 * D @ x + 0.5 * y_in.astype(np.float64)
    assert np.all(np.abs(y - ref) <= 1e-13 * s + 1e-300)
    # and the dequantised matrix is within half a step of the fp16 one
    Df = W.dense_f16().view(np.float16).astype(np.float64)
    assert np.all(np.abs(D - Df) <= 0.5 * sc[:, None].astype(np.float64) * (1 + 1e-6))
