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
* unsorted / duplicate / out-of-range columns are rejected.
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
