"""Pins of the HYB oracle (ELL part + CSR tail; "Why SpMV needs CUDA
optimisation", sections 2.1 and 5).

* the width rule against hand-derived cases (tests/golden/hyb_width.json);
* the split is lossless: ELL part + tail rebuild the CSR arrays exactly;
* at the longest-row width the tail is empty and the ELL part is the ELL
  conversion; at width 0 the tail is the whole CSR matrix;
* the HYB product visits each row's entries in storage order, so it equals
  the CSR oracle bit for bit (fp64), also with alpha / beta.
"""
import json
import os

import numpy as np
import pytest

import gen
import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _rp(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def test_width_golden():
    cases = json.load(open(os.path.join(HERE, "golden", "hyb_width.json")))["cases"]
    for c in cases:
        rp = _rp(c["lens"])
        w = oracle.hyb_width(rp, c["num"], c["den"])
        assert w == c["width"], c
        assert oracle.hyb_tail_size(rp, w) == (c["tail_rows"], c["tail_nnz"]), c


def _rebuild(n, W, ec, ev, tr, trp, tc, tv):
    """CSR arrays back from a HYB split (ELL slots then the tail, per row)."""
    rows_c, rows_v = [], []
    t = 0
    for i in range(n):
        c = [int(ec[k * n + i]) for k in range(W) if ec[k * n + i] >= 0]
        v = [ev[k * n + i] for k in range(W) if ec[k * n + i] >= 0]
        if t < len(tr) and tr[t] == i:
            c += list(tc[trp[t]:trp[t + 1]])
            v += list(tv[trp[t]:trp[t + 1]])
            t += 1
        rows_c.append(c)
        rows_v.append(v)
    rp = _rp([len(c) for c in rows_c])
    return rp, np.array(sum(rows_c, []), np.int32), np.array(sum(rows_v, []), np.float32)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_split_is_lossless(seed):
    rng = np.random.default_rng(seed)
    n = 200
    lens = rng.integers(0, 12, n)
    lens[::17] = 0
    A = gen.random_csr(n, 64, lens, seed)
    for W in [0, 1, 3, oracle.hyb_width(A.row_ptr), int(lens.max())]:
        parts = oracle.hyb_from_csr(A.row_ptr, A.col_idx, A.vals, W)
        rp, ci, v = _rebuild(n, W, *parts)
        assert np.array_equal(rp, A.row_ptr) and np.array_equal(ci, A.col_idx)
        assert np.array_equal(v.view(np.uint32), A.vals.view(np.uint32))
        ec = parts[0]
        assert np.all((ec == -1) | ((ec >= 0) & (ec < 64)))
        assert np.all(parts[1][ec == -1] == 0.0)


def test_extreme_widths():
    lens = np.arange(512) % 9                     # rows of 0..8 entries
    B = gen.random_csr(512, 512, lens, 8)
    W = int(lens.max())
    ec, ev, tr, trp, tc, tv = oracle.hyb_from_csr(B.row_ptr, B.col_idx, B.vals, W)
    assert len(tr) == 0 and len(tc) == 0 and list(trp) == [0]
    ec2, ev2 = oracle.ell_from_csr(B.row_ptr, B.col_idx, B.vals, W)
    assert np.array_equal(ec, ec2) and np.array_equal(ev.view(np.uint32), ev2.view(np.uint32))
    ec, ev, tr, trp, tc, tv = oracle.hyb_from_csr(B.row_ptr, B.col_idx, B.vals, 0)
    nonempty = np.flatnonzero(lens > 0)
    assert len(ec) == 0 and np.array_equal(tr, nonempty)
    assert np.array_equal(tc, B.col_idx) and np.array_equal(tv.view(np.uint32), B.vals.view(np.uint32))
    assert np.array_equal(trp, _rp(lens[nonempty]))


@pytest.mark.parametrize("W", [0, 2, None])
def test_product_equals_csr(W):
    rng = np.random.default_rng(3)
    n = 300
    lens = rng.integers(0, 20, n)
    A = gen.random_csr(n, 300, lens, 3)
    W = oracle.hyb_width(A.row_ptr) if W is None else W
    parts = oracle.hyb_from_csr(A.row_ptr, A.col_idx, A.vals, W)
    y_in = rng.uniform(-1, 1, n).astype(np.float32)
    for alpha, beta in [(1.0, 0.0), (-0.5, 2.0)]:
        y, s = oracle.hyb_spmv(n, W, *parts, A.x, alpha, beta, y_in)
        yr, sr = oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x, alpha, beta, y_in)
        assert np.array_equal(y, yr) and np.array_equal(s, sr)


def test_varlen_config_is_in_the_hyb_range():
    A = gen.varlen_banded(20000, seed=6)
    lens = np.diff(A.row_ptr).astype(np.int64)
    assert oracle.format_choice(len(lens), int(lens.sum()), int((lens ** 2).sum())) == 1
    assert np.all(np.abs(A.col_idx - np.repeat(np.arange(20000), lens)) <= 1000)
