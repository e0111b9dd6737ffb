"""Pins of the row-grouping planner, the row statistics and the CV format rule.

* the hand example built from the page-1 grouping table (tests/golden);
* invariants on random and structured inputs: perm is a permutation, groups
  are contiguous and in order, rows ascend inside a group, counts match a
  NumPy histogram;
* the CV rule on constructed edge cases landing exactly on 0.3 and 0.7, and
  against a floating-point CV away from the edges.
"""
import json
import os

import numpy as np
import pytest

import gen
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rp(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def test_grouping_hand_example():
    g = json.load(open(os.path.join(GOLD, "row_grouping.json")))
    rp = _rp(g["row_lengths"])
    off, perm = oracle.bins(rp, g["thresholds"])
    assert off.tolist() == g["bin_offsets"]
    assert perm.tolist() == g["perm"]
    assert [oracle.row_bin(l, g["thresholds"]) for l in g["row_lengths"]] == g["bins"]


def _check_invariants(rp, thr):
    off, perm = oracle.bins(rp, thr)
    n = len(rp) - 1
    lens = np.diff(rp)
    assert np.array_equal(np.sort(perm), np.arange(n))
    edges = np.array([0] + list(thr) + [np.iinfo(np.int64).max])
    b = np.searchsorted(edges, lens, side="right") - 1      # bin via NumPy
    counts = np.bincount(b, minlength=4)
    assert off.tolist() == [0] + np.cumsum(counts).tolist()
    for g in range(4):
        seg = perm[off[g]:off[g + 1]]
        assert np.all(b[seg] == g)
        assert np.all(np.diff(seg) > 0)


@pytest.mark.parametrize("seed", range(4))
def test_grouping_invariants_random(seed):
    rng = np.random.default_rng(seed)
    lens = rng.choice([0, 1, 5, 31, 32, 33, 511, 512, 600, 8191, 8192, 9000], size=300)
    _check_invariants(_rp(lens), (32, 512, 8192))


def test_grouping_powerlaw_and_custom_thresholds():
    A = gen.powerlaw_csr(n=50000, seed=11)
    _check_invariants(A.row_ptr, (32, 512, 8192))
    _check_invariants(A.row_ptr, (4, 8, 16))
    _check_invariants(np.zeros(1, np.int32), (32, 512, 8192))


def test_cv_rule_golden():
    g = json.load(open(os.path.join(GOLD, "cv_rule.json")))
    for case in g["cases"]:
        lens = np.asarray(case["row_lengths"], dtype=np.int64)
        n, s1, s2 = len(lens), int(lens.sum()), int((lens * lens).sum())
        assert oracle.format_choice(n, s1, s2) == case["choice"], case
        if case["cv"] is not None and len(lens):
            cv = lens.std() / lens.mean()
            assert abs(cv - case["cv"]) < 1e-4


def test_cv_rule_against_float_cv():
    rng = np.random.default_rng(5)
    for _ in range(2000):
        n = int(rng.integers(1, 30))
        lens = rng.integers(0, 50, n)
        if lens.sum() == 0:
            continue
        cv = lens.std() / lens.mean()
        if min(abs(cv - 0.3), abs(cv - 0.7)) < 1e-9:
            continue
        want = 0 if cv < 0.3 else (1 if cv <= 0.7 else 2)
        assert oracle.format_choice(n, int(lens.sum()), int((lens ** 2).sum())) == want


def test_cv_of_configs():
    L = gen.laplacian_2d(1000, with_x=False)
    m, s1, s2 = oracle.row_stats(L.row_ptr)
    assert m == 5 and s1 == 4996000
    cv = np.sqrt(L.n_rows * s2 - s1 * s1) / s1
    assert abs(cv - 0.012647) < 1e-5
    assert oracle.format_choice(L.n_rows, s1, s2) == 0
    T = gen.tiny_csr()
    assert oracle.format_choice(T.n_rows, *oracle.row_stats(T.row_ptr)[1:]) == 0
