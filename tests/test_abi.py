"""CPU-side checks of the C-ABI library (no GPU kernel is launched here).

* the library loads and exports every entry point declared in include/spmv.h;
* the host-only format rule matches the oracle's rule on the golden CV cases
  and on random statistics;
* the host MACKO encoder is bit-exact with the oracle encoder (mrow_ptr,
  codes, values) and rejects unsorted / duplicate / out-of-range columns;
* argument validation that runs before any HIP call returns the documented
  status.
"""
import json
import os
import re

import numpy as np
import pytest

import gen
import oracle
import sparse_matrix_vector_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = os.path.join(ROOT, "tests", "golden")


def _declared():
    text = open(os.path.join(ROOT, "include", "spmv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:spmv_status|const char \*)\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 19
    L = S.lib()
    for n in names:
        assert hasattr(L, n), n
    # and the binding exposes the same names
    for n in names:
        if n != "spmv_last_error":
            assert callable(getattr(S, n)), n


def test_format_recommend_matches_oracle():
    g = json.load(open(os.path.join(GOLD, "cv_rule.json")))
    for case in g["cases"]:
        lens = np.asarray(case["row_lengths"], dtype=np.int64)
        n, s1, s2 = len(lens), int(lens.sum()), int((lens * lens).sum())
        assert S.spmv_format_recommend(n, s1, s2) == case["choice"]
    rng = np.random.default_rng(0)
    for _ in range(3000):
        n = int(rng.integers(0, 40))
        lens = rng.integers(0, 60, n)
        s1, s2 = int(lens.sum()), int((lens * lens).sum())
        assert S.spmv_format_recommend(n, s1, s2) == oracle.format_choice(n, s1, s2)
    big = 2**31 - 1
    assert S.spmv_format_recommend(big, big * 8, big * 64) == oracle.format_choice(big, big * 8, big * 64)


def test_plan_size_validation():
    assert S.spmv_csr_plan_size(1000, 5000) > 0
    with pytest.raises(S.SpmvError) as e:
        S.spmv_csr_plan_size(10, 10, (32, 16, 8192))
    assert e.value.status == 1
    with pytest.raises(S.SpmvError) as e:
        S.spmv_csr_plan_size(10, 10, (300, 512, 8192))
    assert e.value.status == 5
    with pytest.raises(S.SpmvError):
        S.spmv_csr_plan_size(-1, 10)


@pytest.mark.parametrize("s,n_rows,n_cols", [(0.5, 64, 2048), (0.9, 30, 12288), (0.97, 16, 5000),
                                             (0.0, 4, 300), (0.3, 33, 999)])
def test_host_encoder_bit_exact_with_oracle(s, n_rows, n_cols):
    W = gen.pruned_weight(s, n_rows=n_rows, n_cols=n_cols, seed=77)
    mrp, codes, mv = S.macko_encode(n_rows, n_cols, W.row_ptr, W.col_idx, W.vals_f16)
    omrp, ocodes, omv = oracle.macko_encode(n_cols, W.row_ptr, W.col_idx, W.vals_f16)
    assert np.array_equal(mrp, omrp)
    assert np.array_equal(codes, ocodes)
    assert np.array_equal(mv, omv)
    assert S.macko_encode_size(n_rows, n_cols, W.row_ptr, W.col_idx) == oracle.macko_size(n_cols, W.row_ptr, W.col_idx)


@pytest.mark.parametrize("b", [1, 2, 8])
@pytest.mark.parametrize("s,n_rows,n_cols", [(0.5, 40, 2048), (0.9, 20, 12288), (0.0, 4, 300)])
def test_host_encoder_all_widths_bit_exact_with_oracle(b, s, n_rows, n_cols):
    W = gen.pruned_weight(s, n_rows=n_rows, n_cols=n_cols, seed=78)
    got = S.macko_encode(n_rows, n_cols, W.row_ptr, W.col_idx, W.vals_f16, bdelta=b)
    ref = oracle.macko_encode(n_cols, W.row_ptr, W.col_idx, W.vals_f16, bdelta=b)
    assert all(np.array_equal(x, y) for x, y in zip(got, ref))
    assert S.macko_encode_size(n_rows, n_cols, W.row_ptr, W.col_idx, b) == len(ref[2])


def test_host_encoder_width_golden_cases():
    g = json.load(open(os.path.join(GOLD, "macko_widths.json")))
    for case in g["cases"]:
        cols = np.asarray(case["columns"], np.int32)
        rp = np.array([0, len(cols)], np.int32)
        v = np.arange(1, len(cols) + 1).astype(np.float16).view(np.uint16)
        mrp, codes, mv = S.macko_encode(1, 1024, rp, cols, v, bdelta=case["b"])
        assert mrp.tolist() == [0, case["align"]] and int(codes[0]) == case["word0"], case


@pytest.mark.parametrize("b", [0, 3, 16])
def test_host_encoder_rejects_width(b):
    with pytest.raises(S.SpmvError) as e:
        S.macko_encode_size(1, 64, np.array([0, 1], np.int32), np.array([3], np.int32), b)
    assert e.value.status == 1


def test_host_quantizer_bit_exact_with_oracle():
    g = json.load(open(os.path.join(GOLD, "macko_int8.json")))
    rows = g["rows"]
    mrp = np.concatenate([[0], np.cumsum([len(r["values"]) for r in rows])]).astype(np.int32)
    mv = np.concatenate([np.array(r["values"], np.float16) for r in rows]).view(np.uint16)
    q, sc = S.macko_quantize_i8(len(rows), mrp, mv)
    for i, r in enumerate(rows):
        assert float(sc[i]) == r["scale"] and q[mrp[i]:mrp[i + 1]].tolist() == r["q"], r
    for s_, b in [(0.5, 4), (0.7, 2), (0.9, 8)]:
        W = gen.pruned_weight(s_, n_rows=50, n_cols=4000, seed=79)
        mrp, codes, mv = S.macko_encode(50, 4000, W.row_ptr, W.col_idx, W.vals_f16, bdelta=b)
        q, sc = S.macko_quantize_i8(50, mrp, mv)
        oq, osc = oracle.macko_quantize_i8(mrp, mv)
        assert np.array_equal(q, oq) and np.array_equal(sc.view(np.uint32), osc.view(np.uint32))


def test_host_encoder_golden_and_large_gaps():
    g = json.load(open(os.path.join(GOLD, "macko_examples.json")))
    for case in [g["page_example"]] + g["cases"]:
        cols = np.asarray(case["columns"], np.int32)
        rp = np.array([0, len(cols)], np.int32)
        v = np.arange(1, len(cols) + 1).astype(np.float16).view(np.uint16)
        mrp, codes, mv = S.macko_encode(1, 64, rp, cols, v)
        k = len(case["codes"])
        nib = [(int(codes[e // 8]) >> (4 * (e % 8))) & 15 for e in range(k)]
        assert nib == case["codes"]
    # a single row spanning 200,000 columns with 3 entries
    cols = np.array([0, 99_999, 199_999], np.int32)
    rp = np.array([0, 3], np.int32)
    v = np.ones(3, np.float16).view(np.uint16)
    a = S.macko_encode(1, 200_000, rp, cols, v)
    b = oracle.macko_encode(200_000, rp, cols, v)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("cols,status", [([3, 2], 3), ([4, 4], 3), ([-1, 2], 2), ([1, 64], 2)])
def test_host_encoder_rejects(cols, status):
    rp = np.array([0, len(cols)], np.int32)
    v = np.ones(len(cols), np.float16).view(np.uint16)
    with pytest.raises(S.SpmvError) as e:
        S.macko_encode(1, 64, rp, np.asarray(cols, np.int32), v)
    assert e.value.status == status
    with pytest.raises(S.SpmvError) as e:
        S.macko_encode_size(1, 64, rp, np.asarray(cols, np.int32))
    assert e.value.status == status


def test_host_validation_before_any_gpu_call():
    L = S.lib()
    import ctypes
    h = ctypes.c_void_p()
    # negative sizes / NULL pointers are rejected on the host
    assert L.spmv_csr_create(ctypes.byref(h), -1, 4, 0, None, None, None, 0, None, None, 0, None) == 1
    assert L.spmv_csr_create(None, 1, 4, 0, None, None, None, 0, None, None, 0, None) == 1
    assert L.spmv_csr_create(ctypes.byref(h), 4, 4, 4, None, None, None, 0, None, None, 0, None) == 1
    assert L.spmv_csr_create(ctypes.byref(h), 4, 4, 4, 8, 8, 8, 9, None, None, 0, None) == 1
    assert b"variant" in L.spmv_last_error()
    assert L.spmv_csr_apply(None, 1.0, None, 0.0, None, None) == 1
    assert L.spmv_ell_apply(-1, 1, 1, None, None, 1.0, None, 0.0, None, None) == 1
    assert L.spmv_ell_apply(1 << 20, 1, 1 << 12, None, None, 1.0, None, 0.0, None, None) == 4
    assert L.macko_spmv(4, 4, 4, None, None, None, 1.0, None, 0.0, None, None) == 1
    assert L.macko_spmv(4, 4, 4, 16, 16, 18, 1.0, 16, 0.0, 16, None) == 5      # misaligned values
    assert L.macko_spmv(4, 4, 8, 16, 20, 16, 1.0, 16, 0.0, 16, None) == 5      # codes not 8-byte aligned
    assert L.macko_spmv(4, 4, 3, 16, 16, 16, 1.0, 16, 0.0, 16, None) == 1      # code width
    assert L.macko_spmv_i8(4, 4, 2, 16, 16, 20, 16, 1.0, 16, 0.0, 16, None) == 5   # q not 8-byte aligned
    assert L.macko_spmv_i8(4, 4, 2, 16, 16, 16, None, 1.0, 16, 0.0, 16, None) == 1  # no scales
    assert L.macko_decode_columns(4, 16, 16, 16, 16, None) == 1
    assert L.dense_gemv_f16(-1, 4, None, None, 1.0, 0.0, None, None) == 1
    assert L.fem_matvec_apply(4, 10, 16, 16, 9, 16, 1.0, 16, 0.0, 16, None) == 1   # penalty > 8
    assert L.fem_matvec_apply(4, 10, 20, 16, 3, 16, 1.0, 16, 0.0, 16, None) == 5   # edof misaligned
    assert L.fem_matvec_threestage(4, 10, 16, 16, 3, 16, 1.0, 16, 0.0, 16, None, 0, None) == 1
    h = ctypes.c_void_p()
    assert L.spgemm_create(None, 1, 1, 1, 0, 16, None, None, 0, 16, None, None, 16, 1 << 20, None) == 1
    assert L.spgemm_create(ctypes.byref(h), -1, 1, 1, 0, 16, None, None, 0, 16, None, None, 16, 1 << 20, None) == 1
    assert L.spgemm_create(ctypes.byref(h), 2, 2, 2, 3, 16, None, 16, 0, 16, None, None, 16, 1 << 20, None) == 1
    assert L.spgemm_info(None, None, None, None) == 1
    assert L.spgemm_compute(None, None, None, None, None) == 1
    assert L.spgemm_workspace_size(1, 1, 1, 0, None, None, 0, 16, None, ctypes.byref(ctypes.c_size_t()), 256, 512,
                                   None) == 1
    assert L.spgemm_destroy(None) == 0
    # n_rows == 0 applies are no-ops that succeed without touching the GPU
    assert L.macko_spmv(0, 4, 4, None, None, None, 1.0, None, 0.0, None, None) == 0
    assert L.macko_spmv_i8(0, 4, 1, None, None, None, None, 1.0, None, 0.0, None, None) == 0
    assert L.spmv_ell_apply(0, 4, 2, None, None, 1.0, None, 0.0, None, None) == 0
    assert L.dense_gemv_f16(0, 4, None, None, 1.0, 0.0, None, None) == 0


def test_scratch_size_and_validation():
    """The synchronous calls take their device scratch from the caller: its
    size follows the documented formula and a missing, misaligned or short
    buffer is rejected on the host before any GPU call."""
    import ctypes
    L = S.lib()
    for n, want in [(0, 512), (1, 512), (256, 512), (257, 512), (8192, 512), (8193, 768),
                    (1_000_000, 256 + 31488), (2**31 - 1, 256 + 67108864)]:
        assert S.spmv_scratch_size(n) == want, n
    assert L.spmv_scratch_size(-1, ctypes.byref(ctypes.c_size_t())) == 1
    m, s1, s2 = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
    args = (ctypes.byref(m), ctypes.byref(s1), ctypes.byref(s2))
    assert L.spmv_csr_row_stats(10, 4096, *args, None, 512, None) == 1          # no scratch
    assert b"scratch" in L.spmv_last_error()
    assert L.spmv_csr_row_stats(10, 4096, *args, 4096 + 64, 512, None) == 1     # misaligned
    assert L.spmv_csr_row_stats(10, 4096, *args, 4096, 256, None) == 1          # too small
    r, t = ctypes.c_int32(), ctypes.c_int64()
    assert L.spmv_hyb_tail_size(10, 4096, -1, ctypes.byref(r), ctypes.byref(t), 4096, 512, None) == 1
    assert L.spmv_hyb_tail_size(10, 4096, 2, ctypes.byref(r), ctypes.byref(t), None, 512, None) == 1
    assert L.spmv_hyb_width(10, 4096, 7, 10, ctypes.byref(m), ctypes.byref(r), ctypes.byref(t), 4096, 64,
                            None) == 1
    assert L.spmv_ell_from_csr(10, 10, 0, 4096, None, None, 2, 4096, 4096, None, 512, None) == 1
    assert L.spmv_hyb_from_csr(10, 10, 0, 4096, None, None, 2, 4096, 4096, 0, 0, None, 4096, None, None,
                               4096, 8, None) == 1
    p = S._lib.AutoPlan()
    assert L.spmv_auto_plan(10, 10, 0, 4096, ctypes.byref(p), 4096, 100, None) == 1
    # zero rows: valid scratch, nothing to do, no GPU call
    assert L.spmv_csr_row_stats(0, 4096, *args, 4096, 512, None) == 0
    assert (m.value, s1.value, s2.value) == (0, 0, 0)
    assert L.spmv_hyb_tail_size(0, 4096, 3, ctypes.byref(r), ctypes.byref(t), 4096, 512, None) == 0
    # SCALAR / VECTOR handles need a workspace of 256 bytes for the validation flags
    h = ctypes.c_void_p()
    assert L.spmv_csr_create(ctypes.byref(h), 4, 4, 4, 4096, 4096, 4096, 1, None, None, 0, None) == 1
    assert L.spmv_csr_create(ctypes.byref(h), 4, 4, 4, 4096, 4096, 4096, 1, None, 4096, 128, None) == 1
