"""CPU oracle for the SpMV library -- TEST INFRASTRUCTURE ONLY.

A thin ctypes wrapper over ``oracle.c`` (plain serial C, fp64 accumulation).
Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library under
``sparse_matrix_vector_amd/`` never imports it and shares no code with it.

All value-producing functions return ``(y, scale)`` in float64, where
``scale[i] = |alpha| * sum_k |a_ik x_k| + |beta y_in_i|`` is the magnitude
against which a tolerance is applied: ``|y_gpu - y| <= tau * scale``.

Every function here has at least one pin in ``tests/test_oracle_*.py`` that
does not go through this code (closed forms, textbook identities, NumPy
brute force, the pages' worked examples); see each test's docstring.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
u32p = np.ctypeslib.ndpointer(dtype=np.uint32, flags="C_CONTIGUOUS")
u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
i8p = np.ctypeslib.ndpointer(dtype=np.int8, flags="C_CONTIGUOUS")
f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
vp = ctypes.c_void_p


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` with gcc (-O2, no fast-math) into ``liboracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        c_int, c_double, c_i64 = ctypes.c_int, ctypes.c_double, ctypes.c_int64
        sig = {
            "oracle_half_to_double": (c_double, [ctypes.c_uint16]),
            "oracle_csr_spmv": (None, [c_int, i32p, i32p, f32p, f32p, c_double, c_double, vp, f64p, f64p]),
            "oracle_csr_spmv_f64": (None, [c_int, i32p, i32p, f64p, f32p, c_double, c_double, vp, f64p, f64p]),
            "oracle_csr_spmv_f64v": (None, [c_int, i32p, i32p, f64p, f64p, f64p]),
            "oracle_row_stats": (None, [c_int, i32p, ctypes.POINTER(ctypes.c_int32),
                                        ctypes.POINTER(c_i64), ctypes.POINTER(c_i64)]),
            "oracle_row_bin": (c_int, [ctypes.c_int32, i32p]),
            "oracle_bins": (None, [c_int, i32p, i32p, i32p, i32p]),
            "oracle_format_choice": (c_int, [c_i64, c_i64, c_i64]),
            "oracle_ell_from_csr": (c_int, [c_int, i32p, i32p, f32p, c_int, i32p, f32p]),
            "oracle_ell_spmv": (None, [c_int, c_int, i32p, f32p, f32p, c_double, c_double, vp, f64p, f64p]),
            "oracle_hyb_width": (c_int, [c_int, i32p, c_int, c_int]),
            "oracle_hyb_tail_size": (None, [c_int, i32p, c_int, ctypes.POINTER(c_int), ctypes.POINTER(ctypes.c_longlong)]),
            "oracle_hyb_from_csr": (None, [c_int, i32p, i32p, f32p, c_int, i32p, f32p, i32p, i32p, i32p, f32p]),
            "oracle_hyb_spmv": (None, [c_int, c_int, i32p, f32p, c_int, i32p, i32p, i32p, f32p, f32p,
                                       c_double, c_double, vp, f64p, f64p]),
            "oracle_macko_size": (c_i64, [c_int, c_int, c_int, i32p, i32p]),
            "oracle_macko_encode": (c_int, [c_int, c_int, c_int, i32p, i32p, u16p, i32p, u32p, u16p]),
            "oracle_macko_decode": (None, [c_int, c_int, i32p, u32p, i32p]),
            "oracle_macko_spmv": (None, [c_int, c_int, c_int, i32p, u32p, u16p, u16p, c_double, c_double, vp,
                                         f64p, f64p]),
            "oracle_macko_quantize_i8": (None, [c_int, i32p, u16p, i8p, f32p]),
            "oracle_spgemm_ip": (None, [c_int, i32p, i32p, i32p, i64p]),
            "oracle_spgemm_rows": (c_i64, [c_int, c_int, i32p, i32p, i32p, i32p, i64p]),
            "oracle_spgemm_fill": (c_int, [c_int, c_int, i32p, i32p, f32p, i32p, i32p, f32p, i64p, i32p, f64p,
                                           f64p]),
            "oracle_macko_spmv_i8": (None, [c_int, c_int, c_int, i32p, u32p, i8p, f32p, u16p, c_double, c_double,
                                            vp, f64p, f64p]),
            "oracle_gemv_f16": (None, [c_int, c_int, u16p, u16p, c_double, c_double, vp, f64p, f64p]),
            "oracle_fe_matvec": (None, [c_int, c_int, i32p, f32p, c_int, f32p, f32p, c_double, c_double, vp, f64p, f64p]),
            "oracle_fe_assemble": (c_i64, [c_int, c_int, i32p, f32p, c_int, f32p, vp, vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def _yin(y_in, n, beta):
    if beta == 0.0:
        return None, None
    y = _c(y_in, np.float32)
    assert y.shape == (n,)
    return y, y.ctypes.data


# --------------------------------------------------------------------------
def half_to_double(h: int) -> float:
    return lib().oracle_half_to_double(int(h))


def csr_spmv(row_ptr, col_idx, vals, x, alpha=1.0, beta=0.0, y_in=None):
    """fp64 reference of y = alpha*A*x + beta*y for fp32 CSR."""
    rp = _c(row_ptr, np.int32)
    n = len(rp) - 1
    keep, yp = _yin(y_in, n, beta)
    y = np.empty(n, np.float64)
    s = np.empty(n, np.float64)
    lib().oracle_csr_spmv(n, rp, _c(col_idx, np.int32), _c(vals, np.float32), _c(x, np.float32),
                          float(alpha), float(beta), yp, y, s)
    return y, s


def csr_spmv_f64(row_ptr, col_idx, vals64, x, alpha=1.0, beta=0.0, y_in=None):
    rp = _c(row_ptr, np.int32)
    n = len(rp) - 1
    keep, yp = _yin(y_in, n, beta)
    y = np.empty(n, np.float64)
    s = np.empty(n, np.float64)
    lib().oracle_csr_spmv_f64(n, rp, _c(col_idx, np.int32), _c(vals64, np.float64), _c(x, np.float32),
                              float(alpha), float(beta), yp, y, s)
    return y, s


def csr_spmv_f64v(row_ptr, col_idx, vals64, x64):
    """y = A x with fp64 values and an fp64 vector (rows summed in storage order)."""
    rp = _c(row_ptr, np.int32)
    y = np.empty(len(rp) - 1, np.float64)
    lib().oracle_csr_spmv_f64v(len(rp) - 1, rp, _c(col_idx, np.int32), _c(vals64, np.float64),
                               _c(x64, np.float64), y)
    return y


def row_stats(row_ptr):
    rp = _c(row_ptr, np.int32)
    m = ctypes.c_int32()
    s = ctypes.c_int64()
    q = ctypes.c_int64()
    lib().oracle_row_stats(len(rp) - 1, rp, ctypes.byref(m), ctypes.byref(s), ctypes.byref(q))
    return m.value, s.value, q.value


DEFAULT_THRESHOLDS = (32, 512, 8192)


def row_bin(length, thresholds=DEFAULT_THRESHOLDS):
    return lib().oracle_row_bin(int(length), _c(thresholds, np.int32))


def bins(row_ptr, thresholds=DEFAULT_THRESHOLDS):
    """(bin_offsets int32[5], perm int32[n]) of the row-grouping planner."""
    rp = _c(row_ptr, np.int32)
    n = len(rp) - 1
    off = np.empty(5, np.int32)
    perm = np.empty(n, np.int32)
    lib().oracle_bins(n, rp, _c(thresholds, np.int32), off, perm)
    return off, perm


FORMAT_NAMES = {0: "ELL", 1: "HYB", 2: "CSR"}


def format_choice(n, s1, s2) -> int:
    return lib().oracle_format_choice(int(n), int(s1), int(s2))


def ell_from_csr(row_ptr, col_idx, vals, width):
    rp = _c(row_ptr, np.int32)
    n = len(rp) - 1
    ec = np.empty(n * width, np.int32)
    ev = np.empty(n * width, np.float32)
    rc = lib().oracle_ell_from_csr(n, rp, _c(col_idx, np.int32), _c(vals, np.float32), int(width), ec, ev)
    if rc != 0:
        raise ValueError("row longer than the ELL width")
    return ec, ev


def ell_spmv(n_rows, width, ell_col, ell_val, x, alpha=1.0, beta=0.0, y_in=None):
    keep, yp = _yin(y_in, n_rows, beta)
    y = np.empty(n_rows, np.float64)
    s = np.empty(n_rows, np.float64)
    lib().oracle_ell_spmv(int(n_rows), int(width), _c(ell_col, np.int32), _c(ell_val, np.float32),
                          _c(x, np.float32), float(alpha), float(beta), yp, y, s)
    return y, s


HYB_FRACTION = (7, 10)   # ELL share of the nonzeros in the HYB split


def hyb_width(row_ptr, num=HYB_FRACTION[0], den=HYB_FRACTION[1]) -> int:
    """Smallest W with den * sum_i min(len_i, W) >= num * nnz."""
    rp = _c(row_ptr, np.int32)
    return int(lib().oracle_hyb_width(len(rp) - 1, rp, int(num), int(den)))


def hyb_tail_size(row_ptr, width):
    """(rows with len > width, entries past width)."""
    rp = _c(row_ptr, np.int32)
    r, t = ctypes.c_int(), ctypes.c_longlong()
    lib().oracle_hyb_tail_size(len(rp) - 1, rp, int(width), ctypes.byref(r), ctypes.byref(t))
    return r.value, t.value


def hyb_from_csr(row_ptr, col_idx, vals, width):
    """(ell_col, ell_val, tail_rows, tail_rp, tail_col, tail_val)."""
    rp = _c(row_ptr, np.int32)
    n = len(rp) - 1
    nt, tn = hyb_tail_size(rp, width)
    ec = np.empty(max(width * n, 1), np.int32)
    ev = np.empty(max(width * n, 1), np.float32)
    tr = np.empty(max(nt, 1), np.int32)
    trp = np.empty(nt + 1, np.int32)
    tc = np.empty(max(tn, 1), np.int32)
    tv = np.empty(max(tn, 1), np.float32)
    lib().oracle_hyb_from_csr(n, rp, _c(col_idx, np.int32), _c(vals, np.float32), int(width), ec, ev, tr, trp, tc, tv)
    return ec[:width * n], ev[:width * n], tr[:nt], trp, tc[:tn], tv[:tn]


def hyb_spmv(n_rows, width, ell_col, ell_val, tail_rows, tail_rp, tail_col, tail_val, x,
             alpha=1.0, beta=0.0, y_in=None):
    keep, yp = _yin(y_in, n_rows, beta)
    y = np.empty(n_rows, np.float64)
    s = np.empty(n_rows, np.float64)
    z32 = np.zeros(1, np.int32)
    zf = np.zeros(1, np.float32)
    ec = _c(ell_col, np.int32) if width * n_rows else z32
    ev = _c(ell_val, np.float32) if width * n_rows else zf
    tr = _c(tail_rows, np.int32) if len(tail_rows) else z32
    tc = _c(tail_col, np.int32) if len(tail_col) else z32
    tv = _c(tail_val, np.float32) if len(tail_val) else zf
    lib().oracle_hyb_spmv(int(n_rows), int(width), ec, ev, len(tail_rows), tr, _c(tail_rp, np.int32), tc, tv,
                          _c(x, np.float32), float(alpha), float(beta), yp, y, s)
    return y, s


MACKO_BITS = (1, 2, 4, 8)


def macko_align(bdelta=4) -> int:
    """Row alignment in entries: 1024 / b (one 128-byte block of codes)."""
    return 1024 // bdelta


def macko_size(n_cols, row_ptr, col_idx, bdelta=4) -> int:
    rp = _c(row_ptr, np.int32)
    return int(lib().oracle_macko_size(len(rp) - 1, int(n_cols), int(bdelta), rp, _c(col_idx, np.int32)))


def macko_encode(n_cols, row_ptr, col_idx, vals_f16, bdelta=4):
    """(mrow_ptr int32[R+1], codes uint32[E*b/32], mvals uint16[E])."""
    rp = _c(row_ptr, np.int32)
    n = len(rp) - 1
    ci = _c(col_idx, np.int32)
    E = macko_size(n_cols, rp, ci, bdelta)
    if E == -2:
        raise ValueError("code width must be 1, 2, 4 or 8")
    if E < 0:
        raise ValueError("columns must be strictly increasing per row and in range")
    mrp = np.empty(n + 1, np.int32)
    codes = np.zeros(E * bdelta // 32, np.uint32)
    mv = np.zeros(E, np.uint16)
    rc = lib().oracle_macko_encode(n, int(n_cols), int(bdelta), rp, ci, _c(vals_f16, np.uint16), mrp, codes, mv)
    if rc != 0:
        raise ValueError("MACKO encode failed")
    return mrp, codes, mv


def macko_decode(mrow_ptr, codes, bdelta=4):
    mrp = _c(mrow_ptr, np.int32)
    cols = np.empty(int(mrp[-1]), np.int32)
    lib().oracle_macko_decode(len(mrp) - 1, int(bdelta), mrp, _c(codes, np.uint32), cols)
    return cols


def macko_spmv(n_cols, mrow_ptr, codes, mvals, x_f16, alpha=1.0, beta=0.0, y_in=None, bdelta=4):
    mrp = _c(mrow_ptr, np.int32)
    n = len(mrp) - 1
    keep, yp = _yin(y_in, n, beta)
    y = np.empty(n, np.float64)
    s = np.empty(n, np.float64)
    lib().oracle_macko_spmv(n, int(n_cols), int(bdelta), mrp, _c(codes, np.uint32), _c(mvals, np.uint16),
                            _c(x_f16, np.uint16), float(alpha), float(beta), yp, y, s)
    return y, s


def macko_quantize_i8(mrow_ptr, mvals):
    """(q int8[E], row_scale float32[R]) of the 8-bit value mode."""
    mrp = _c(mrow_ptr, np.int32)
    n = len(mrp) - 1
    q = np.empty(int(mrp[-1]), np.int8)
    sc = np.empty(n, np.float32)
    lib().oracle_macko_quantize_i8(n, mrp, _c(mvals, np.uint16), q, sc)
    return q, sc


def macko_spmv_i8(n_cols, mrow_ptr, codes, q, row_scale, x_f16, alpha=1.0, beta=0.0, y_in=None, bdelta=4):
    mrp = _c(mrow_ptr, np.int32)
    n = len(mrp) - 1
    keep, yp = _yin(y_in, n, beta)
    y = np.empty(n, np.float64)
    s = np.empty(n, np.float64)
    lib().oracle_macko_spmv_i8(n, int(n_cols), int(bdelta), mrp, _c(codes, np.uint32), _c(q, np.int8),
                               _c(row_scale, np.float32), _c(x_f16, np.uint16), float(alpha), float(beta), yp,
                               y, s)
    return y, s


def gemv_f16(W_f16, x_f16, alpha=1.0, beta=0.0, y_in=None):
    W = _c(W_f16, np.uint16)
    m, n = W.shape
    keep, yp = _yin(y_in, m, beta)
    y = np.empty(m, np.float64)
    s = np.empty(m, np.float64)
    lib().oracle_gemv_f16(m, n, W.reshape(-1), _c(x_f16, np.uint16), float(alpha), float(beta), yp, y, s)
    return y, s


def fe_matvec(edof, rho, Ke, x, n_dof, penalty=3, alpha=1.0, beta=0.0, y_in=None):
    ed = _c(edof, np.int32).reshape(-1)
    n_elem = len(ed) // 24
    keep, yp = _yin(y_in, n_dof, beta)
    y = np.empty(n_dof, np.float64)
    s = np.empty(n_dof, np.float64)
    lib().oracle_fe_matvec(n_elem, int(n_dof), ed, _c(rho, np.float32), int(penalty),
                           _c(Ke, np.float32).reshape(-1), _c(x, np.float32),
                           float(alpha), float(beta), yp, y, s)
    return y, s


def fe_assemble(edof, rho, Ke, n_dof, penalty=3):
    """Assembled fp64 CSR (row_ptr, col_idx, vals) of the FE operator."""
    ed = _c(edof, np.int32).reshape(-1)
    n_elem = len(ed) // 24
    r = _c(rho, np.float32)
    K = _c(Ke, np.float32).reshape(-1)
    nnz = lib().oracle_fe_assemble(n_elem, int(n_dof), ed, r, int(penalty), K, None, None, None)
    if nnz < 0:
        raise MemoryError("oracle_fe_assemble")
    rp = np.empty(n_dof + 1, np.int32)
    ci = np.empty(nnz, np.int32)
    v = np.empty(nnz, np.float64)
    lib().oracle_fe_assemble(n_elem, int(n_dof), ed, r, int(penalty), K,
                             rp.ctypes.data, ci.ctypes.data, v.ctypes.data)
    return rp, ci, v


def spgemm_ip(rp_a, ci_a, rp_b):
    """Intermediate products per row of A*B (int64[m])."""
    rpa = _c(rp_a, np.int32)
    ip = np.empty(len(rpa) - 1, np.int64)
    lib().oracle_spgemm_ip(len(rpa) - 1, rpa, _c(ci_a, np.int32), _c(rp_b, np.int32), ip)
    return ip


def spgemm(n_cols_b, rp_a, ci_a, v_a, rp_b, ci_b, v_b):
    """C = A*B: (rp_c int64[m+1], ci_c int32[nnz], v_c float64[nnz], scale float64[nnz]),
    columns increasing in each row."""
    rpa, cia, rpb, cib = (_c(x, np.int32) for x in (rp_a, ci_a, rp_b, ci_b))
    m = len(rpa) - 1
    rpc = np.empty(m + 1, np.int64)
    nnz = lib().oracle_spgemm_rows(m, int(n_cols_b), rpa, cia, rpb, cib, rpc)
    if nnz < 0:
        raise MemoryError("oracle_spgemm_rows")
    cic = np.empty(max(nnz, 1), np.int32)
    vc = np.empty(max(nnz, 1), np.float64)
    sc = np.empty(max(nnz, 1), np.float64)
    if lib().oracle_spgemm_fill(m, int(n_cols_b), rpa, cia, _c(v_a, np.float32), rpb, cib, _c(v_b, np.float32),
                                rpc, cic, vc, sc) != 0:
        raise MemoryError("oracle_spgemm_fill")
    return rpc, cic[:nnz], vc[:nnz], sc[:nnz]


from .solver import fe_diagonal, pcg_jacobi, power_lambda_max, inverse_lambda_min  # noqa: E402
