"""ctypes loader and signatures of libspmv_amd.so (the C ABI in include/spmv.h).

The library must have been built (``__graft_entry__.build()`` or
``python -m sparse_matrix_vector_amd.csrc.build``); loading fails loudly
otherwise.  There is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspmv_amd.so")

c_i32, c_i64, c_f32, c_sz, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
P_i32 = ctypes.POINTER(ctypes.c_int32)
P_i64 = ctypes.POINTER(ctypes.c_int64)
P_sz = ctypes.POINTER(ctypes.c_size_t)
P_f64 = ctypes.POINTER(ctypes.c_double)
P_vp = ctypes.POINTER(ctypes.c_void_p)



class AutoPlan(ctypes.Structure):
    """spmv_auto_plan_t."""
    _fields_ = [("format", ctypes.c_int32), ("width", ctypes.c_int32), ("n_tail_rows", ctypes.c_int32),
                ("tail_nnz", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t)]


P_plan = ctypes.POINTER(AutoPlan)

# name -> argument types (every function returns spmv_status, an int)
SIGNATURES = {
    "spmv_scratch_size": [c_i32, P_sz],
    "spmv_csr_row_stats": [c_i32, vp, P_i32, P_i64, P_i64, vp, c_sz, vp],
    "spmv_format_recommend": [c_i64, c_i64, c_i64, P_i32],
    "spmv_csr_plan_size": [c_i32, c_i32, vp, P_sz],
    "spmv_csr_create": [P_vp, c_i32, c_i32, c_i32, vp, vp, vp, c_i32, vp, vp, c_sz, vp],
    "spmv_csr_apply": [vp, c_f32, vp, c_f32, vp, vp],
    "spmv_csr_apply_rows": [vp, c_f32, vp, c_f32, vp, vp, vp],
    "spmv_csr_get_plan": [vp, P_i32, vp, vp],
    "spmv_csr_info": [vp, P_i32, P_i32, P_i32],
    "spmv_csr_destroy": [vp],
    "spmv_ell_from_csr": [c_i32, c_i32, c_i32, vp, vp, vp, c_i32, vp, vp, vp, c_sz, vp],
    "spmv_ell_apply": [c_i32, c_i32, c_i32, vp, vp, c_f32, vp, c_f32, vp, vp],
    "spmv_hyb_width": [c_i32, vp, c_i32, c_i32, P_i32, P_i32, P_i64, vp, c_sz, vp],
    "spmv_hyb_tail_size": [c_i32, vp, c_i32, P_i32, P_i64, vp, c_sz, vp],
    "spmv_hyb_from_csr": [c_i32, c_i32, c_i32, vp, vp, vp, c_i32, vp, vp, c_i32, c_i64, vp, vp, vp, vp, vp, c_sz,
                          vp],
    "spmv_hyb_apply": [c_i32, c_i32, c_i32, vp, vp, c_i32, c_i64, vp, vp, vp, vp, c_f32, vp, c_f32, vp, vp],
    "spmv_auto_plan": [c_i32, c_i32, c_i32, vp, P_plan, vp, c_sz, vp],
    "spmv_auto_create": [P_vp, P_plan, c_i32, c_i32, c_i32, vp, vp, vp, vp, c_sz, vp],
    "spmv_auto_apply": [vp, c_f32, vp, c_f32, vp, vp],
    "spmv_auto_destroy": [vp],
    "macko_encode_size": [c_i32, c_i32, c_i32, vp, vp, P_i64],
    "macko_encode": [c_i32, c_i32, c_i32, vp, vp, vp, vp, vp, vp],
    "macko_quantize_i8": [c_i32, vp, vp, vp, vp],
    "macko_spmv": [c_i32, c_i32, c_i32, vp, vp, vp, c_f32, vp, c_f32, vp, vp],
    "macko_spmv_i8": [c_i32, c_i32, c_i32, vp, vp, vp, vp, c_f32, vp, c_f32, vp, vp],
    "macko_decode_columns": [c_i32, c_i32, vp, vp, vp, vp],
    "dense_gemv_f16": [c_i32, c_i32, vp, vp, c_f32, c_f32, vp, vp],
    "fem_matvec_apply": [c_i32, c_i32, vp, vp, c_i32, vp, c_f32, vp, c_f32, vp, vp],
    "fem_threestage_size": [c_i32, P_sz],
    "fem_blocks_size": [c_i32, c_i32, P_sz],
    "fem_blocks_create": [vp, c_i32, c_i32, vp, c_i32, vp, c_sz, vp],
    "fem_blocks_apply": [vp, vp, c_i32, vp, c_f32, vp, c_f32, vp, vp],
    "fem_blocks_info": [vp, vp],
    "fem_blocks_destroy": [vp],
    "fem_blocks_plan_host": [c_i32, c_i32, vp, c_i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
    "fem_matvec_threestage": [c_i32, c_i32, vp, vp, c_i32, vp, c_f32, vp, c_f32, vp, vp, c_sz, vp],
    "fem_matvec_threestage_noalloc": [c_i32, c_i32, vp, vp, c_i32, vp, c_f32, vp, c_f32, vp, vp],
    "fem_assemble_size": [c_i32, c_i32, P_sz],
    "fem_assemble_pattern": [c_i32, c_i32, vp, vp, P_i64, vp, c_sz, vp],
    "fem_assemble_values": [c_i32, c_i32, vp, vp, c_i32, vp, vp, vp, vp, vp, c_sz, vp],
    "spmv_stream_copy": [vp, vp, c_sz, vp],
    "spmv_stream_read": [vp, c_sz, vp, c_sz, vp],
    "spgemm_workspace_size": [c_i32, c_i32, c_i32, c_i32, vp, vp, c_i32, vp, vp, P_sz, vp, c_sz, vp],
    "spgemm_create": [P_vp, c_i32, c_i32, c_i32, c_i32, vp, vp, vp, c_i32, vp, vp, vp, vp, c_sz, vp],
    "spgemm_info": [vp, P_i64, P_i64, P_i32],
    "spgemm_compute": [vp, vp, vp, vp, vp],
    "spgemm_destroy": [vp],
    "fem_jacobi_diagonal": [c_i32, c_i32, vp, vp, c_i32, vp, vp, vp],
    "fem_solver_workspace_size": [c_i32, c_i32, P_sz],
    "fem_pcg_solve": [c_i32, c_i32, vp, vp, c_i32, vp, vp, vp, c_f32, c_i32, vp, c_sz, P_i32, P_f64, vp],
    "fem_lambda_max": [c_i32, c_i32, vp, vp, c_i32, vp, vp, c_i32, vp, c_sz, vp, vp],
    "fem_lambda_min": [c_i32, c_i32, vp, vp, c_i32, vp, vp, c_i32, c_f32, c_i32, vp, c_sz, vp, vp, vp],
}

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m sparse_matrix_vector_amd.csrc.build)")
        L = ctypes.CDLL(LIB_PATH)
        L.spmv_last_error.restype = ctypes.c_char_p
        L.spmv_last_error.argtypes = []
        for name, args in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = ctypes.c_int
            fn.argtypes = args
        _lib = L
    return _lib
