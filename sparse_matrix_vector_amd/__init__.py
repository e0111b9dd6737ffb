"""Python binding of the MI355X SpMV library (libspmv_amd.so, C ABI in
include/spmv.h).

Each function has the name of the C entry point it calls and only marshals
arguments: torch tensors (or NumPy arrays for the host-side MACKO encoder)
become pointers, ``stream=None`` becomes torch's current stream on the
tensors' device.  Every step of the computation runs in the library's HIP
kernels; nothing here computes.  A non-zero status raises ``SpmvError`` with
the library's message.

``CSRMatrix`` is a small convenience wrapper that owns the plan workspace and
the handle of ``spmv_csr_create``.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib

__all__ = [
    "SpmvError", "STATUS", "CSR_AUTO", "CSR_SCALAR", "CSR_VECTOR", "CSR_BINNED",
    "FORMAT_ELL", "FORMAT_HYB", "FORMAT_CSR", "lib",
    "spmv_scratch_size", "spmv_csr_row_stats", "spmv_format_recommend", "spmv_csr_plan_size", "spmv_csr_create",
    "spmv_csr_apply", "spmv_csr_get_plan", "spmv_csr_info", "spmv_csr_destroy",
    "spmv_ell_from_csr", "spmv_ell_apply", "macko_encode_size", "macko_encode", "macko_spmv",
    "macko_quantize_i8", "macko_spmv_i8", "macko_decode_columns", "dense_gemv_f16", "fem_matvec_apply", "fem_threestage_size", "fem_blocks_size", "fem_blocks_plan_host", "FEBlocks",
    "fem_blocks_create", "fem_blocks_apply", "fem_blocks_info", "fem_blocks_destroy",
    "fem_matvec_threestage", "fem_matvec_threestage_noalloc", "spmv_stream_copy", "spmv_stream_read",
    "fem_assemble_size", "fem_assemble_pattern", "fem_assemble_values", "fem_assemble_csr",
    "fem_jacobi_diagonal", "fem_solver_workspace_size", "fem_pcg_solve",
    "fem_lambda_max", "fem_lambda_min", "spgemm_workspace_size", "spgemm_create", "spgemm_info",
    "spgemm_compute", "spgemm_destroy", "SpGEMM", "CSRMatrix", "spmv_hyb_width", "spmv_hyb_tail_size",
    "spmv_hyb_from_csr", "spmv_hyb_apply", "HYBMatrix", "spmv_auto_plan", "spmv_auto_create", "spmv_auto_apply",
    "spmv_auto_destroy", "AutoMatrix",
]

STATUS = {0: "SPMV_OK", 1: "SPMV_ERR_INVALID_VALUE", 2: "SPMV_ERR_INVALID_MATRIX",
          3: "SPMV_ERR_UNSORTED", 4: "SPMV_ERR_OVERFLOW", 5: "SPMV_ERR_UNSUPPORTED", 6: "SPMV_ERR_HIP"}
CSR_AUTO, CSR_SCALAR, CSR_VECTOR, CSR_BINNED = 0, 1, 2, 3
FORMAT_ELL, FORMAT_HYB, FORMAT_CSR = 0, 1, 2


class SpmvError(RuntimeError):
    def __init__(self, status: int, func: str, message: str):
        self.status = status
        super().__init__(f"{func}: {STATUS.get(status, status)}: {message}")


def lib():
    return _lib.load()


def _check(status: int, func: str):
    if status != 0:
        msg = lib().spmv_last_error().decode(errors="replace")
        raise SpmvError(status, func, msg)


def _call(name: str, *args):
    _check(getattr(lib(), name)(*args), name)


def _dev(t, dtype, name, allow_none=False):
    """Device pointer of a contiguous CUDA tensor of the given dtype."""
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    ok = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in ok:
        raise TypeError(f"{name} must be one of {ok}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _host(a, dtype, name):
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"{name} must be {np.dtype(dtype)}, got {a.dtype}")
    if not a.flags.c_contiguous:
        raise ValueError(f"{name} must be C-contiguous")
    return a


def _stream(stream, like=None):
    if stream is None:
        import torch
        dev = like.device if like is not None else None
        return torch.cuda.current_stream(dev).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _i32_dtype():
    import torch
    return torch.int32


def _f32_dtype():
    import torch
    return torch.float32


def _u16_dtype():
    """fp16 data may come as float16 or as its raw bits (uint16 / int16)."""
    import torch
    return (torch.float16, torch.uint16, torch.int16)


def _u32_dtype():
    """Packed code words: uint32 or int32 with the same bits."""
    import torch
    return (torch.uint32, torch.int32)


# ---------------------------------------------------------------------------
# Device scratch of the synchronous calls
# ---------------------------------------------------------------------------
def spmv_scratch_size(n_rows) -> int:
    out = ctypes.c_size_t()
    _call("spmv_scratch_size", int(n_rows), ctypes.byref(out))
    return out.value


def _scratch(scratch, n_rows, like):
    """(pointer, bytes) of the caller's scratch tensor, or of a new one of
    spmv_scratch_size(n_rows) bytes on like's device (torch allocates it)."""
    if scratch is None:
        import torch
        scratch = torch.empty(spmv_scratch_size(n_rows), dtype=torch.uint8, device=like.device)
    return scratch, scratch.data_ptr(), scratch.numel() * scratch.element_size()


# ---------------------------------------------------------------------------
# Row statistics and format choice
# ---------------------------------------------------------------------------
def spmv_csr_row_stats(row_ptr, stream=None, scratch=None):
    """(max_len, sum_len, sum_len_sq) of a device int32 row_ptr."""
    n = row_ptr.numel() - 1
    m, s, q = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
    keep, sp, sb = _scratch(scratch, n, row_ptr)
    _call("spmv_csr_row_stats", n, _dev(row_ptr, _i32_dtype(), "row_ptr"), ctypes.byref(m),
          ctypes.byref(s), ctypes.byref(q), sp, sb, _stream(stream, row_ptr))
    return m.value, s.value, q.value


def spmv_format_recommend(n_rows, sum_len, sum_len_sq) -> int:
    f = ctypes.c_int32()
    _call("spmv_format_recommend", int(n_rows), int(sum_len), int(sum_len_sq), ctypes.byref(f))
    return f.value


# ---------------------------------------------------------------------------
# CSR
# ---------------------------------------------------------------------------
def _thr(thresholds):
    if thresholds is None:
        return None, None
    a = (ctypes.c_int32 * 3)(*[int(t) for t in thresholds])
    return a, ctypes.addressof(a)


def spmv_csr_plan_size(n_rows, nnz, thresholds=None) -> int:
    keep, p = _thr(thresholds)
    out = ctypes.c_size_t()
    _call("spmv_csr_plan_size", int(n_rows), int(nnz), p, ctypes.byref(out))
    return out.value


def spmv_csr_create(n_rows, n_cols, row_ptr, col_idx, vals, variant=CSR_AUTO, thresholds=None,
                    workspace=None, stream=None):
    """Returns an opaque handle (int).  workspace: a CUDA uint8 tensor of at
    least spmv_csr_plan_size() bytes (needed by BINNED / AUTO)."""
    keep, p = _thr(thresholds)
    h = ctypes.c_void_p()
    nnz = col_idx.numel()
    ws = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call("spmv_csr_create", ctypes.byref(h), int(n_rows), int(n_cols), int(nnz),
          _dev(row_ptr, _i32_dtype(), "row_ptr"), _dev(col_idx, _i32_dtype(), "col_idx"),
          _dev(vals, _f32_dtype(), "vals"), int(variant), p, ws, ws_bytes, _stream(stream, row_ptr))
    return h.value


def spmv_csr_apply(h, alpha, x, beta, y, stream=None):
    _call("spmv_csr_apply", h, float(alpha), _dev(x, _f32_dtype(), "x"), float(beta),
          _dev(y, _f32_dtype(), "y"), _stream(stream, y))


def spmv_csr_apply_rows(h, alpha, x, beta, y, row_map, stream=None):
    """Scatter form: y[row_map[i]] = alpha * (A x)_i + beta * y[row_map[i]]."""
    _call("spmv_csr_apply_rows", h, float(alpha), _dev(x, _f32_dtype(), "x"), float(beta),
          _dev(y, _f32_dtype(), "y"), _dev(row_map, _i32_dtype(), "row_map"), _stream(stream, y))


def spmv_csr_get_plan(h, perm_out=None, stream=None):
    """bin_offsets (list of 5 ints); fills perm_out (CUDA int32 [n_rows]) if given."""
    off = (ctypes.c_int32 * 5)()
    _call("spmv_csr_get_plan", h, off, _dev(perm_out, _i32_dtype(), "perm_out", allow_none=True),
          _stream(stream, perm_out))
    return list(off)


def spmv_csr_info(h):
    v, g, b = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _call("spmv_csr_info", h, ctypes.byref(v), ctypes.byref(g), ctypes.byref(b))
    return {"variant": v.value, "group_lanes": g.value, "n_short_blocks": b.value}


def spmv_csr_destroy(h):
    _call("spmv_csr_destroy", h)


class CSRMatrix:
    """Owns the plan workspace and handle of one CSR matrix (device tensors)."""

    def __init__(self, n_rows, n_cols, row_ptr, col_idx, vals, variant=CSR_AUTO, thresholds=None,
                 stream=None):
        import torch
        self.n_rows, self.n_cols = int(n_rows), int(n_cols)
        self._arrays = (row_ptr, col_idx, vals)          # borrowed by the handle: keep alive
        # BINNED / AUTO keep their plan here; SCALAR / VECTOR use 256 bytes
        # of it while the handle is created
        nb = spmv_csr_plan_size(n_rows, col_idx.numel(), thresholds) if variant in (CSR_AUTO, CSR_BINNED) else 256
        self.workspace = torch.empty(max(nb, 256), dtype=torch.uint8, device=row_ptr.device)
        self.handle = spmv_csr_create(n_rows, n_cols, row_ptr, col_idx, vals, variant, thresholds,
                                      self.workspace, stream)

    def apply(self, x, y, alpha=1.0, beta=0.0, stream=None):
        spmv_csr_apply(self.handle, alpha, x, beta, y, stream)
        return y

    def apply_rows(self, x, y, row_map, alpha=1.0, beta=0.0, stream=None):
        spmv_csr_apply_rows(self.handle, alpha, x, beta, y, row_map, stream)
        return y

    def plan(self, perm_out=None):
        return spmv_csr_get_plan(self.handle, perm_out)

    def info(self):
        return spmv_csr_info(self.handle)

    def close(self):
        if getattr(self, "handle", None):
            spmv_csr_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------------------
# ELL
# ---------------------------------------------------------------------------
def spmv_ell_from_csr(n_rows, n_cols, row_ptr, col_idx, vals, width, ell_col, ell_val, stream=None, scratch=None):
    keep, sp, sb = _scratch(scratch, n_rows, row_ptr)
    _call("spmv_ell_from_csr", int(n_rows), int(n_cols), int(col_idx.numel()),
          _dev(row_ptr, _i32_dtype(), "row_ptr"), _dev(col_idx, _i32_dtype(), "col_idx"),
          _dev(vals, _f32_dtype(), "vals"), int(width), _dev(ell_col, _i32_dtype(), "ell_col"),
          _dev(ell_val, _f32_dtype(), "ell_val"), sp, sb, _stream(stream, row_ptr))


def spmv_ell_apply(n_rows, n_cols, width, ell_col, ell_val, alpha, x, beta, y, stream=None):
    _call("spmv_ell_apply", int(n_rows), int(n_cols), int(width),
          _dev(ell_col, _i32_dtype(), "ell_col"), _dev(ell_val, _f32_dtype(), "ell_val"),
          float(alpha), _dev(x, _f32_dtype(), "x"), float(beta), _dev(y, _f32_dtype(), "y"),
          _stream(stream, y))


# ---------------------------------------------------------------------------
# HYB (ELL part + CSR tail) and the CV-driven format choice
# ---------------------------------------------------------------------------
HYB_ELL_NUM, HYB_ELL_DEN = 7, 10


def spmv_hyb_width(n_rows, row_ptr, num=HYB_ELL_NUM, den=HYB_ELL_DEN, stream=None, scratch=None):
    """(width, n_tail_rows, tail_nnz) of the width rule.  Synchronises."""
    w, r, t = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    keep, sp, sb = _scratch(scratch, n_rows, row_ptr)
    _call("spmv_hyb_width", int(n_rows), _dev(row_ptr, _i32_dtype(), "row_ptr"), int(num), int(den),
          ctypes.byref(w), ctypes.byref(r), ctypes.byref(t), sp, sb, _stream(stream, row_ptr))
    return w.value, r.value, t.value


def spmv_hyb_tail_size(n_rows, row_ptr, width, stream=None, scratch=None):
    """(n_tail_rows, tail_nnz) of the HYB split at an explicit width.  Synchronises."""
    r, t = ctypes.c_int32(), ctypes.c_int64()
    keep, sp, sb = _scratch(scratch, n_rows, row_ptr)
    _call("spmv_hyb_tail_size", int(n_rows), _dev(row_ptr, _i32_dtype(), "row_ptr"), int(width),
          ctypes.byref(r), ctypes.byref(t), sp, sb, _stream(stream, row_ptr))
    return r.value, t.value


def spmv_hyb_from_csr(n_rows, n_cols, row_ptr, col_idx, vals, width, n_tail_rows, tail_nnz,
                      ell_col, ell_val, tail_rows, tail_rp, tail_col, tail_val, stream=None, scratch=None):
    keep, sp, sb = _scratch(scratch, n_rows, row_ptr)
    _call("spmv_hyb_from_csr", int(n_rows), int(n_cols), int(col_idx.numel()),
          _dev(row_ptr, _i32_dtype(), "row_ptr"), _dev(col_idx, _i32_dtype(), "col_idx"),
          _dev(vals, _f32_dtype(), "vals"), int(width), _dev(ell_col, _i32_dtype(), "ell_col"),
          _dev(ell_val, _f32_dtype(), "ell_val"), int(n_tail_rows), int(tail_nnz),
          _dev(tail_rows, _i32_dtype(), "tail_rows"), _dev(tail_rp, _i32_dtype(), "tail_rp"),
          _dev(tail_col, _i32_dtype(), "tail_col"), _dev(tail_val, _f32_dtype(), "tail_val"), sp, sb,
          _stream(stream, row_ptr))


def spmv_hyb_apply(n_rows, n_cols, width, ell_col, ell_val, n_tail_rows, tail_nnz, tail_rows, tail_rp,
                   tail_col, tail_val, alpha, x, beta, y, stream=None):
    _call("spmv_hyb_apply", int(n_rows), int(n_cols), int(width), _dev(ell_col, _i32_dtype(), "ell_col"),
          _dev(ell_val, _f32_dtype(), "ell_val"), int(n_tail_rows), int(tail_nnz),
          _dev(tail_rows, _i32_dtype(), "tail_rows"), _dev(tail_rp, _i32_dtype(), "tail_rp"),
          _dev(tail_col, _i32_dtype(), "tail_col"), _dev(tail_val, _f32_dtype(), "tail_val"),
          float(alpha), _dev(x, _f32_dtype(), "x"), float(beta), _dev(y, _f32_dtype(), "y"),
          _stream(stream, y))


class HYBMatrix:
    """A CSR matrix split into HYB (device tensors it owns)."""

    def __init__(self, n_rows, n_cols, row_ptr, col_idx, vals, width=None, num=HYB_ELL_NUM, den=HYB_ELL_DEN,
                 stream=None):
        import torch
        self.n_rows, self.n_cols = int(n_rows), int(n_cols)
        scratch = torch.empty(spmv_scratch_size(n_rows), dtype=torch.uint8, device=row_ptr.device)
        if width is None:
            w, r, t = spmv_hyb_width(n_rows, row_ptr, num, den, stream, scratch)
        else:
            w = int(width)
            r, t = spmv_hyb_tail_size(n_rows, row_ptr, w, stream, scratch)
        self.width, self.n_tail_rows, self.tail_nnz = w, r, t
        d = row_ptr.device
        self.ell_col = torch.empty(w * self.n_rows, dtype=torch.int32, device=d)
        self.ell_val = torch.empty(w * self.n_rows, dtype=torch.float32, device=d)
        self.tail_rows = torch.empty(r, dtype=torch.int32, device=d)
        self.tail_rp = torch.empty(r + 1, dtype=torch.int32, device=d)
        self.tail_col = torch.empty(t, dtype=torch.int32, device=d)
        self.tail_val = torch.empty(t, dtype=torch.float32, device=d)
        spmv_hyb_from_csr(n_rows, n_cols, row_ptr, col_idx, vals, w, r, t, self.ell_col, self.ell_val,
                          self.tail_rows, self.tail_rp, self.tail_col, self.tail_val, stream, scratch)

    def apply(self, x, y, alpha=1.0, beta=0.0, stream=None):
        spmv_hyb_apply(self.n_rows, self.n_cols, self.width, self.ell_col, self.ell_val, self.n_tail_rows,
                       self.tail_nnz, self.tail_rows, self.tail_rp, self.tail_col, self.tail_val, alpha, x,
                       beta, y, stream)
        return y


def spmv_auto_plan(n_rows, n_cols, nnz, row_ptr, stream=None, scratch=None):
    """The CV rule's choice for this matrix: an AutoPlan (format, width, tail sizes, workspace bytes)."""
    p = _lib.AutoPlan()
    keep, sp, sb = _scratch(scratch, n_rows, row_ptr)
    _call("spmv_auto_plan", int(n_rows), int(n_cols), int(nnz), _dev(row_ptr, _i32_dtype(), "row_ptr"),
          ctypes.byref(p), sp, sb, _stream(stream, row_ptr))
    return p


def spmv_auto_create(plan, n_rows, n_cols, row_ptr, col_idx, vals, workspace, stream=None):
    """Handle (int) of the planned format built in `workspace` (a uint8 CUDA tensor).  Synchronises."""
    h = ctypes.c_void_p()
    _call("spmv_auto_create", ctypes.byref(h), ctypes.byref(plan), int(n_rows), int(n_cols),
          int(col_idx.numel()), _dev(row_ptr, _i32_dtype(), "row_ptr"), _dev(col_idx, _i32_dtype(), "col_idx"),
          _dev(vals, _f32_dtype(), "vals"), workspace.data_ptr(), int(workspace.numel()),
          _stream(stream, row_ptr))
    return h.value


def spmv_auto_apply(handle, alpha, x, beta, y, stream=None):
    _call("spmv_auto_apply", handle, float(alpha), _dev(x, _f32_dtype(), "x"), float(beta),
          _dev(y, _f32_dtype(), "y"), _stream(stream, y))


def spmv_auto_destroy(handle):
    _call("spmv_auto_destroy", handle)


class AutoMatrix:
    """ELL, HYB or binned CSR, as the CV rule chooses, behind one handle."""

    def __init__(self, n_rows, n_cols, row_ptr, col_idx, vals, stream=None):
        import torch
        self.n_rows, self.n_cols = int(n_rows), int(n_cols)
        self._arrays = (row_ptr, col_idx, vals)          # borrowed when the format is CSR
        self.plan = spmv_auto_plan(n_rows, n_cols, col_idx.numel(), row_ptr, stream)
        self.workspace = torch.empty(max(int(self.plan.workspace_bytes), 256), dtype=torch.uint8,
                                     device=row_ptr.device)
        self.handle = spmv_auto_create(self.plan, n_rows, n_cols, row_ptr, col_idx, vals, self.workspace, stream)

    @property
    def format(self):
        return int(self.plan.format)

    def apply(self, x, y, alpha=1.0, beta=0.0, stream=None):
        spmv_auto_apply(self.handle, alpha, x, beta, y, stream)
        return y

    def close(self):
        if getattr(self, "handle", None):
            spmv_auto_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------------------
# SpGEMM C = A * B (hash-based, multi-phase)
# ---------------------------------------------------------------------------
def spgemm_workspace_size(m, k, n, rp_a, ci_a, rp_b, ci_b, stream=None, scratch=None) -> int:
    out = ctypes.c_size_t()
    keep, sp, sb = _scratch(scratch, m, rp_a)
    _call("spgemm_workspace_size", int(m), int(k), int(n), int(ci_a.numel()), _dev(rp_a, _i32_dtype(), "rp_a"),
          _dev(ci_a, _i32_dtype(), "ci_a"), int(ci_b.numel()), _dev(rp_b, _i32_dtype(), "rp_b"),
          _dev(ci_b, _i32_dtype(), "ci_b"), ctypes.byref(out), sp, sb, _stream(stream, rp_a))
    return out.value


def spgemm_create(m, k, n, rp_a, ci_a, v_a, rp_b, ci_b, v_b, workspace, stream=None):
    """Handle (int) after the grouping and allocation phases.  Synchronises."""
    h = ctypes.c_void_p()
    _call("spgemm_create", ctypes.byref(h), int(m), int(k), int(n), int(ci_a.numel()),
          _dev(rp_a, _i32_dtype(), "rp_a"), _dev(ci_a, _i32_dtype(), "ci_a"), _dev(v_a, _f32_dtype(), "v_a"),
          int(ci_b.numel()), _dev(rp_b, _i32_dtype(), "rp_b"), _dev(ci_b, _i32_dtype(), "ci_b"),
          _dev(v_b, _f32_dtype(), "v_b"), workspace.data_ptr(), int(workspace.numel()), _stream(stream, rp_a))
    return h.value


def spgemm_info(handle):
    """(nnz_c, intermediate products, rows per IP group [4])."""
    nnz, ip = ctypes.c_int64(), ctypes.c_int64()
    g = (ctypes.c_int32 * 4)()
    _call("spgemm_info", handle, ctypes.byref(nnz), ctypes.byref(ip), g)
    return nnz.value, ip.value, list(g)


def spgemm_compute(handle, rp_c, ci_c, v_c, stream=None):
    _call("spgemm_compute", handle, _dev(rp_c, _i32_dtype(), "rp_c"),
          _dev(ci_c, _i32_dtype(), "ci_c", allow_none=True) if ci_c is not None and ci_c.numel() else None,
          _dev(v_c, _f32_dtype(), "v_c", allow_none=True) if v_c is not None and v_c.numel() else None,
          _stream(stream, rp_c))


def spgemm_destroy(handle):
    _call("spgemm_destroy", handle)


class SpGEMM:
    """C = A * B for device CSR matrices (A m x k, B k x n): the grouping and
    allocation phases run at construction; compute() runs the accumulation
    phase into new (or given) output tensors."""

    def __init__(self, m, k, n, rp_a, ci_a, v_a, rp_b, ci_b, v_b, stream=None):
        import torch
        self.m, self.k, self.n = int(m), int(k), int(n)
        self._arrays = (rp_a, ci_a, v_a, rp_b, ci_b, v_b)      # borrowed by the handle
        nbytes = spgemm_workspace_size(m, k, n, rp_a, ci_a, rp_b, ci_b, stream)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=rp_a.device)
        self.handle = spgemm_create(m, k, n, rp_a, ci_a, v_a, rp_b, ci_b, v_b, self.workspace, stream)
        self.nnz, self.intermediate_products, self.group_rows = spgemm_info(self.handle)

    def compute(self, out=None, stream=None):
        import torch
        dev = self._arrays[0].device
        if out is None:
            out = (torch.empty(self.m + 1, dtype=torch.int32, device=dev),
                   torch.empty(self.nnz, dtype=torch.int32, device=dev),
                   torch.empty(self.nnz, dtype=torch.float32, device=dev))
        spgemm_compute(self.handle, *out, stream)
        return out

    def close(self):
        if getattr(self, "handle", None):
            spgemm_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------------------
# MACKO (encoder on the host, kernels on the device)
# ---------------------------------------------------------------------------
def macko_encode_size(n_rows, n_cols, row_ptr, col_idx, bdelta=4) -> int:
    rp = _host(row_ptr, np.int32, "row_ptr")
    ci = _host(col_idx, np.int32, "col_idx")
    out = ctypes.c_int64()
    _call("macko_encode_size", int(n_rows), int(n_cols), int(bdelta), rp.ctypes.data, ci.ctypes.data,
          ctypes.byref(out))
    return out.value


def macko_encode(n_rows, n_cols, row_ptr, col_idx, vals_f16, bdelta=4):
    """Host encode with b-bit codes: (mrow_ptr int32[R+1], codes uint32[E*b/32], mvals uint16[E])."""
    rp = _host(row_ptr, np.int32, "row_ptr")
    ci = _host(col_idx, np.int32, "col_idx")
    vv = _host(vals_f16, np.uint16, "vals_f16")
    E = macko_encode_size(n_rows, n_cols, rp, ci, bdelta)
    nw = E * int(bdelta) // 32
    mrp = np.empty(n_rows + 1, np.int32)
    codes = np.empty(max(nw, 1), np.uint32)[:nw]
    mv = np.empty(max(E, 1), np.uint16)[:E]
    _call("macko_encode", int(n_rows), int(n_cols), int(bdelta), rp.ctypes.data, ci.ctypes.data, vv.ctypes.data,
          mrp.ctypes.data, codes.ctypes.data, mv.ctypes.data)
    return mrp, codes, mv


def macko_quantize_i8(n_rows, mrow_ptr, mvals):
    """Host int8 values of an encoded matrix: (q int8[E], row_scale float32[R])."""
    mrp = _host(mrow_ptr, np.int32, "mrow_ptr")
    mv = _host(mvals, np.uint16, "mvals")
    E = int(mrp[n_rows]) if n_rows > 0 else 0
    q = np.empty(max(E, 1), np.int8)[:E]
    sc = np.empty(max(n_rows, 1), np.float32)[:n_rows]
    _call("macko_quantize_i8", int(n_rows), mrp.ctypes.data, mv.ctypes.data, q.ctypes.data, sc.ctypes.data)
    return q, sc


def macko_spmv(n_rows, n_cols, mrow_ptr, codes, mvals, alpha, x_f16, beta, y, stream=None, bdelta=4):
    _call("macko_spmv", int(n_rows), int(n_cols), int(bdelta), _dev(mrow_ptr, _i32_dtype(), "mrow_ptr"),
          _dev(codes, _u32_dtype(), "codes"), _dev(mvals, _u16_dtype(), "mvals"), float(alpha),
          _dev(x_f16, _u16_dtype(), "x_f16"), float(beta), _dev(y, _f32_dtype(), "y"), _stream(stream, y))


def macko_spmv_i8(n_rows, n_cols, mrow_ptr, codes, q, row_scale, alpha, x_f16, beta, y, stream=None, bdelta=4):
    import torch
    _call("macko_spmv_i8", int(n_rows), int(n_cols), int(bdelta), _dev(mrow_ptr, _i32_dtype(), "mrow_ptr"),
          _dev(codes, _u32_dtype(), "codes"), _dev(q, (torch.int8, torch.uint8), "q"),
          _dev(row_scale, _f32_dtype(), "row_scale"), float(alpha), _dev(x_f16, _u16_dtype(), "x_f16"),
          float(beta), _dev(y, _f32_dtype(), "y"), _stream(stream, y))


def macko_decode_columns(n_rows, mrow_ptr, codes, cols_out, stream=None, bdelta=4):
    _call("macko_decode_columns", int(n_rows), int(bdelta), _dev(mrow_ptr, _i32_dtype(), "mrow_ptr"),
          _dev(codes, _u32_dtype(), "codes"), _dev(cols_out, _i32_dtype(), "cols_out"),
          _stream(stream, cols_out))


# ---------------------------------------------------------------------------
# Dense fp16 GEMV
# ---------------------------------------------------------------------------
def dense_gemv_f16(m, n, W, x_f16, alpha, beta, y, stream=None):
    _call("dense_gemv_f16", int(m), int(n), _dev(W, _u16_dtype(), "W"), _dev(x_f16, _u16_dtype(), "x_f16"),
          float(alpha), float(beta), _dev(y, _f32_dtype(), "y"), _stream(stream, y))


# ---------------------------------------------------------------------------
# Finite-element matvec
# ---------------------------------------------------------------------------
def fem_matvec_apply(n_elem, n_dof, edof, rho, penalty, Ke, alpha, x, beta, y, stream=None):
    _call("fem_matvec_apply", int(n_elem), int(n_dof), _dev(edof, _i32_dtype(), "edof"),
          _dev(rho, _f32_dtype(), "rho"), int(penalty), _dev(Ke, _f32_dtype(), "Ke"), float(alpha),
          _dev(x, _f32_dtype(), "x"), float(beta), _dev(y, _f32_dtype(), "y"), _stream(stream, y))


def fem_blocks_size(n_elem, n_dof) -> int:
    out = ctypes.c_size_t()
    _call("fem_blocks_size", int(n_elem), int(n_dof), ctypes.byref(out))
    return out.value


def fem_blocks_plan_host(n_elem, n_dof, edof, group=0):
    """The element-block plan from a host (NumPy) edof: a dict of NumPy
    arrays (blk_elem_off, perm, blk_dof_off, ldof, ldst, crun, lidx, lpos,
    shr_ptr, shr_dof, shr_cnt) and the counts.  group: 0 (3 when the numbering has
    the node structure, else 1), 1 or 3.  For inspection and tests."""
    import numpy as np
    E, n = int(n_elem), int(n_dof)
    ed = np.ascontiguousarray(edof, dtype=np.int32).reshape(-1)
    counts = np.zeros(9, np.int32)
    ent = max(24 * E, 1)
    names = ("blk_elem_off", "perm", "blk_dof_off", "ldof", "ldst", "crun", "lidx", "lpos", "shr_ptr", "shr_dof",
             "shr_cnt")
    a = {"blk_elem_off": np.zeros(E + 1, np.int32), "perm": np.zeros(max(E, 1), np.int32),
         "blk_dof_off": np.zeros(E + 1, np.int32), "ldof": np.zeros(ent, np.int32), "ldst": np.zeros(ent, np.int32),
         "crun": np.zeros(ent, np.uint32), "lidx": np.zeros(ent, np.uint16), "lpos": np.zeros(ent, np.uint16),
         "shr_ptr": np.zeros(n + 1, np.int32), "shr_dof": np.zeros(max(n, 1), np.int32),
         "shr_cnt": np.zeros(max(n, 1), np.int32)}
    _call("fem_blocks_plan_host", E, n, ed.ctypes.data, int(group), counts.ctypes.data,
          *[a[k].ctypes.data for k in names])
    nb, sum_l, n_sh, n_slots, lmax, pmax, G, planes, block = (int(c) for c in counts)
    U = 24 // G
    return {"group": G, "block": block, "n_blocks": nb, "Lmax": lmax, "Pmax": pmax, "n_slots": n_slots,
            "planes": planes,
            "blk_elem_off": a["blk_elem_off"][:nb + 1], "perm": a["perm"][:E],
            "blk_dof_off": a["blk_dof_off"][:nb + 1], "ldof": a["ldof"][:sum_l], "ldst": a["ldst"][:sum_l],
            "crun": a["crun"][:sum_l], "lidx": a["lidx"][:U * E], "lpos": a["lpos"][:U * E],
            "shr_ptr": a["shr_ptr"][:n_sh + 1], "shr_dof": a["shr_dof"][:n_sh], "shr_cnt": a["shr_cnt"][:n_sh]}


def fem_blocks_create(n_elem, n_dof, edof, workspace, stream=None, group=0):
    """Opaque handle (int) of the element-block plan, kept in `workspace` (a
    CUDA uint8 tensor of at least fem_blocks_size() bytes); group as for
    fem_blocks_plan_host."""
    h = ctypes.c_void_p()
    _call("fem_blocks_create", ctypes.byref(h), int(n_elem), int(n_dof), _dev(edof, _i32_dtype(), "edof"), int(group),
          workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream, edof))
    return h.value


def fem_blocks_apply(handle, rho, penalty, Ke, alpha, x, beta, y, stream=None):
    _call("fem_blocks_apply", handle, _dev(rho, _f32_dtype(), "rho"), int(penalty), _dev(Ke, _f32_dtype(), "Ke"),
          float(alpha), _dev(x, _f32_dtype(), "x"), float(beta), _dev(y, _f32_dtype(), "y"), _stream(stream, y))
    return y


def fem_blocks_info(handle):
    import numpy as np
    c = np.zeros(7, np.int32)
    _call("fem_blocks_info", handle, c.ctypes.data)
    return {"n_blocks": int(c[0]), "Lmax": int(c[1]), "n_shared": int(c[2]), "Pmax": int(c[3]), "group": int(c[4]),
            "planes": int(c[5]), "block": int(c[6])}


def fem_blocks_destroy(handle):
    _call("fem_blocks_destroy", handle)


class FEBlocks:
    """The element-block plan of one mesh (edof: a device int32 tensor of
    n_elem * 24 entries), built once; apply() runs the two-kernel matvec.
    group: 0 (per node when the numbering allows it), 1 or 3."""

    def __init__(self, n_elem, n_dof, edof, stream=None, group=0):
        import torch
        self.n_elem, self.n_dof = int(n_elem), int(n_dof)
        self.workspace = torch.empty(max(fem_blocks_size(n_elem, n_dof), 256), dtype=torch.uint8,
                                     device=edof.device)
        self.handle = fem_blocks_create(n_elem, n_dof, edof, self.workspace, stream, group)

    def info(self):
        return fem_blocks_info(self.handle)

    def apply(self, rho, penalty, Ke, alpha, x, beta, y, stream=None):
        return fem_blocks_apply(self.handle, rho, penalty, Ke, alpha, x, beta, y, stream)

    def close(self):
        if getattr(self, "handle", None):
            fem_blocks_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def fem_threestage_size(n_elem) -> int:
    out = ctypes.c_size_t()
    _call("fem_threestage_size", int(n_elem), ctypes.byref(out))
    return out.value


def fem_jacobi_diagonal(n_elem, n_dof, edof, rho, penalty, Ke, diag, stream=None):
    _call("fem_jacobi_diagonal", int(n_elem), int(n_dof), _dev(edof, _i32_dtype(), "edof"),
          _dev(rho, _f32_dtype(), "rho"), int(penalty), _dev(Ke, _f32_dtype(), "Ke"),
          _dev(diag, _f32_dtype(), "diag"), _stream(stream, diag))


def fem_solver_workspace_size(n_dof, max_history=0) -> int:
    out = ctypes.c_size_t()
    _call("fem_solver_workspace_size", int(n_dof), int(max_history), ctypes.byref(out))
    return out.value


def _workspace(nbytes, like):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=like.device)


def fem_pcg_solve(n_elem, n_dof, edof, rho, penalty, Ke, f, u, rtol=1e-6, max_iter=1000, workspace=None,
                  stream=None):
    """Jacobi-PCG for K u = f (u: initial guess in, solution out).  Returns
    (iterations, ||r|| / ||f||).  Synchronises."""
    ws = workspace if workspace is not None else _workspace(fem_solver_workspace_size(n_dof), u)
    it = ctypes.c_int32()
    rr = ctypes.c_double()
    _call("fem_pcg_solve", int(n_elem), int(n_dof), _dev(edof, _i32_dtype(), "edof"),
          _dev(rho, _f32_dtype(), "rho"), int(penalty), _dev(Ke, _f32_dtype(), "Ke"), _dev(f, _f32_dtype(), "f"),
          _dev(u, _f32_dtype(), "u"), float(rtol), int(max_iter), ws.data_ptr(),
          ws.numel() * ws.element_size(), ctypes.byref(it), ctypes.byref(rr), _stream(stream, u))
    return it.value, rr.value


def fem_lambda_max(n_elem, n_dof, edof, rho, penalty, Ke, v0, iterations, workspace=None, stream=None):
    """Power iteration: the Rayleigh quotient of every iterate (float64[iterations])."""
    ws = workspace if workspace is not None else _workspace(fem_solver_workspace_size(n_dof, iterations), v0)
    lam = np.zeros(int(iterations), np.float64)
    _call("fem_lambda_max", int(n_elem), int(n_dof), _dev(edof, _i32_dtype(), "edof"),
          _dev(rho, _f32_dtype(), "rho"), int(penalty), _dev(Ke, _f32_dtype(), "Ke"), _dev(v0, _f32_dtype(), "v0"),
          int(iterations), ws.data_ptr(), ws.numel() * ws.element_size(), lam.ctypes.data, _stream(stream, v0))
    return lam


def fem_lambda_min(n_elem, n_dof, edof, rho, penalty, Ke, v0, iterations, inner_rtol=1e-6, inner_max_iter=5000,
                   workspace=None, stream=None):
    """Inverse iteration with Jacobi-PCG solves: (Rayleigh quotients
    float64[iterations], PCG iterations int32[iterations])."""
    ws = workspace if workspace is not None else _workspace(fem_solver_workspace_size(n_dof, iterations), v0)
    lam = np.zeros(int(iterations), np.float64)
    inner = np.zeros(int(iterations), np.int32)
    _call("fem_lambda_min", int(n_elem), int(n_dof), _dev(edof, _i32_dtype(), "edof"),
          _dev(rho, _f32_dtype(), "rho"), int(penalty), _dev(Ke, _f32_dtype(), "Ke"), _dev(v0, _f32_dtype(), "v0"),
          int(iterations), float(inner_rtol), int(inner_max_iter), ws.data_ptr(), ws.numel() * ws.element_size(),
          lam.ctypes.data, inner.ctypes.data, _stream(stream, v0))
    return lam, inner


def fem_matvec_threestage(n_elem, n_dof, edof, rho, penalty, Ke, alpha, x, beta, y, workspace,
                          stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _call("fem_matvec_threestage", int(n_elem), int(n_dof), _dev(edof, _i32_dtype(), "edof"),
          _dev(rho, _f32_dtype(), "rho"), int(penalty), _dev(Ke, _f32_dtype(), "Ke"), float(alpha),
          _dev(x, _f32_dtype(), "x"), float(beta), _dev(y, _f32_dtype(), "y"), workspace.data_ptr(),
          ws_bytes, _stream(stream, y))


def fem_matvec_threestage_noalloc(n_elem, n_dof, edof, rho, penalty, Ke, alpha, x, beta, y, stream=None):
    """The three-stage FE matvec with the library's static device scratch
    (no workspace, no allocation); calls overlapping on one GPU race."""
    _call("fem_matvec_threestage_noalloc", int(n_elem), int(n_dof), _dev(edof, _i32_dtype(), "edof"),
          _dev(rho, _f32_dtype(), "rho"), int(penalty), _dev(Ke, _f32_dtype(), "Ke"), float(alpha),
          _dev(x, _f32_dtype(), "x"), float(beta), _dev(y, _f32_dtype(), "y"), _stream(stream, y))


# ---------------------------------------------------------------------------
# Reference streams (the measured bandwidth denominator)
# ---------------------------------------------------------------------------
def spmv_stream_copy(src, dst, stream=None):
    """dst = src byte for byte (CUDA tensors of equal size, multiple of 16 bytes)."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst must have the same size in bytes")
    _call("spmv_stream_copy", src.data_ptr(), dst.data_ptr(), n, _stream(stream, dst))


def spmv_stream_read(src, partial, stream=None):
    """Reads src once; one fp32 sum per workgroup into partial (2048 floats always suffice)."""
    _call("spmv_stream_read", src.data_ptr(), src.numel() * src.element_size(),
          _dev(partial, _f32_dtype(), "partial"), partial.numel(), _stream(stream, partial))


# ---------------------------------------------------------------------------
# Assembled stiffness matrix (CSR) of the FE operator
# ---------------------------------------------------------------------------
def fem_assemble_size(n_elem, n_dof) -> int:
    out = ctypes.c_size_t()
    _call("fem_assemble_size", int(n_elem), int(n_dof), ctypes.byref(out))
    return out.value


def fem_assemble_pattern(n_elem, n_dof, edof, row_ptr, workspace, stream=None) -> int:
    """Fills row_ptr (CUDA int32[n_dof + 1]); returns nnz.  Synchronises."""
    nnz = ctypes.c_int64()
    _call("fem_assemble_pattern", int(n_elem), int(n_dof), _dev(edof, _i32_dtype(), "edof"),
          _dev(row_ptr, _i32_dtype(), "row_ptr"), ctypes.byref(nnz), workspace.data_ptr(),
          workspace.numel() * workspace.element_size(), _stream(stream, row_ptr))
    return nnz.value


def fem_assemble_values(n_elem, n_dof, edof, rho, penalty, Ke, row_ptr, col_idx, vals, workspace, stream=None):
    _call("fem_assemble_values", int(n_elem), int(n_dof), _dev(edof, _i32_dtype(), "edof"),
          _dev(rho, _f32_dtype(), "rho"), int(penalty), _dev(Ke, _f32_dtype(), "Ke"),
          _dev(row_ptr, _i32_dtype(), "row_ptr"), _dev(col_idx, _i32_dtype(), "col_idx"),
          _dev(vals, _f32_dtype(), "vals"), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
          _stream(stream, row_ptr))


def fem_assemble_csr(n_elem, n_dof, edof, rho, penalty, Ke, stream=None):
    """(row_ptr, col_idx, vals) of the assembled K as new CUDA tensors."""
    import torch
    dev = edof.device
    ws = torch.empty(max(fem_assemble_size(n_elem, n_dof), 256), dtype=torch.uint8, device=dev)
    rp = torch.empty(int(n_dof) + 1, dtype=torch.int32, device=dev)
    nnz = fem_assemble_pattern(n_elem, n_dof, edof, rp, ws, stream)
    ci = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)[:nnz]
    v = torch.empty(max(nnz, 1), dtype=torch.float32, device=dev)[:nnz]
    fem_assemble_values(n_elem, n_dof, edof, rho, penalty, Ke, rp, ci, v, ws, stream)
    return rp, ci, v
