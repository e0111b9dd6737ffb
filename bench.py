#!/usr/bin/env python3
"""Benchmark of the MI355X SpMV library: y = alpha * A * x + beta * y.

Default run (N = 1): every configuration in one JSON line.  The headline is
the 2-D 5-point Laplacian on a 1000 x 1000 grid (1,000,000 rows, 4,996,000
nonzeros, fp32), CSR path with the row-grouping planner (spmv_csr_apply,
AUTO variant); one step = one apply, and exactly --steps of them are timed.
Under "configs" the line then carries, with the same step count, its own
parity check and a short oracle timing: the Laplacian's ELL path, the tiny
CSR, the power-law CSR, the pruned 12288 x 12288 weights at 50 / 70 / 90 %
sparsity (MACKO) and the dense fp16 GEMV comparator, and the FE matvec
(fused, three-stage, and the assembled stiffness matrix through the binned
CSR path).  Under "next_rows": the moderate-CV matrix through the CV-driven
choice (HYB), Jacobi-PCG on the elasticity cantilever, and the hash SpGEMM
C = A * A of the power-law matrix (at most 20 whole products).

Cold-cache protocol ("rotate", the default): the inputs are replicated R
times in HBM so that R copies span >= 1 GiB (4x the 256 MB Infinity Cache
plus the L2s); step i applies copy i mod R, so every apply streams a matrix
that was last touched >= 3/4 GiB of traffic earlier, i.e. from HBM.  K steps
run back to back on one stream between two HIP events recorded on that
stream (no host synchronisation inside), replayed from HIP graphs (one of
the R copies, one of the first K mod R), so per-launch host cost does not
enter the per-step time.  "flush" mode instead writes 1 GiB before every
apply and brackets each apply with its own event pair.  "warm" repeats copy
0 (data cached in the Infinity Cache).  Inputs are resident in HBM before
the timed region.

Printed: ONE JSON line with the metric (GFLOP/s), effective GB/s over the
algorithmic bytes, the roofline of the dominant kernel against the 8 TB/s
HBM peak, the library's reference streams (copy, read) at the same size,
and the CPU oracle timed on the host (serial fp64 C on one core, bounded
sample; and the same function on row blocks in one thread per core).

One workload only (--config, optionally --path; used for the profiles):
  --config tiny | laplacian | powerlaw | varlen | pruned50 | pruned70 | pruned90 | fe | cantilever
  --path   csr | csr-binned | csr-vector | csr-scalar | ell | hyb | auto | macko | dense | fem | fem-blocks
           | fem-blocks-dof (the element-block plan on single DOFs instead of nodes) | fem-3stage
           | fem-csr (the assembled stiffness matrix through the binned CSR path)
           (MACKO variants: macko-b1 | macko-b2 | macko-b8 for 1-, 2- or 8-bit
           codes instead of 4, macko-i8 and macko-i8-bN for int8 values)
  (varlen: 1M rows of 2..10 entries in a +-1000 band, CV 0.43, the HYB range
  of the CV rule; auto: the format that rule picks)
  powerlaw | laplacian / spgemm: C = A * A by the hash-based multi-phase
  SpGEMM; one step = one whole product (row grouping, allocation phase,
  accumulation phase into fresh output), host-synchronous, as a caller runs
  it; the accumulation phase alone is also timed with HIP events.
  cantilever / fem-pcg: Jacobi-PCG on the 216k-element elasticity cantilever
  (rho = 0.5); one step = one PCG iteration (fixed count, rtol = 0), timed
  warm, as a solver runs it; the line also carries a solve to rtol 1e-6 and
  the condition-number estimate.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "SpMV GFLOP/s and effective HBM GB/s (% of MI355X peak) per config, 1 GPU"
FLUSH_BYTES = 1 << 30
ROTATE_BYTES = 1 << 30

DEFAULT_PATH = {"tiny": "csr", "laplacian": "csr", "powerlaw": "csr", "varlen": "auto", "pruned50": "macko",
                "pruned70": "macko", "pruned90": "macko", "fe": "fem", "cantilever": "fem-pcg"}
CSR_CONFIGS = ("tiny", "laplacian", "powerlaw", "varlen")
# further paths the config itself names, measured beside the default one when
# no --path is given (the Laplacian config names a CSR and an ELL path)
OTHER_PATHS = {"laplacian": ("ell",)}

# kernel (as rocprofv3 names it) that dominates each path
KERNEL = {"csr": "k_csr_tasks", "csr-binned": "k_csr_tasks", "csr-vector": "k_csr_vector",
          "csr-scalar": "k_csr_scalar", "ell": "k_ell_apply4t", "macko": "k_macko_spmv",
          "dense": "k_gemv_f16", "fem": "k_fe_fused", "fem-blocks": "k_fe_block", "fem-blocks-dof": "k_fe_block",
          "fem-3stage": "k_fe_elem",
          "fem-csr": "k_csr_tasks",
          "hyb": "k_ell_apply",
          "auto": None, "fem-pcg": "k_fe_matvec64 + k_cg_dot + k_cg_step",
          "spgemm": "k_sg_* (grouping, allocation, accumulation)"}

# source file of each path's kernels (for the traffic-record freshness check)
SOURCE = {"csr": ("csr.hip",), "csr-binned": ("csr.hip",), "csr-vector": ("csr.hip",),
          "csr-scalar": ("csr.hip",), "ell": ("ell.hip",), "macko": ("macko.hip",), "dense": ("dense.hip",),
          "fem": ("fem.hip", "fem_common.hpp"), "fem-blocks": ("fem_blocks.hip", "fem_blocks.cpp", "fem_blocks.hpp"),
          "fem-blocks-dof": ("fem_blocks.hip", "fem_blocks.cpp", "fem_blocks.hpp"),
          "fem-3stage": ("fem.hip",), "fem-csr": ("csr.hip",),
          "hyb": ("ell.hip", "hyb.hip"),
          "auto": ("csr.hip", "ell.hip", "hyb.hip"), "fem-pcg": ("fem_solver.hip", "fem_common.hpp"), "spgemm": ("spgemm.hip",)}
for _v in ("b1", "b2", "b8", "i8", "i8-b1", "i8-b2", "i8-b8"):
    KERNEL["macko-" + _v] = "k_macko_spmv"
    SOURCE["macko-" + _v] = ("macko.hip",)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(path_name):
    """Hash of the path's kernel sources without their // comments and blank
    lines, so that a comment edit does not retire the recorded counters."""
    h = hashlib.sha256()
    for f in SOURCE[path_name]:
        with open(os.path.join(ROOT, "sparse_matrix_vector_amd", "csrc", f), encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


class Workload:
    """Inputs on the GPU (replicated `copies` times) plus one launch closure
    per copy for one path."""

    def __init__(self, config, path, copies=None):
        import numpy as np
        import torch
        import gen
        import sparse_matrix_vector_amd as S
        self.config, self.path = config, path
        self.np, self.torch, self.S = np, torch, S
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.alpha, self.beta = 1.0, 0.0
        t0 = time.time()
        if config in CSR_CONFIGS:
            A = {"tiny": gen.tiny_csr, "laplacian": gen.laplacian_2d, "powerlaw": gen.powerlaw_csr,
                 "varlen": gen.varlen_banded}[config]()
            self.A = A
            self.workload = {"tiny": "tiny_csr_4096x4096_8perrow", "laplacian": "laplacian_2d_1000x1000",
                             "powerlaw": "powerlaw_916428_zipf1.9931",
                             "varlen": "varlen_banded_1000000_len2-10_band1000"}[config]
            self.flops = 2 * A.nnz
            csr_bytes = 8 * A.nnz + 4 * (A.n_rows + 1) + 4 * A.n_cols + 4 * A.n_rows
            ell_bytes = lambda W: 8 * W * A.n_rows + 4 * A.n_cols + 4 * A.n_rows
            # HYB: ELL part (padding included), tail arrays, x, y, and y read
            # and written again for the tail rows
            hyb_bytes = lambda W, r, t: ell_bytes(W) + 8 * t + 4 * r + 4 * (r + 1) + 8 * r
            if path.startswith("csr"):
                var = {"csr": S.CSR_AUTO, "csr-binned": S.CSR_BINNED, "csr-vector": S.CSR_VECTOR,
                       "csr-scalar": S.CSR_SCALAR}[path]
                self.bytes = csr_bytes
                base = (dev(A.row_ptr), dev(A.col_idx), dev(A.vals), dev(A.x))

                def make(arrs):
                    rp, ci, v, x = arrs
                    M = S.CSRMatrix(A.n_rows, A.n_cols, rp, ci, v, var)
                    y = torch.zeros(A.n_rows, device="cuda")
                    return (lambda: M.apply(x, y, self.alpha, self.beta)), y, M
                self._setup(base, make, copies)
                self.shape = {"n_rows": A.n_rows, "n_cols": A.n_cols, "nnz": A.nnz,
                              "plan": self.extra[0].info()}
            elif path == "ell":
                W = S.spmv_csr_row_stats(dev(A.row_ptr))[0]   # ELL width = the longest row
                self.W = W
                ec = torch.empty(A.n_rows * W, dtype=torch.int32, device="cuda")
                ev = torch.empty(A.n_rows * W, dtype=torch.float32, device="cuda")
                S.spmv_ell_from_csr(A.n_rows, A.n_cols, dev(A.row_ptr), dev(A.col_idx), dev(A.vals), W, ec, ev)
                self.bytes = ell_bytes(W)

                def make(arrs):
                    ec, ev, x = arrs
                    y = torch.zeros(A.n_rows, device="cuda")
                    return (lambda: S.spmv_ell_apply(A.n_rows, A.n_cols, W, ec, ev, self.alpha, x, self.beta,
                                                     y)), y, None
                self._setup((ec, ev, dev(A.x)), make, copies)
                self.shape = {"n_rows": A.n_rows, "nnz": A.nnz, "ell_width": W}
            elif path == "hyb":
                rp0 = dev(A.row_ptr)
                W, r, t = S.spmv_hyb_width(A.n_rows, rp0)
                self.W, self.hyb = W, (W, r, t)
                self.bytes = hyb_bytes(W, r, t)
                H = S.HYBMatrix(A.n_rows, A.n_cols, rp0, dev(A.col_idx), dev(A.vals))
                base = (H.ell_col, H.ell_val, H.tail_rows, H.tail_rp, H.tail_col, H.tail_val, dev(A.x))

                def make(arrs):
                    ec, ev, tr, trp, tc, tv, x = arrs
                    y = torch.zeros(A.n_rows, device="cuda")
                    return (lambda: S.spmv_hyb_apply(A.n_rows, A.n_cols, W, ec, ev, r, t, tr, trp, tc, tv,
                                                     self.alpha, x, self.beta, y)), y, None
                self._setup(base, make, copies)
                self.shape = {"n_rows": A.n_rows, "nnz": A.nnz, "ell_width": W, "tail_rows": r, "tail_nnz": t}
            elif path == "auto":
                plan = S.spmv_auto_plan(A.n_rows, A.n_cols, A.nnz, dev(A.row_ptr))
                fmt = int(plan.format)
                self.auto_format = ["ell", "hyb", "csr"][fmt]
                self.kernel = ["k_ell_apply", "k_ell_apply", "k_csr_tasks"][fmt]
                self.bytes = [ell_bytes(plan.width), hyb_bytes(plan.width, plan.n_tail_rows, plan.tail_nnz),
                              csr_bytes][fmt]
                base = (dev(A.row_ptr), dev(A.col_idx), dev(A.vals), dev(A.x))

                def make(arrs):
                    rp, ci, v, x = arrs
                    M = S.AutoMatrix(A.n_rows, A.n_cols, rp, ci, v)
                    y = torch.zeros(A.n_rows, device="cuda")
                    return (lambda: M.apply(x, y, self.alpha, self.beta)), y, M
                self._setup(base, make, copies)
                self.shape = {"n_rows": A.n_rows, "nnz": A.nnz, "format": self.auto_format,
                              "width": int(plan.width), "tail_rows": int(plan.n_tail_rows),
                              "tail_nnz": int(plan.tail_nnz)}
            else:
                raise SystemExit(f"path {path} does not apply to config {config}")
        elif config.startswith("pruned"):
            s = int(config[6:]) / 100.0
            P = gen.pruned_weight(s)
            self.P = P
            self.workload = f"pruned_weight_12288x12288_sparsity{int(s * 100)}"
            if path.startswith("macko"):
                i8, bd = macko_variant(path)
                mrp, codes, mv = S.macko_encode(P.n_rows, P.n_cols, P.row_ptr, P.col_idx, P.vals_f16, bdelta=bd)
                self.enc = (mrp, codes, mv)
                E = int(mrp[-1])
                # codes + values (+ row scales) + row pointers + x + y
                self.bytes = (E * bd // 8 + (E + 4 * P.n_rows if i8 else 2 * E) + 4 * (P.n_rows + 1)
                              + 2 * P.n_cols + 4 * P.n_rows)
                self.flops = 2 * P.nnz
                if i8:
                    q, rsc = S.macko_quantize_i8(P.n_rows, mrp, mv)
                    vals = (dev(q), dev(rsc))
                else:
                    vals = (dev(mv),)

                def make(arrs):
                    mrp_d, codes_d, xh = arrs[0], arrs[1], arrs[-1]
                    y = torch.zeros(P.n_rows, device="cuda")
                    if i8:
                        q_d, s_d = arrs[2], arrs[3]
                        return (lambda: S.macko_spmv_i8(P.n_rows, P.n_cols, mrp_d, codes_d, q_d, s_d, self.alpha,
                                                        xh, self.beta, y, bdelta=bd)), y, None
                    mv_d = arrs[2]
                    return (lambda: S.macko_spmv(P.n_rows, P.n_cols, mrp_d, codes_d, mv_d, self.alpha, xh,
                                                 self.beta, y, bdelta=bd)), y, None
                self._setup((dev(mrp), dev(codes)) + vals + (dev(P.x_f16),), make, copies)
                self.shape = {"n_rows": P.n_rows, "n_cols": P.n_cols, "nnz": P.nnz, "entries": E,
                              "bdelta": bd, "values": "int8" if i8 else "fp16"}
            elif path == "dense":
                self.bytes = 2 * P.n_rows * P.n_cols + 2 * P.n_cols + 4 * P.n_rows
                self.flops = 2 * P.n_rows * P.n_cols

                def make(arrs):
                    D, xh = arrs
                    y = torch.zeros(P.n_rows, device="cuda")
                    return (lambda: S.dense_gemv_f16(P.n_rows, P.n_cols, D, xh, self.alpha, self.beta, y)), y, None
                self._setup((dev(P.dense_f16()), dev(P.x_f16)), make, copies)
                self.shape = {"m": P.n_rows, "n": P.n_cols}
            else:
                raise SystemExit(f"path {path} does not apply to config {config}")
        elif config == "fe":
            M = gen.fe_mesh()
            self.Mesh = M
            self.workload = "fe_hex8_cantilever_120x60x30"
            self.bytes = 96 * M.n_elem + 4 * M.n_elem + 2304 + 8 * M.n_dof
            self.flops = 1176 * M.n_elem
            if path not in ("fem", "fem-blocks", "fem-blocks-dof", "fem-3stage", "fem-csr"):
                raise SystemExit(f"path {path} does not apply to config {config}")
            if path == "fem-csr":
                # the assembled K, built by the library on the GPU once, then the binned CSR apply
                rp, ci, v = S.fem_assemble_csr(M.n_elem, M.n_dof, dev(M.edof.reshape(-1)), dev(M.rho), M.penalty,
                                               dev(M.Ke.reshape(-1)))
                nnz = int(ci.numel())
                self.bytes = 8 * nnz + 4 * (M.n_dof + 1) + 8 * M.n_dof
                self.flops = 2 * nnz

                def make_csr(arrs):
                    rp_, ci_, v_, x = arrs
                    A = S.CSRMatrix(M.n_dof, M.n_dof, rp_, ci_, v_)
                    y = torch.zeros(M.n_dof, device="cuda")
                    return (lambda: A.apply(x, y, self.alpha, self.beta)), y, A
                self._setup((rp, ci, v, dev(M.x)), make_csr, copies)
                self.shape = {"n_elem": M.n_elem, "n_dof": M.n_dof, "assembled_nnz": nnz,
                              "note": "K assembled by fem_assemble_pattern / fem_assemble_values"}
                torch.cuda.synchronize()
                log(f"[bench] setup {config}/{path}: {len(self.launches)} copies, {time.time() - t0:.1f}s")
                return
            ws = None
            if path == "fem-3stage":
                ws = torch.empty(S.fem_threestage_size(M.n_elem), dtype=torch.uint8, device="cuda")

            def make(arrs):
                edof, rho, Ke, x = arrs
                y = torch.zeros(M.n_dof, device="cuda")
                a = (M.n_elem, M.n_dof, edof, rho, M.penalty, Ke)
                if path in ("fem-blocks", "fem-blocks-dof"):
                    # the plan is built once per copy, outside the timed region
                    P = S.FEBlocks(M.n_elem, M.n_dof, edof, group=1 if path == "fem-blocks-dof" else 0)
                    return (lambda: P.apply(rho, M.penalty, Ke, self.alpha, x, self.beta, y)), y, P
                if path == "fem":
                    return (lambda: S.fem_matvec_apply(*a, self.alpha, x, self.beta, y)), y, None
                return (lambda: S.fem_matvec_threestage(*a, self.alpha, x, self.beta, y, ws)), y, None
            self._setup((dev(M.edof.reshape(-1)), dev(M.rho), dev(M.Ke.reshape(-1)), dev(M.x)), make, copies)
            self.shape = {"n_elem": M.n_elem, "n_dof": M.n_dof}
            if path in ("fem", "fem-3stage"):
                self.shape["atomics"] = int((M.edof >= 0).sum())
            elif path in ("fem-blocks", "fem-blocks-dof"):
                self.shape["plan"] = self.extra[0].info()
        else:
            raise SystemExit(f"unknown config {config}")
        torch.cuda.synchronize()
        log(f"[bench] setup {config}/{path}: {len(self.launches)} copies, {time.time() - t0:.1f}s")

    def _setup(self, base, make, copies):
        """Replicates the input tensors so that all copies span >= ROTATE_BYTES."""
        import math
        n = copies or max(2, math.ceil(ROTATE_BYTES / self.bytes))
        self.launches, self.outputs, self.extra = [], [], []
        for i in range(n):
            arrs = base if i == 0 else tuple(t.clone() for t in base)
            launch, y, extra = make(arrs)
            self.launches.append(launch)
            self.outputs.append(y)
            self.extra.append(extra)
        self.launch = self.launches[0]
        self.y = self.outputs[0]

    # -- oracle (the CPU baseline and the parity check) --
    def oracle_call(self):
        import oracle
        if self.config in CSR_CONFIGS:
            A = self.A
            if self.path == "ell":
                ec, ev = oracle.ell_from_csr(A.row_ptr, A.col_idx, A.vals, self.W)
                return lambda: oracle.ell_spmv(A.n_rows, self.W, ec, ev, A.x)
            if self.path == "hyb":
                parts = oracle.hyb_from_csr(A.row_ptr, A.col_idx, A.vals, self.W)
                return lambda: oracle.hyb_spmv(A.n_rows, self.W, *parts, A.x)
            return lambda: oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x)
        if self.config.startswith("pruned"):
            P = self.P
            if self.path.startswith("macko"):
                i8, bd = macko_variant(self.path)
                mrp, codes, mv = oracle.macko_encode(P.n_cols, P.row_ptr, P.col_idx, P.vals_f16, bdelta=bd)
                if i8:
                    q, rsc = oracle.macko_quantize_i8(mrp, mv)
                    return lambda: oracle.macko_spmv_i8(P.n_cols, mrp, codes, q, rsc, P.x_f16, bdelta=bd)
                return lambda: oracle.macko_spmv(P.n_cols, mrp, codes, mv, P.x_f16, bdelta=bd)
            D = P.dense_f16()
            return lambda: oracle.gemv_f16(D, P.x_f16)
        M = self.Mesh
        return lambda: oracle.fe_matvec(M.edof, M.rho, M.Ke, M.x, M.n_dof)


def macko_variant(path):
    """(int8 values?, code width) of a MACKO path name such as macko-i8-b2."""
    parts = path.split("-")[1:]
    i8 = "i8" in parts
    bd = 4
    for p in parts:
        if p.startswith("b") and p[1:] in ("1", "2", "4", "8"):
            bd = int(p[1:])
        elif p != "i8":
            raise SystemExit(f"unknown MACKO variant {path}")
    return i8, bd


def parity(w, ref_fn):
    """The GPU result of one apply against the oracle, element by element:
    |y - y_ref| <= tau * scale (tau 1e-5 for fp32 values, 4e-3 for fp16
    values), and for MACKO the library's encoding bit-exact with the
    oracle's."""
    np = w.np
    w.torch.cuda.synchronize()
    w.launch()
    w.torch.cuda.synchronize()
    y = w.y.cpu().numpy().astype(np.float64)
    yr, sc = ref_fn()
    tau = 4e-3 if w.config.startswith("pruned") else 1e-5
    nz = sc > 0
    err = np.abs(y - yr)
    worst = float(np.max(err[nz] / sc[nz])) if nz.any() else 0.0
    ok = bool(np.all(err <= tau * sc))
    out = {"ok": ok, "tau": tau, "max_err_over_scale": worst, "outputs": int(len(y))}
    if getattr(w, "enc", None) is not None:
        import oracle
        i8, bd = macko_variant(w.path)
        P = w.P
        oenc = oracle.macko_encode(P.n_cols, P.row_ptr, P.col_idx, P.vals_f16, bdelta=bd)
        same = all(np.array_equal(a, b) for a, b in zip(w.enc, oenc))
        out["encoding_bit_exact"] = bool(same)
        out["ok"] = bool(ok and same)
    return out


def _rate(w, per_call_s):
    """CPU rate in the metric's unit (GFLOP/s) and per-call milliseconds."""
    return round(w.flops / per_call_s / 1e9, 4), round(per_call_s * 1e3, 3)


def _repeat(fn, seconds):
    """Calls fn until `seconds` have passed (at least once); seconds per call."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return el / reps, reps, el


def rowpar_oracle(w):
    """(callable, threads) running the oracle's serial C function on T
    nonzero-balanced row blocks in T threads at once (ctypes releases the
    GIL), T = the host cores this process may use; every row is still summed
    serially, so the result equals the serial oracle's bit for bit.  None
    for paths without independent rows (ELL's slot-major layout, the FE
    element loop)."""
    import concurrent.futures
    import oracle
    np = w.np
    L = oracle.lib()
    T = len(os.sched_getaffinity(0))
    if w.config in CSR_CONFIGS and w.path.startswith("csr"):
        A = w.A
        rp, ci, v, x = (np.ascontiguousarray(a) for a in (A.row_ptr, A.col_idx, A.vals, A.x))
        n, weight = A.n_rows, rp.astype(np.int64) + np.arange(A.n_rows + 1)

        def part(r0, r1, y, s):
            L.oracle_csr_spmv(r1 - r0, rp[r0:r1 + 1], ci, v, x, 1.0, 0.0, None, y[r0:r1], s[r0:r1])
    elif w.config.startswith("pruned") and w.path.startswith("macko") and not macko_variant(w.path)[0]:
        P = w.P
        i8, bd = macko_variant(w.path)
        mrp, codes, mv = oracle.macko_encode(P.n_cols, P.row_ptr, P.col_idx, P.vals_f16, bdelta=bd)
        x = np.ascontiguousarray(P.x_f16)
        n, weight = P.n_rows, mrp.astype(np.int64)

        def part(r0, r1, y, s):
            L.oracle_macko_spmv(r1 - r0, P.n_cols, bd, mrp[r0:r1 + 1], codes, mv, x, 1.0, 0.0, None, y[r0:r1],
                                s[r0:r1])
    elif w.config.startswith("pruned") and w.path == "dense":
        P = w.P
        D = np.ascontiguousarray(P.dense_f16())
        x = np.ascontiguousarray(P.x_f16)
        n, weight = P.n_rows, np.arange(P.n_rows + 1, dtype=np.int64)

        def part(r0, r1, y, s):
            L.oracle_gemv_f16(r1 - r0, P.n_cols, D[r0:r1].reshape(-1), x, 1.0, 0.0, None, y[r0:r1], s[r0:r1])
    else:
        return None, 0
    cuts = np.searchsorted(weight, np.linspace(0, weight[-1], T + 1), side="left").clip(0, n)
    cuts[0], cuts[-1] = 0, n
    blocks = [(int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    y, s = np.empty(n), np.empty(n)
    pool = concurrent.futures.ThreadPoolExecutor(T)

    def run():
        list(pool.map(lambda b: part(b[0], b[1], y, s), blocks))
        return y, s
    return run, T


def cpu_baseline(w, fn, seconds, par_seconds=None):
    """The oracle as it stands (serial C, fp64, one core) on the full input,
    repeated for `seconds`; and, where the path has independent rows, the
    same function on row blocks in one thread per host core (the identical
    result is checked)."""
    per, reps, el = _repeat(fn, seconds)
    value, ms = _rate(w, per)
    out = {"value": value, "unit": "GFLOP/s", "cores": 1, "kind": "oracle", "ms_per_apply": ms,
           "sample": f"{reps} full applies of the same {w.workload} input ({el:.1f} s, {ms:.2f} ms each)"}
    run, T = rowpar_oracle(w)
    if run is not None:
        np = w.np
        ys, _ = fn()
        yp, _ = run()
        per_p, reps_p, el_p = _repeat(run, par_seconds if par_seconds is not None else seconds / 2)
        v2, ms2 = _rate(w, per_p)
        out["row_parallel"] = {"value": v2, "unit": "GFLOP/s", "cores": T, "kind": "oracle", "ms_per_apply": ms2,
                               "identical_to_serial": bool(np.array_equal(ys, yp)),
                               "sample": f"{reps_p} full applies on {T} threads, nonzero-balanced row blocks "
                                         f"({el_p:.1f} s)"}
    return out


def traffic_record(w):
    """HBM bytes per launch from a committed rocprofv3 counter record, if it
    was taken on the current kernel source; otherwise None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    recs = json.load(open(p))
    key = f"{w.config}/{w.path}"
    r = recs.get(key)
    if not r or r.get("source_sha") != source_sha(w.path):
        return None
    return int(r["bytes_per_launch"])


def _capture(torch, launches):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for L in launches:
            L()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for L in launches:
            L()
    return g.replay


def timed_rotate(w, steps, warmup, launches, graph=True):
    """Exactly `steps` applies back to back, step i on launches[i % R],
    between one pair of HIP events on the launch stream, with a device
    synchronisation on both sides.  With `graph`, one pass over the R
    launches is captured in a HIP graph (and the first steps % R launches
    in a second one) and replayed, so host launch cost does not throttle
    the GPU; the captured kernels are the same launches."""
    torch = w.torch
    R = len(launches)
    full_passes, rest = divmod(steps, R)
    if graph:
        run_all = _capture(torch, launches)
        run_rest = _capture(torch, launches[:rest]) if rest else None
    else:
        def run_all():
            for L in launches:
                L()

        def run_rest():
            for L in launches[:rest]:
                L()
    for _ in range(max(1, -(-warmup // R))):
        run_all()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(full_passes):
        run_all()
    if rest:
        run_rest()
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n = max(steps, 1)
    return {"ms_per_apply": a.elapsed_time(b) / n, "wall_ms_per_apply": wall * 1e3 / n, "applies": steps,
            "copies": R, "graph": graph}


def timed_flush(w, steps, warmup):
    """1 GiB write before every apply; each apply between its own event pair."""
    torch = w.torch
    buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        buf.zero_()
        w.launch()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        buf.zero_()
        a.record()
        w.launch()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return {"ms_per_apply": sum(ms) / len(ms), "median_ms": ms[len(ms) // 2], "applies": steps}


def launch_spread(w, launches, n=200):
    """Spread of single applies: n launches (rotating over the copies, so each
    finds its inputs out of cache), each between its own HIP event pair on
    the launch stream; p10 / median / p90 in microseconds.  A single launch
    also holds its own ramp and drain, which back-to-back launches overlap."""
    torch = w.torch
    for L in launches[: min(len(launches), 8)]:
        L()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        a.record()
        launches[i % len(launches)]()
        b.record()
    torch.cuda.synchronize()
    us = sorted(1e3 * a.elapsed_time(b) for a, b in ev)
    q = lambda f: round(us[min(n - 1, int(f * n))], 3)  # noqa: E731
    return {"p10": q(0.1), "p50": q(0.5), "p90": q(0.9), "launches": n}


def stream_reference(nbytes, steps=400):
    """The library's own reference streams (spmv_stream_copy, spmv_stream_read)
    at the workload's size, under the same rotation protocol and graph
    replay: what a plain streaming kernel of this size reaches on this GPU.
    copy: nbytes / 2 read + nbytes / 2 written; read: nbytes read."""
    import torch
    import sparse_matrix_vector_amd as S
    out = {}
    for kind in ("copy", "read"):
        elems = max(((nbytes // 2 if kind == "copy" else nbytes) // 4) // 4 * 4, 4)
        moved = 4 * elems * (2 if kind == "copy" else 1)
        R = max(2, -(-ROTATE_BYTES // moved))
        bufs = [(torch.ones(elems, dtype=torch.float32, device="cuda"),
                 torch.empty(elems if kind == "copy" else 4096, dtype=torch.float32, device="cuda"))
                for _ in range(R)]
        if kind == "copy":
            launches = [(lambda b=b: S.spmv_stream_copy(b[0], b[1])) for b in bufs]
        else:
            launches = [(lambda b=b: S.spmv_stream_read(b[0], b[1])) for b in bufs]

        class _W:
            pass
        w = _W()
        w.torch = torch
        r = timed_rotate(w, steps, 2 * R, launches, graph=True)
        out[kind] = {"bytes": moved, "copies": R, "us": round(r["ms_per_apply"] * 1e3, 3),
                     "gbs": round(moved / (r["ms_per_apply"] * 1e-3) / 1e9, 1),
                     "kernel": "k_stream_" + kind}
        del bufs, launches
    return out


def pmc_calibration_copies(nbytes=256 << 20, reps=3):
    """Plain device copies of a known size (nbytes read + nbytes written),
    launched outside any graph so that a rocprofv3 counter run records them:
    the ratio of bytes to the FETCH_SIZE / WRITE_SIZE the copy kernel shows
    calibrates those counters for the kernels of the same run."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] calibration copies: {reps} x {nbytes} bytes read and written")


def bench_pcg(args, emit=True):
    """One JSON line for Jacobi-PCG on the cantilever (see the module docstring);
    returns it (and prints it when `emit`)."""
    import numpy as np
    import torch
    import gen
    import sparse_matrix_vector_amd as S
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    dims = (120, 60, 30)
    m = gen.fe_cantilever(*dims)
    E, n = m.n_elem, m.n_dof
    op = (E, n, dev(m.edof.reshape(-1)), dev(m.rho), m.penalty, dev(m.Ke.reshape(-1)))
    f = dev(m.f)
    ws = torch.empty(S.fem_solver_workspace_size(n, 400), dtype=torch.uint8, device="cuda")
    u = torch.zeros(n, device="cuda")
    stream = torch.cuda.current_stream()
    # per iteration (fp64 vectors, int64 fixed-point accumulator; the one-reduction CG form): matvec
    # w = K z (edof 96 B + rho 4 B per element; z 8 B, accumulator read + write 16 B per DOF), w.z
    # (accumulator and z in: 16 B), step (accumulator, p, s, x, r, dinv in; p, s, x, r, z and the cleared
    # accumulator out: 96 B)
    nbytes = 100 * E + 136 * n
    flops = 2 * 576 * E + 13 * n
    S.fem_pcg_solve(*op, f, u, 0.0, max(args.warmup, 1), workspace=ws)
    u.zero_()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    it, _ = S.fem_pcg_solve(*op, f, u, 0.0, args.steps, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / max(it, 1)
    gbs = nbytes / (ms * 1e-3) / 1e9
    # a solve to rtol 1e-6 and the condition number, as the page reports them
    u.zero_()
    torch.cuda.synchronize()
    t0 = time.time()
    it6, rr6 = S.fem_pcg_solve(*op, f, u, 1e-6, 20000, workspace=ws)
    t_solve = time.time() - t0
    comp = float(m.f.astype(np.float64) @ u.cpu().numpy().astype(np.float64))
    v0 = dev(np.random.default_rng(5).standard_normal(n).astype(np.float32))
    t0 = time.time()
    lam = S.fem_lambda_max(*op, v0, 400, workspace=ws)
    mu, inner = S.fem_lambda_min(*op, v0, 4, 1e-6, 20000, workspace=ws)
    t_kappa = time.time() - t0
    par = None
    gpath = os.path.join(ROOT, "tests", "golden", "fe_cantilever.json")
    if not args.no_parity and os.path.exists(gpath):
        g = json.load(open(gpath))["cases"]["120x60x30"]
        par = {"ok": bool(abs(comp - g["compliance"]) <= 1e-4 * abs(g["compliance"])
                          and abs(it6 - g["pcg_iterations_rtol_1e-6"]) <= 0.05 * g["pcg_iterations_rtol_1e-6"]),
               "compliance": comp, "compliance_fp64_oracle": g["compliance"],
               "iterations": it6, "iterations_fp64_oracle": g["pcg_iterations_rtol_1e-6"],
               "source": "tests/golden/fe_cantilever.json (written by the fp64 oracle)"}
    line = {
        "metric": METRIC, "value": round(flops / (ms * 1e-3) / 1e9, 3), "unit": "GFLOP/s", "n_gpus": 1,
        "steps": it, "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32 operator, f64 vectors", "data": "synthetic (gen.fe_cantilever)",
        "config": {"workload": "fe_elasticity_cantilever_120x60x30_rho0.5", "path": "fem-pcg", "n_elem": E,
                   "n_dof": n, "step": "one Jacobi-PCG iteration", "protocol": "warm (the solver's own vectors)",
                   "timing": "HIP events on the launch stream around a fixed-count solve",
                   "algorithmic_bytes": nbytes, "flops": flops},
        "effective_gbs": round(gbs, 2), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": KERNEL["fem-pcg"]},
        "solve": {"rtol": 1e-6, "iterations": it6, "rel_residual": rr6, "seconds": round(t_solve, 4),
                  "compliance": comp},
        "kappa": {"lambda_max": lam[-1], "lambda_min": float(mu[-1]), "kappa": lam[-1] / mu[-1],
                  "page_kappa_216k": 1.3e6, "power_steps": 400, "inverse_steps": 4,
                  "inner_pcg_iterations": inner.tolist(), "seconds": round(t_kappa, 3)},
        "parity": par,
    }
    if args.cpu_seconds > 0:
        import oracle
        rp, ci, v = oracle.fe_assemble(m.edof, m.rho, m.Ke, n, m.penalty)
        v64 = np.asarray(v, np.float64)
        d = oracle.fe_diagonal(m.edof, m.rho, m.Ke, n, m.penalty)
        k, t0 = 0, time.time()
        while time.time() - t0 < args.cpu_seconds:
            oracle.pcg_jacobi(lambda x: oracle.csr_spmv_f64v(rp, ci, v64, x), d, m.f.astype(np.float64), rtol=0.0,
                              max_iter=10)
            k += 10
        el = time.time() - t0
        line["cpu_baseline"] = {"value": round(flops * k / el / 1e9, 3), "unit": "GFLOP/s", "cores": 1,
                                "kind": "oracle", "ms_per_step": round(1e3 * el / k, 3),
                                "sample": f"{k} fp64 PCG iterations on the assembled CSR (oracle matvec), same mesh"}
    if emit:
        print(json.dumps(line), flush=True)
    return line


def bench_spgemm(args, emit=True):
    """One JSON line for C = A * A (see the module docstring); returns it
    (and prints it when `emit`)."""
    import numpy as np
    import torch
    import gen
    import sparse_matrix_vector_amd as S
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    A = gen.powerlaw_csr() if args.config == "powerlaw" else gen.laplacian_2d(1000, with_x=False)
    workload = {"powerlaw": "powerlaw_916428_zipf1.9931", "laplacian": "laplacian_2d_1000x1000"}[args.config]
    arrs = [dev(A.row_ptr), dev(A.col_idx), dev(A.vals)]
    m = A.n_rows
    steps = max(1, min(args.steps, 20))

    def full():
        G = S.SpGEMM(m, A.n_cols, A.n_cols, *arrs, *arrs)
        out = G.compute()
        torch.cuda.synchronize()
        return G, out
    for _ in range(max(1, min(args.warmup, 3))):
        G, out = full()
        G.close()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        G, out = full()
        G.close()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    G, out = full()
    nnz_c, ip, groups = G.nnz, G.intermediate_products, G.group_rows
    # the accumulation phase alone, HIP events on the stream
    stream = torch.cuda.current_stream()
    k = max(10, min(args.steps, 100))
    G.compute(out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(k):
        G.compute(out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_acc = e0.elapsed_time(e1) / k
    # bytes the accumulation phase must move: A (row pointers, columns, values), the reached rows of B (their
    # row-pointer pairs, and columns and values once per intermediate product), and C written once
    nnz = A.nnz
    nbytes = 4 * (m + 1) + 8 * nnz + 8 * nnz + 8 * ip + 4 * (m + 1) + 8 * nnz_c
    flops = 2 * ip
    gbs_acc = nbytes / (ms_acc * 1e-3) / 1e9
    par = None
    if not args.no_parity:
        import oracle
        rp, ci, v = (t.cpu().numpy() for t in out)
        ipr = oracle.spgemm_ip(A.row_ptr, A.col_idx, A.row_ptr)
        g = np.digitize(ipr, [32, 512, 8192])
        rng = np.random.default_rng(11)
        rows = np.sort(np.concatenate([np.flatnonzero(g == q) if (g == q).sum() <= 300 else
                                       rng.choice(np.flatnonzero(g == q), 300, replace=False) for q in range(4)]))
        sub_rp = np.concatenate([[0], np.cumsum(A.row_ptr[rows + 1] - A.row_ptr[rows])]).astype(np.int32)
        sub_ci = np.concatenate([A.col_idx[A.row_ptr[r]:A.row_ptr[r + 1]] for r in rows])
        sub_v = np.concatenate([A.vals[A.row_ptr[r]:A.row_ptr[r + 1]] for r in rows])
        orp, oci, ov, osc = oracle.spgemm(A.n_cols, sub_rp, sub_ci, sub_v, A.row_ptr, A.col_idx, A.vals)
        ok, worst = True, 0.0
        for q, r in enumerate(rows):
            a, b = rp[r], rp[r + 1]
            oa, ob = orp[q], orp[q + 1]
            ok = ok and (b - a == ob - oa) and np.array_equal(ci[a:b], oci[oa:ob])
            if ok and ob > oa:
                e = np.abs(v[a:b].astype(np.float64) - ov[oa:ob])
                ok = ok and bool(np.all(e <= 1e-5 * osc[oa:ob]))
                worst = max(worst, float(np.max(e / np.maximum(osc[oa:ob], 1e-300))))
        par = {"ok": bool(ok and rp[-1] == nnz_c), "rows_checked": int(len(rows)), "tau": 1e-5,
               "max_err_over_scale": worst}
    G.close()
    line = {
        "metric": METRIC, "value": round(flops / (ms * 1e-3) / 1e9, 3), "unit": "GFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": max(1, min(args.warmup, 3)), "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded generators in gen/)",
        "config": {"workload": workload, "path": "spgemm", "product": "C = A * A", "n_rows": m, "nnz_a": nnz,
                   "intermediate_products": ip, "nnz_c": nnz_c, "ip_groups": groups,
                   "step": "one whole product (grouping, allocation, accumulation), host-synchronous",
                   "timing": "host clock around synchronous products; accumulation phase: HIP events",
                   "algorithmic_bytes_accumulation": nbytes, "flops": flops},
        "accumulation_phase": {"ms": round(ms_acc, 6), "gflops": round(flops / (ms_acc * 1e-3) / 1e9, 3),
                               "effective_gbs": round(gbs_acc, 2)},
        "effective_gbs": round(gbs_acc, 2), "pct_hbm_peak": round(100 * gbs_acc / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs_acc, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs_acc / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "accumulation phase (k_sg_g0_fill, k_sg_tb_fill, k_sg_g3_fill)"},
        "parity": par,
    }
    if args.cpu_seconds > 0:
        import oracle
        n_sample, t0 = 0, time.time()
        while time.time() - t0 < args.cpu_seconds and n_sample < m:
            r0, r1 = n_sample, min(m, n_sample + 50000)
            base = A.row_ptr[r0]
            sub_rp = (A.row_ptr[r0:r1 + 1] - base).astype(np.int32)
            oracle.spgemm(A.n_cols, sub_rp, A.col_idx[base:A.row_ptr[r1]], A.vals[base:A.row_ptr[r1]],
                          A.row_ptr, A.col_idx, A.vals)
            n_sample = r1
        el = time.time() - t0
        ip_s = int(oracle.spgemm_ip(A.row_ptr[:n_sample + 1], A.col_idx, A.row_ptr).sum())
        line["cpu_baseline"] = {"value": round(2 * ip_s / el / 1e9, 4), "unit": "GFLOP/s", "cores": 1,
                                "kind": "oracle", "sample": f"rows 0..{n_sample} of the same product "
                                f"({ip_s} intermediate products, {el:.1f} s)"}
    if emit:
        print(json.dumps(line), flush=True)
    return line


# The default run: the headline (Laplacian CSR) in full detail, then every
# other path the five configurations name, each with its own parity check,
# timing over the same number of steps, and a short oracle timing.  Targets
# are % of the 8 TB/s HBM peak over the algorithmic bytes.
HEADLINE = ("laplacian", "csr", 60.0, None)
SUITE = [
    ("laplacian", "ell", 60.0, "the Laplacian config's ELL path (width 5)"),
    ("tiny", "csr", None, "parity config: 311 KB, launch-bound, no % target"),
    ("tiny", "csr-scalar", None, "the pages' scalar CSR kernel on the parity config"),
    ("tiny", "csr-vector", None, "the pages' vector (lanes per row) CSR kernel on the parity config"),
    ("tiny", "ell", None, "ELL (W = 8) on the parity config"),
    ("powerlaw", "csr", 35.0, None),
    ("pruned50", "macko", 60.0, None),
    ("pruned70", "macko", 60.0, None),
    ("pruned90", "macko", 60.0, None),
    ("pruned50", "dense", None, "dense fp16 GEMV comparator of the MACKO configs (same W densified)"),
    ("fe", "fem", None, "fused FE matvec: parity config, atomic-bound, no % target"),
    ("fe", "fem-blocks", None, "element-block FE matvec: plan built once per copy, no atomics, fixed-order sums"),
    ("fe", "fem-3stage", None, "unfused three-stage comparator of the fused FE matvec"),
    ("fe", "fem-csr", None, "the assembled K (53.1M nonzeros, built on the GPU) through the binned CSR path"),
]


def measure(config, path, args, target=None, note=None, detail=False, cpu_seconds=0.0, par_seconds=None):
    """One path of one config: parity, timing over args.steps applies, the
    oracle on the host; returns the result record."""
    import torch
    w = Workload(config, path, args.copies if args.protocol == "rotate" else 1)
    ref_fn = w.oracle_call() if (not args.no_parity or cpu_seconds > 0) else None
    par = None
    if not args.no_parity:
        par = parity(w, ref_fn)
        log(f"[bench] parity {config}/{path} {par}")
    graph = not args.no_graph
    if args.protocol == "rotate":
        meas = timed_rotate(w, args.steps, args.warmup, w.launches, graph)
    elif args.protocol == "flush":
        meas = timed_flush(w, args.steps, args.warmup)
    else:
        meas = timed_rotate(w, args.steps, args.warmup, [w.launches[0]] * min(len(w.launches), 16), graph)
    ms = meas["ms_per_apply"]
    gbs = w.bytes / (ms * 1e-3) / 1e9
    pct = 100 * gbs / HBM_PEAK_GBS
    rec = {"workload": w.workload, "path": path, "kernel": getattr(w, "kernel", None) or KERNEL[path],
           "us_per_apply": round(ms * 1e3, 3), "algorithmic_bytes": w.bytes, "flops": w.flops,
           "gflops": round(w.flops / (ms * 1e-3) / 1e9, 3), "effective_gbs": round(gbs, 2),
           "pct_hbm_peak": round(pct, 2), "target_pct": target,
           "target_met": None if target is None else bool(pct >= target),
           "traffic": traffic_record(w), "parity": par, "shape": w.shape,
           "timing_ms": {k: (round(v, 6) if isinstance(v, float) else v) for k, v in meas.items()}}
    if note:
        rec["note"] = note
    if detail:
        warm = timed_rotate(w, args.steps, args.warmup, [w.launches[0]] * min(len(w.launches), 16), graph)
        rec["warm_timing_ms"] = {k: (round(v, 6) if isinstance(v, float) else v) for k, v in warm.items()}
        rec["single_launch_us"] = launch_spread(w, w.launches)
    if cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(w, ref_fn, cpu_seconds, par_seconds)
    log(f"[bench] {config}/{path}: {rec['us_per_apply']} us per apply, {rec['pct_hbm_peak']}% of peak")
    del w
    torch.cuda.empty_cache()
    return rec, meas


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default=None, choices=sorted(DEFAULT_PATH),
                    help="one configuration only (default: all of them, headline first)")
    ap.add_argument("--path", default=None, choices=sorted(KERNEL))
    ap.add_argument("--protocol", default="rotate", choices=["rotate", "flush", "warm"],
                    help="cold-cache protocol (see the module docstring)")
    ap.add_argument("--copies", type=int, default=None, help="input copies for the rotate protocol")
    ap.add_argument("--no-graph", action="store_true", help="launch from Python instead of a HIP graph")
    ap.add_argument("--pmc-calibrate", action="store_true",
                    help="first run known-size device copies (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time spent on the headline's serial oracle baseline (0 = skip every CPU timing)")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-copy-ref", action="store_true", help="skip the reference-stream bandwidth")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        raise SystemExit("--steps must be >= 1")

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(2)
    config = args.config or HEADLINE[0]
    path = args.path or (DEFAULT_PATH[config] if args.config else HEADLINE[1])
    if path == "spgemm":
        if config not in ("powerlaw", "laplacian"):
            raise SystemExit("the spgemm path runs on the powerlaw and laplacian configs")
        args.config = config
        bench_spgemm(args)
        return
    if config == "cantilever" or path == "fem-pcg":
        if config != "cantilever" or path != "fem-pcg":
            raise SystemExit("the fem-pcg path runs on the cantilever config only")
        bench_pcg(args)
        return
    if args.pmc_calibrate:
        pmc_calibration_copies()
    suite = args.config is None and args.path is None
    target = HEADLINE[2] if (config, path) == HEADLINE[:2] else None
    head, meas = measure(config, path, args, target=target, detail=True, cpu_seconds=args.cpu_seconds,
                         par_seconds=args.cpu_seconds / 2)
    ms = meas["ms_per_apply"]
    line = {
        "metric": METRIC,
        "value": head["gflops"],
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": meas["applies"],
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xf16->f32" if config.startswith("pruned") else "f32",
        "data": "synthetic (seeded generators in gen/)",
        "config": {"workload": head["workload"], "path": path, **head["shape"], "alpha": 1.0, "beta": 0.0,
                   "protocol": args.protocol, "copies": meas.get("copies", 1),
                   "timing": "HIP events on the launch stream around exactly `steps` applies"
                             + (", replayed from HIP graphs" if not args.no_graph and args.protocol != "flush"
                                else ""),
                   "algorithmic_bytes": head["algorithmic_bytes"], "flops": head["flops"]},
        "effective_gbs": head["effective_gbs"],
        "pct_hbm_peak": head["pct_hbm_peak"],
        "roofline": {"bound": "hbm", "achieved": head["effective_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head["effective_gbs"] / HBM_PEAK_GBS, 4), "traffic": head["traffic"],
                     "kernel": head["kernel"]},
        "timing_ms": head["timing_ms"],
        "warm_timing_ms": head["warm_timing_ms"],
        "single_launch_us": head["single_launch_us"],
        "parity": head["parity"],
        "target_pct": head["target_pct"],
        "target_met": head["target_met"],
    }
    if not args.no_copy_ref:
        line["stream_reference"] = stream_reference(head["algorithmic_bytes"])
    if "cpu_baseline" in head:
        line["cpu_baseline"] = head["cpu_baseline"]
    if suite:
        configs = {f"{config}/{path}": {k: v for k, v in head.items()
                                        if k not in ("warm_timing_ms", "single_launch_us", "cpu_baseline")}}
        for c, p, tgt, note in SUITE:
            rec, _ = measure(c, p, args, target=tgt, note=note, detail=True,
                             cpu_seconds=min(args.cpu_seconds, 1.5), par_seconds=min(args.cpu_seconds, 1.0))
            configs[f"{c}/{p}"] = rec
        line["configs"] = configs
        # the MACKO speed-up over the dense fp16 GEMV of the same 12288 x 12288
        # shape (one dense time serves every sparsity: the dense matrix is the same size)
        dense = configs.get("pruned50/dense")
        if dense:
            line["macko_speedup_vs_dense"] = {
                c: round(dense["us_per_apply"] / configs[f"{c}/macko"]["us_per_apply"], 3)
                for c in ("pruned50", "pruned70", "pruned90") if f"{c}/macko" in configs}
        met = [r["target_met"] for r in configs.values() if r["target_met"] is not None]
        line["targets_met"] = f"{sum(met)} of {len(met)}"
        # the adjacent rows built beside the hot path: HYB chosen by the CV
        # rule, Jacobi-PCG on the elasticity cantilever, hash SpGEMM (C = A * A)
        import copy
        nxt = {}
        rec, _ = measure("varlen", "auto", args, note="HYB chosen by the CV rule (CV 0.43, W = 5)", detail=True,
                         cpu_seconds=min(args.cpu_seconds, 1.5), par_seconds=min(args.cpu_seconds, 1.0))
        nxt["varlen/auto"] = rec
        drop = ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data")
        a = copy.copy(args)
        a.config, a.cpu_seconds = "cantilever", min(args.cpu_seconds, 1.5)
        nxt["cantilever/fem-pcg"] = {k: v for k, v in bench_pcg(a, emit=False).items() if k not in drop}
        a = copy.copy(args)
        a.config, a.steps, a.warmup = "powerlaw", min(args.steps, 20), min(args.warmup, 3)
        a.cpu_seconds = min(args.cpu_seconds, 1.5)
        nxt["powerlaw/spgemm"] = {k: v for k, v in bench_spgemm(a, emit=False).items() if k not in drop}
        line["next_rows"] = nxt
        line["parity_all_ok"] = (all((r["parity"] or {}).get("ok", False) for r in configs.values())
                                 and all((r.get("parity") or {}).get("ok", False) for r in nxt.values()))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
