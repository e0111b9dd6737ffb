#!/usr/bin/env python3
"""Benchmark of the MI355X SpMV library: y = alpha * A * x + beta * y.

Default run (N = 1): the 2-D 5-point Laplacian on a 1000 x 1000 grid
(1,000,000 rows, 4,996,000 nonzeros, fp32), CSR path with the row-grouping
planner (spmv_csr_apply, AUTO variant).  One step = a cache flush (a 1 GiB
write, larger than the 256 MB Infinity Cache plus the L2s, so the matrix
comes from HBM) followed by one apply; the apply alone is timed with HIP
events recorded on the stream it is launched on.  Inputs are resident in HBM
before the timed region.

Printed: ONE JSON line with the metric (GFLOP/s), effective GB/s over the
algorithmic bytes, the roofline of the dominant kernel against the 8 TB/s
HBM peak, and the CPU oracle timed on the host (serial fp64 C, bounded
sample).

Other workloads (parity-test configs, also used for profiles):
  --config tiny | laplacian | powerlaw | pruned50 | pruned70 | pruned90 | fe
  --path   csr | csr-binned | csr-vector | csr-scalar | ell | macko | dense | fem | fem-3stage
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

DEFAULT_PATH = {"tiny": "csr", "laplacian": "csr", "powerlaw": "csr", "pruned50": "macko",
                "pruned70": "macko", "pruned90": "macko", "fe": "fem"}

# kernel (as rocprofv3 names it) that dominates each path
KERNEL = {"csr": "k_csr_binned", "csr-binned": "k_csr_binned", "csr-vector": "k_csr_vector",
          "csr-scalar": "k_csr_scalar", "ell": "k_ell_apply", "macko": "k_macko_spmv",
          "dense": "k_gemv_f16", "fem": "k_fe_fused", "fem-3stage": "k_fe_elem"}

# source file of each path's kernels (for the traffic-record freshness check)
SOURCE = {"csr": "csr.hip", "csr-binned": "csr.hip", "csr-vector": "csr.hip", "csr-scalar": "csr.hip",
          "ell": "ell.hip", "macko": "macko.hip", "dense": "dense.hip", "fem": "fem.hip",
          "fem-3stage": "fem.hip"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(path_name):
    p = os.path.join(ROOT, "sparse_matrix_vector_amd", "csrc", SOURCE[path_name])
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


class Workload:
    """Inputs on the GPU plus a launch closure for one path."""

    def __init__(self, config, path):
        import numpy as np
        import torch
        import gen
        import sparse_matrix_vector_amd as S
        self.config, self.path = config, path
        self.np, self.torch, self.S = np, torch, S
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.alpha, self.beta = 1.0, 0.0
        t0 = time.time()
        if config in ("tiny", "laplacian", "powerlaw"):
            A = {"tiny": gen.tiny_csr, "laplacian": gen.laplacian_2d, "powerlaw": gen.powerlaw_csr}[config]()
            self.A = A
            self.n_out = A.n_rows
            self.workload = {"tiny": "tiny_csr_4096x4096_8perrow", "laplacian": "laplacian_2d_1000x1000",
                             "powerlaw": "powerlaw_916428_zipf1.9931"}[config]
            self.rp, self.ci, self.v, self.x = dev(A.row_ptr), dev(A.col_idx), dev(A.vals), dev(A.x)
            self.y = torch.zeros(A.n_rows, device="cuda")
            self.flops = 2 * A.nnz
            if path.startswith("csr"):
                var = {"csr": S.CSR_AUTO, "csr-binned": S.CSR_BINNED, "csr-vector": S.CSR_VECTOR,
                       "csr-scalar": S.CSR_SCALAR}[path]
                self.M = S.CSRMatrix(A.n_rows, A.n_cols, self.rp, self.ci, self.v, var)
                self.bytes = 8 * A.nnz + 4 * (A.n_rows + 1) + 4 * A.n_cols + 4 * A.n_rows
                self.launch = lambda: self.M.apply(self.x, self.y, self.alpha, self.beta)
                self.shape = {"n_rows": A.n_rows, "n_cols": A.n_cols, "nnz": A.nnz,
                              "plan": self.M.info()}
            elif path == "ell":
                import oracle
                W = oracle.row_stats(A.row_ptr)[0]
                self.W = W
                self.ec = torch.empty(A.n_rows * W, dtype=torch.int32, device="cuda")
                self.ev = torch.empty(A.n_rows * W, dtype=torch.float32, device="cuda")
                S.spmv_ell_from_csr(A.n_rows, A.n_cols, self.rp, self.ci, self.v, W, self.ec, self.ev)
                self.bytes = 8 * W * A.n_rows + 4 * A.n_cols + 4 * A.n_rows
                self.launch = lambda: S.spmv_ell_apply(A.n_rows, A.n_cols, W, self.ec, self.ev, self.alpha,
                                                       self.x, self.beta, self.y)
                self.shape = {"n_rows": A.n_rows, "nnz": A.nnz, "ell_width": W}
            else:
                raise SystemExit(f"path {path} does not apply to config {config}")
        elif config.startswith("pruned"):
            s = int(config[6:]) / 100.0
            P = gen.pruned_weight(s)
            self.P = P
            self.n_out = P.n_rows
            self.workload = f"pruned_weight_12288x12288_sparsity{int(s * 100)}"
            self.xh = dev(P.x_f16)
            self.y = torch.zeros(P.n_rows, device="cuda")
            if path == "macko":
                mrp, codes, mv = S.macko_encode(P.n_rows, P.n_cols, P.row_ptr, P.col_idx, P.vals_f16)
                self.enc = (mrp, codes, mv)
                self.mrp, self.codes, self.mv = dev(mrp), dev(codes), dev(mv)
                E = int(mrp[-1])
                self.bytes = 2 * E + E // 2 + 4 * (P.n_rows + 1) + 2 * P.n_cols + 4 * P.n_rows
                self.flops = 2 * P.nnz
                self.launch = lambda: S.macko_spmv(P.n_rows, P.n_cols, self.mrp, self.codes, self.mv,
                                                   self.alpha, self.xh, self.beta, self.y)
                self.shape = {"n_rows": P.n_rows, "n_cols": P.n_cols, "nnz": P.nnz, "entries": E}
            elif path == "dense":
                self.D = dev(P.dense_f16())
                self.bytes = 2 * P.n_rows * P.n_cols + 2 * P.n_cols + 4 * P.n_rows
                self.flops = 2 * P.n_rows * P.n_cols
                self.launch = lambda: S.dense_gemv_f16(P.n_rows, P.n_cols, self.D, self.xh, self.alpha,
                                                       self.beta, self.y)
                self.shape = {"m": P.n_rows, "n": P.n_cols}
            else:
                raise SystemExit(f"path {path} does not apply to config {config}")
        elif config == "fe":
            M = gen.fe_mesh()
            self.Mesh = M
            self.n_out = M.n_dof
            self.workload = "fe_hex8_cantilever_120x60x30"
            self.edof, self.rho, self.Ke = dev(M.edof.reshape(-1)), dev(M.rho), dev(M.Ke.reshape(-1))
            self.x = dev(M.x)
            self.y = torch.zeros(M.n_dof, device="cuda")
            self.bytes = 96 * M.n_elem + 4 * M.n_elem + 2304 + 8 * M.n_dof
            self.flops = 1176 * M.n_elem
            args = lambda: (M.n_elem, M.n_dof, self.edof, self.rho, M.penalty, self.Ke, self.alpha, self.x,
                            self.beta, self.y)
            if path == "fem":
                self.launch = lambda: S.fem_matvec_apply(*args())
            elif path == "fem-3stage":
                self.ws = torch.empty(S.fem_threestage_size(M.n_elem), dtype=torch.uint8, device="cuda")
                self.launch = lambda: S.fem_matvec_threestage(*args(), self.ws)
            else:
                raise SystemExit(f"path {path} does not apply to config {config}")
            self.shape = {"n_elem": M.n_elem, "n_dof": M.n_dof, "atomics": int((M.edof >= 0).sum())}
        else:
            raise SystemExit(f"unknown config {config}")
        torch.cuda.synchronize()
        log(f"[bench] setup {config}/{path}: {time.time() - t0:.1f}s")

    # -- oracle (the CPU baseline and the parity check) --
    def oracle_call(self):
        import oracle
        if self.config in ("tiny", "laplacian", "powerlaw"):
            A = self.A
            if self.path == "ell":
                ec, ev = oracle.ell_from_csr(A.row_ptr, A.col_idx, A.vals, self.W)
                return lambda: oracle.ell_spmv(A.n_rows, self.W, ec, ev, A.x)
            return lambda: oracle.csr_spmv(A.row_ptr, A.col_idx, A.vals, A.x)
        if self.config.startswith("pruned"):
            P = self.P
            if self.path == "macko":
                mrp, codes, mv = oracle.macko_encode(P.n_cols, P.row_ptr, P.col_idx, P.vals_f16)
                return lambda: oracle.macko_spmv(P.n_cols, mrp, codes, mv, P.x_f16)
            D = P.dense_f16()
            return lambda: oracle.gemv_f16(D, P.x_f16)
        M = self.Mesh
        return lambda: oracle.fe_matvec(M.edof, M.rho, M.Ke, M.x, M.n_dof)


def parity(w, ref_fn):
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
    return {"ok": ok, "tau": tau, "max_err_over_scale": worst}


def cpu_baseline(w, fn, seconds):
    """The oracle as it stands (serial C, fp64), repeated on the full input
    until `seconds` of CPU time have passed (at least one call)."""
    reps = 0
    t0 = time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / reps
    return {"value": round(w.flops / per / 1e9, 4), "unit": "GFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} full applies of the same {w.workload} input ({el:.1f} s, {per * 1e3:.2f} ms each)"}


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


def timed(w, steps, warmup, flush):
    torch = w.torch
    buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda") if flush else None
    for _ in range(warmup):
        if flush:
            buf.zero_()
        w.launch()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        if flush:
            buf.zero_()
        a.record()
        w.launch()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return {"mean_ms": sum(ms) / len(ms), "median_ms": ms[len(ms) // 2], "p10_ms": ms[len(ms) // 10],
            "p90_ms": ms[(9 * len(ms)) // 10], "wall_ms_per_step": wall * 1e3 / steps}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="laplacian", choices=sorted(DEFAULT_PATH))
    ap.add_argument("--path", default=None, choices=sorted(KERNEL))
    ap.add_argument("--no-flush", action="store_true", help="time with warm caches only")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time spent on the oracle baseline (0 = skip)")
    ap.add_argument("--no-parity", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(2)
    path = args.path or DEFAULT_PATH[args.config]
    w = Workload(args.config, path)

    par = None
    ref_fn = w.oracle_call() if (not args.no_parity or args.cpu_seconds > 0) else None
    if not args.no_parity:
        par = parity(w, ref_fn)
        log(f"[bench] parity {par}")

    cold = timed(w, args.steps, args.warmup, flush=not args.no_flush)
    warm = timed(w, args.steps, args.warmup, flush=False) if not args.no_flush else cold
    ms = cold["mean_ms"]
    gflops = w.flops / (ms * 1e-3) / 1e9
    gbs = w.bytes / (ms * 1e-3) / 1e9
    traffic = traffic_record(w)
    line = {
        "metric": METRIC,
        "value": round(gflops, 3),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xf16->f32" if args.config.startswith("pruned") else "f32",
        "data": "synthetic (seeded generators in gen/)",
        "config": {"workload": w.workload, "path": path, **w.shape, "alpha": w.alpha, "beta": w.beta,
                   "cache": "warm" if args.no_flush else "cold: 1 GiB write before each timed apply",
                   "timing": "HIP events around each apply on its launch stream",
                   "algorithmic_bytes": w.bytes, "flops": w.flops},
        "effective_gbs": round(gbs, 2),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": KERNEL[path]},
        "timing_ms": {k: round(v, 6) for k, v in cold.items()},
        "warm_timing_ms": {k: round(v, 6) for k, v in warm.items()},
        "parity": par,
    }
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(w, ref_fn, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
