"""Shared helpers of the GPU parity tests: device copies and the tolerance check.

Tolerance (applied element by element): |y_gpu - y_ref| <= tau * scale,
where y_ref and scale = |alpha| sum_k |a_ik x_k| + |beta y_in_i| come from the
fp64 oracle; tau = 1e-5 for fp32 values, 4e-3 for fp16 values with fp32
accumulation.
"""
from __future__ import annotations

import numpy as np

TAU_F32 = 1e-5
TAU_F16 = 4e-3


def dev(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t):
    return t.detach().cpu().numpy()


def assert_close(y_gpu, y_ref, scale, tau, what=""):
    y = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y - y_ref)
    bad = err > tau * scale
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {len(y)} outside tolerance; first at {i}: "
            f"gpu={y[i]!r} ref={y_ref[i]!r} scale={scale[i]!r} tau={tau}")
    nz = scale > 0
    return float(np.max(err[nz] / scale[nz])) if nz.any() else 0.0
