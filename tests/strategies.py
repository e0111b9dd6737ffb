"""Hypothesis strategies shared by the property tests: small random CSR
matrices with the awkward cases the kernels must handle -- no rows, empty
rows, unsorted and repeated columns within a row, and (optionally) one row of
8,192 to 12,000 entries, longer than the 16 chunks of 512 entries that one
workgroup takes, so it is split into chunk tasks.  Values and x are fp32."""
from __future__ import annotations

import numpy as np
from hypothesis import strategies as st

from gen import CSR


@st.composite
def csr_matrices(draw, max_rows=24, max_cols=64, long_row=True, sorted_distinct=False):
    n_rows = draw(st.integers(0, max_rows))
    n_cols = draw(st.integers(1, max_cols))
    seed = draw(st.integers(0, 2**32 - 1))
    rng = np.random.default_rng(seed)
    lens = [draw(st.integers(0, min(n_cols, 12) if sorted_distinct else 12)) for _ in range(n_rows)]
    if long_row and n_rows > 0 and draw(st.booleans()):
        r = draw(st.integers(0, n_rows - 1))
        lens[r] = min(n_cols, 20) if sorted_distinct else draw(st.integers(8192, 12000))
    rows = []
    for k in lens:
        if sorted_distinct:
            c = np.sort(rng.choice(n_cols, size=k, replace=False))
        else:
            c = rng.integers(0, n_cols, k)                 # repeats and any order
        rows.append(c.astype(np.int32))
    rp = np.zeros(n_rows + 1, np.int32)
    rp[1:] = np.cumsum(lens) if n_rows else rp[1:]
    ci = np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, np.int32)
    vals = rng.uniform(-2.0, 2.0, len(ci)).astype(np.float32)
    x = rng.uniform(-1.0, 1.0, n_cols).astype(np.float32)
    return CSR(n_rows, n_cols, rp, ci, vals, x, {"name": "hypothesis", "seed": seed})
