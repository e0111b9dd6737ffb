"""Seeded synthetic inputs for the SpMV library and its CPU oracle.

This package produces *inputs only*: sparsity patterns, values, vectors,
finite-element meshes and the shared element matrix.  It holds none of the
arithmetic of y = alpha*A*x + beta*y, none of the format encoders and none of
the kernels' planning logic, so both the HIP path and the oracle can consume
it without sharing code with each other.

Every generator is deterministic for a given seed (NumPy ``default_rng``) and
draws its random numbers in a fixed, documented order.  The shapes follow the
workloads the source pages measure:

* ``tiny_csr``       small uniform-degree CSR (8 per row),
* ``laplacian_2d``   2-D 5-point Laplacian on an N x N grid (the regular
                     FE/FD-style matrix of "Why SpMV needs CUDA optimisation",
                     section 2.1 table, stands in for the ecology2 matrix),
* ``powerlaw_csr``   a web-graph-like matrix with truncated-Zipf out-degrees
                     (the page-1 SpGEMM article's web-Google row, 916,428 rows,
                     ~5.1M nnz, max degree 4,334),
* ``pruned_weight``  a 12288 x 12288 fp16 weight with exactly k nonzeros per
                     row at uniform random positions (MACKO-SpMV page, section
                     3.1 table shape),
* ``fe_mesh``        a structured hex8 cantilever mesh with a shared seeded SPD
                     24x24 element matrix and SIMP densities (fused FE matvec
                     page, sections 2 and 3.2; 120x60x30 is its 216k case).
* ``fe_cantilever``  the same mesh with the linear-elasticity element matrix
                     of a unit hex8 (``hex8_elasticity_ke``), uniform density
                     and an end load: the system the page's Jacobi-PCG solves
                     and whose condition number it reports (sections 4.1, 6.1).
"""
from __future__ import annotations

from dataclasses import dataclass, field
import numpy as np

__all__ = [
    "CSR", "tiny_csr", "laplacian_2d", "powerlaw_csr", "powerlaw_pmf",
    "random_csr", "PrunedWeight", "pruned_weight", "FEMesh", "fe_mesh",
    "fe_ke_translation_free", "hex8_elasticity_ke", "fe_cantilever", "sine_mode", "SPARSITY_INDEX",
    "POWERLAW_ALPHA", "POWERLAW_KMAX",
]


@dataclass
class CSR:
    """A CSR matrix as plain host arrays (int32 indices, fp32 values)."""
    n_rows: int
    n_cols: int
    row_ptr: np.ndarray          # int32[n_rows + 1]
    col_idx: np.ndarray          # int32[nnz]
    vals: np.ndarray             # float32[nnz]
    x: np.ndarray                # float32[n_cols]
    meta: dict = field(default_factory=dict)

    @property
    def nnz(self) -> int:
        return int(self.row_ptr[-1])


def _rows_from_lengths(lens: np.ndarray) -> np.ndarray:
    rp = np.zeros(len(lens) + 1, dtype=np.int64)
    np.cumsum(lens, out=rp[1:])
    if rp[-1] >= 2**31:
        raise ValueError("nnz does not fit int32")
    return rp.astype(np.int32)


def _distinct_sorted_columns(rng, lens: np.ndarray, n_cols: int) -> np.ndarray:
    """Uniform random *distinct* columns per row, sorted ascending per row.

    Draw all columns with replacement (``rng.integers``), then repeatedly
    redraw every entry that duplicates an earlier one in the same row until no
    duplicates remain.  The final multiset per row is a uniform random k-subset
    (rejection of duplicates keeps uniformity), and the draw order is fixed, so
    the result is reproducible.
    """
    lens = np.asarray(lens, dtype=np.int64)
    if np.any(lens > n_cols):
        raise ValueError("row longer than the number of columns")
    nnz = int(lens.sum())
    row_of = np.repeat(np.arange(len(lens), dtype=np.int64), lens)
    cols = rng.integers(0, n_cols, size=nnz, dtype=np.int64)
    while True:
        key = row_of * n_cols + cols
        order = np.argsort(key, kind="stable")
        ks = key[order]
        dup_sorted = np.zeros(nnz, dtype=bool)
        dup_sorted[1:] = ks[1:] == ks[:-1]
        if not dup_sorted.any():
            break
        dup_idx = np.sort(order[dup_sorted])
        cols[dup_idx] = rng.integers(0, n_cols, size=len(dup_idx), dtype=np.int64)
    key = row_of * n_cols + cols
    cols = cols[np.argsort(key, kind="stable")]
    return cols.astype(np.int32)


# ---------------------------------------------------------------------------
# Config 0: tiny CSR, 4096 x 4096, exactly 8 distinct columns per row
# ---------------------------------------------------------------------------
def tiny_csr(n: int = 4096, per_row: int = 8, seed: int = 0) -> CSR:
    """Draw order: columns row by row (``rng.choice(n, per_row, replace=False)``,
    then sorted), then all values U[-1,1], then x U[-1,1]; fp32."""
    rng = np.random.default_rng(seed)
    cols = np.empty(n * per_row, dtype=np.int32)
    for i in range(n):
        cols[i * per_row:(i + 1) * per_row] = np.sort(rng.choice(n, per_row, replace=False))
    vals = rng.uniform(-1.0, 1.0, n * per_row).astype(np.float32)
    x = rng.uniform(-1.0, 1.0, n).astype(np.float32)
    rp = np.arange(0, n * per_row + 1, per_row, dtype=np.int32)
    return CSR(n, n, rp, cols, vals, x, {"name": "tiny", "seed": seed})


# ---------------------------------------------------------------------------
# Config 1: 2-D 5-point Laplacian on an N x N grid
# ---------------------------------------------------------------------------
def laplacian_2d(N: int = 1000, seed: int = 1, with_x: bool = True) -> CSR:
    """Row i = iy*N + ix; diagonal 4, the (up to) four grid neighbours -1,
    Dirichlet boundary (no ghost entries), columns ascending.
    nnz = 5 N^2 - 4 N.  x ~ U[-1,1] fp32 from ``default_rng(seed)``."""
    n = N * N
    iy, ix = np.divmod(np.arange(n, dtype=np.int64), N)
    # candidate columns in ascending order: up, left, diag, right, down
    cand = np.stack([
        np.where(iy > 0, np.arange(n) - N, -1),
        np.where(ix > 0, np.arange(n) - 1, -1),
        np.arange(n),
        np.where(ix < N - 1, np.arange(n) + 1, -1),
        np.where(iy < N - 1, np.arange(n) + N, -1),
    ], axis=1)
    valc = np.array([-1.0, -1.0, 4.0, -1.0, -1.0], dtype=np.float32)
    mask = cand >= 0
    lens = mask.sum(axis=1)
    cols = cand[mask].astype(np.int32)
    vals = np.broadcast_to(valc, cand.shape)[mask].astype(np.float32)
    rp = _rows_from_lengths(lens)
    if with_x:
        x = np.random.default_rng(seed).uniform(-1.0, 1.0, n).astype(np.float32)
    else:
        x = np.zeros(n, dtype=np.float32)
    return CSR(n, n, rp, cols, vals, x, {"name": f"laplacian{N}", "N": N, "seed": seed})


def sine_mode(N: int, p: int, q: int) -> tuple[np.ndarray, float]:
    """The (p, q) eigenvector of the N x N Dirichlet 5-point Laplacian in fp64,
    v(ix, iy) = sin(p pi (ix+1)/(N+1)) sin(q pi (iy+1)/(N+1)), with its
    eigenvalue 4 - 2cos(p pi/(N+1)) - 2cos(q pi/(N+1)).  Used only as a test
    input whose image under A is known in closed form."""
    t = np.arange(1, N + 1, dtype=np.float64) / (N + 1)
    vx = np.sin(p * np.pi * t)
    vy = np.sin(q * np.pi * t)
    v = np.outer(vy, vx).reshape(-1)        # row index iy*N + ix
    lam = 4.0 - 2.0 * np.cos(p * np.pi / (N + 1)) - 2.0 * np.cos(q * np.pi / (N + 1))
    return v, float(lam)


# ---------------------------------------------------------------------------
# Config 2: power-law graph
# ---------------------------------------------------------------------------
POWERLAW_ALPHA = 1.9931     # calibrated: E[k] = 5,105,039 / 916,428 on [1, 4334]
POWERLAW_KMAX = 4334


def powerlaw_pmf(alpha: float = POWERLAW_ALPHA, kmax: int = POWERLAW_KMAX) -> np.ndarray:
    k = np.arange(1, kmax + 1, dtype=np.float64)
    p = k ** (-alpha)
    return p / p.sum()


def powerlaw_csr(n: int = 916_428, alpha: float = POWERLAW_ALPHA,
                 kmax: int = POWERLAW_KMAX, seed: int = 2) -> CSR:
    """Out-degrees k_i ~ truncated Zipf, P(k) proportional to k^-alpha on
    [1, kmax] (``rng.choice`` with the pmf); then per row k_i distinct uniform
    columns (see ``_distinct_sorted_columns``), sorted; vals U[0,1) fp32;
    x U[-1,1] fp32.  Draw order: degrees, columns, vals, x."""
    rng = np.random.default_rng(seed)
    kmax = min(kmax, n)
    pmf = powerlaw_pmf(alpha, kmax)
    lens = rng.choice(np.arange(1, kmax + 1, dtype=np.int64), size=n, p=pmf)
    cols = _distinct_sorted_columns(rng, lens, n)
    vals = rng.random(len(cols), dtype=np.float32)
    x = rng.uniform(-1.0, 1.0, n).astype(np.float32)
    rp = _rows_from_lengths(lens)
    return CSR(n, n, rp, cols, vals, x, {"name": "powerlaw", "alpha": alpha, "seed": seed})


def random_csr(n_rows: int, n_cols: int, lens, seed: int, sorted_cols: bool = True,
               value_range=(-1.0, 1.0)) -> CSR:
    """General helper for edge-case tests: given row lengths, uniform distinct
    columns per row (sorted unless ``sorted_cols`` is False, in which case each
    row is randomly permuted), values and x uniform in ``value_range``."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    cols = _distinct_sorted_columns(rng, lens, n_cols) if len(lens) and lens.sum() else np.zeros(0, np.int32)
    rp = _rows_from_lengths(lens) if len(lens) else np.zeros(1, np.int32)
    if not sorted_cols:
        for i in range(n_rows):
            a, b = rp[i], rp[i + 1]
            cols[a:b] = rng.permutation(cols[a:b])
    vals = rng.uniform(value_range[0], value_range[1], len(cols)).astype(np.float32)
    x = rng.uniform(-1.0, 1.0, n_cols).astype(np.float32)
    return CSR(n_rows, n_cols, rp, cols, vals, x, {"name": "random", "seed": seed})


# ---------------------------------------------------------------------------
# Moderate row-length variation (the HYB regime of the CV rule)
# ---------------------------------------------------------------------------
def stencil_csr(n: int, offsets, seed: int) -> CSR:
    """Row i holds columns i + d for each offset d (those inside [0, n)),
    ascending; values and x uniform in [-1, 1].  A banded matrix whose
    entries fall in a few narrow bands far apart (edge-case tests)."""
    rng = np.random.default_rng(seed)
    offs = np.unique(np.asarray(offsets, dtype=np.int64))
    cand = np.arange(n, dtype=np.int64)[:, None] + offs[None, :]
    mask = (cand >= 0) & (cand < n)
    lens = mask.sum(axis=1)
    cols = cand[mask].astype(np.int32)
    rp = _rows_from_lengths(lens)
    vals = rng.uniform(-1.0, 1.0, len(cols)).astype(np.float32)
    x = rng.uniform(-1.0, 1.0, n).astype(np.float32)
    return CSR(n, n, rp, cols, vals, x, {"name": f"stencil{n}", "offsets": offs.tolist(), "seed": seed})


def varlen_banded(n: int = 1_000_000, lo: int = 2, hi: int = 10, band: int = 1000, seed: int = 6) -> CSR:
    """Square matrix whose row lengths are uniform on {lo..hi} (for 2..10:
    mean 6, CV = sqrt(80/12)/6 = 0.430, inside the HYB range 0.3..0.7), with
    distinct columns drawn uniformly from the band [i - band, i + band]
    clipped to [0, n) and sorted: a PDE-like locality with irregular rows.
    Values U[-1, 1), x U[-1, 1).  Draw order: lengths, columns, values, x."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, size=n).astype(np.int64)
    start = np.maximum(np.arange(n, dtype=np.int64) - band, 0)
    stop = np.minimum(np.arange(n, dtype=np.int64) + band + 1, n)
    width = stop - start
    lens = np.minimum(lens, width)
    # distinct offsets within each row's window, redrawn on duplicates
    nnz = int(lens.sum())
    row_of = np.repeat(np.arange(n, dtype=np.int64), lens)
    off = (rng.random(nnz) * width[row_of]).astype(np.int64)
    while True:
        key = row_of * (2 * band + 1) + off
        order = np.argsort(key, kind="stable")
        ks = key[order]
        dup = np.zeros(nnz, dtype=bool)
        dup[1:] = ks[1:] == ks[:-1]
        if not dup.any():
            break
        idx = np.sort(order[dup])
        off[idx] = (rng.random(len(idx)) * width[row_of[idx]]).astype(np.int64)
    key = row_of * (2 * band + 1) + off
    off = off[np.argsort(key, kind="stable")]
    cols = (start[row_of] + off).astype(np.int32)
    rp = _rows_from_lengths(lens)
    vals = rng.uniform(-1.0, 1.0, nnz).astype(np.float32)
    x = rng.uniform(-1.0, 1.0, n).astype(np.float32)
    return CSR(n, n, rp, cols, vals, x, {"name": f"varlen_banded_{n}_len{lo}-{hi}_band{band}", "seed": seed})


# ---------------------------------------------------------------------------
# Config 3: pruned fp16 weight matrix (MACKO input)
# ---------------------------------------------------------------------------
SPARSITY_INDEX = {0.3: 0, 0.5: 1, 0.7: 2, 0.9: 3}


@dataclass
class PrunedWeight:
    n_rows: int
    n_cols: int
    sparsity: float
    row_ptr: np.ndarray          # int32[R+1]
    col_idx: np.ndarray          # int32[nnz], strictly increasing per row
    vals_f16: np.ndarray         # uint16[nnz], fp16 bit patterns, never +-0
    x_f16: np.ndarray            # uint16[C], fp16 bit patterns

    @property
    def nnz(self) -> int:
        return int(self.row_ptr[-1])

    def dense_f16(self) -> np.ndarray:
        """The same weight densified (zeros off the pattern), fp16 bits, row-major."""
        W = np.zeros((self.n_rows, self.n_cols), dtype=np.uint16)
        rows = np.repeat(np.arange(self.n_rows), np.diff(self.row_ptr))
        W[rows, self.col_idx] = self.vals_f16
        return W


def pruned_weight(sparsity: float = 0.5, n_rows: int = 12288, n_cols: int | None = None,
                  seed: int = 3, std: float = 0.02) -> PrunedWeight:
    """W ~ N(0, std) in fp16 with exactly k = round((1-s) * n_cols) nonzeros per
    row at uniform random positions (``rng.choice(n_cols, k, replace=False)``,
    sorted).  Values that round to +-0 in fp16 are redrawn so every stored
    value is nonzero.  x ~ U[-1,1] in fp16.  Stream: ``default_rng([seed,
    SPARSITY_INDEX[s]])``; draw order: positions row by row, values, redraws,
    x."""
    n_cols = n_rows if n_cols is None else n_cols
    sidx = SPARSITY_INDEX.get(round(sparsity, 6), int(round(sparsity * 1000)))
    rng = np.random.default_rng([seed, sidx])
    k = int(round((1.0 - sparsity) * n_cols))
    cols = np.empty(n_rows * k, dtype=np.int32)
    for i in range(n_rows):
        cols[i * k:(i + 1) * k] = np.sort(rng.choice(n_cols, k, replace=False))
    v = (rng.standard_normal(n_rows * k) * std).astype(np.float16)
    while True:
        z = np.flatnonzero(v == 0)
        if len(z) == 0:
            break
        v[z] = (rng.standard_normal(len(z)) * std).astype(np.float16)
    x = rng.uniform(-1.0, 1.0, n_cols).astype(np.float16)
    rp = np.arange(0, n_rows * k + 1, k, dtype=np.int64)
    if rp[-1] >= 2**31:
        raise ValueError("nnz does not fit int32")
    return PrunedWeight(n_rows, n_cols, sparsity, rp.astype(np.int32), cols,
                        v.view(np.uint16), x.view(np.uint16))


# ---------------------------------------------------------------------------
# Config 4: structured hex8 mesh for the FE stiffness matvec
# ---------------------------------------------------------------------------
# Local node order of a hex8 element (offsets in x, y, z).
HEX8_LOCAL_NODES = np.array([
    (0, 0, 0), (1, 0, 0), (1, 1, 0), (0, 1, 0),
    (0, 0, 1), (1, 0, 1), (1, 1, 1), (0, 1, 1)], dtype=np.int64)


@dataclass
class FEMesh:
    nx: int
    ny: int
    nz: int
    n_elem: int
    n_dof: int                   # free (unconstrained) DOFs
    edof: np.ndarray             # int32[n_elem, 24]; -1 = constrained DOF
    rho: np.ndarray              # float32[n_elem]
    Ke: np.ndarray               # float32[24, 24], symmetric positive definite
    x: np.ndarray                # float32[n_dof]
    penalty: int = 3
    f: np.ndarray | None = None  # float32[n_dof] load (fe_cantilever only)


def _fe_structure(nx, ny, nz, clamp_x0):
    nnx, nny, nnz_ = nx + 1, ny + 1, nz + 1
    n_nodes = nnx * nny * nnz_
    ex, ey, ez = np.meshgrid(np.arange(nx), np.arange(ny), np.arange(nz), indexing="ij")
    # element id = ix + nx*(iy + ny*iz): flatten with ix fastest
    ex = ex.transpose(2, 1, 0).reshape(-1)
    ey = ey.transpose(2, 1, 0).reshape(-1)
    ez = ez.transpose(2, 1, 0).reshape(-1)
    nodes = ((ex[:, None] + HEX8_LOCAL_NODES[None, :, 0])
             + nnx * ((ey[:, None] + HEX8_LOCAL_NODES[None, :, 1])
                      + nny * (ez[:, None] + HEX8_LOCAL_NODES[None, :, 2])))
    full_dof = (3 * nodes[:, :, None] + np.arange(3)[None, None, :]).reshape(len(ex), 24)
    if clamp_x0:
        node_ix = np.arange(n_nodes) % nnx
        free = np.repeat(node_ix != 0, 3)
    else:
        free = np.ones(3 * n_nodes, dtype=bool)
    newid = np.full(3 * n_nodes, -1, dtype=np.int64)
    newid[free] = np.arange(int(free.sum()))
    edof = newid[full_dof].astype(np.int32)
    return edof, int(free.sum())


def fe_mesh(nx: int = 120, ny: int = 60, nz: int = 30, seed: int = 4,
            clamp_x0: bool = True, penalty: int = 3) -> FEMesh:
    """Hex8 mesh on an nx x ny x nz grid of unit cubes.

    Nodes are numbered ix + (nx+1)*(iy + (ny+1)*iz); global DOF = 3*node + comp
    (comp = x, y, z); local DOF of an element = 3*a + comp with the local node
    order of ``HEX8_LOCAL_NODES``.  With ``clamp_x0`` every DOF of the nodes on
    the ix = 0 face is constrained (a cantilever's fixed end) and the free DOFs
    are renumbered in increasing order; constrained entries of ``edof`` are -1.

    Random draws from ``default_rng(seed)`` in this order: G (24x24 standard
    normal) giving Ke = G G^T / 24 + I (symmetrised in fp64, stored fp32);
    rho ~ U[0.001, 1] fp32 per element; x ~ U[-1, 1] fp32 per free DOF.
    """
    rng = np.random.default_rng(seed)
    G = rng.standard_normal((24, 24))
    Ke = G @ G.T / 24.0 + np.eye(24)
    Ke = 0.5 * (Ke + Ke.T)
    edof, n_dof = _fe_structure(nx, ny, nz, clamp_x0)
    n_elem = nx * ny * nz
    rho = rng.uniform(0.001, 1.0, n_elem).astype(np.float32)
    x = rng.uniform(-1.0, 1.0, n_dof).astype(np.float32)
    return FEMesh(nx, ny, nz, n_elem, n_dof, edof, rho, Ke.astype(np.float32), x, penalty)


def fe_ke_translation_free(seed: int = 5) -> np.ndarray:
    """A seeded symmetric 24x24 element matrix whose null space contains the
    three rigid translations: Ke_t = Q (G G^T) Q with Q the orthogonal
    projector that removes the translation vectors (1 at every local DOF of
    one component).  A test input: any assembled operator built from it must
    map a global translation to zero."""
    rng = np.random.default_rng(seed)
    G = rng.standard_normal((24, 24))
    T = np.zeros((24, 3))
    for c in range(3):
        T[c::3, c] = 1.0 / np.sqrt(8.0)
    Q = np.eye(24) - T @ T.T
    K = Q @ (G @ G.T) @ Q
    return 0.5 * (K + K.T)


def hex8_elasticity_ke(E: float = 1.0, nu: float = 0.3) -> np.ndarray:
    """fp64 24x24 stiffness matrix of a unit-cube trilinear hex8 element in
    isotropic linear elasticity (Young's modulus E, Poisson ratio nu):
    Ke = sum over the 2 x 2 x 2 Gauss points (weight 1/8) of B^T D B, which
    is exact for this element.  Local DOF 3a + comp with the node order of
    ``HEX8_LOCAL_NODES``; strains in Voigt order (xx, yy, zz, xy, yz, zx) with
    engineering shears.  Symmetric, positive semidefinite with the six rigid
    motions as its null space."""
    lam = E * nu / ((1 + nu) * (1 - 2 * nu))
    mu = E / (2 * (1 + nu))
    D = np.zeros((6, 6))
    D[:3, :3] = lam
    D[np.arange(3), np.arange(3)] = lam + 2 * mu
    D[np.arange(3, 6), np.arange(3, 6)] = mu
    g = (0.5 - 0.5 / np.sqrt(3.0), 0.5 + 0.5 / np.sqrt(3.0))
    Ke = np.zeros((24, 24))
    for px in g:
        for py in g:
            for pz in g:
                B = np.zeros((6, 24))
                for a, (ax, ay, az) in enumerate(HEX8_LOCAL_NODES):
                    fx = px if ax else 1 - px
                    fy = py if ay else 1 - py
                    fz = pz if az else 1 - pz
                    sx, sy, sz = (1 if ax else -1), (1 if ay else -1), (1 if az else -1)
                    dx, dy, dz = sx * fy * fz, fx * sy * fz, fx * fy * sz
                    c = 3 * a
                    B[0, c] = dx
                    B[1, c + 1] = dy
                    B[2, c + 2] = dz
                    B[3, c], B[3, c + 1] = dy, dx
                    B[4, c + 1], B[4, c + 2] = dz, dy
                    B[5, c], B[5, c + 2] = dz, dx
                Ke += 0.125 * (B.T @ D @ B)
    return 0.5 * (Ke + Ke.T)


def fe_cantilever(nx: int = 120, ny: int = 60, nz: int = 30, rho: float = 0.5, E: float = 1.0,
                  nu: float = 0.3, penalty: int = 3) -> FEMesh:
    """The cantilever the fused-FE page solves: the hex8 mesh of ``fe_mesh``
    with the ix = 0 face clamped, the elasticity element matrix (fp32), the
    same density rho in every element, and a load of total -1 in z spread
    evenly over the nodes of the free end face ix = nx (``f``; ``x`` holds
    the same vector).  No random draws."""
    edof, n_dof = _fe_structure(nx, ny, nz, True)
    n_elem = nx * ny * nz
    nnx, nny, nnz_ = nx + 1, ny + 1, nz + 1
    node = np.arange(nnx * nny * nnz_)
    free = np.repeat(node % nnx != 0, 3)
    newid = np.full(3 * len(node), -1, dtype=np.int64)
    newid[free] = np.arange(int(free.sum()))
    end = node[node % nnx == nx]
    f = np.zeros(n_dof, np.float32)
    f[newid[3 * end + 2]] = np.float32(-1.0 / len(end))
    Ke = hex8_elasticity_ke(E, nu).astype(np.float32)
    return FEMesh(nx, ny, nz, n_elem, n_dof, edof, np.full(n_elem, rho, np.float32), Ke, f.copy(), penalty, f)
