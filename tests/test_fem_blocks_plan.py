"""The element-block plan of the FE matvec, on the host (no GPU): its
structure checked against brute force on small meshes under several
numberings, and the two-kernel apply emulated in NumPy from the plan alone
against the oracle's element loop.

Pins: every element in exactly one block of at most 512 elements (256 where
512 would overflow the LDS), the chosen size's LDS need within 64 KB; each element's 16-bit
local indices map back to its edof; a DOF is private exactly when all its
elements lie in one block (set of blocks per DOF by brute force), and then
its destination is the DOF itself; the private DOFs and the second kernel's
DOFs partition all DOFs (untouched DOFs go to the second kernel); each
second-kernel DOF owns one slot per block that touches it, numbered in
increasing block order, and each of those blocks writes its own slot; the
product positions of a block fill its runs, each local unit's run holds
exactly its entries in (element, entry) order and is followed by a padding
word when its length is even; and the product
rebuilt from these arrays equals the oracle within the FE tolerance.
"""
import numpy as np
import pytest

import gen
import oracle
from helpers import TAU_F32, assert_close

S = pytest.importorskip("sparse_matrix_vector_amd")

NONE = 0xFFFF


def _renumber(M, how, seed=3):
    rng = np.random.default_rng(seed)
    ed = M.edof.reshape(M.n_elem, 24)
    if how == "shuffled":
        return ed[rng.permutation(M.n_elem)].copy()
    if how == "relabelled":
        q = rng.permutation(M.n_dof)
        return np.where(ed >= 0, q[np.maximum(ed, 0)], -1).astype(np.int32)
    return ed.copy()


def _check(ed, n_dof, group=0):
    E = ed.shape[0]
    P = S.fem_blocks_plan_host(E, n_dof, ed, group)
    G = P["group"]
    assert group in (0, G)
    U = 24 // G
    nb = P["n_blocks"]
    beo, perm, bdo = P["blk_elem_off"], P["perm"], P["blk_dof_off"]
    g, dst = P["ldof"].astype(np.int64), P["ldst"].astype(np.int64)
    starts, ends = (P["crun"] & 0xFFFF).astype(np.int64), (P["crun"] >> 16).astype(np.int64)
    # unit of each element entry (the entry's first DOF / G), -1 if constrained
    first = ed.reshape(E, U, G)[:, :, 0].astype(np.int64)
    unit = np.where((first >= 0) & (first < n_dof), first // G, -1)
    if G == 3:   # every corner a whole node or wholly constrained
        ok = (first >= 0) & (first < n_dof)
        e3 = ed.reshape(E, 8, 3).astype(np.int64)
        assert np.all(np.where(ok, (first % 3 == 0) & (e3[:, :, 1] == first + 1) & (e3[:, :, 2] == first + 2),
                               (e3[:, :, 1] < 0) | (e3[:, :, 1] >= n_dof)))
    # blocks: a permutation of the elements, at most 256 each
    assert P["block"] in (256, 512)
    assert beo[0] == 0 and beo[-1] == E and np.all(np.diff(beo) >= 1) and np.all(np.diff(beo) <= P["block"])
    # the chosen size fits the workgroup's LDS; 256 is taken only when 512 would not
    assert 4 * (G * max(P["Lmax"], 1) + max(P["Pmax"], 1)) <= 65536
    assert np.array_equal(np.sort(perm), np.arange(E))
    block_of = np.empty(E, np.int64)
    for b in range(nb):
        block_of[perm[beo[b]:beo[b + 1]]] = b
    # local indices map back to the units; local unit lists sorted and
    # distinct; product positions: runs in local-unit order, (element, entry)
    # order inside, G products per entry
    L = P["lidx"].reshape(E, U).astype(np.int64)
    Q = P["lpos"].reshape(E, U).astype(np.int64)
    up = unit[perm]
    lmax = pmax = 0
    for b in range(nb):
        loc = g[bdo[b]:bdo[b + 1]]
        assert np.all(np.diff(loc) > 0) and np.all(loc % G == 0)
        rows = slice(beo[b], beo[b + 1])
        valid = up[rows] >= 0
        assert np.all((L[rows] == NONE) == ~valid) and np.all((Q[rows] == NONE) == ~valid)
        assert np.array_equal(loc[L[rows][valid]] // G, up[rows][valid])
        li, q = L[rows][valid], Q[rows][valid]   # flattened in (element, entry) order
        # runs in local-unit order, each followed by one padding word when its
        # length is even, starting at 0; each holds its unit's entries
        s_b, e_b = starts[bdo[b]:bdo[b + 1]], ends[bdo[b]:bdo[b + 1]]
        size = 0
        for l in range(len(loc)):
            assert s_b[l] == size
            assert np.array_equal(q[li == l], np.arange(s_b[l], e_b[l], G)), (b, l)
            size = e_b[l] + (1 if (e_b[l] - s_b[l]) % 2 == 0 else 0)
        assert G * len(li) == (e_b - s_b).sum()
        lmax, pmax = max(lmax, len(loc)), max(pmax, size)
    assert P["Lmax"] == lmax and P["Pmax"] == pmax
    # private units against the set of blocks per unit
    n_units = (n_dof + G - 1) // G
    nblk = np.zeros(n_units, np.int64)
    inc = np.repeat(np.arange(E), U)[unit.reshape(-1) >= 0]
    us = unit.reshape(-1)[unit.reshape(-1) >= 0]
    pairs = np.unique(np.stack([us, block_of[inc]], 1), axis=0)
    np.add.at(nblk, pairs[:, 0], 1)
    private = dst >= 0
    assert np.array_equal(dst[private], g[private])
    assert np.array_equal(nblk[g[private] // G], np.ones(private.sum(), np.int64))
    assert np.all(nblk[g[~private] // G] != 1)
    # second-kernel units: the complement of the private ones, each with its
    # block count; the slots of each, G per block in block order (rank planes
    # first, the overflow list after), written by exactly those blocks
    priv_set = np.zeros(n_units, bool)
    priv_set[g[private] // G] = True
    assert np.array_equal(P["shr_dof"], G * np.flatnonzero(~priv_set))
    assert np.array_equal(P["shr_cnt"], nblk[P["shr_dof"] // G])
    ns, planes, sp = len(P["shr_dof"]), P["planes"], P["shr_ptr"]
    assert planes == min(8, int(P["shr_cnt"].max(initial=0)))
    assert np.array_equal(np.diff(sp), G * np.maximum(P["shr_cnt"] - planes, 0))
    assert P["n_slots"] == planes * ns * G + sp[-1]
    written = np.sort(~dst[~private])
    for i, d in enumerate(P["shr_dof"]):
        mine = ~dst[(g == d) & ~private]   # in block order
        want = [G * (r * ns + i) if r < planes else planes * ns * G + sp[i] + G * (r - planes)
                for r in range(P["shr_cnt"][i])]
        assert np.array_equal(mine, want), d
    assert len(np.unique(written)) == len(written)
    return P


def _emulate(P, ed, n_dof, rho, Ke, x, alpha, beta, y_in, penalty=3):
    """The two kernels in NumPy (fp64), from the plan's arrays only."""
    G = P["group"]
    U = 24 // G
    beo, perm, bdo = P["blk_elem_off"], P["perm"], P["blk_dof_off"]
    g, dst = P["ldof"].astype(np.int64), P["ldst"].astype(np.int64)
    starts, ends = (P["crun"] & 0xFFFF).astype(np.int64), (P["crun"] >> 16).astype(np.int64)
    slots = np.zeros(P["n_slots"])
    y = np.array(y_in, np.float64) if beta != 0 else np.zeros(n_dof)
    Kd = Ke.astype(np.float64).reshape(24, 24)
    L = P["lidx"].reshape(-1, U).astype(np.int64)
    Q = P["lpos"].reshape(-1, U).astype(np.int64)
    comp = np.arange(G)
    for b in range(P["n_blocks"]):
        loc = g[bdo[b]:bdo[b + 1]]
        xs = x[(loc[:, None] + comp).reshape(-1)].astype(np.float64)   # unit l, component c at G l + c
        pb = np.full(max(P["Pmax"], 1), np.nan)
        for k in range(beo[b], beo[b + 1]):
            on = np.repeat(L[k] != NONE, G)
            idx = (G * np.where(L[k] != NONE, L[k], 0)[:, None] + comp).reshape(-1)
            u = np.where(on, xs[idx] if len(xs) else 0.0, 0.0)
            f = alpha * float(rho[perm[k]]) ** penalty * (Kd @ u)
            pos = (np.where(L[k] != NONE, Q[k], 0)[:, None] + comp).reshape(-1)
            pb[pos[on]] = f[on]
        for l in range(len(loc)):
            j = bdo[b] + l
            v = np.zeros(G)
            for q in range(starts[j], ends[j], G):
                v += pb[q:q + G]
            for c in range(G):
                if dst[j] >= 0:
                    y[dst[j] + c] = (beta * y[dst[j] + c] if beta != 0 else 0.0) + v[c]
                else:
                    slots[~dst[j] + c] = v[c]
    ns, planes = len(P["shr_dof"]), P["planes"]
    for i, d in enumerate(P["shr_dof"]):
        s = np.zeros(G)
        for r in range(P["shr_cnt"][i]):
            at = G * (r * ns + i) if r < planes else planes * ns * G + P["shr_ptr"][i] + G * (r - planes)
            s += slots[at:at + G]
        for c in range(G):
            if d + c < n_dof:
                y[d + c] = (beta * y[d + c] if beta != 0 else 0.0) + s[c]
    return y


@pytest.mark.parametrize("how", ["identity", "shuffled", "relabelled"])
@pytest.mark.parametrize("dims,clamp", [((13, 7, 5), True), ((16, 16, 1), False), ((1, 1, 1), False)])
def test_plan_structure_and_product(dims, clamp, how):
    M = gen.fe_mesh(*dims, clamp_x0=clamp, seed=8)
    ed = _renumber(M, how)
    # the node plan applies unless the DOFs were relabelled; the DOF plan always
    groups = [0, 1] + ([3] if how != "relabelled" else [])
    y_in = np.random.default_rng(4).uniform(-1, 1, M.n_dof).astype(np.float32)
    for group in groups:
        P = _check(ed, M.n_dof, group)
        assert P["group"] == (group or (1 if how == "relabelled" else 3))
        for alpha, beta in [(1.0, 0.0), (0.5, -2.0)]:
            y = _emulate(P, ed, M.n_dof, M.rho, M.Ke, M.x, alpha, beta, y_in, M.penalty)
            yr, sc = oracle.fe_matvec(ed, M.rho, M.Ke, M.x, M.n_dof, M.penalty, alpha, beta, y_in)
            assert_close(y, yr, sc, TAU_F32, f"emulated blocks {dims} {how} G={P['group']} {alpha} {beta}")
    if how == "relabelled":
        with pytest.raises(S.SpmvError):
            S.fem_blocks_plan_host(ed.shape[0], M.n_dof, ed, 3)


def test_plan_node_groups_need_whole_nodes():
    """One constrained component on an otherwise free node, nodes whose DOFs
    do not start at a multiple of 3, or a node's components swapped in its
    elements: the automatic choice falls back to single DOFs, and forcing
    G = 3 fails."""
    M = gen.fe_mesh(5, 3, 2, clamp_x0=False, seed=1)
    base = M.edof.reshape(M.n_elem, 24).copy()
    cases = []
    e = base.copy(); e[e == 7] = -1; cases.append((e, M.n_dof))                 # a roller
    cases.append((np.where(base >= 0, base + 1, -1).astype(np.int32), M.n_dof + 1))  # shifted by one
    e = base.copy(); e[:, 3:6] = e[:, [4, 3, 5]]; cases.append((e, M.n_dof))     # components swapped
    for e, n in cases:
        P = _check(e, n, 0)
        assert P["group"] == 1
        with pytest.raises(S.SpmvError):
            S.fem_blocks_plan_host(e.shape[0], n, e, 3)
        x = np.random.default_rng(2).uniform(-1, 1, n).astype(np.float32)
        y = _emulate(P, e, n, M.rho, M.Ke, x, 1.0, 0.0, None, M.penalty)
        yr, sc = oracle.fe_matvec(e, M.rho, M.Ke, x, n, M.penalty)
        assert_close(y, yr, sc, TAU_F32, "fallback to single DOFs")
    # n_dof not a multiple of 3: the last unit is cut, its missing DOFs unused
    P = _check(base, M.n_dof + 2, 3)
    y = _emulate(P, base, M.n_dof + 2, M.rho, M.Ke, np.concatenate([M.x, [5.0, 6.0]]).astype(np.float32),
                 1.0, 0.0, None, M.penalty)
    yr, sc = oracle.fe_matvec(base, M.rho, M.Ke, np.concatenate([M.x, [5.0, 6.0]]).astype(np.float32),
                              M.n_dof + 2, M.penalty)
    assert_close(y, yr, sc, TAU_F32, "cut last node")


def _hub_mesh():
    """A 40 x 24 x 6 mesh whose elements all list one extra node (DOFs n..n+2)
    in place of their first corner: that node lies in every block, so its
    partial sums run past the rank planes into the overflow list."""
    M = gen.fe_mesh(40, 24, 6, clamp_x0=True, seed=6)
    ed = M.edof.reshape(M.n_elem, 24).copy()
    n = M.n_dof + 3
    ed[:, 0:3] = [M.n_dof, M.n_dof + 1, M.n_dof + 2]
    x = np.random.default_rng(9).uniform(-1, 1, n).astype(np.float32)
    return M, ed, n, x


@pytest.mark.parametrize("group", [1, 3])
def test_plan_partial_sums_past_the_rank_planes(group):
    M, ed, n, x = _hub_mesh()
    P = _check(ed, n, group)
    assert P["planes"] == 8 and P["shr_cnt"].max() == P["n_blocks"] > 8 and P["shr_ptr"][-1] > 0
    y_in = np.random.default_rng(4).uniform(-1, 1, n).astype(np.float32)
    y = _emulate(P, ed, n, M.rho, M.Ke, x, 0.5, 2.0, y_in, M.penalty)
    yr, sc = oracle.fe_matvec(ed, M.rho, M.Ke, x, n, M.penalty, 0.5, 2.0, y_in)
    assert_close(y, yr, sc, TAU_F32, f"hub node, G={group}")


def _chain_mesh(E=600):
    """Elements in a chain, each sharing one node with the next: a block of
    256 holds ~1,800 nodes (~5,400 DOFs), more local units than a lane's
    registers stage, so the apply's remainder loops run."""
    M = gen.fe_mesh(1, 1, 1, clamp_x0=False, seed=5)
    nodes = 7 * np.arange(E)[:, None] + np.arange(8)[None, :]
    ed = (3 * nodes[:, :, None] + np.arange(3)[None, None, :]).reshape(E, 24).astype(np.int32)
    n = 3 * (7 * E + 1)
    rng = np.random.default_rng(11)
    rho = rng.uniform(0.1, 1.0, E).astype(np.float32)
    x = rng.uniform(-1, 1, n).astype(np.float32)
    return M.Ke, ed, n, rho, x


@pytest.mark.parametrize("group", [1, 3])
def test_plan_long_blocks(group):
    Ke, ed, n, rho, x = _chain_mesh()
    P = _check(ed, n, group)
    assert P["Lmax"] > (1792 if group == 1 else 768)
    y = _emulate(P, ed, n, rho, Ke, x, 1.0, 0.0, None)
    yr, sc = oracle.fe_matvec(ed, rho, Ke, x, n)
    assert_close(y, yr, sc, TAU_F32, f"chain, G={group}")


def test_plan_blocks_are_compact_on_the_cantilever_slice():
    """A 40 x 20 x 10 slice: the breadth-first blocks keep about half of the
    DOFs private (a regression guard on the partition, not a correctness pin)."""
    M = gen.fe_mesh(40, 20, 10, seed=2)
    P = _check(M.edof.reshape(M.n_elem, 24), M.n_dof)
    frac = 1.0 - 3 * len(P["shr_dof"]) / M.n_dof
    print(f"[blocks] 40x20x10: {P['n_blocks']} blocks of <= {P['block']}, Lmax {P['Lmax']}, private {frac:.2f}")
    assert frac > 0.4 and P["block"] == 512


def test_plan_edge_cases():
    # no elements: every DOF goes to the second kernel with no slots
    P = S.fem_blocks_plan_host(0, 5, np.zeros(0, np.int32), 1)
    assert P["n_blocks"] == 0 and list(P["shr_dof"]) == [0, 1, 2, 3, 4] and list(P["shr_cnt"]) == [0] * 5
    assert P["planes"] == 0 and P["n_slots"] == 0 and list(P["shr_ptr"]) == [0] * 6
    P = S.fem_blocks_plan_host(0, 5, np.zeros(0, np.int32))
    assert P["group"] == 3 and list(P["shr_dof"]) == [0, 3] and list(P["shr_cnt"]) == [0, 0]
    # one element, all DOFs constrained: a block with no local units
    for group in (0, 1, 3):
        P = S.fem_blocks_plan_host(1, 3, np.full(24, -1, np.int32), group)
        assert P["n_blocks"] == 1 and len(P["ldof"]) == 0 and np.all(P["lidx"] == NONE)
        assert np.all(P["lpos"] == NONE) and P["Lmax"] == 0 and P["Pmax"] == 0 and P["n_slots"] == 0
    # repeated DOFs inside one element share one local index
    ed = np.arange(24, dtype=np.int32) % 6
    P = S.fem_blocks_plan_host(1, 6, ed, 1)
    assert P["group"] == 1 and len(P["ldof"]) == 6
    assert np.array_equal(P["lidx"].astype(np.int64), ed.astype(np.int64))
    # ... and each local DOF's run holds its four entries in DOF order, each
    # run of four followed by a padding word
    assert list(P["crun"] & 0xFFFF) == [0, 5, 10, 15, 20, 25] and list(P["crun"] >> 16) == [4, 9, 14, 19, 24, 29]
    assert P["Pmax"] == 30
    assert np.array_equal(P["lpos"].astype(np.int64), 5 * (ed % 6) + np.arange(24) // 6)
    # the same with whole nodes (the automatic choice): two nodes, each on
    # four corners
    P = S.fem_blocks_plan_host(1, 6, ed)
    assert P["group"] == 3 and list(P["ldof"]) == [0, 3]
    assert list(P["crun"] & 0xFFFF) == [0, 13] and list(P["crun"] >> 16) == [12, 25] and P["Pmax"] == 26
    assert np.array_equal(P["lidx"].astype(np.int64), np.arange(8) % 2)
    assert np.array_equal(P["lpos"].astype(np.int64), 13 * (np.arange(8) % 2) + 3 * (np.arange(8) // 2))
    # bad group
    with pytest.raises(S.SpmvError):
        S.fem_blocks_plan_host(1, 6, ed, 2)
