"""Property test of the element-block FE plan on random connectivities (no
GPU): for every drawn edof the plan passes the structural checks of
test_fem_blocks_plan (against brute force) and the two kernels emulated from
the plan alone give the oracle's product, in both unit sizes where the node
structure holds.  Connectivities: element corners drawn from a random node
pool (whole nodes, some wholly constrained), or single DOFs at random with
constrained entries and repeats; elements in a random order; up to ~1,200
elements, so that plans hold several blocks and shared nodes."""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import gen
import oracle
from helpers import TAU_F32, assert_close
from test_fem_blocks_plan import _check, _emulate

S = pytest.importorskip("sparse_matrix_vector_amd")


@st.composite
def connectivities(draw):
    seed = draw(st.integers(0, 2**32 - 1))
    rng = np.random.default_rng(seed)
    E = draw(st.sampled_from([0, 1, 2, 7, 64, 300, 600, 1200]))
    nodes = draw(st.integers(1, 400))
    nodewise = draw(st.booleans())
    if nodewise:
        # corners from a node pool; a node is either free (DOFs 3i..3i+2) or clamped
        clamped = rng.random(nodes) < 0.1
        corner = rng.integers(0, nodes, (E, 8))
        ed = 3 * corner[:, :, None] + np.arange(3)[None, None, :]
        ed = np.where(clamped[corner][:, :, None], -1, ed).reshape(E, 24)
        n_dof = 3 * nodes + draw(st.integers(0, 2))
    else:
        n_dof = draw(st.integers(1, 3 * nodes))
        ed = rng.integers(0, n_dof, (E, 24))
        ed = np.where(rng.random((E, 24)) < 0.1, -1, ed)
    rho = rng.uniform(0.05, 1.0, E).astype(np.float32)
    x = rng.uniform(-1, 1, n_dof).astype(np.float32)
    y_in = rng.uniform(-1, 1, n_dof).astype(np.float32)
    return ed.astype(np.int32).reshape(E, 24), n_dof, rho, x, y_in, nodewise


KE = gen.fe_mesh(1, 1, 1, clamp_x0=False, seed=5).Ke


@settings(max_examples=40, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(connectivities(), st.sampled_from([(1.0, 0.0), (0.5, -1.5)]))
def test_random_plans(c, ab):
    ed, n_dof, rho, x, y_in, nodewise = c
    alpha, beta = ab
    groups = (0, 1, 3) if nodewise else (0, 1)
    for group in groups:
        P = _check(ed, n_dof, group)
        if group == 0:
            assert P["group"] == (3 if nodewise else P["group"])
        y = _emulate(P, ed, n_dof, rho, KE, x, alpha, beta, y_in)
        yr, sc = oracle.fe_matvec(ed, rho, KE, x, n_dof, 3, alpha, beta, y_in)
        assert_close(y, yr, sc, TAU_F32, f"random plan G={P['group']}")


@pytest.mark.parametrize("nodewise", [True, False])
def test_random_plan_with_several_blocks(nodewise):
    """A fixed draw of 1,500 elements over 300 nodes (the strategy above may
    shrink towards small meshes): several blocks, most nodes shared."""
    rng = np.random.default_rng(42)
    E, nodes = 1500, 300
    if nodewise:
        corner = rng.integers(0, nodes, (E, 8))
        ed = (3 * corner[:, :, None] + np.arange(3)[None, None, :]).reshape(E, 24)
        n_dof = 3 * nodes
    else:
        n_dof = 3 * nodes
        ed = np.where(rng.random((E, 24)) < 0.1, -1, rng.integers(0, n_dof, (E, 24)))
    ed = ed.astype(np.int32)
    rho = rng.uniform(0.05, 1.0, E).astype(np.float32)
    x = rng.uniform(-1, 1, n_dof).astype(np.float32)
    for group in ((0, 1, 3) if nodewise else (0, 1)):
        P = _check(ed, n_dof, group)
        assert P["n_blocks"] >= 3
        y = _emulate(P, ed, n_dof, rho, KE, x, 1.0, 0.0, None)
        yr, sc = oracle.fe_matvec(ed, rho, KE, x, n_dof)
        assert_close(y, yr, sc, TAU_F32, f"random plan G={P['group']}")
