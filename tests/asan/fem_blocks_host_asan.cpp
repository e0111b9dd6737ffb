// Host-side memory check of the element-block FE planner (fem_blocks.cpp),
// built with AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_asan_host.py compiles and runs it).  Every output buffer of
// fem_blocks_plan_host is allocated with exactly the upper-bound size the
// header documents, so a write one element past it is caught.  Meshes:
// structured hexahedra with a clamped face (node units), the same with the
// DOFs relabelled (DOF units), a chain of elements sharing one node each
// (blocks with ~1,800 nodes), a node shared by every element (partial sums
// past the rank planes), repeated DOFs inside an element, fully constrained
// elements, no elements; and the error paths.  Light invariants are checked
// on every plan; the full structural checks are in test_fem_blocks_plan.py.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <numeric>
#include <random>
#include <vector>

#include "spmv.h"

static int failures = 0;
#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            ++failures;                                   \
            std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
            std::printf(__VA_ARGS__);                     \
            std::printf("\n");                            \
        }                                                 \
    } while (0)

struct Mesh {
    int32_t n_elem = 0, n_dof = 0;
    std::vector<int32_t> edof;
};

// nx x ny x nz hexahedra, node = ix + (nx+1)(iy + (ny+1) iz), DOF = 3 node + c;
// with `clamp` the ix = 0 nodes are constrained (-1) and the rest renumbered
static Mesh hex(int nx, int ny, int nz, bool clamp) {
    Mesh m;
    const int nnx = nx + 1, nny = ny + 1, nnz = nz + 1, nodes = nnx * nny * nnz;
    std::vector<int32_t> id(3 * nodes, -1);
    int32_t next = 0;
    for (int n = 0; n < nodes; ++n)
        for (int c = 0; c < 3; ++c)
            if (!(clamp && n % nnx == 0)) id[3 * n + c] = next++;
    m.n_dof = next;
    const int corner[8][3] = {{0, 0, 0}, {1, 0, 0}, {1, 1, 0}, {0, 1, 0}, {0, 0, 1}, {1, 0, 1}, {1, 1, 1}, {0, 1, 1}};
    for (int z = 0; z < nz; ++z)
        for (int y = 0; y < ny; ++y)
            for (int x = 0; x < nx; ++x) {
                for (int a = 0; a < 8; ++a) {
                    const int n = (x + corner[a][0]) + nnx * ((y + corner[a][1]) + nny * (z + corner[a][2]));
                    for (int c = 0; c < 3; ++c) m.edof.push_back(id[3 * n + c]);
                }
                ++m.n_elem;
            }
    return m;
}

// the plan into buffers of exactly the documented upper-bound sizes
static void plan(const char *name, const Mesh &m, int group, int want_group) {
    const int64_t E = m.n_elem, n = m.n_dof, ent = std::max<int64_t>(24 * E, 1);
    std::vector<int32_t> counts(9, -7), beo(E + 1), perm(std::max<int64_t>(E, 1)), bdo(E + 1), ldof(ent), ldst(ent);
    std::vector<uint32_t> crun(ent);
    std::vector<uint16_t> lidx(ent), lpos(ent);
    std::vector<int32_t> sptr(n + 1), sdof(std::max<int64_t>(n, 1)), scnt(std::max<int64_t>(n, 1));
    const spmv_status s = fem_blocks_plan_host(m.n_elem, m.n_dof, m.edof.data(), group, counts.data(), beo.data(),
                                               perm.data(), bdo.data(), ldof.data(), ldst.data(), crun.data(),
                                               lidx.data(), lpos.data(), sptr.data(), sdof.data(), scnt.data());
    CHECK(s == SPMV_OK, "%s: status %d (%s)", name, (int)s, spmv_last_error());
    if (s != SPMV_OK) return;
    const int nb = counts[0], sum_l = counts[1], ns = counts[2], n_slots = counts[3], pmax = counts[5];
    const int G = counts[6], U = 24 / G;
    CHECK(G == want_group, "%s: group %d, want %d", name, G, want_group);
    CHECK(nb >= 0 && nb <= E && sum_l >= 0 && sum_l <= ent && ns >= 0 && ns <= n, "%s: counts", name);
    // elements: a permutation, blocks of at most 256
    std::vector<int32_t> p(perm.begin(), perm.begin() + E);
    std::sort(p.begin(), p.end());
    for (int64_t k = 0; k < E; ++k) CHECK(p[k] == k, "%s: perm", name);
    CHECK(beo[0] == 0 && beo[nb] == E && bdo[0] == 0 && bdo[nb] == sum_l, "%s: offsets", name);
    for (int b = 0; b < nb; ++b) {
        CHECK(beo[b + 1] - beo[b] >= 1 && beo[b + 1] - beo[b] <= counts[8], "%s: block size", name);
        const int L = bdo[b + 1] - bdo[b];
        for (int64_t k = beo[b]; k < beo[b + 1]; ++k)
            for (int j = 0; j < U; ++j) {
                const uint16_t li = lidx[k * U + j], lp = lpos[k * U + j];
                CHECK((li == 0xFFFF) == (lp == 0xFFFF), "%s: constrained entries", name);
                if (li != 0xFFFF) {
                    const uint32_t r = crun[bdo[b] + li];
                    CHECK(li < L && lp >= (r & 0xFFFFu) && lp + G <= (r >> 16) && (int)(r >> 16) <= pmax,
                          "%s: entry out of its run", name);
                }
            }
    }
    for (int l = 0; l < sum_l; ++l) {
        CHECK(ldof[l] >= 0 && ldof[l] < n && ldof[l] % G == 0, "%s: ldof", name);
        CHECK(ldst[l] >= 0 ? ldst[l] == ldof[l] : ~ldst[l] + G <= n_slots, "%s: ldst", name);
    }
    for (int i = 0; i < ns; ++i) CHECK(sdof[i] >= 0 && sdof[i] < n && scnt[i] >= 0 && sptr[i] <= sptr[i + 1], "%s: shared", name);
    // NULL buffers: counts only
    std::vector<int32_t> c2(9, -7);
    CHECK(fem_blocks_plan_host(m.n_elem, m.n_dof, m.edof.data(), group, c2.data(), nullptr, nullptr, nullptr, nullptr,
                               nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == SPMV_OK &&
              std::equal(c2.begin(), c2.end(), counts.begin()),
          "%s: counts without buffers", name);
}

int main() {
    const Mesh cube = hex(13, 7, 5, true);
    plan("hex 13x7x5 auto", cube, 0, 3);
    plan("hex 13x7x5 dofs", cube, 1, 1);
    plan("hex 16x16x1 free", hex(16, 16, 1, false), 3, 3);
    plan("hex 40x20x10", hex(40, 20, 10, true), 0, 3);
    {   // DOFs relabelled at random: no node structure
        Mesh m = cube;
        std::vector<int32_t> q(m.n_dof);
        std::iota(q.begin(), q.end(), 0);
        std::shuffle(q.begin(), q.end(), std::mt19937(7));
        for (auto &d : m.edof)
            if (d >= 0) d = q[d];
        plan("hex relabelled", m, 0, 1);
        std::vector<int32_t> c(9);
        CHECK(fem_blocks_plan_host(m.n_elem, m.n_dof, m.edof.data(), 3, c.data(), nullptr, nullptr, nullptr, nullptr,
                                   nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) ==
                  SPMV_ERR_INVALID_VALUE,
              "group 3 on relabelled DOFs must fail");
    }
    {   // a chain: element e owns nodes 7e .. 7e + 7
        Mesh m;
        m.n_elem = 600;
        m.n_dof = 3 * (7 * m.n_elem + 1);
        for (int e = 0; e < m.n_elem; ++e)
            for (int a = 0; a < 8; ++a)
                for (int c = 0; c < 3; ++c) m.edof.push_back(3 * (7 * e + a) + c);
        plan("chain nodes", m, 0, 3);
        plan("chain dofs", m, 1, 1);
    }
    {   // one node in every element: past the rank planes
        Mesh m = hex(40, 24, 6, true);
        const int32_t hub = m.n_dof;
        m.n_dof += 3;
        for (int e = 0; e < m.n_elem; ++e)
            for (int c = 0; c < 3; ++c) m.edof[24 * e + c] = hub + c;
        plan("hub nodes", m, 3, 3);
        plan("hub dofs", m, 1, 1);
    }
    {   // repeated DOFs inside one element; fully constrained elements; no elements
        Mesh m;
        m.n_elem = 1;
        m.n_dof = 6;
        for (int a = 0; a < 24; ++a) m.edof.push_back(a % 6);
        plan("repeated", m, 1, 1);
        plan("repeated nodes", m, 0, 3);
        Mesh c;
        c.n_elem = 3;
        c.n_dof = 5;
        c.edof.assign(72, -1);
        plan("constrained", c, 0, 3);
        Mesh z;
        z.n_dof = 7;
        plan("no elements", z, 1, 1);
    }
    {   // error paths
        std::vector<int32_t> c(9), ed(24, 0);
        CHECK(fem_blocks_plan_host(-1, 5, ed.data(), 0, c.data(), nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, nullptr, nullptr, nullptr, nullptr) == SPMV_ERR_INVALID_VALUE,
              "negative n_elem");
        CHECK(fem_blocks_plan_host(1, 5, nullptr, 0, c.data(), nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, nullptr, nullptr, nullptr, nullptr) == SPMV_ERR_INVALID_VALUE,
              "NULL edof");
        CHECK(fem_blocks_plan_host(1, 5, ed.data(), 2, c.data(), nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, nullptr, nullptr, nullptr, nullptr) == SPMV_ERR_INVALID_VALUE,
              "group 2");
        CHECK(fem_blocks_plan_host(1, 5, ed.data(), 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, nullptr, nullptr, nullptr, nullptr) == SPMV_ERR_INVALID_VALUE,
              "NULL counts");
        CHECK(fem_blocks_plan_host(100000000, 5, ed.data(), 0, c.data(), nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == SPMV_ERR_OVERFLOW,
              "n_elem * 24 past int32");
    }
    std::printf("fem_blocks host check: %d failures\n", failures);
    return failures != 0;
}
