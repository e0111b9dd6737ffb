// Element blocks of the finite-element matvec: the host planner.
//
// "Fused GPU SpMV kernel optimisation", section 2.2: the fused matvec keeps
// every element's gather, product and scatter on chip, and its cost is the
// scatter (atomic adds) and the index traffic.  A plan built once from the
// mesh connectivity (edof) takes most of that off the apply:
//   - the elements are cut into compact blocks of at most 512 elements (256
//     when a 512-element block would not fit a workgroup's LDS)
//     (greedy breadth-first growth over elements that share a DOF, from the
//     lowest-numbered element not yet taken), one workgroup each;
//   - the plan works on units of G DOFs: a node's three DOFs (G = 3) when
//     the numbering gives every node the DOFs 3i, 3i+1, 3i+2 (a third of the
//     index data), single DOFs (G = 1) for any other numbering;
//   - each block numbers the units its elements touch (its local units, in
//     increasing global order) and stores every element's 24 / G units as
//     16-bit local indices;
//   - each element entry gets a 16-bit position in the block's product
//     buffer, so that the entries of one local unit form a run (ordered by
//     element, then by the element's entry, G products each; a run of even
//     length is followed by one unused word, which keeps the lanes that sum
//     neighbouring runs on different LDS banks): the apply then sums each
//     run in a fixed order instead of adding into shared memory with
//     atomics;
//   - a unit whose elements all lie in one block is private to it: the block
//     writes y there with plain stores.  Every other unit (shared by several
//     blocks, or touched by none) is finished by a second kernel that adds
//     the blocks' partial sums in increasing block order; the sums sit in
//     planes by rank (the r-th block of every shared unit in plane r, units
//     in increasing order), which keeps both the blocks' writes and the
//     second kernel's reads on consecutive words.
// The plan depends on edof only (rho, Ke, x, alpha, beta come with each
// apply).  Any numbering is valid; compact blocks only make more units
// private.
#include "fem_blocks.hpp"

#include <algorithm>
#include <deque>

namespace spmv {

bool fb_node_structured(int32_t n_elem, int32_t n_dof, const int32_t *edof) {
    auto valid = [n_dof](int32_t d) { return (uint32_t)d < (uint32_t)n_dof; };
    for (int64_t k = 0; k < (int64_t)n_elem * FB_NDOF; k += 3) {
        const int32_t d = edof[k];
        if (!valid(d)) {
            if (valid(edof[k + 1]) || valid(edof[k + 2])) return false;
        } else if (d % 3 != 0 || edof[k + 1] != d + 1 || edof[k + 2] != d + 2 || !valid(d + 2)) {
            return false;
        }
    }
    return true;
}

bool fb_plan_build(int32_t n_elem, int32_t n_dof, const int32_t *edof, int32_t group, int32_t cap,
                   FbPlanHost &P) {
    P = FbPlanHost{};
    const int E = n_elem, n = n_dof, G = group, U = FB_NDOF / group;
    P.group = G;
    P.block = cap;
    auto valid = [n](int32_t d) { return (uint32_t)d < (uint32_t)n; };
    // DOF -> elements (each element listed once per DOF entry, in element order)
    std::vector<int32_t> ptr(n + 1, 0);
    for (int64_t k = 0; k < (int64_t)E * FB_NDOF; ++k)
        if (valid(edof[k])) ++ptr[edof[k] + 1];
    for (int d = 0; d < n; ++d) ptr[d + 1] += ptr[d];
    std::vector<int32_t> elems(ptr[n]);
    {
        std::vector<int32_t> at(ptr.begin(), ptr.end() - 1);
        for (int e = 0; e < E; ++e)
            for (int a = 0; a < FB_NDOF; ++a) {
                const int32_t d = edof[(int64_t)e * FB_NDOF + a];
                if (valid(d)) elems[at[d]++] = e;
            }
    }
    // breadth-first blocks
    std::vector<int32_t> block(E, -1);
    P.perm.reserve(E);
    P.blk_elem_off.push_back(0);
    std::deque<int32_t> q;
    for (int s = 0; s < E; ++s) {
        if (block[s] >= 0) continue;
        const int32_t b = (int32_t)P.blk_elem_off.size() - 1;
        int size = 1;
        block[s] = b;
        P.perm.push_back(s);
        q.clear();
        q.push_back(s);
        while (!q.empty() && size < cap) {
            const int32_t e = q.front();
            q.pop_front();
            for (int a = 0; a < FB_NDOF && size < cap; ++a) {
                const int32_t d = edof[(int64_t)e * FB_NDOF + a];
                if (!valid(d)) continue;
                for (int32_t k = ptr[d]; k < ptr[d + 1] && size < cap; ++k) {
                    const int32_t f = elems[k];
                    if (block[f] >= 0) continue;
                    block[f] = b;
                    ++size;
                    P.perm.push_back(f);
                    q.push_back(f);
                }
            }
        }
        P.blk_elem_off.push_back((int32_t)P.perm.size());
    }
    const int nb = (int)P.blk_elem_off.size() - 1;
    // units: u covers DOFs G u .. G u + G - 1 (the last may be cut by n)
    const int n_units = (n + G - 1) / G;
    // private units: every element on the unit's first DOF in one block (with
    // G = 3 the node's three DOFs have the same elements)
    std::vector<uint8_t> priv(n_units, 0);
    for (int u = 0; u < n_units; ++u) {
        const int d = G * u;
        if (ptr[d] == ptr[d + 1]) continue;   // touched by no element: finished by the second kernel
        const int32_t b0 = block[elems[ptr[d]]];
        bool one = true;
        for (int32_t k = ptr[d] + 1; k < ptr[d + 1] && one; ++k) one = block[elems[k]] == b0;
        priv[u] = one;
    }
    // the unit of entry j of element e, or -1
    auto unit_of = [&](int32_t e, int j) -> int32_t {
        const int32_t d = edof[(int64_t)e * FB_NDOF + G * j];
        return valid(d) ? d / G : -1;
    };
    // units the second kernel finishes (increasing), each with G slots per
    // block that touches it, in rank planes (overflow past FB_PLANES ranks)
    std::vector<int32_t> nblk(n_units, 0), shr_index(n_units, -1), rank(n_units, 0);
    {
        std::vector<int32_t> last(n_units, -1);
        for (int b = 0; b < nb; ++b)
            for (int32_t k = P.blk_elem_off[b]; k < P.blk_elem_off[b + 1]; ++k)
                for (int j = 0; j < U; ++j) {
                    const int32_t u = unit_of(P.perm[k], j);
                    if (u >= 0 && last[u] != b) {
                        last[u] = b;
                        ++nblk[u];
                    }
                }
    }
    int32_t most = 0;
    for (int u = 0; u < n_units; ++u) {
        if (priv[u]) continue;
        shr_index[u] = (int32_t)P.shr_dof.size();
        P.shr_dof.push_back(G * u);
        P.shr_cnt.push_back(nblk[u]);
        most = std::max(most, nblk[u]);
    }
    const int64_t n_shared = (int64_t)P.shr_dof.size();
    P.planes = std::min<int32_t>(most, FB_PLANES);
    P.shr_ptr.assign(1, 0);
    for (int64_t i = 0; i < n_shared; ++i)
        P.shr_ptr.push_back(P.shr_ptr.back() + G * std::max<int32_t>(P.shr_cnt[i] - P.planes, 0));
    const int64_t plane_slots = (int64_t)P.planes * n_shared * G;
    if (plane_slots + P.shr_ptr.back() > INT32_MAX) return false;
    P.n_slots = (int32_t)(plane_slots + P.shr_ptr.back());
    auto slot_of = [&](int32_t u, int32_t r) -> int32_t {   // first slot of rank r of unit u
        const int64_t i = shr_index[u];
        if (r < P.planes) return (int32_t)(((int64_t)r * n_shared + i) * G);
        return (int32_t)(plane_slots + P.shr_ptr[i] + (int64_t)(r - P.planes) * G);
    };
    // per block: local units (sorted, distinct), the entries' local indices,
    // the product runs and the entries' positions in them
    P.blk_dof_off.push_back(0);
    P.lidx.assign((size_t)E * U, FB_NONE);
    P.lpos.assign((size_t)E * U, FB_NONE);
    std::vector<int32_t> loc, run;
    for (int b = 0; b < nb; ++b) {
        const int32_t k0 = P.blk_elem_off[b], k1 = P.blk_elem_off[b + 1];
        loc.clear();
        for (int32_t k = k0; k < k1; ++k)
            for (int j = 0; j < U; ++j) {
                const int32_t u = unit_of(P.perm[k], j);
                if (u >= 0) loc.push_back(u);
            }
        std::sort(loc.begin(), loc.end());
        loc.erase(std::unique(loc.begin(), loc.end()), loc.end());
        if ((int)loc.size() > FB_NONE) return false;   // cannot happen: at most 512 * 24
        P.Lmax = std::max<int32_t>(P.Lmax, (int32_t)loc.size());
        run.assign(loc.size(), 0);
        for (int32_t k = k0; k < k1; ++k)
            for (int j = 0; j < U; ++j) {
                const int32_t u = unit_of(P.perm[k], j);
                if (u < 0) continue;
                const int32_t l = (int32_t)(std::lower_bound(loc.begin(), loc.end(), u) - loc.begin());
                P.lidx[(size_t)k * U + j] = (uint16_t)l;
                ++run[l];
            }
        int32_t at = 0;   // run l starts after run l - 1 and its padding word, if any
        for (size_t l = 0; l < loc.size(); ++l) {
            const int32_t u = loc[l];
            P.ldof.push_back(G * u);
            if (priv[u])
                P.ldst.push_back(G * u);
            else
                P.ldst.push_back(~slot_of(u, rank[u]++));   // blocks come in increasing order
            const int32_t c = G * run[l];
            run[l] = at;   // next free position in the run
            P.crun.push_back((uint32_t)at | (uint32_t)(at + c) << 16);
            at += c + (c % 2 == 0 ? 1 : 0);
        }
        if (at > FB_NONE) return false;   // cannot happen: at most 512 * 24 products and as many pads
        P.Pmax = std::max<int32_t>(P.Pmax, at);
        for (int32_t k = k0; k < k1; ++k)
            for (int j = 0; j < U; ++j) {
                const uint16_t l = P.lidx[(size_t)k * U + j];
                if (l == FB_NONE) continue;
                P.lpos[(size_t)k * U + j] = (uint16_t)run[l];
                run[l] += G;
            }
        P.blk_dof_off.push_back((int32_t)P.ldof.size());
    }
    P.n_blocks = nb;
    return true;
}

bool fb_plan_choose(int32_t n_elem, int32_t n_dof, const int32_t *edof, int32_t group, FbPlanHost &P) {
    if (!fb_plan_build(n_elem, n_dof, edof, group, FB_BLOCK_MAX, P)) return false;
    if (fb_lds_bytes(P) <= FB_LDS_MAX) return true;
    return fb_plan_build(n_elem, n_dof, edof, group, FB_BLOCK_MIN, P);
}

}  // namespace spmv

using namespace spmv;

extern "C" spmv_status fem_blocks_plan_host(int32_t n_elem, int32_t n_dof, const int32_t *edof, int32_t group,
                                            int32_t *counts, int32_t *blk_elem_off, int32_t *perm,
                                            int32_t *blk_dof_off, int32_t *ldof, int32_t *ldst, uint32_t *crun,
                                            uint16_t *lidx, uint16_t *lpos, int32_t *shr_ptr, int32_t *shr_dof,
                                            int32_t *shr_cnt) {
    if (n_elem < 0 || n_dof < 0 || !counts) return fail(SPMV_ERR_INVALID_VALUE, "bad size or NULL counts");
    if ((int64_t)n_elem * FB_NDOF > INT32_MAX) return fail(SPMV_ERR_OVERFLOW, "n_elem * 24 exceeds int32");
    if (n_elem > 0 && !edof) return fail(SPMV_ERR_INVALID_VALUE, "edof is NULL");
    if (group != 0 && group != 1 && group != 3) return fail(SPMV_ERR_INVALID_VALUE, "group must be 0, 1 or 3");
    const bool nodes = fb_node_structured(n_elem, n_dof, edof);
    if (group == 3 && !nodes)
        return fail(SPMV_ERR_INVALID_VALUE, "group 3 needs every element corner to be one node's DOFs 3i..3i+2");
    FbPlanHost P;
    if (!fb_plan_choose(n_elem, n_dof, edof, group ? group : nodes ? 3 : 1, P))
        return fail(SPMV_ERR_UNSUPPORTED, "a block has too many DOFs");
    counts[6] = P.group;
    counts[7] = P.planes;
    counts[8] = P.block;
    counts[0] = P.n_blocks;
    counts[1] = (int32_t)P.ldof.size();
    counts[2] = (int32_t)P.shr_dof.size();
    counts[3] = P.n_slots;
    counts[4] = P.Lmax;
    counts[5] = P.Pmax;
    auto put = [](auto *dst, const auto &v) {
        if (dst) std::copy(v.begin(), v.end(), dst);
    };
    put(blk_elem_off, P.blk_elem_off);
    put(perm, P.perm);
    put(blk_dof_off, P.blk_dof_off);
    put(ldof, P.ldof);
    put(ldst, P.ldst);
    put(crun, P.crun);
    put(lidx, P.lidx);
    put(lpos, P.lpos);
    put(shr_ptr, P.shr_ptr);
    put(shr_dof, P.shr_dof);
    put(shr_cnt, P.shr_cnt);
    return SPMV_OK;
}
