// Element blocks of the finite-element matvec: plan layout shared by the
// host planner (fem_blocks.cpp) and the apply (fem_blocks.hip).
#pragma once

#include "common.hpp"

#include <algorithm>
#include <cstdint>
#include <vector>

namespace spmv {

constexpr int FB_BLOCK_MAX = 512;             // most elements per block (one workgroup, a lane each)
constexpr int FB_BLOCK_MIN = 256;             // the size taken when larger blocks overflow the LDS
constexpr size_t FB_LDS_MAX = 65536;          // LDS bytes a workgroup may take
constexpr int FB_NDOF = 24;                   // DOFs per element
constexpr uint16_t FB_NONE = 0xFFFF;          // local index / position of a constrained DOF

// The plan works on units of G consecutive DOFs: G = 1 (a unit is a DOF) for
// any numbering, or G = 3 (a unit is a node) when every element corner lists
// either three constrained DOFs or the DOFs 3i, 3i+1, 3i+2 of one node i.
// An element has U = 24 / G corner entries (k, j); component c of entry j
// is the element's DOF G * j + c.
//
// The plan on the host.  Blocks b = 0..n_blocks-1:
//   elements perm[blk_elem_off[b] .. blk_elem_off[b+1])  (caller's element ids;
//     the k-th element of the list is "element k" below)
//   local units l = 0..L-1 at blk_dof_off[b] + l: first DOF ldof (increasing),
//     destination ldst of the first component (the DOF itself when every
//     element on the unit lies in this block, else ~slot; component c goes
//     to that + c), and crun = start | end << 16, the unit's run in the
//     block's product buffer (runs follow the local units; a run of even
//     length is followed by one unused word, so that neighbouring lanes
//     summing neighbouring runs read different LDS banks)
//   lidx[k * U + j]: local unit of entry j of element k
//   lpos[k * U + j]: where that entry's G products go in the block's product
//     buffer (component c at lpos + c): a unit's run holds its entries in
//     (k, j) order, G products each
// Units finished by the second kernel: shr_dof[i] (first DOF, increasing;
// shared by several blocks or touched by none), touched by shr_cnt[i]
// blocks.  Their partial sums (G floats per block, in block order r =
// 0, 1, ...) sit in rank planes: for r < planes, component c at
// (r * n_shared + i) * G + c, so that a block writing rank r of neighbouring
// units and the second kernel reading unit after unit both touch
// consecutive words; ranks r >= planes (only when a unit lies in more than
// FB_PLANES blocks) at planes * n_shared * G + shr_ptr[i] + (r - planes) * G + c.
// Lmax: the most local units of a block; Pmax: the largest product buffer
// of one (products and padding words).
constexpr int FB_PLANES = 8;   // most rank planes of the partial sums (a hexahedral node lies in <= 8 blocks)

struct FbPlanHost {
    int32_t group = 1, block = FB_BLOCK_MIN, n_blocks = 0, Lmax = 0, Pmax = 0, planes = 0, n_slots = 0;
    std::vector<int32_t> blk_elem_off, perm, blk_dof_off, ldof, ldst, shr_ptr, shr_dof, shr_cnt;
    std::vector<uint32_t> crun;
    std::vector<uint16_t> lidx, lpos;
};

// True when every element corner is three constrained DOFs or the three DOFs
// of one node (3i, 3i+1, 3i+2), so that G = 3 applies.
bool fb_node_structured(int32_t n_elem, int32_t n_dof, const int32_t *edof);

// Builds the plan from host edof (int32[n_elem * 24], entries outside
// [0, n_dof) constrained) for group 1 or 3 (3 only when fb_node_structured)
// with blocks of at most `cap` elements.  False only if a block had more
// local units or products than 16-bit indices hold (not possible with
// FB_BLOCK_MAX * 48 < 65535) or the partial sums would need more than 2^31
// slots.
bool fb_plan_build(int32_t n_elem, int32_t n_dof, const int32_t *edof, int32_t group, int32_t cap,
                   FbPlanHost &P);

// LDS bytes a block's workgroup takes: x of its units and its product
// buffer (at least one word each).
inline size_t fb_lds_bytes(const FbPlanHost &P) {
    return sizeof(float) * ((size_t)P.group * std::max(P.Lmax, 1) + std::max(P.Pmax, 1));
}

// The plan with the largest block size whose workgroups fit the LDS limit:
// FB_BLOCK_MAX elements (fewer nodes shared between blocks), else
// FB_BLOCK_MIN, which always fits (at most 256 * 24 units and products).
bool fb_plan_choose(int32_t n_elem, int32_t n_dof, const int32_t *edof, int32_t group, FbPlanHost &P);

}  // namespace spmv
