// Element blocks of the finite-element matvec: the apply on gfx950.
//
// "Fused GPU SpMV kernel optimisation", sections 2.2 and 5.2: one fused
// pass gathers, multiplies and scatters; fast on-chip memory should hold
// what the elements share.  With the plan of fem_blocks.cpp a block of up to
// 512 elements (256 where a larger one would overflow the LDS) is one
// workgroup, a lane per element:
//   k_fe_block  stages x of the block's local units (G DOFs each: a node's
//               three, or one) in LDS, one load per DOF instead of one per
//               element entry; reads each element's 24 / G 16-bit local
//               indices and product positions (32 bytes per element with
//               nodes, against edof's 96); forms the 24 x 24 product in
//               registers (Ke through the scalar cache, as in the fused
//               kernel); writes the 24 products to their planned positions
//               in an LDS product buffer; then sums each local unit's run in
//               a fixed order and writes it once: y = beta y + sum for a
//               private unit (plain stores), the partial sums into the
//               unit's slots otherwise;
//   k_fe_shared  y = beta y + the unit's partial sums (one per block, in
//               increasing block order), for every unit that is not private
//               to one block.
// No atomics anywhere (LDS float atomics serialise badly on this part: the
// same kernel adding into an LDS accumulator ran more than twice as long),
// no separate beta pass, every DOF of y written exactly once, and every sum
// taken in an order fixed by the plan, so y is the same bits on every call.
#include "fem_blocks.hpp"

#include <algorithm>
#include <cstring>

namespace spmv {
namespace {

constexpr int FB_MAX_PENALTY = 8;
__device__ __forceinline__ float fb_simp(float r, int p) {
    float s = 1.0f;
    for (int k = 0; k < p; ++k) s *= r;
    return s;
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// N 16-bit values (N a multiple of 8, 16-byte aligned) in N / 8 loads
template <int N>
__device__ __forceinline__ void fb_load16(const uint16_t *p, unsigned (&o)[N]) {
    const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
        const u32x4 w = __builtin_nontemporal_load(q + i);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            o[8 * i + 2 * h] = w[h] & 0xFFFFu;
            o[8 * i + 2 * h + 1] = w[h] >> 16;
        }
    }
}

// G DOFs per unit: U = 24 / G entries per element, PER local units per
// thread held in registers (all of them when L <= PER * NT, NT the block size)
template <int G>
struct FbShape {
    static constexpr int U = FB_NDOF / G;
    static constexpr int PER = G == 1 ? 7 : 3;
};

template <int G, int NT>
__global__ __launch_bounds__(NT) void k_fe_block(const int *__restrict__ blk_elem_off,
                                                      const int *__restrict__ perm,
                                                      const int *__restrict__ blk_dof_off,
                                                      const int *__restrict__ ldof, const int *__restrict__ ldst,
                                                      const unsigned *__restrict__ crun,
                                                      const uint16_t *__restrict__ lidx,
                                                      const uint16_t *__restrict__ lpos, int Lmax,
                                                      const float *__restrict__ rho, int penalty,
                                                      const float *__restrict__ Ke, float alpha,
                                                      const float *__restrict__ x, float beta,
                                                      float *__restrict__ y, float *__restrict__ slots) {
    constexpr int U = FbShape<G>::U, PER = FbShape<G>::PER;
    extern __shared__ float fb_lds[];
    float *xs = fb_lds, *pb = fb_lds + G * Lmax;
    const int t = threadIdx.x;
    // the workgroups one XCD receives (workgroup i goes to XCD i % 8) take a
    // contiguous range of blocks: neighbouring blocks share nodes, whose x
    // and partial-sum lines then stay in that XCD's L2
    int b;
    {
        const int nw = gridDim.x, w = blockIdx.x, q = nw / 8, r = nw % 8, xcd = w % 8, idx = w / 8;
        b = xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
    }
    const int e0 = blk_elem_off[b], ne = blk_elem_off[b + 1] - e0;
    const int d0 = blk_dof_off[b], L = blk_dof_off[b + 1] - d0;
    // the lane's element: local units and product positions of its entries, rho
    const bool live = t < ne;
    const int k = e0 + (live ? t : 0);
    unsigned li[U], lp[U];
    fb_load16<U>(lidx + (size_t)k * U, li);
    fb_load16<U>(lpos + (size_t)k * U, lp);
    const float r = rho[perm[k]];
    // Ke (2304 bytes) is read through the scalar cache a few lines at a
    // time as the products go; when it is cold in L2 every line is a miss in
    // that chain.  One lane per 64-byte line touches it now, beside the
    // staging loads, and the value is kept until the barrier
    const float ke_touch = t < FB_NDOF * FB_NDOF / 16 ? Ke[16 * t] : 0.0f;
    // the thread's local units l = j * NT + t: first DOF, destination and
    // run bounds; x of the block's units into LDS.  The loads take no branch
    // (a lane past the block's last unit reads that unit again and drops
    // it), so that all of them are in flight together instead of one
    // memory latency after another
    int g[PER], dst[PER], c0[PER], c1[PER];
    if (L > 0) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int l = min(j * NT + t, L - 1);
            g[j] = ldof[d0 + l];
            dst[j] = ldst[d0 + l];
            const unsigned q = crun[d0 + l];
            c0[j] = q & 0xFFFFu;
            c1[j] = q >> 16;
        }
        float xv[PER][G];
#pragma unroll
        for (int j = 0; j < PER; ++j)
#pragma unroll
            for (int c = 0; c < G; ++c) xv[j][c] = x[(unsigned)g[j] + c];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int l = j * NT + t;
            if (l < L)
#pragma unroll
                for (int c = 0; c < G; ++c) xs[G * l + c] = xv[j][c];
        }
    }
    for (int l = PER * NT + t; l < L; l += NT)
#pragma unroll
        for (int c = 0; c < G; ++c) xs[G * l + c] = x[ldof[d0 + l] + c];
    asm volatile("" ::"v"(ke_touch));
    __syncthreads();
    float u[FB_NDOF];
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const bool on = live && li[j] != FB_NONE;
#pragma unroll
        for (int c = 0; c < G; ++c) {
            const float v = xs[on ? G * li[j] + c : 0];
            u[G * j + c] = on ? v : 0.0f;
        }
    }
    const float s = alpha * fb_simp(r, penalty);
    float fa[FB_NDOF];
#pragma unroll
    for (int a = 0; a < FB_NDOF; ++a) {
        float f = 0.0f;
#pragma unroll
        for (int c = 0; c < FB_NDOF; ++c) f = fmaf(Ke[a * FB_NDOF + c], u[c], f);
        fa[a] = s * f;
    }
    // products finished before the stores (else the compiler sinks them into
    // the store loop, where Ke no longer fits the scalar registers)
#pragma unroll
    for (int a = 0; a < FB_NDOF; ++a) asm volatile("" : "+v"(fa[a]));
#pragma unroll
    for (int j = 0; j < U; ++j)
        if (live && lp[j] != FB_NONE)
#pragma unroll
            for (int c = 0; c < G; ++c) pb[lp[j] + c] = fa[G * j + c];
    __syncthreads();
    // each local unit: its run's entries added in order, component by
    // component, then written once
    auto put = [&](int m, int q0, int q1) {
        float v[G];
#pragma unroll
        for (int c = 0; c < G; ++c) v[c] = 0.0f;
        for (int q = q0; q < q1; q += G)
#pragma unroll
            for (int c = 0; c < G; ++c) v[c] += pb[q + c];
        if (m >= 0) {
#pragma unroll
            for (int c = 0; c < G; ++c) y[m + c] = beta != 0.0f ? fmaf(beta, y[m + c], v[c]) : v[c];
        } else {
#pragma unroll
            for (int c = 0; c < G; ++c) slots[~m + c] = v[c];
        }
    };
#pragma unroll
    for (int j = 0; j < PER; ++j)
        if (j * NT + t < L) put(dst[j], c0[j], c1[j]);
    for (int l = PER * NT + t; l < L; l += NT) {
        const unsigned q = crun[d0 + l];
        put(ldst[d0 + l], q & 0xFFFFu, q >> 16);
    }
}

// y = beta y + the unit's partial sums (G per block, in increasing block
// order: ranks below `planes` in the rank planes, the rest in the overflow
// list)
template <int G>
__global__ __launch_bounds__(256) void k_fe_shared(int n_shared, int planes, int n_dof,
                                                  const int *__restrict__ shr_dof, const int *__restrict__ shr_cnt,
                                                  const int *__restrict__ shr_ptr,
                                                  const float *__restrict__ slots, float beta,
                                                  float *__restrict__ y) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n_shared) return;
    const int d = shr_dof[i], cnt = shr_cnt[i];
    // all plane loads issued together (a hexahedral node lies in at most 8
    // blocks), added in rank order
    float w[FB_PLANES][G];
#pragma unroll
    for (int r = 0; r < FB_PLANES; ++r)
#pragma unroll
        for (int c = 0; c < G; ++c)
            w[r][c] = r < cnt && r < planes ? slots[((size_t)r * n_shared + i) * G + c] : 0.0f;
    float v[G];
#pragma unroll
    for (int c = 0; c < G; ++c) v[c] = 0.0f;
#pragma unroll
    for (int r = 0; r < FB_PLANES; ++r)
        if (r < cnt && r < planes)
#pragma unroll
            for (int c = 0; c < G; ++c) v[c] += w[r][c];
    if (cnt > planes) {
        const float *o = slots + (size_t)planes * n_shared * G + shr_ptr[i];
        for (int r = 0; r < cnt - planes; ++r)
#pragma unroll
            for (int c = 0; c < G; ++c) v[c] += o[G * r + c];
    }
#pragma unroll
    for (int c = 0; c < G; ++c)
        if (d + c < n_dof) y[d + c] = beta != 0.0f ? fmaf(beta, y[d + c], v[c]) : v[c];
}

size_t fb_align(size_t v) { return (v + 255) & ~size_t(255); }

// Device workspace, every array sized by its upper bound for the shape (a
// block holds at most 256 * 24 local units and products; the partial sums
// take at most FB_PLANES planes of n_dof + 2 words plus one overflow slot
// per local unit).
struct FbLayout {
    size_t blk_elem_off, perm, blk_dof_off, ldof, ldst, crun, lidx, lpos, slots, shr_ptr, shr_dof, shr_cnt, total;
};

FbLayout fb_layout(int64_t E, int64_t n) {
    FbLayout L{};
    size_t at = 0;
    auto take = [&](size_t bytes) {
        const size_t p = at;
        at = fb_align(at + std::max<size_t>(bytes, 4));
        return p;
    };
    const size_t ent = (size_t)E * FB_NDOF;
    L.blk_elem_off = take(4 * ((size_t)E + 1));
    L.perm = take(4 * (size_t)E);
    L.blk_dof_off = take(4 * ((size_t)E + 1));
    L.ldof = take(4 * ent);
    L.ldst = take(4 * ent);
    L.crun = take(4 * ent);
    L.lidx = take(2 * ent);
    L.lpos = take(2 * ent);
    L.slots = take(4 * (ent + (size_t)FB_PLANES * ((size_t)n + 2)));
    L.shr_ptr = take(4 * ((size_t)n + 1));
    L.shr_dof = take(4 * (size_t)n);
    L.shr_cnt = take(4 * (size_t)n);
    L.total = at;
    return L;
}

spmv_status fb_check_shape(int32_t n_elem, int32_t n_dof) {
    if (n_elem < 0 || n_dof < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if ((int64_t)n_elem * FB_NDOF > INT32_MAX) return fail(SPMV_ERR_OVERFLOW, "n_elem * 24 exceeds int32");
    return SPMV_OK;
}

}  // namespace
}  // namespace spmv

using namespace spmv;

struct fem_blocks {
    int32_t n_elem = 0, n_dof = 0, group = 1, block = FB_BLOCK_MIN, n_blocks = 0, Lmax = 0, Pmax = 0, n_shared = 0, planes = 0;
    int32_t *blk_elem_off = nullptr, *perm = nullptr, *blk_dof_off = nullptr, *ldof = nullptr, *ldst = nullptr;
    int32_t *shr_ptr = nullptr, *shr_dof = nullptr, *shr_cnt = nullptr;
    uint32_t *crun = nullptr;
    uint16_t *lidx = nullptr, *lpos = nullptr;
    float *slots = nullptr;
};

extern "C" spmv_status fem_blocks_size(int32_t n_elem, int32_t n_dof, size_t *bytes) {
    if (!bytes) return fail(SPMV_ERR_INVALID_VALUE, "bytes is NULL");
    spmv_status s = fb_check_shape(n_elem, n_dof);
    if (s != SPMV_OK) return s;
    *bytes = fb_layout(n_elem, n_dof).total;
    return SPMV_OK;
}

extern "C" spmv_status fem_blocks_create(fem_blocks_t *out, int32_t n_elem, int32_t n_dof, const int32_t *edof,
                                         int32_t group, void *workspace, size_t workspace_bytes, void *stream) {
    if (!out) return fail(SPMV_ERR_INVALID_VALUE, "handle pointer is NULL");
    *out = nullptr;
    spmv_status s = fb_check_shape(n_elem, n_dof);
    if (s != SPMV_OK) return s;
    if (n_elem > 0 && !edof) return fail(SPMV_ERR_INVALID_VALUE, "edof is NULL");
    if (group != 0 && group != 1 && group != 3) return fail(SPMV_ERR_INVALID_VALUE, "group must be 0, 1 or 3");
    const FbLayout L = fb_layout(n_elem, n_dof);
    if (workspace_bytes < L.total)
        return fail(SPMV_ERR_INVALID_VALUE, "workspace of %zu bytes is smaller than %zu", workspace_bytes, L.total);
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return fail(SPMV_ERR_INVALID_VALUE, "workspace must be non-NULL and 256-byte aligned");
    hipStream_t st = as_stream(stream);
    std::vector<int32_t> h_edof((size_t)n_elem * FB_NDOF);
    if (n_elem > 0) {
        SPMV_HIP(hipMemcpyAsync(h_edof.data(), edof, h_edof.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st));
        SPMV_HIP(hipStreamSynchronize(st));
    }
    const bool nodes = fb_node_structured(n_elem, n_dof, h_edof.data());
    if (group == 3 && !nodes)
        return fail(SPMV_ERR_INVALID_VALUE, "group 3 needs every element corner to be one node's DOFs 3i..3i+2");
    FbPlanHost P;
    if (!fb_plan_choose(n_elem, n_dof, h_edof.data(), group ? group : nodes ? 3 : 1, P))
        return fail(SPMV_ERR_UNSUPPORTED, "a block has too many DOFs");
    fem_blocks *h = new fem_blocks();
    char *ws = static_cast<char *>(workspace);
    h->n_elem = n_elem;
    h->n_dof = n_dof;
    h->group = P.group;
    h->block = P.block;
    h->n_blocks = P.n_blocks;
    h->Lmax = P.Lmax;
    h->Pmax = P.Pmax;
    h->n_shared = (int32_t)P.shr_dof.size();
    h->planes = P.planes;
    h->blk_elem_off = reinterpret_cast<int32_t *>(ws + L.blk_elem_off);
    h->perm = reinterpret_cast<int32_t *>(ws + L.perm);
    h->blk_dof_off = reinterpret_cast<int32_t *>(ws + L.blk_dof_off);
    h->ldof = reinterpret_cast<int32_t *>(ws + L.ldof);
    h->ldst = reinterpret_cast<int32_t *>(ws + L.ldst);
    h->crun = reinterpret_cast<uint32_t *>(ws + L.crun);
    h->lidx = reinterpret_cast<uint16_t *>(ws + L.lidx);
    h->lpos = reinterpret_cast<uint16_t *>(ws + L.lpos);
    h->slots = reinterpret_cast<float *>(ws + L.slots);
    h->shr_ptr = reinterpret_cast<int32_t *>(ws + L.shr_ptr);
    h->shr_dof = reinterpret_cast<int32_t *>(ws + L.shr_dof);
    h->shr_cnt = reinterpret_cast<int32_t *>(ws + L.shr_cnt);
    auto put = [&](void *dst, const void *src, size_t bytes) -> hipError_t {
        return bytes ? hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, st) : hipSuccess;
    };
    hipError_t e = hipSuccess;
    auto chk = [&](hipError_t r) {
        if (e == hipSuccess) e = r;
    };
    chk(put(h->blk_elem_off, P.blk_elem_off.data(), P.blk_elem_off.size() * 4));
    chk(put(h->perm, P.perm.data(), P.perm.size() * 4));
    chk(put(h->blk_dof_off, P.blk_dof_off.data(), P.blk_dof_off.size() * 4));
    chk(put(h->ldof, P.ldof.data(), P.ldof.size() * 4));
    chk(put(h->ldst, P.ldst.data(), P.ldst.size() * 4));
    chk(put(h->crun, P.crun.data(), P.crun.size() * 4));
    chk(put(h->lidx, P.lidx.data(), P.lidx.size() * 2));
    chk(put(h->lpos, P.lpos.data(), P.lpos.size() * 2));
    chk(put(h->shr_ptr, P.shr_ptr.data(), P.shr_ptr.size() * 4));
    chk(put(h->shr_dof, P.shr_dof.data(), P.shr_dof.size() * 4));
    chk(put(h->shr_cnt, P.shr_cnt.data(), P.shr_cnt.size() * 4));
    chk(hipStreamSynchronize(st));   // the host vectors go out of scope below
    if (e != hipSuccess) {
        delete h;
        return fail(SPMV_ERR_HIP, "plan upload: %s", hipGetErrorString(e));
    }
    *out = h;
    return SPMV_OK;
}

extern "C" spmv_status fem_blocks_apply(fem_blocks_t h, const float *rho, int32_t penalty, const float *Ke,
                                        float alpha, const float *x, float beta, float *y, void *stream) {
    if (!h) return fail(SPMV_ERR_INVALID_VALUE, "handle is NULL");
    if (penalty < 0 || penalty > FB_MAX_PENALTY)
        return fail(SPMV_ERR_INVALID_VALUE, "penalty must be in [0, %d]", FB_MAX_PENALTY);
    if (h->n_dof == 0) return SPMV_OK;
    if (!y) return fail(SPMV_ERR_INVALID_VALUE, "y is NULL");
    if (h->n_blocks > 0 && (!rho || !Ke || !x)) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    hipStream_t st = as_stream(stream);
    if (h->n_blocks > 0) {
        // at least one word each, so that the masked read of x at local index 0
        // stays inside the allocation when no block has a free DOF
        const int lmax = std::max(h->Lmax, 1), pmax = std::max(h->Pmax, 1);
        const size_t lds = sizeof(float) * ((size_t)h->group * lmax + pmax);
        auto launch = [&](auto kernel, int nt) {
            kernel<<<h->n_blocks, nt, lds, st>>>(h->blk_elem_off, h->perm, h->blk_dof_off, h->ldof, h->ldst, h->crun,
                                                 h->lidx, h->lpos, lmax, rho, penalty, Ke, alpha, x, beta, y,
                                                 h->slots);
        };
        if (h->group == 3)
            h->block == FB_BLOCK_MAX ? launch(k_fe_block<3, FB_BLOCK_MAX>, FB_BLOCK_MAX)
                                     : launch(k_fe_block<3, FB_BLOCK_MIN>, FB_BLOCK_MIN);
        else
            h->block == FB_BLOCK_MAX ? launch(k_fe_block<1, FB_BLOCK_MAX>, FB_BLOCK_MAX)
                                     : launch(k_fe_block<1, FB_BLOCK_MIN>, FB_BLOCK_MIN);
        SPMV_LAUNCHED("k_fe_block");
    }
    if (h->n_shared > 0) {
        const int grid = (int)ceil_div(h->n_shared, 256);
        if (h->group == 3)
            k_fe_shared<3><<<grid, 256, 0, st>>>(h->n_shared, h->planes, h->n_dof, h->shr_dof, h->shr_cnt, h->shr_ptr,
                                                 h->slots, beta, y);
        else
            k_fe_shared<1><<<grid, 256, 0, st>>>(h->n_shared, h->planes, h->n_dof, h->shr_dof, h->shr_cnt, h->shr_ptr,
                                                 h->slots, beta, y);
        SPMV_LAUNCHED("k_fe_shared");
    }
    return SPMV_OK;
}

extern "C" spmv_status fem_blocks_info(fem_blocks_t h, int32_t *counts) {
    if (!h || !counts) return fail(SPMV_ERR_INVALID_VALUE, "NULL handle or counts");
    counts[0] = h->n_blocks;
    counts[1] = h->Lmax;
    counts[2] = h->n_shared;
    counts[3] = h->Pmax;
    counts[4] = h->group;
    counts[5] = h->planes;
    counts[6] = h->block;
    return SPMV_OK;
}

extern "C" spmv_status fem_blocks_destroy(fem_blocks_t h) {
    delete h;
    return SPMV_OK;
}
