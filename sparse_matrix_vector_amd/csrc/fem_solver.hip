// Jacobi-preconditioned CG and extreme-eigenvalue estimates around the FE
// stiffness matvec, on gfx950.
//
// "Fused GPU SpMV kernel optimisation: from bandwidth bottleneck to BF16
// precision", section 6.1: the fused matvec serves a conjugate-gradient
// solver preconditioned by the operator's diagonal (Jacobi), run up to an
// iteration cap; section 4.1: the condition number of K is measured by
// power iteration.  Here the largest eigenvalue comes from power iteration
// on K and the smallest from the same iteration on K^-1, each step of which
// is a Jacobi-PCG solve.
//
// Vectors are fp32, every inner product is accumulated in fp64 and the
// scalars of the iteration are fp64, so an iteration needs no host round
// trip.  The matvec inside the solver (k_fe_matvec64) is the fused one with
// fp64 element products and fp64 atomic adds into an fp64 accumulator: a
// stiffness operator applied to a smooth vector cancels most of each sum
// (the element matrix annihilates rigid motions), and with fp32 sums that
// cancellation error more than doubles the iteration count already at
// kappa ~ 2e4; with fp64 sums the fp32 iteration tracks the fp64 one.  The
// kernel that consumes K p next reads the accumulator, rounds it to fp32
// and clears it for the following product.
//
// Inner products: every workgroup stores its partial sums; the next kernel
// in the stream, in every one of its workgroups, adds all partials in the
// same fixed order and so obtains the same scalar (alpha, beta, norms)
// bit for bit.  Kernel boundaries make the partials visible across the
// XCDs' L2 caches; no device-scope fence, which on gfx950 writes back and
// invalidates the L2, is issued inside a kernel.  Partials of consecutive
// iterations alternate between two slots, so a kernel never overwrites
// sums that a workgroup of the same kernel still reads.  One PCG iteration
// k is: the matvec acc = K p; k_pcg_pq (q = acc, partial p.q);
// k_pcg_update (alpha = r.z(k-1) / p.q; u, r, z = D^-1 r; partial r.z, r.r
// into slot k & 1); k_pcg_direction (convergence test, beta, p = z + beta p).
// Once the state says "done", these kernels return at once; the host checks
// the state every PCG_CHECK iterations.  The reductions are deterministic;
// the matvec's atomic adds are not (their order varies), so two solves
// agree to rounding, not bit for bit.
#include "common.hpp"
#include "fem_common.hpp"

#include <algorithm>
#include <cmath>

namespace spmv {
namespace {

constexpr int SV_WG = 256;
constexpr int SV_MAX_BLOCKS = 1024;
constexpr int SV_NQ = 3;                 // inner products per partial slot
constexpr int PCG_CHECK = 8;             // iterations launched between host checks
constexpr int NDOF_E = 24;
constexpr int MAX_PENALTY = 8;

// Scalars kept between kernels, at the start of the workspace.  Written by
// workgroup 0 of a kernel, read by later kernels.
struct SolverState {
    double ff;          // f . f
    double rr;          // r . r of the last residual
    double rtol2;       // rtol^2
    int iter, max_iter;
    int done;           // converged, capped or broken down
    int bad;            // 1: diagonal entry not positive, 2: p.Kp <= 0, 4: zero vector
};

size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

// Workspace: state | partials: 2 slots x SV_NQ x SV_MAX_BLOCKS doubles, then
// SV_MAX_BLOCKS more for p.q | lambda history (max_history doubles) |
// vectors of n_dof floats: dinv r z p q (PCG) and v w (eigenvalue
// iterations) | the fp64 matvec accumulator (n_dof doubles, all zero
// between uses).
struct Layout {
    size_t state, partials, hist, vec[7], acc, total;
};

Layout layout(int64_t n_dof, int64_t max_history) {
    Layout L;
    size_t at = 0;
    L.state = at;
    at += round256(sizeof(SolverState));
    L.partials = at;
    at += round256(sizeof(double) * (2 * SV_NQ + 1) * SV_MAX_BLOCKS);
    L.hist = at;
    at += round256(sizeof(double) * (size_t)std::max<int64_t>(max_history, 1));
    for (int k = 0; k < 7; ++k) {
        L.vec[k] = at;
        at += round256(sizeof(float) * (size_t)std::max<int64_t>(n_dof, 1));
    }
    L.acc = at;
    at += round256(sizeof(double) * (size_t)std::max<int64_t>(n_dof, 1));
    L.total = at;
    return L;
}

// Workgroups of the vector kernels: 2 per CU once the vector is long
// enough (every workgroup of the next kernel re-adds all the partials, so
// more workgroups cost more of that).
int vec_blocks(int64_t n) {
    const int64_t cap = std::min<int64_t>(SV_MAX_BLOCKS, 2 * (int64_t)device_cu_count());
    return (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(n, 2 * SV_WG), cap));
}

// Partial-sum slots: slot s, quantity q, one entry per workgroup.
__device__ __forceinline__ double *slot(double *partials, int s, int q) {
    return partials + (size_t)(s * SV_NQ + q) * SV_MAX_BLOCKS;
}
__device__ __forceinline__ const double *slot(const double *partials, int s, int q) {
    return partials + (size_t)(s * SV_NQ + q) * SV_MAX_BLOCKS;
}
__device__ __forceinline__ double *pq_slot(double *partials) {
    return partials + (size_t)2 * SV_NQ * SV_MAX_BLOCKS;
}

// Sum over the workgroup of NQ values per thread, in a fixed order; the
// totals are returned in every thread.
template <int NQ>
__device__ void block_sum(double (&v)[NQ]) {
    __shared__ double red[NQ][SV_WG / 64];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v[q] += __shfl_xor(v[q], off, 64);
    }
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) red[q][wv] = v[q];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        double s = 0.0;
        for (int k = 0; k < SV_WG / 64; ++k) s += red[q][k];
        v[q] = s;
    }
}

// This workgroup's sums of v, one per quantity, into dst[q][blockIdx.x].
template <int NQ>
__device__ void store_partials(double (&v)[NQ], double *const (&dst)[NQ]) {
    block_sum<NQ>(v);
    if (threadIdx.x == 0) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) dst[q][blockIdx.x] = v[q];
    }
}

// Totals of `nb` partials per quantity, the same in every workgroup.
template <int NQ>
__device__ void total_partials(const double *const (&src)[NQ], int nb, double (&tot)[NQ]) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        tot[q] = 0.0;
        for (int b = threadIdx.x; b < nb; b += SV_WG) tot[q] += src[q][b];
    }
    block_sum<NQ>(tot);
}

__global__ void k_sv_fill(int n, float v, float *__restrict__ y) {
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) y[i] = v;
}

__global__ void k_sv_zero64(int n, double *__restrict__ y) {
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) y[i] = 0.0;
}

// acc += sum_e rho_e^p P_e^T Ke P_e x, with the element product and the
// scatter in fp64 (products of fp32 values are exact in fp64).  The fused
// shape of fem_matvec_apply: one lane per element, Ke through the scalar
// cache, 24 gathers, and the contributions merged along x-lines of nodes in
// LDS before the fp64 atomic adds.  Does nothing when `st` says the
// iteration is done.
__global__ __launch_bounds__(SV_WG) void k_fe_matvec64(int n_elem, int n_dof, const int *__restrict__ edof,
                                                       const float *__restrict__ rho, int penalty,
                                                       const float *__restrict__ Ke, const float *__restrict__ x,
                                                       double *__restrict__ acc, const SolverState *st) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    if (st && st->done) return;   // uniform
    __shared__ int line_dof[SV_WG / 64][3 * 65];
    __shared__ double line_val[SV_WG / 64][3 * 65];
    // lanes past the last element stay for the wave exchange, with index -1
    const int e = blockIdx.x * SV_WG + threadIdx.x;
    const bool live = e < n_elem;
    const int ec = live ? e : n_elem - 1;
    int d[NDOF_E];
    const i32x4 *ep = reinterpret_cast<const i32x4 *>(edof + (size_t)ec * NDOF_E);
#pragma unroll
    for (int k = 0; k < NDOF_E / 4; ++k) {
        const i32x4 q = __builtin_nontemporal_load(ep + k);
        d[4 * k] = q.x;
        d[4 * k + 1] = q.y;
        d[4 * k + 2] = q.z;
        d[4 * k + 3] = q.w;
    }
#pragma unroll
    for (int b = 0; b < NDOF_E; ++b) d[b] = live ? d[b] : -1;
    float u[NDOF_E];
#pragma unroll
    for (int b = 0; b < NDOF_E; ++b) u[b] = x[(unsigned)d[b] < (unsigned)n_dof ? d[b] : 0];
#pragma unroll
    for (int b = 0; b < NDOF_E; ++b) u[b] = (unsigned)d[b] < (unsigned)n_dof ? u[b] : 0.0f;
    double s = 1.0;
    for (int k = 0; k < penalty; ++k) s *= (double)rho[ec];
    double fa[NDOF_E];
#pragma unroll
    for (int a = 0; a < NDOF_E; ++a) {
        double f = 0.0;
#pragma unroll
        for (int b = 0; b < NDOF_E; ++b) f = fma((double)Ke[a * NDOF_E + b], (double)u[b], f);
        fa[a] = s * f;
    }
    fe_scatter_lines(d, fa, n_dof, acc, line_dof[threadIdx.x >> 6], line_val[threadIdx.x >> 6]);
}

// diag[edof[e][a]] += rho_e^p Ke[a][a] over the element's free DOFs.
__global__ void k_fe_diag(int n_elem, int n_dof, const int *__restrict__ edof, const float *__restrict__ rho,
                          int penalty, const float *__restrict__ Ke, float *__restrict__ diag) {
    const int e = blockIdx.x * SV_WG + threadIdx.x;
    if (e >= n_elem) return;
    float s = 1.0f;
    for (int k = 0; k < penalty; ++k) s *= rho[e];
#pragma unroll 4
    for (int a = 0; a < NDOF_E; ++a) {
        const int d = edof[(size_t)e * NDOF_E + a];
        if ((unsigned)d < (unsigned)n_dof) atomicAdd(diag + d, s * Ke[a * NDOF_E + a]);
    }
}

// dinv = 1 / diag, flagging an entry that is not positive and finite.
__global__ void k_pcg_dinv(int n, const float *__restrict__ diag, float *__restrict__ dinv, SolverState *st) {
    bool ok = true;
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) {
        const float d = diag[i];
        ok = ok && (d > 0.0f) && (d < INFINITY);
        dinv[i] = 1.0f / d;
    }
    if (!ok) atomicOr(&st->bad, 1);
}

// Start of PCG, with acc = K u: r = f - acc (acc cleared), z = D^-1 r,
// p = z; partial r.z, r.r, f.f into slot 1 (read as "iteration -1").
__global__ void k_pcg_start(int n, const float *__restrict__ f, double *__restrict__ acc, float *__restrict__ r,
                            const float *__restrict__ dinv, float *__restrict__ z, float *__restrict__ p,
                            double *__restrict__ partials) {
    double v[3] = {0.0, 0.0, 0.0};
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) {
        const float fi = f[i];
        const float ri = (float)((double)fi - acc[i]);
        acc[i] = 0.0;
        const float zi = dinv[i] * ri;
        r[i] = ri;
        z[i] = zi;
        p[i] = zi;
        v[0] += (double)ri * zi;
        v[1] += (double)ri * ri;
        v[2] += (double)fi * fi;
    }
    double *const dst[3] = {slot(partials, 1, 0), slot(partials, 1, 1), slot(partials, 1, 2)};
    store_partials<3>(v, dst);
}

// One workgroup: f.f and r.r of the start, and whether there is anything to do.
__global__ void k_pcg_start_fin(int nb, const double *__restrict__ partials, SolverState *st) {
    const double *const src[2] = {slot(partials, 1, 1), slot(partials, 1, 2)};
    double t[2];
    total_partials<2>(src, nb, t);
    if (threadIdx.x == 0) {
        st->rr = t[0];
        st->ff = t[1];
        st->iter = 0;
        st->done = (st->bad != 0) || st->max_iter <= 0 || t[0] <= st->rtol2 * t[1];
    }
}

// q = acc = K p (acc cleared); partial p.q.
__global__ void k_pcg_pq(int n, const float *__restrict__ p, double *__restrict__ acc, float *__restrict__ q,
                         double *__restrict__ partials, const SolverState *st) {
    if (st->done) return;   // uniform: set by an earlier launch
    double v[1] = {0.0};
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) {
        const float qi = (float)acc[i];
        acc[i] = 0.0;
        q[i] = qi;
        v[0] += (double)p[i] * qi;
    }
    double *const dst[1] = {pq_slot(partials)};
    store_partials<1>(v, dst);
}

// Iteration k: alpha = r.z (slot (k+1)&1) / p.q; u += alpha p,
// r -= alpha q, z = D^-1 r; partial r.z, r.r into slot k&1.  A p.q that is
// not positive stops the iteration (the operator is not SPD).
__global__ void k_pcg_update(int n, int k, const float *__restrict__ p, const float *__restrict__ q,
                             const float *__restrict__ dinv, float *__restrict__ u, float *__restrict__ r,
                             float *__restrict__ z, double *__restrict__ partials, SolverState *st) {
    if (st->done) return;
    const double *const src[2] = {pq_slot(partials), slot(partials, (k + 1) & 1, 0)};
    double t[2];
    total_partials<2>(src, gridDim.x, t);
    if (!(t[0] > 0.0)) {   // uniform: every workgroup has the same totals
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            st->bad |= 2;
            st->done = 1;
        }
        return;
    }
    const float a = (float)(t[1] / t[0]);
    double v[2] = {0.0, 0.0};
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) {
        u[i] = fmaf(a, p[i], u[i]);
        const float ri = fmaf(-a, q[i], r[i]);
        r[i] = ri;
        const float zi = dinv[i] * ri;
        z[i] = zi;
        v[0] += (double)ri * zi;
        v[1] += (double)ri * ri;
    }
    double *const dst[2] = {slot(partials, k & 1, 0), slot(partials, k & 1, 1)};
    store_partials<2>(v, dst);
}

// Iteration k: stop when r.r <= rtol^2 f.f or the cap is reached, else
// beta = r.z (slot k&1) / r.z (slot (k+1)&1) and p = z + beta p.
__global__ void k_pcg_direction(int n, int k, const float *__restrict__ z, float *__restrict__ p,
                                const double *__restrict__ partials, SolverState *st) {
    if (st->done) return;
    const double *const src[3] = {slot(partials, k & 1, 0), slot(partials, k & 1, 1),
                                  slot(partials, (k + 1) & 1, 0)};
    double t[3];
    total_partials<3>(src, gridDim.x, t);
    const bool stop = t[1] <= st->rtol2 * st->ff || k + 1 >= st->max_iter;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        st->iter = k + 1;
        st->rr = t[1];
        if (stop) st->done = 1;
    }
    if (stop) return;
    const float b = (float)(t[0] / t[2]);
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) p[i] = fmaf(b, p[i], z[i]);
}

// Partial ||v||^2 into slot 0.
__global__ void k_sv_norm(int n, const float *__restrict__ v, double *__restrict__ partials) {
    double s[1] = {0.0};
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) s[0] += (double)v[i] * v[i];
    double *const dst[1] = {slot(partials, 0, 0)};
    store_partials<1>(s, dst);
}

// dst = src / ||src|| with ||src||^2 from slot 0 (a zero vector is flagged
// and gives zeros).
__global__ void k_sv_scale(int n, const float *__restrict__ src, float *__restrict__ dst,
                           const double *__restrict__ partials, SolverState *st) {
    const double *const in[1] = {slot(partials, 0, 0)};
    double t[1];
    total_partials<1>(in, gridDim.x, t);
    if (!(t[0] > 0.0) && blockIdx.x == 0 && threadIdx.x == 0) st->bad |= 4;
    const float s = t[0] > 0.0 ? (float)(1.0 / sqrt(t[0])) : 0.0f;
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) dst[i] = src[i] * s;
}

// Power-iteration step after acc = K v (v of unit length): w = acc (acc
// cleared); partial v.w, w.w into slot 0.
__global__ void k_pow_dots(int n, const float *__restrict__ v, double *__restrict__ acc, float *__restrict__ w,
                           double *__restrict__ partials) {
    double s[2] = {0.0, 0.0};
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) {
        const double wi = acc[i];
        acc[i] = 0.0;
        w[i] = (float)wi;
        s[0] += (double)v[i] * wi;
        s[1] += wi * wi;
    }
    double *const dst[2] = {slot(partials, 0, 0), slot(partials, 0, 1)};
    store_partials<2>(s, dst);
}

// v = w / ||w||, and the Rayleigh quotient v.w of the previous v into
// hist[k] (both from slot 0).
__global__ void k_pow_next(int n, int k, const float *__restrict__ w, float *__restrict__ v,
                           const double *__restrict__ partials, double *__restrict__ hist, SolverState *st) {
    const double *const in[2] = {slot(partials, 0, 0), slot(partials, 0, 1)};
    double t[2];
    total_partials<2>(in, gridDim.x, t);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        hist[k] = t[0];
        if (!(t[1] > 0.0)) st->bad |= 4;
    }
    const float s = t[1] > 0.0 ? (float)(1.0 / sqrt(t[1])) : 0.0f;
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) v[i] = w[i] * s;
}

// Partial v.acc (acc = K v; acc cleared) into slot 0.
__global__ void k_rayleigh(int n, const float *__restrict__ v, double *__restrict__ acc,
                           double *__restrict__ partials) {
    double s[1] = {0.0};
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) {
        s[0] += (double)v[i] * acc[i];
        acc[i] = 0.0;
    }
    double *const dst[1] = {slot(partials, 0, 0)};
    store_partials<1>(s, dst);
}

// One workgroup: hist[k] = the total of slot 0.
__global__ void k_hist_fin(int nb, int k, const double *__restrict__ partials, double *__restrict__ hist) {
    const double *const in[1] = {slot(partials, 0, 0)};
    double t[1];
    total_partials<1>(in, nb, t);
    if (threadIdx.x == 0) hist[k] = t[0];
}

// ---- host side ----

struct Operator {
    int32_t n_elem, n_dof;
    const int32_t *edof;
    const float *rho;
    int32_t penalty;
    const float *Ke;
};

struct Work {
    SolverState *st;
    double *partials, *hist, *acc;
    float *dinv, *r, *z, *p, *q, *v, *w;
};

Work carve(void *ws, const Layout &L) {
    char *b = static_cast<char *>(ws);
    Work W;
    W.st = reinterpret_cast<SolverState *>(b + L.state);
    W.partials = reinterpret_cast<double *>(b + L.partials);
    W.hist = reinterpret_cast<double *>(b + L.hist);
    W.acc = reinterpret_cast<double *>(b + L.acc);
    float **v[7] = {&W.dinv, &W.r, &W.z, &W.p, &W.q, &W.v, &W.w};
    for (int k = 0; k < 7; ++k) *v[k] = reinterpret_cast<float *>(b + L.vec[k]);
    return W;
}

spmv_status check_op(const Operator &A) {
    if (A.n_elem < 0 || A.n_dof < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if ((int64_t)A.n_elem * NDOF_E > INT32_MAX) return fail(SPMV_ERR_OVERFLOW, "n_elem * 24 exceeds int32");
    if (A.penalty < 0 || A.penalty > MAX_PENALTY)
        return fail(SPMV_ERR_INVALID_VALUE, "penalty must be in [0, %d]", MAX_PENALTY);
    if (A.n_elem > 0 && (!A.edof || !A.rho || !A.Ke)) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    if (A.n_elem > 0 && (!aligned16(A.edof) || !aligned16(A.Ke)))
        return fail(SPMV_ERR_UNSUPPORTED, "edof and Ke must be 16-byte aligned");
    return SPMV_OK;
}

spmv_status check_ws(const Layout &L, void *ws, size_t bytes) {
    if (!ws || bytes < L.total)
        return fail(SPMV_ERR_INVALID_VALUE, "workspace of %zu bytes is smaller than %zu", bytes, L.total);
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(SPMV_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
    return SPMV_OK;
}

// acc += K x (acc must hold zeros, or a sum to add to); skipped once
// `state` (if given) says done.
spmv_status matvec64(const Operator &A, const float *x, double *acc, hipStream_t st,
                     const SolverState *state = nullptr) {
    if (A.n_elem == 0) return SPMV_OK;
    k_fe_matvec64<<<(int)ceil_div(A.n_elem, SV_WG), SV_WG, 0, st>>>(A.n_elem, A.n_dof, A.edof, A.rho, A.penalty,
                                                                    A.Ke, x, acc, state);
    SPMV_LAUNCHED("k_fe_matvec64");
    return SPMV_OK;
}

spmv_status read_state(const Work &W, SolverState *h, hipStream_t st) {
    SPMV_HIP(hipMemcpyAsync(h, W.st, sizeof(SolverState), hipMemcpyDeviceToHost, st));
    SPMV_HIP(hipStreamSynchronize(st));
    return SPMV_OK;
}

spmv_status write_state(const Work &W, const SolverState &h, hipStream_t st) {
    SPMV_HIP(hipMemcpyAsync(W.st, &h, sizeof(SolverState), hipMemcpyHostToDevice, st));
    SPMV_HIP(hipStreamSynchronize(st));   // the source lives on the caller's stack
    return SPMV_OK;
}

spmv_status diag_into(const Operator &A, float *diag, hipStream_t st) {
    k_sv_fill<<<vec_blocks(A.n_dof), SV_WG, 0, st>>>(A.n_dof, 0.0f, diag);
    SPMV_LAUNCHED("k_sv_fill");
    if (A.n_elem > 0) {
        k_fe_diag<<<(int)ceil_div(A.n_elem, SV_WG), SV_WG, 0, st>>>(A.n_elem, A.n_dof, A.edof, A.rho, A.penalty,
                                                                    A.Ke, diag);
        SPMV_LAUNCHED("k_fe_diag");
    }
    return SPMV_OK;
}

// Sets up D^-1 (once per operator) in W.dinv, using W.q as scratch.
spmv_status prepare_dinv(const Operator &A, const Work &W, hipStream_t st) {
    spmv_status s = diag_into(A, W.q, st);
    if (s != SPMV_OK) return s;
    k_pcg_dinv<<<vec_blocks(A.n_dof), SV_WG, 0, st>>>(A.n_dof, W.q, W.dinv, W.st);
    SPMV_LAUNCHED("k_pcg_dinv");
    return SPMV_OK;
}

// Solves K u = f by Jacobi-PCG from the initial u, with W.dinv ready, the
// accumulator zero and W.st's bad flags set.  Synchronises.
spmv_status pcg_run(const Operator &A, const Work &W, const float *f, float *u, float rtol, int32_t max_iter,
                    int32_t *iters, double *relres, hipStream_t st) {
    const int n = A.n_dof, nb = vec_blocks(n);
    SolverState h{};
    spmv_status s = read_state(W, &h, st);
    if (s != SPMV_OK) return s;
    h.rtol2 = (double)rtol * (double)rtol;
    h.max_iter = max_iter;
    h.done = 0;
    h.iter = 0;
    s = write_state(W, h, st);
    if (s != SPMV_OK) return s;
    // r = f - K u
    s = matvec64(A, u, W.acc, st);
    if (s != SPMV_OK) return s;
    k_pcg_start<<<nb, SV_WG, 0, st>>>(n, f, W.acc, W.r, W.dinv, W.z, W.p, W.partials);
    SPMV_LAUNCHED("k_pcg_start");
    k_pcg_start_fin<<<1, SV_WG, 0, st>>>(nb, W.partials, W.st);
    SPMV_LAUNCHED("k_pcg_start_fin");
    s = read_state(W, &h, st);
    if (s != SPMV_OK) return s;
    int k = 0;
    while (!h.done && k < max_iter) {
        const int batch = std::min(PCG_CHECK, max_iter - k);
        for (int j = 0; j < batch; ++j, ++k) {
            s = matvec64(A, W.p, W.acc, st, W.st);
            if (s != SPMV_OK) return s;
            k_pcg_pq<<<nb, SV_WG, 0, st>>>(n, W.p, W.acc, W.q, W.partials, W.st);
            SPMV_LAUNCHED("k_pcg_pq");
            k_pcg_update<<<nb, SV_WG, 0, st>>>(n, k, W.p, W.q, W.dinv, u, W.r, W.z, W.partials, W.st);
            SPMV_LAUNCHED("k_pcg_update");
            k_pcg_direction<<<nb, SV_WG, 0, st>>>(n, k, W.z, W.p, W.partials, W.st);
            SPMV_LAUNCHED("k_pcg_direction");
        }
        s = read_state(W, &h, st);
        if (s != SPMV_OK) return s;
    }
    if (h.bad & 1) return fail(SPMV_ERR_INVALID_MATRIX, "a diagonal entry of the operator is not positive");
    if (h.bad & 2) return fail(SPMV_ERR_INVALID_MATRIX, "p.Kp <= 0: the operator is not positive definite");
    if (iters) *iters = h.iter;
    if (relres) *relres = h.ff > 0.0 ? std::sqrt(h.rr / h.ff) : std::sqrt(h.rr);
    return SPMV_OK;
}

// Clears the state and the fp64 accumulator.
spmv_status reset_state(const Work &W, int n, hipStream_t st) {
    k_sv_zero64<<<vec_blocks(n), SV_WG, 0, st>>>(n, W.acc);
    SPMV_LAUNCHED("k_sv_zero64");
    return write_state(W, SolverState{}, st);
}

// dst = src / ||src||.
spmv_status normalise_into(const Work &W, int n, const float *src, float *dst, hipStream_t st) {
    const int nb = vec_blocks(n);
    k_sv_norm<<<nb, SV_WG, 0, st>>>(n, src, W.partials);
    SPMV_LAUNCHED("k_sv_norm");
    k_sv_scale<<<nb, SV_WG, 0, st>>>(n, src, dst, W.partials, W.st);
    SPMV_LAUNCHED("k_sv_scale");
    return SPMV_OK;
}

}  // namespace
}  // namespace spmv

using namespace spmv;

extern "C" spmv_status fem_jacobi_diagonal(int32_t n_elem, int32_t n_dof, const int32_t *edof, const float *rho,
                                           int32_t penalty, const float *Ke, float *diag, void *stream) {
    const Operator A{n_elem, n_dof, edof, rho, penalty, Ke};
    spmv_status s = check_op(A);
    if (s != SPMV_OK) return s;
    if (n_dof == 0) return SPMV_OK;
    if (!diag) return fail(SPMV_ERR_INVALID_VALUE, "diag is NULL");
    return diag_into(A, diag, as_stream(stream));
}

extern "C" spmv_status fem_solver_workspace_size(int32_t n_dof, int32_t max_history, size_t *bytes) {
    if (!bytes) return fail(SPMV_ERR_INVALID_VALUE, "bytes is NULL");
    if (n_dof < 0 || max_history < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    *bytes = layout(n_dof, max_history).total;
    return SPMV_OK;
}

extern "C" spmv_status fem_pcg_solve(int32_t n_elem, int32_t n_dof, const int32_t *edof, const float *rho,
                                     int32_t penalty, const float *Ke, const float *f, float *u, float rtol,
                                     int32_t max_iter, void *workspace, size_t workspace_bytes, int32_t *iterations,
                                     double *rel_residual, void *stream) {
    const Operator A{n_elem, n_dof, edof, rho, penalty, Ke};
    spmv_status s = check_op(A);
    if (s != SPMV_OK) return s;
    if (!(rtol >= 0.0f) || max_iter < 0) return fail(SPMV_ERR_INVALID_VALUE, "rtol must be >= 0 and max_iter >= 0");
    if (n_dof == 0) {
        if (iterations) *iterations = 0;
        if (rel_residual) *rel_residual = 0.0;
        return SPMV_OK;
    }
    if (!f || !u) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    const Layout L = layout(n_dof, 0);
    s = check_ws(L, workspace, workspace_bytes);
    if (s != SPMV_OK) return s;
    hipStream_t st = as_stream(stream);
    const Work W = carve(workspace, L);
    s = reset_state(W, n_dof, st);
    if (s != SPMV_OK) return s;
    s = prepare_dinv(A, W, st);
    if (s != SPMV_OK) return s;
    return pcg_run(A, W, f, u, rtol, max_iter, iterations, rel_residual, st);
}

extern "C" spmv_status fem_lambda_max(int32_t n_elem, int32_t n_dof, const int32_t *edof, const float *rho,
                                      int32_t penalty, const float *Ke, const float *v0, int32_t iterations,
                                      void *workspace, size_t workspace_bytes, double *h_lambda, void *stream) {
    const Operator A{n_elem, n_dof, edof, rho, penalty, Ke};
    spmv_status s = check_op(A);
    if (s != SPMV_OK) return s;
    if (iterations < 1 || n_dof < 1) return fail(SPMV_ERR_INVALID_VALUE, "need iterations >= 1 and n_dof >= 1");
    if (!v0 || !h_lambda) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    const Layout L = layout(n_dof, iterations);
    s = check_ws(L, workspace, workspace_bytes);
    if (s != SPMV_OK) return s;
    hipStream_t st = as_stream(stream);
    const Work W = carve(workspace, L);
    const int n = n_dof, nb = vec_blocks(n);
    s = reset_state(W, n_dof, st);
    if (s != SPMV_OK) return s;
    s = normalise_into(W, n, v0, W.v, st);
    if (s != SPMV_OK) return s;
    for (int k = 0; k < iterations; ++k) {
        s = matvec64(A, W.v, W.acc, st);
        if (s != SPMV_OK) return s;
        k_pow_dots<<<nb, SV_WG, 0, st>>>(n, W.v, W.acc, W.w, W.partials);
        SPMV_LAUNCHED("k_pow_dots");
        k_pow_next<<<nb, SV_WG, 0, st>>>(n, k, W.w, W.v, W.partials, W.hist, W.st);
        SPMV_LAUNCHED("k_pow_next");
    }
    SolverState h;
    s = read_state(W, &h, st);
    if (s != SPMV_OK) return s;
    if (h.bad & 4) return fail(SPMV_ERR_INVALID_VALUE, "the iteration reached a zero vector");
    SPMV_HIP(hipMemcpyAsync(h_lambda, W.hist, sizeof(double) * (size_t)iterations, hipMemcpyDeviceToHost, st));
    SPMV_HIP(hipStreamSynchronize(st));
    return SPMV_OK;
}

extern "C" spmv_status fem_lambda_min(int32_t n_elem, int32_t n_dof, const int32_t *edof, const float *rho,
                                      int32_t penalty, const float *Ke, const float *v0, int32_t iterations,
                                      float inner_rtol, int32_t inner_max_iter, void *workspace,
                                      size_t workspace_bytes, double *h_lambda, int32_t *h_inner_iterations,
                                      void *stream) {
    const Operator A{n_elem, n_dof, edof, rho, penalty, Ke};
    spmv_status s = check_op(A);
    if (s != SPMV_OK) return s;
    if (iterations < 1 || n_dof < 1) return fail(SPMV_ERR_INVALID_VALUE, "need iterations >= 1 and n_dof >= 1");
    if (!(inner_rtol >= 0.0f) || inner_max_iter < 1)
        return fail(SPMV_ERR_INVALID_VALUE, "inner_rtol must be >= 0 and inner_max_iter >= 1");
    if (!v0 || !h_lambda) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    const Layout L = layout(n_dof, iterations);
    s = check_ws(L, workspace, workspace_bytes);
    if (s != SPMV_OK) return s;
    hipStream_t st = as_stream(stream);
    const Work W = carve(workspace, L);
    const int n = n_dof, nb = vec_blocks(n);
    s = reset_state(W, n_dof, st);
    if (s != SPMV_OK) return s;
    s = prepare_dinv(A, W, st);
    if (s != SPMV_OK) return s;
    s = normalise_into(W, n, v0, W.v, st);
    if (s != SPMV_OK) return s;
    for (int k = 0; k < iterations; ++k) {
        // w = K^-1 v by PCG from zero
        k_sv_fill<<<nb, SV_WG, 0, st>>>(n, 0.0f, W.w);
        SPMV_LAUNCHED("k_sv_fill");
        int32_t it = 0;
        s = pcg_run(A, W, W.v, W.w, inner_rtol, inner_max_iter, &it, nullptr, st);
        if (s != SPMV_OK) return s;
        if (h_inner_iterations) h_inner_iterations[k] = it;
        // v = w / ||w||, then the Rayleigh quotient v.Kv
        s = normalise_into(W, n, W.w, W.v, st);
        if (s != SPMV_OK) return s;
        s = matvec64(A, W.v, W.acc, st);
        if (s != SPMV_OK) return s;
        k_rayleigh<<<nb, SV_WG, 0, st>>>(n, W.v, W.acc, W.partials);
        SPMV_LAUNCHED("k_rayleigh");
        k_hist_fin<<<1, SV_WG, 0, st>>>(nb, k, W.partials, W.hist);
        SPMV_LAUNCHED("k_hist_fin");
    }
    SolverState h;
    s = read_state(W, &h, st);
    if (s != SPMV_OK) return s;
    if (h.bad & 4) return fail(SPMV_ERR_INVALID_VALUE, "the iteration reached a zero vector");
    SPMV_HIP(hipMemcpyAsync(h_lambda, W.hist, sizeof(double) * (size_t)iterations, hipMemcpyDeviceToHost, st));
    SPMV_HIP(hipStreamSynchronize(st));
    return SPMV_OK;
}
