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
// The operator's data (edof, rho, Ke) are those of the fp32 matvec; the
// iteration's vectors (u, r, z, p, q and the Jacobi scaling) are fp64, every
// inner product is accumulated in fp64 and the scalars are fp64, so an
// iteration needs no host round trip.  The matvec inside the solver
// (k_fe_matvec64) is the fused one with fp64 element products: a stiffness
// operator applied to a smooth vector cancels most of each sum (the element
// matrix annihilates rigid motions), and with fp32 sums that cancellation
// error more than doubles the iteration count already at kappa ~ 2e4.  With
// fp32 vectors the iteration still lost conjugacy at kappa ~ 1e6 (the
// rounding of r and p each step is ~1e-7 against kappa * 1e-16 for fp64)
// and needed 1.0x-1.6x the fp64 count depending on rounding details; with
// fp64 vectors it follows the fp64 iteration.  The caller's f and u stay
// fp32: u is read once at the start and written once at the end.
//
// Its scatter adds 64-bit fixed-point integers, not floating-point values:
// each contribution v becomes round(v * 2^k) and is added with an integer
// atomic, and integer addition does not depend on the order of the adds.
// The product K x is therefore the same bit for bit in every run, and so is
// the whole iteration, its count included.  The scale 2^k is set per
// product from a bound on |(K x)_i|: G * max|x|, with G = (most elements on
// one DOF) * max_e rho_e^p * max_a sum_b |Ke_ab| computed once per operator,
// and k chosen so that the bound times 2^k stays below 2^62.  The rounding
// of one contribution is at most 2^-(k+1) <= G max|x| 2^-63, below the
// rounding of an fp64 running sum of the same terms.  Every kernel that
// produces a vector the matvec takes next also stores per-workgroup maxima
// of |x|; the matvec reduces them, and the kernel that consumes K x reads
// the accumulator back with the same k, rounds it to fp32 and clears it.
// The Jacobi diagonal is summed the same way.
//
// Inner products: every workgroup stores its partial sums; the next kernel
// in the stream, in every one of its workgroups, adds all partials in the
// same fixed order and so obtains the same scalar (alpha, beta, norms)
// bit for bit.  Kernel boundaries make the partials visible across the
// XCDs' L2 caches; no device-scope fence, which on gfx950 writes back and
// invalidates the L2, is issued inside a kernel.  Partials of consecutive
// iterations alternate between two slots, so a kernel never overwrites
// sums that a workgroup of the same kernel still reads.  The CG recurrences
// are taken in the one-reduction form of Chronopoulos and Gear (the same
// iterates as the textbook form in exact arithmetic): besides r and
// z = D^-1 r it carries w = K z and s = K p, so that r.z and w.z, the only
// inner products of an iteration, are both known before the vector
// updates.  One iteration i is three launches: the matvec acc = K z_i;
// k_cg_dot (convergence test on r_i.r_i, partial w.z); k_cg_step (beta,
// alpha, p = z + beta p, s = w + beta s, x += alpha p, r -= alpha s,
// z = D^-1 r; partial r.z, r.r into slot (i + 1) & 1).
// Once the state says "done", these kernels return at once; the host checks
// the state every PCG_CHECK iterations.  Reductions and matvecs are both
// deterministic, so two solves of the same system agree bit for bit.
#include "common.hpp"
#include "fem_common.hpp"

#include <algorithm>
#include <cmath>

namespace spmv {
namespace {

typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef long long i64x2 __attribute__((ext_vector_type(2)));

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
    double op_bound;    // G: |(K x)_i| <= G max|x| for every i
    int iter, max_iter;
    int done;           // converged, capped or broken down
    int bad;            // 1: diagonal entry not positive, 2: p.Kp <= 0, 4: zero vector
    int acc_exp;        // k of the accumulator's fixed point (value = acc * 2^-k)
    double cg_gamma[2]; // r.z of CG step i, in slot i & 1 (read by step i + 1)
    double cg_alpha[2]; // alpha of CG step i, in slot i & 1
};

size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

// Workspace: state | partials: 2 slots x SV_NQ x SV_MAX_BLOCKS doubles, then
// SV_MAX_BLOCKS more for w.z (CG) and SV_MAX_BLOCKS for the maxima of |x| of the
// next matvec's input | lambda history (max_history doubles) | vectors of
// n_dof doubles: dinv r z p kp u (PCG; kp = K p) | vectors of n_dof floats: v w
// (eigenvalue iterations) | the fixed-point matvec accumulator (n_dof
// int64, all zero between uses).
constexpr int NVEC64 = 6, NVEC32 = 2;
struct Layout {
    size_t state, partials, hist, vec64[NVEC64], vec32[NVEC32], acc, total;
};

Layout layout(int64_t n_dof, int64_t max_history) {
    Layout L;
    size_t at = 0;
    L.state = at;
    at += round256(sizeof(SolverState));
    L.partials = at;
    at += round256(sizeof(double) * (2 * SV_NQ + 2) * SV_MAX_BLOCKS);
    L.hist = at;
    at += round256(sizeof(double) * (size_t)std::max<int64_t>(max_history, 1));
    for (int k = 0; k < NVEC64; ++k) {
        L.vec64[k] = at;
        at += round256(sizeof(double) * (size_t)std::max<int64_t>(n_dof, 1));
    }
    for (int k = 0; k < NVEC32; ++k) {
        L.vec32[k] = at;
        at += round256(sizeof(float) * (size_t)std::max<int64_t>(n_dof, 1));
    }
    L.acc = at;
    at += round256(sizeof(long long) * (size_t)std::max<int64_t>(n_dof, 1));
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
// The partials of w.z = (K z).z of a CG iteration.
__device__ __forceinline__ double *wz_slot(double *partials) {
    return partials + (size_t)2 * SV_NQ * SV_MAX_BLOCKS;
}
// Per-workgroup maxima of |x| of the vector the next matvec takes.
__device__ __forceinline__ double *xmax_slot(double *partials) {
    return partials + (size_t)(2 * SV_NQ + 1) * SV_MAX_BLOCKS;
}
__device__ __forceinline__ const double *xmax_slot(const double *partials) {
    return partials + (size_t)(2 * SV_NQ + 1) * SV_MAX_BLOCKS;
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

// Maximum over the workgroup, returned in every thread.
__device__ double block_max(double v) {
    __shared__ double red[SV_WG / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    double m = red[0];
    for (int k = 1; k < SV_WG / 64; ++k) m = fmax(m, red[k]);
    return m;
}

// This workgroup's max |x| (m: this thread's) into the xmax slot.
__device__ void store_xmax(double m, double *partials) {
    m = block_max(m);
    if (threadIdx.x == 0) xmax_slot(partials)[blockIdx.x] = m;
}

// 2^-k as a double (k may be negative).
__device__ __forceinline__ double fix_unit(int k) { return ldexp(1.0, -k); }

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

__global__ void k_sv_zero64(int n, long long *__restrict__ y) {
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) y[i] = 0;
}

// Per-workgroup maxima of |x| into the xmax slot (for a matvec whose input
// was not produced by one of the iteration kernels).
template <typename X>
__global__ void k_sv_absmax(int n, const X *__restrict__ x, double *__restrict__ partials) {
    double m = 0.0;
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) m = fmax(m, fabs((double)x[i]));
    store_xmax(m, partials);
}

// The operator bound G (see the file comment), in three steps.  1: counts
// of elements per DOF into cnt (int32, zero on entry).
__global__ void k_op_count(int n_elem, int n_dof, const int *__restrict__ edof, int *__restrict__ cnt) {
    const int64_t k = (int64_t)blockIdx.x * SV_WG + threadIdx.x;
    if (k >= (int64_t)n_elem * NDOF_E) return;
    const int d = edof[k];
    if ((unsigned)d < (unsigned)n_dof) atomicAdd(cnt + d, 1);
}

// 2: per-workgroup maxima of the counts (cleared for the accumulator again)
// into slot 0 quantity 0 and of rho_e^p into slot 0 quantity 1.
__global__ void k_op_partials(int n_elem, int n_dof, const float *__restrict__ rho, int penalty,
                              int *__restrict__ cnt, double *__restrict__ partials) {
    double mc = 0.0, ms = 0.0;
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n_dof; i += gridDim.x * SV_WG) {
        mc = fmax(mc, (double)cnt[i]);
        cnt[i] = 0;
    }
    for (int e = blockIdx.x * SV_WG + threadIdx.x; e < n_elem; e += gridDim.x * SV_WG) {
        double sv = 1.0;
        for (int k = 0; k < penalty; ++k) sv *= (double)rho[e];
        ms = fmax(ms, fabs(sv));
    }
    mc = block_max(mc);
    ms = block_max(ms);
    if (threadIdx.x == 0) {
        slot(partials, 0, 0)[blockIdx.x] = mc;
        slot(partials, 0, 1)[blockIdx.x] = ms;
    }
}

// 3 (one workgroup): G = max count * max rho^p * max_a sum_b |Ke_ab|.
__global__ void k_op_bound(int nb, const double *__restrict__ partials, const float *__restrict__ Ke,
                           SolverState *st) {
    double mc = 0.0, ms = 0.0, mk = 0.0;
    for (int b = threadIdx.x; b < nb; b += SV_WG) {
        mc = fmax(mc, slot(partials, 0, 0)[b]);
        ms = fmax(ms, slot(partials, 0, 1)[b]);
    }
    if (threadIdx.x < NDOF_E) {
        for (int b = 0; b < NDOF_E; ++b) mk += fabs((double)Ke[threadIdx.x * NDOF_E + b]);
    }
    mc = block_max(mc);
    ms = block_max(ms);
    mk = block_max(mk);
    if (threadIdx.x == 0) st->op_bound = mc * ms * mk;
}

// Fixed-point exponent for a product whose input has max|x| = xm: the
// largest k with G * xm * 2^k < 2^62 (0 when the bound is 0, i.e. K x = 0).
__device__ __forceinline__ int fix_exponent(double G, double xm) {
    const double b = G * xm;
    if (!(b > 0.0) || !(b < INFINITY)) return 0;
    int e;
    (void)frexp(b, &e);   // b < 2^e
    return 62 - e;
}

// acc += sum_e rho_e^p P_e^T Ke P_e x in fixed point, with the element
// product in fp64 (products of fp32 values are exact in fp64).  The fused
// shape of fem_matvec_apply: one lane per element, Ke through the scalar
// cache, 24 gathers, and the contributions merged along x-lines of nodes in
// LDS before the integer atomic adds.  The scale comes from the nb maxima
// of |x| in the xmax slot and the operator bound; workgroup 0 records its
// exponent for the consumer.  x is fp32 (power iteration, the initial
// guess) or fp64 (the PCG direction).  Does nothing when `check_done` and
// the state says the iteration is done.
template <typename X>
__global__ __launch_bounds__(SV_WG) void k_fe_matvec64(int n_elem, int n_dof, const int *__restrict__ edof,
                                                       const float *__restrict__ rho, int penalty,
                                                       const float *__restrict__ Ke, const X *__restrict__ x,
                                                       long long *__restrict__ acc, const double *__restrict__ partials,
                                                       int nb, SolverState *st, int check_done) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    if (check_done && st->done) return;   // uniform
    __shared__ int line_dof[SV_WG / 64][4 * 3 * 65];
    __shared__ double line_val[SV_WG / 64][4 * 3 * 65];
    double xm = 0.0;
    for (int b = threadIdx.x; b < nb; b += SV_WG) xm = fmax(xm, xmax_slot(partials)[b]);
    const int kx = fix_exponent(st->op_bound, block_max(xm));
    if (blockIdx.x == 0 && threadIdx.x == 0) st->acc_exp = kx;
    const double unit = ldexp(1.0, kx);
    // lanes past the last element stay for the wave exchange, with index -1
    // the workgroups one XCD receives (workgroup i goes to XCD i % 8) take a
    // contiguous range of elements, whose x and accumulator lines then stay
    // in that XCD's L2 (0.8 us per PCG iteration; the fused fp32 kernel,
    // whose memory-side atomics dominate, is slower this way)
    int wg;
    {
        const int nw = gridDim.x, w = blockIdx.x, q = nw / 8, r = nw % 8, xcd = w % 8, idx = w / 8;
        wg = xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
    }
    const int e = wg * SV_WG + threadIdx.x;
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
    X u[NDOF_E];
#pragma unroll
    for (int b = 0; b < NDOF_E; ++b) u[b] = x[(unsigned)d[b] < (unsigned)n_dof ? d[b] : 0];
#pragma unroll
    for (int b = 0; b < NDOF_E; ++b) u[b] = (unsigned)d[b] < (unsigned)n_dof ? u[b] : X(0);
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
    // products finished before the scatter (else the compiler sinks them
    // into it and spills Ke from the scalar registers to vector lanes)
#pragma unroll
    for (int a = 0; a < NDOF_E; ++a) asm volatile("" : "+v"(fa[a]));
    fe_scatter_lines(
        d, fa, n_dof,
        [acc, unit](int i, bool on, double v) {
            if (on)
                atomicAdd(reinterpret_cast<unsigned long long *>(acc + i),
                          (unsigned long long)__double2ll_rn(v * unit));
        },
        line_dof[threadIdx.x >> 6], line_val[threadIdx.x >> 6]);
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

// The solver's diagonal in fixed point: acc[edof[e][a]] += rho_e^p Ke[a][a]
// scaled by 2^k with k from the operator bound (Ke_aa <= sum_b |Ke_ab|, so
// each DOF's sum is within G), added with integer atomics.
__global__ void k_fe_diag_fixed(int n_elem, int n_dof, const int *__restrict__ edof, const float *__restrict__ rho,
                                int penalty, const float *__restrict__ Ke, long long *__restrict__ acc,
                                const SolverState *st) {
    const int e = blockIdx.x * SV_WG + threadIdx.x;
    if (e >= n_elem) return;
    const double unit = ldexp(1.0, fix_exponent(st->op_bound, 1.0));
    double s = 1.0;
    for (int k = 0; k < penalty; ++k) s *= (double)rho[e];
#pragma unroll 4
    for (int a = 0; a < NDOF_E; ++a) {
        const int d = edof[(size_t)e * NDOF_E + a];
        if ((unsigned)d < (unsigned)n_dof)
            atomicAdd(reinterpret_cast<unsigned long long *>(acc + d),
                      (unsigned long long)__double2ll_rn(s * (double)Ke[a * NDOF_E + a] * unit));
    }
}

// dinv = 1 / diag with diag read from the fixed-point accumulator (which is
// cleared), flagging an entry that is not positive and finite.
__global__ void k_pcg_dinv(int n, long long *__restrict__ acc, double *__restrict__ dinv, SolverState *st) {
    const double inv_unit = fix_unit(fix_exponent(st->op_bound, 1.0));
    bool ok = true;
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) {
        const double d = (double)acc[i] * inv_unit;
        acc[i] = 0;
        ok = ok && (d > 0.0) && (d < INFINITY);
        dinv[i] = 1.0 / d;
    }
    if (!ok) atomicOr(&st->bad, 1);
}

// Start of PCG, with acc = K u: u64 = u, r = f - acc (acc cleared),
// z = D^-1 r; partial r.z, r.r, f.f into slot 0 (read by CG step 0), and the
// maxima of |z| for the first matvec.
__global__ void k_pcg_start(int n, const float *__restrict__ f, const float *__restrict__ u, long long *__restrict__ acc,
                            double *__restrict__ u64, double *__restrict__ r, const double *__restrict__ dinv,
                            double *__restrict__ z, double *__restrict__ partials, const SolverState *st) {
    const double inv_unit = fix_unit(st->acc_exp);
    double v[3] = {0.0, 0.0, 0.0};
    double m = 0.0;
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) {
        const double fi = f[i];
        const double ri = fi - (double)acc[i] * inv_unit;
        acc[i] = 0;
        const double zi = dinv[i] * ri;
        u64[i] = u[i];
        r[i] = ri;
        z[i] = zi;
        v[0] += ri * zi;
        v[1] += ri * ri;
        v[2] += fi * fi;
        m = fmax(m, fabs(zi));
    }
    double *const dst[3] = {slot(partials, 0, 0), slot(partials, 0, 1), slot(partials, 0, 2)};
    store_partials<3>(v, dst);
    store_xmax(m, partials);
}

// One workgroup: f.f and r.r of the start, and whether there is anything to do.
__global__ void k_pcg_start_fin(int nb, const double *__restrict__ partials, SolverState *st) {
    const double *const src[2] = {slot(partials, 0, 1), slot(partials, 0, 2)};
    double t[2];
    total_partials<2>(src, nb, t);
    if (threadIdx.x == 0) {
        st->rr = t[0];
        st->ff = t[1];
        st->iter = 0;
        st->done = (st->bad != 0) || st->max_iter <= 0 || t[0] <= st->rtol2 * t[1];
    }
}

// CG iteration i, first part (acc = K z_i from the matvec, left in place):
// stop when r_i.r_i <= rtol^2 f.f or i reached the cap (i steps taken so
// far), clearing the accumulator, else partial w.z with w = acc.
__global__ void k_cg_dot(int n, int i, long long *__restrict__ acc, const double *__restrict__ z,
                         double *__restrict__ partials, SolverState *st) {
    if (st->done) return;   // uniform: set by an earlier launch
    const double *const src[1] = {slot(partials, i & 1, 1)};
    double t[1];
    total_partials<1>(src, gridDim.x, t);
    const bool stop = t[0] <= st->rtol2 * st->ff || i >= st->max_iter;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        st->iter = i;
        st->rr = t[0];
        if (stop) st->done = 1;
    }
    if (stop) {   // uniform: every workgroup has the same totals; the accumulator is left all zero
        for (int j = blockIdx.x * SV_WG + threadIdx.x; j < n; j += gridDim.x * SV_WG) acc[j] = 0;
        return;
    }
    const double inv_unit = fix_unit(st->acc_exp);
    double v[1] = {0.0};
    // two DOFs per thread and step, 16-byte loads (the workspace vectors are 256-byte aligned)
    const int n2 = n >> 1;
    const i64x2 *acc2 = reinterpret_cast<const i64x2 *>(acc);
    const f64x2 *z2 = reinterpret_cast<const f64x2 *>(z);
    for (int j = blockIdx.x * SV_WG + threadIdx.x; j < n2; j += gridDim.x * SV_WG) {
        const i64x2 a = acc2[j];
        const f64x2 zz = z2[j];
        v[0] += ((double)a.x * inv_unit) * zz.x;
        v[0] += ((double)a.y * inv_unit) * zz.y;
    }
    if ((n & 1) && blockIdx.x == 0 && threadIdx.x == 0) v[0] += ((double)acc[n - 1] * inv_unit) * z[n - 1];
    double *const dst[1] = {wz_slot(partials)};
    store_partials<1>(v, dst);
}

// CG iteration i, second part: gamma = r_i.z_i (slot i & 1), delta = w.z;
// beta = gamma / gamma_{i-1}, alpha = gamma / (delta - beta gamma /
// alpha_{i-1}) (step 0: beta = 0, alpha = gamma / delta, p = z, s = w);
// p = z + beta p, s = w + beta s (w = acc, which is cleared), x += alpha p,
// r -= alpha s, z = D^-1 r; partial r.z and r.r into slot (i + 1) & 1 and
// the maxima of |z| for the next matvec.  A denominator that is not
// positive stops the iteration (the operator is not SPD).
__global__ void k_cg_step(int n, int i, long long *__restrict__ acc, const double *__restrict__ dinv,
                          double *__restrict__ x, double *__restrict__ r, double *__restrict__ z,
                          double *__restrict__ p, double *__restrict__ s, double *__restrict__ partials,
                          SolverState *st) {
    if (st->done) return;
    const double *const src[2] = {slot(partials, i & 1, 0), wz_slot(partials)};
    double t[2];
    total_partials<2>(src, gridDim.x, t);
    const double g = t[0], d = t[1];
    double beta = 0.0, den = d;
    if (i > 0) {
        beta = g / st->cg_gamma[(i - 1) & 1];
        den = d - beta * g / st->cg_alpha[(i - 1) & 1];
    }
    if (!(den > 0.0)) {   // uniform; the accumulator is left all zero
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            st->bad |= 2;
            st->done = 1;
        }
        for (int j = blockIdx.x * SV_WG + threadIdx.x; j < n; j += gridDim.x * SV_WG) acc[j] = 0;
        return;
    }
    const double alpha = g / den;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        st->cg_gamma[i & 1] = g;
        st->cg_alpha[i & 1] = alpha;
    }
    const double inv_unit = fix_unit(st->acc_exp);
    double v[2] = {0.0, 0.0};
    double m = 0.0;
    // one DOF: w = acc (cleared), p, s, x, r, z updated; r.z, r.r, max|z| collected
    auto dof = [&](long long a, double &pj, double &sj, double &xj, double &rj, double dj, double &zj) {
        const double wj = (double)a * inv_unit;
        pj = i > 0 ? fma(beta, pj, zj) : zj;
        sj = i > 0 ? fma(beta, sj, wj) : wj;
        xj = fma(alpha, pj, xj);
        rj = fma(-alpha, sj, rj);
        zj = dj * rj;
        v[0] += rj * zj;
        v[1] += rj * rj;
        m = fmax(m, fabs(zj));
    };
    // two DOFs per thread and step, 16-byte accesses (the workspace vectors are 256-byte aligned)
    const int n2 = n >> 1;
    for (int j = blockIdx.x * SV_WG + threadIdx.x; j < n2; j += gridDim.x * SV_WG) {
        const i64x2 a = reinterpret_cast<const i64x2 *>(acc)[j];
        const f64x2 pv = reinterpret_cast<const f64x2 *>(p)[j];
        const f64x2 sv = i > 0 ? reinterpret_cast<const f64x2 *>(s)[j] : f64x2{0.0, 0.0};
        const f64x2 xv = reinterpret_cast<const f64x2 *>(x)[j];
        const f64x2 rv = reinterpret_cast<const f64x2 *>(r)[j];
        const f64x2 dv = reinterpret_cast<const f64x2 *>(dinv)[j];
        const f64x2 zv = reinterpret_cast<const f64x2 *>(z)[j];
        double pp[2] = {pv.x, pv.y}, ss[2] = {sv.x, sv.y}, xx[2] = {xv.x, xv.y}, rr[2] = {rv.x, rv.y},
               zz[2] = {zv.x, zv.y};
        dof(a.x, pp[0], ss[0], xx[0], rr[0], dv.x, zz[0]);
        dof(a.y, pp[1], ss[1], xx[1], rr[1], dv.y, zz[1]);
        reinterpret_cast<i64x2 *>(acc)[j] = i64x2{0, 0};
        reinterpret_cast<f64x2 *>(p)[j] = f64x2{pp[0], pp[1]};
        reinterpret_cast<f64x2 *>(s)[j] = f64x2{ss[0], ss[1]};
        reinterpret_cast<f64x2 *>(x)[j] = f64x2{xx[0], xx[1]};
        reinterpret_cast<f64x2 *>(r)[j] = f64x2{rr[0], rr[1]};
        reinterpret_cast<f64x2 *>(z)[j] = f64x2{zz[0], zz[1]};
    }
    if ((n & 1) && blockIdx.x == 0 && threadIdx.x == 0) {
        const int j = n - 1;
        double pj = p[j], sj = i > 0 ? s[j] : 0.0, xj = x[j], rj = r[j], zj = z[j];
        dof(acc[j], pj, sj, xj, rj, dinv[j], zj);
        acc[j] = 0;
        p[j] = pj;
        s[j] = sj;
        x[j] = xj;
        r[j] = rj;
        z[j] = zj;
    }
    double *const dst[2] = {slot(partials, (i + 1) & 1, 0), slot(partials, (i + 1) & 1, 1)};
    store_partials<2>(v, dst);
    store_xmax(m, partials);
}

// The solution back into the caller's fp32 u.
__global__ void k_pcg_store_u(int n, const double *__restrict__ u64, float *__restrict__ u) {
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) u[i] = (float)u64[i];
}

// Partial ||v||^2 into slot 0.
__global__ void k_sv_norm(int n, const float *__restrict__ v, double *__restrict__ partials) {
    double s[1] = {0.0};
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) s[0] += (double)v[i] * v[i];
    double *const dst[1] = {slot(partials, 0, 0)};
    store_partials<1>(s, dst);
}

// dst = src / ||src|| with ||src||^2 from slot 0 (a zero vector is flagged
// and gives zeros); the maxima of |dst| for the next matvec.
__global__ void k_sv_scale(int n, const float *__restrict__ src, float *__restrict__ dst,
                           double *__restrict__ partials, SolverState *st) {
    const double *const in[1] = {slot(partials, 0, 0)};
    double t[1];
    total_partials<1>(in, gridDim.x, t);
    if (!(t[0] > 0.0) && blockIdx.x == 0 && threadIdx.x == 0) st->bad |= 4;
    const float s = t[0] > 0.0 ? (float)(1.0 / sqrt(t[0])) : 0.0f;
    double m = 0.0;
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) {
        const float di = src[i] * s;
        dst[i] = di;
        m = fmax(m, fabs((double)di));
    }
    store_xmax(m, partials);
}

// Power-iteration step after acc = K v (v of unit length): w = acc (acc
// cleared); partial v.w, w.w into slot 0.
__global__ void k_pow_dots(int n, const float *__restrict__ v, long long *__restrict__ acc, float *__restrict__ w,
                           double *__restrict__ partials, const SolverState *st) {
    const double inv_unit = fix_unit(st->acc_exp);
    double s[2] = {0.0, 0.0};
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) {
        const double wi = (double)acc[i] * inv_unit;
        acc[i] = 0;
        w[i] = (float)wi;
        s[0] += (double)v[i] * wi;
        s[1] += wi * wi;
    }
    double *const dst[2] = {slot(partials, 0, 0), slot(partials, 0, 1)};
    store_partials<2>(s, dst);
}

// v = w / ||w||, and the Rayleigh quotient v.w of the previous v into
// hist[k] (both from slot 0); the maxima of |v| for the next matvec.
__global__ void k_pow_next(int n, int k, const float *__restrict__ w, float *__restrict__ v,
                           double *__restrict__ partials, double *__restrict__ hist, SolverState *st) {
    const double *const in[2] = {slot(partials, 0, 0), slot(partials, 0, 1)};
    double t[2];
    total_partials<2>(in, gridDim.x, t);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        hist[k] = t[0];
        if (!(t[1] > 0.0)) st->bad |= 4;
    }
    const float s = t[1] > 0.0 ? (float)(1.0 / sqrt(t[1])) : 0.0f;
    double m = 0.0;
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) {
        const float vi = w[i] * s;
        v[i] = vi;
        m = fmax(m, fabs((double)vi));
    }
    store_xmax(m, partials);
}

// Partial v.acc (acc = K v; acc cleared) into slot 0.
__global__ void k_rayleigh(int n, const float *__restrict__ v, long long *__restrict__ acc,
                           double *__restrict__ partials, const SolverState *st) {
    const double inv_unit = fix_unit(st->acc_exp);
    double s[1] = {0.0};
    for (int i = blockIdx.x * SV_WG + threadIdx.x; i < n; i += gridDim.x * SV_WG) {
        s[0] += (double)v[i] * ((double)acc[i] * inv_unit);
        acc[i] = 0;
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
    double *partials, *hist;
    long long *acc;
    double *dinv, *r, *z, *p, *kp, *u;  // PCG (kp: K p, the CG recurrence's s)
    float *v, *w;                       // eigenvalue iterations
};

Work carve(void *ws, const Layout &L) {
    char *b = static_cast<char *>(ws);
    Work W;
    W.st = reinterpret_cast<SolverState *>(b + L.state);
    W.partials = reinterpret_cast<double *>(b + L.partials);
    W.hist = reinterpret_cast<double *>(b + L.hist);
    W.acc = reinterpret_cast<long long *>(b + L.acc);
    double **v64[NVEC64] = {&W.dinv, &W.r, &W.z, &W.p, &W.kp, &W.u};
    for (int k = 0; k < NVEC64; ++k) *v64[k] = reinterpret_cast<double *>(b + L.vec64[k]);
    float **v32[NVEC32] = {&W.v, &W.w};
    for (int k = 0; k < NVEC32; ++k) *v32[k] = reinterpret_cast<float *>(b + L.vec32[k]);
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

// acc = K x in fixed point (acc must hold zeros).  The maxima of |x| must
// be in the xmax slot (from the kernel that wrote x) unless `find_max`, in
// which case they are computed first.  With `check_done`, skipped once the
// state says done.
template <typename X>
spmv_status matvec64(const Operator &A, const Work &W, const X *x, hipStream_t st, bool find_max,
                     bool check_done) {
    const int nb = vec_blocks(A.n_dof);
    if (find_max) {
        k_sv_absmax<X><<<nb, SV_WG, 0, st>>>(A.n_dof, x, W.partials);
        SPMV_LAUNCHED("k_sv_absmax");
    }
    if (A.n_elem == 0) return SPMV_OK;   // K x = 0: the accumulator holds zeros at any exponent
    k_fe_matvec64<X><<<(int)ceil_div(A.n_elem, SV_WG), SV_WG, 0, st>>>(A.n_elem, A.n_dof, A.edof, A.rho,
                                                                       A.penalty, A.Ke, x, W.acc, W.partials, nb,
                                                                       W.st, check_done ? 1 : 0);
    SPMV_LAUNCHED("k_fe_matvec64");
    return SPMV_OK;
}

// The operator bound G into the state (the accumulator must hold zeros;
// it does again afterwards).
spmv_status prepare_bound(const Operator &A, const Work &W, hipStream_t st) {
    const int nb = vec_blocks(std::max(A.n_dof, A.n_elem));
    if (A.n_elem > 0) {
        k_op_count<<<(int)ceil_div((int64_t)A.n_elem * NDOF_E, SV_WG), SV_WG, 0, st>>>(
            A.n_elem, A.n_dof, A.edof, reinterpret_cast<int *>(W.acc));
        SPMV_LAUNCHED("k_op_count");
    }
    k_op_partials<<<nb, SV_WG, 0, st>>>(A.n_elem, A.n_dof, A.rho, A.penalty, reinterpret_cast<int *>(W.acc),
                                       W.partials);
    SPMV_LAUNCHED("k_op_partials");
    k_op_bound<<<1, SV_WG, 0, st>>>(nb, W.partials, A.Ke, W.st);
    SPMV_LAUNCHED("k_op_bound");
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

// Sets up D^-1 (once per operator) in W.dinv from the fixed-point
// diagonal; the operator bound must be in the state.
spmv_status prepare_dinv(const Operator &A, const Work &W, hipStream_t st) {
    if (A.n_elem > 0) {
        k_fe_diag_fixed<<<(int)ceil_div(A.n_elem, SV_WG), SV_WG, 0, st>>>(A.n_elem, A.n_dof, A.edof, A.rho,
                                                                          A.penalty, A.Ke, W.acc, W.st);
        SPMV_LAUNCHED("k_fe_diag_fixed");
    }
    k_pcg_dinv<<<vec_blocks(A.n_dof), SV_WG, 0, st>>>(A.n_dof, W.acc, W.dinv, W.st);
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
    s = matvec64(A, W, u, st, true, false);
    if (s != SPMV_OK) return s;
    k_pcg_start<<<nb, SV_WG, 0, st>>>(n, f, u, W.acc, W.u, W.r, W.dinv, W.z, W.partials, W.st);
    SPMV_LAUNCHED("k_pcg_start");
    k_pcg_start_fin<<<1, SV_WG, 0, st>>>(nb, W.partials, W.st);
    SPMV_LAUNCHED("k_pcg_start_fin");
    s = read_state(W, &h, st);
    if (s != SPMV_OK) return s;
    int k = 0;
    while (!h.done && k < max_iter) {
        const int batch = std::min(PCG_CHECK, max_iter - k);
        for (int j = 0; j < batch; ++j, ++k) {
            s = matvec64(A, W, W.z, st, false, true);   // w = K z_k
            if (s != SPMV_OK) return s;
            k_cg_dot<<<nb, SV_WG, 0, st>>>(n, k, W.acc, W.z, W.partials, W.st);
            SPMV_LAUNCHED("k_cg_dot");
            k_cg_step<<<nb, SV_WG, 0, st>>>(n, k, W.acc, W.dinv, W.u, W.r, W.z, W.p, W.kp, W.partials, W.st);
            SPMV_LAUNCHED("k_cg_step");
        }
        s = read_state(W, &h, st);
        if (s != SPMV_OK) return s;
    }
    if (!h.done) {   // the cap: the last residual's norm and the count (the accumulator is already clear)
        k_cg_dot<<<nb, SV_WG, 0, st>>>(n, k, W.acc, W.z, W.partials, W.st);
        SPMV_LAUNCHED("k_cg_dot");
        s = read_state(W, &h, st);
        if (s != SPMV_OK) return s;
    }
    k_pcg_store_u<<<nb, SV_WG, 0, st>>>(n, W.u, u);
    SPMV_LAUNCHED("k_pcg_store_u");
    if (h.bad & 1) return fail(SPMV_ERR_INVALID_MATRIX, "a diagonal entry of the operator is not positive");
    if (h.bad & 2) return fail(SPMV_ERR_INVALID_MATRIX, "p.Kp <= 0: the operator is not positive definite");
    if (iters) *iters = h.iter;
    if (relres) *relres = h.ff > 0.0 ? std::sqrt(h.rr / h.ff) : std::sqrt(h.rr);
    return SPMV_OK;
}

// Clears the state and the accumulator, then puts the operator bound in
// the state.
spmv_status reset_state(const Operator &A, const Work &W, hipStream_t st) {
    const int n = A.n_dof;
    k_sv_zero64<<<vec_blocks(n), SV_WG, 0, st>>>(n, W.acc);
    SPMV_LAUNCHED("k_sv_zero64");
    spmv_status s = write_state(W, SolverState{}, st);
    if (s != SPMV_OK) return s;
    return prepare_bound(A, W, st);
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
    s = reset_state(A, W, st);
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
    s = reset_state(A, W, st);
    if (s != SPMV_OK) return s;
    s = normalise_into(W, n, v0, W.v, st);
    if (s != SPMV_OK) return s;
    for (int k = 0; k < iterations; ++k) {
        s = matvec64(A, W, W.v, st, false, false);
        if (s != SPMV_OK) return s;
        k_pow_dots<<<nb, SV_WG, 0, st>>>(n, W.v, W.acc, W.w, W.partials, W.st);
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
    s = reset_state(A, W, st);
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
        s = matvec64(A, W, W.v, st, false, false);
        if (s != SPMV_OK) return s;
        k_rayleigh<<<nb, SV_WG, 0, st>>>(n, W.v, W.acc, W.partials, W.st);
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
