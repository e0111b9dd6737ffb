// Finite-element stiffness matvec on gfx950.
//
// "Fused GPU SpMV kernel optimisation: from bandwidth bottleneck to BF16
// precision", section 2.1: the unfused form gathers every element's 24 DOFs
// into a per-element vector, multiplies by the element matrix, and scatters
// the result with atomic adds, one kernel per stage with the intermediates
// in DRAM.  Section 2.2: the fused form keeps the gathered vector and the
// product in registers and issues one launch.  Section 5.1 gives the fused
// kernel's shape (one thread per element), section 5.2 notes that a Ke shared
// by all elements belongs in fast on-chip memory.
//
// Operator: y = alpha * sum_e rho_e^p * P_e^T Ke P_e x + beta * y, with one
// shared Ke (24 x 24, row-major) scaled per element by the SIMP factor
// rho_e^p.  An edof entry outside [0, n_dof) (the mesh uses -1 for a
// clamped DOF) contributes no gather and no scatter.
//
// gfx950 shape of the fused kernel: one lane per element; Ke is the same
// for every lane, so the product reads it with scalar loads (the constant
// cache is the on-chip home of section 5.2 here) and uses it as scalar
// operands of the FMAs, with no LDS staging and no barrier; the element's
// 24 DOF indices are read with six 16-byte loads, 24 gathers of x,
// 576 FMAs, then the wave's contributions are merged along x-lines of
// nodes in LDS (the face shared with the next lane's element is summed
// there, all four node lines in one pass) and go out as fp32 atomic adds
// (hardware buffer atomics, issued unconditionally with out-of-range
// offsets where there is nothing to add) with consecutive lanes on
// consecutive DOFs: 12 instead of 24 adds per element when elements are
// numbered x-fastest, ~16 lanes per memory-side request.  The beta pass
// runs first as a separate small kernel, because atomics only add.
#include "common.hpp"
#include "fem_common.hpp"

#include <algorithm>
#include <mutex>

// Device scratch of fem_matvec_threestage_noalloc: the per-element vectors U
// and F of one chunk of at most FE_NOALLOC_CHUNK elements (2 * 65536 * 24
// floats = 12 MiB).  Each GPU the library runs on holds its own copy until
// the process ends.  Host code never uses this name as an address: the
// entry point takes the device address from hipGetSymbolAddress once per
// device.
constexpr int FE_NOALLOC_CHUNK = 65536;
static __device__ __align__(256) float scratch[2 * FE_NOALLOC_CHUNK * 24];

namespace spmv {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int FE_WG = 256;
constexpr int NDOF_E = 24;
constexpr int MAX_PENALTY = 8;

__device__ __forceinline__ float simp(float r, int p) {
    float s = 1.0f;
    for (int k = 0; k < p; ++k) s *= r;
    return s;
}

// y = beta * y, and y = 0 without reading y when beta = 0.  With y 16-byte
// aligned: 16-byte accesses over a grid-stride loop of 8 workgroups per CU
// (the streaming kernels' shape; as fast as a device fill at 2.7 MB and
// 1.5x faster than one float per thread at 43 MB), the last n % 4 entries
// by block 0; otherwise one float per thread.
__global__ __launch_bounds__(256) void k_fe_beta(int n, float beta, float *__restrict__ y) {
    const int n4 = n >> 2;
    f32x4 *y4 = reinterpret_cast<f32x4 *>(y);
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n4; i += gridDim.x * 256) {
        f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
        if (beta != 0.0f) v = beta * y4[i];
        y4[i] = v;
    }
    if (blockIdx.x == 0 && (int)threadIdx.x < (n & 3)) {
        const int i = 4 * n4 + threadIdx.x;
        y[i] = beta != 0.0f ? beta * y[i] : 0.0f;
    }
}

__global__ void k_fe_beta1(int n, float beta, float *__restrict__ y) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) y[i] = beta != 0.0f ? beta * y[i] : 0.0f;
}

void beta_launch(int n, float beta, float *y, hipStream_t st) {
    if (aligned16(y)) {
        const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(n, 1024), 8 * (int64_t)device_cu_count()));
        k_fe_beta<<<grid, 256, 0, st>>>(n, beta, y);
    } else {
        k_fe_beta1<<<(int)ceil_div(n, 256), 256, 0, st>>>(n, beta, y);
    }
}

// Ke (576 floats, 16-byte aligned) into LDS: 144 16-byte vectors, all loads
// issued before the barrier.
__device__ __forceinline__ void stage_ke(float *ke, const float *__restrict__ Ke) {
    if (threadIdx.x < NDOF_E * NDOF_E / 4)
        reinterpret_cast<f32x4 *>(ke)[threadIdx.x] = reinterpret_cast<const f32x4 *>(Ke)[threadIdx.x];
    __syncthreads();
}

__device__ __forceinline__ void load_edof(const int *__restrict__ edof, int e, int (&d)[NDOF_E]) {
    const i32x4 *p = reinterpret_cast<const i32x4 *>(edof + (size_t)e * NDOF_E);
#pragma unroll
    for (int k = 0; k < NDOF_E / 4; ++k) {
        const i32x4 q = __builtin_nontemporal_load(p + k);
        d[4 * k + 0] = q.x;
        d[4 * k + 1] = q.y;
        d[4 * k + 2] = q.z;
        d[4 * k + 3] = q.w;
    }
}

// Buffer resources for x and y (byte offsets below 2 GiB): an offset of
// FE_OOB is out of range, so a load there returns 0 and an atomic there is
// dropped, with no memory access and no branch.
constexpr int FE_BUF_DWORD3 = 0x00020000;   // gfx9-family buffer resource word 3 (raw 32-bit data)
constexpr int FE_OOB = 0x7FFFFFF0;

// BUF: x and y are addressed through buffer resources (4 * n_dof <= FE_OOB),
// so every gather and every atomic add is issued unconditionally, with an
// out-of-range offset where a DOF is constrained or has nothing to add;
// otherwise through pointers with the same results.
template <bool BUF>
__global__ __launch_bounds__(FE_WG) void k_fe_fused(int n_elem, int n_dof, const int *__restrict__ edof,
                                                    const float *__restrict__ rho, int penalty,
                                                    const float *__restrict__ Ke, float alpha,
                                                    const float *__restrict__ x, float *__restrict__ y) {
    __shared__ int line_dof[FE_WG / 64][4 * 3 * 65];
    __shared__ float line_val[FE_WG / 64][4 * 3 * 65];
    // lanes past the last element stay (the wave exchange below needs all
    // 64) with every DOF index -1
    const int e = blockIdx.x * FE_WG + threadIdx.x;
    const bool live = e < n_elem;
    const int ec = live ? e : n_elem - 1;
    int d[NDOF_E];
    load_edof(edof, ec, d);
#pragma unroll
    for (int b = 0; b < NDOF_E; ++b) d[b] = live ? d[b] : -1;
    // 24 gathers issued together; a constrained DOF contributes 0
    float u[NDOF_E];
    __amdgpu_buffer_rsrc_t xr, yr;
    if (BUF) {
        xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(x), 0, 4 * n_dof, FE_BUF_DWORD3);
        yr = __builtin_amdgcn_make_buffer_rsrc(y, 0, 4 * n_dof, FE_BUF_DWORD3);
#pragma unroll
        for (int b = 0; b < NDOF_E; ++b)
            u[b] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                 xr, (unsigned)d[b] < (unsigned)n_dof ? 4 * d[b] : FE_OOB, 0, 0));
    } else {
#pragma unroll
        for (int b = 0; b < NDOF_E; ++b) u[b] = x[(unsigned)d[b] < (unsigned)n_dof ? d[b] : 0];
#pragma unroll
        for (int b = 0; b < NDOF_E; ++b) u[b] = (unsigned)d[b] < (unsigned)n_dof ? u[b] : 0.0f;
    }
    const float s = alpha * simp(rho[ec], penalty);
    float fa[NDOF_E];
#pragma unroll
    for (int a = 0; a < NDOF_E; ++a) {
        float f = 0.0f;
#pragma unroll
        for (int b = 0; b < NDOF_E; ++b) f = fmaf(Ke[a * NDOF_E + b], u[b], f);
        fa[a] = s * f;
    }
    // all 24 products are finished here: left to itself the compiler sinks
    // them into the scatter, where Ke no longer fits the scalar registers and
    // is spilled to vector-register lanes and reloaded around every add
#pragma unroll
    for (int a = 0; a < NDOF_E; ++a) asm volatile("" : "+v"(fa[a]));
    const int w = threadIdx.x >> 6;
    if (BUF)
        fe_scatter_lines(
            d, fa, n_dof,
            [yr](int i, bool on, float v) {
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v, yr, on ? 4 * i : FE_OOB, 0, 0);
            },
            line_dof[w], line_val[w]);
    else
        fe_scatter_lines(
            d, fa, n_dof,
            [y](int i, bool on, float v) {
                if (on) atomicAdd(y + i, v);
            },
            line_dof[w], line_val[w]);
}

// ---- three-stage comparator ----

// U[e][b] = x[edof[e][b]] (0 for a constrained DOF); one thread per entry.
__global__ void k_fe_gather(int n_elem, int n_dof, const int *__restrict__ edof, const float *__restrict__ x,
                            float *__restrict__ U) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= (int64_t)n_elem * NDOF_E) return;
    const int d = edof[k];
    const float xv = x[(unsigned)d < (unsigned)n_dof ? d : 0];
    U[k] = (unsigned)d < (unsigned)n_dof ? xv : 0.0f;
}

// F[e] = alpha * rho_e^p * Ke U[e]; one thread per element.
__global__ __launch_bounds__(FE_WG) void k_fe_elem(int n_elem, const float *__restrict__ rho, int penalty,
                                                   const float *__restrict__ Ke, float alpha,
                                                   const float *__restrict__ U, float *__restrict__ F) {
    __shared__ __attribute__((aligned(16))) float ke[NDOF_E * NDOF_E];
    stage_ke(ke, Ke);
    const int e = blockIdx.x * FE_WG + threadIdx.x;
    if (e >= n_elem) return;
    float u[NDOF_E];
    const f32x4 *up = reinterpret_cast<const f32x4 *>(U + (size_t)e * NDOF_E);
#pragma unroll
    for (int k = 0; k < NDOF_E / 4; ++k) {
        const f32x4 q = up[k];
        u[4 * k] = q.x;
        u[4 * k + 1] = q.y;
        u[4 * k + 2] = q.z;
        u[4 * k + 3] = q.w;
    }
    const float s = alpha * simp(rho[e], penalty);
    f32x4 *fp = reinterpret_cast<f32x4 *>(F + (size_t)e * NDOF_E);
#pragma unroll
    for (int a4 = 0; a4 < NDOF_E; a4 += 4) {
        f32x4 o;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float f = 0.0f;
#pragma unroll
            for (int b = 0; b < NDOF_E; ++b) f = fmaf(ke[(a4 + t) * NDOF_E + b], u[b], f);
            o[t] = s * f;
        }
        fp[a4 / 4] = o;
    }
}

// y[edof[e][a]] += F[e][a]; one thread per entry.
__global__ void k_fe_scatter(int n_elem, int n_dof, const int *__restrict__ edof, const float *__restrict__ F,
                             float *__restrict__ y) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= (int64_t)n_elem * NDOF_E) return;
    const int d = edof[k];
    if ((unsigned)d < (unsigned)n_dof) atomicAdd(y + d, F[k]);
}

// The three launches of the unfused form for elements [0, n_elem) of the
// given arrays (already offset to a chunk), U and F holding n_elem * 24
// floats each.
spmv_status threestage_launch(int n_elem, int n_dof, const int32_t *edof, const float *rho, int penalty,
                              const float *Ke, float alpha, const float *x, float *y, float *U, float *F,
                              hipStream_t st) {
    const int entries = n_elem * NDOF_E;
    k_fe_gather<<<(int)ceil_div(entries, 256), 256, 0, st>>>(n_elem, n_dof, edof, x, U);
    SPMV_LAUNCHED("k_fe_gather");
    k_fe_elem<<<(int)ceil_div(n_elem, FE_WG), FE_WG, 0, st>>>(n_elem, rho, penalty, Ke, alpha, U, F);
    SPMV_LAUNCHED("k_fe_elem");
    k_fe_scatter<<<(int)ceil_div(entries, 256), 256, 0, st>>>(n_elem, n_dof, edof, F, y);
    SPMV_LAUNCHED("k_fe_scatter");
    return SPMV_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
spmv_status scratch_address(float **out) {
    static std::mutex mu;
    static float *addr[64] = {};
    int dev = -1;
    SPMV_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= 64) return fail(SPMV_ERR_UNSUPPORTED, "device %d: at most 64 devices", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(SPMV_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        addr[dev] = static_cast<float *>(p);
    }
    *out = addr[dev];
    return SPMV_OK;
}

spmv_status check_fe(int32_t n_elem, int32_t n_dof, const int32_t *edof, const float *rho, int32_t penalty,
                     const float *Ke, const float *x, float *y) {
    if (n_elem < 0 || n_dof < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if ((int64_t)n_elem * NDOF_E > INT32_MAX) return fail(SPMV_ERR_OVERFLOW, "n_elem * 24 exceeds int32");
    if (penalty < 0 || penalty > MAX_PENALTY) return fail(SPMV_ERR_INVALID_VALUE, "penalty must be in [0, %d]", MAX_PENALTY);
    if (n_dof > 0 && !y) return fail(SPMV_ERR_INVALID_VALUE, "y is NULL");
    if (n_elem > 0 && (!edof || !rho || !Ke || !x)) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    if (n_elem > 0 && (!aligned16(edof) || !aligned16(Ke)))
        return fail(SPMV_ERR_UNSUPPORTED, "edof and Ke must be 16-byte aligned");
    return SPMV_OK;
}

}  // namespace
}  // namespace spmv

using namespace spmv;

extern "C" spmv_status fem_matvec_apply(int32_t n_elem, int32_t n_dof, const int32_t *edof, const float *rho,
                                        int32_t penalty, const float *Ke, float alpha, const float *x, float beta,
                                        float *y, void *stream) {
    spmv_status s = check_fe(n_elem, n_dof, edof, rho, penalty, Ke, x, y);
    if (s != SPMV_OK) return s;
    if (n_dof == 0) return SPMV_OK;
    hipStream_t st = as_stream(stream);
    if (beta != 1.0f) {
        beta_launch(n_dof, beta, y, st);
        SPMV_LAUNCHED("k_fe_beta");
    }
    if (n_elem == 0) return SPMV_OK;
    const int grid = (int)ceil_div(n_elem, FE_WG);
    if (4 * (int64_t)n_dof <= FE_OOB)
        k_fe_fused<true><<<grid, FE_WG, 0, st>>>(n_elem, n_dof, edof, rho, penalty, Ke, alpha, x, y);
    else
        k_fe_fused<false><<<grid, FE_WG, 0, st>>>(n_elem, n_dof, edof, rho, penalty, Ke, alpha, x, y);
    SPMV_LAUNCHED("k_fe_fused");
    return SPMV_OK;
}

extern "C" spmv_status fem_threestage_size(int32_t n_elem, size_t *bytes) {
    if (!bytes) return fail(SPMV_ERR_INVALID_VALUE, "bytes is NULL");
    if (n_elem < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    *bytes = 2 * (size_t)n_elem * NDOF_E * sizeof(float);
    return SPMV_OK;
}

extern "C" spmv_status fem_matvec_threestage(int32_t n_elem, int32_t n_dof, const int32_t *edof, const float *rho,
                                             int32_t penalty, const float *Ke, float alpha, const float *x,
                                             float beta, float *y, void *workspace, size_t workspace_bytes,
                                             void *stream) {
    spmv_status s = check_fe(n_elem, n_dof, edof, rho, penalty, Ke, x, y);
    if (s != SPMV_OK) return s;
    const size_t need = 2 * (size_t)n_elem * NDOF_E * sizeof(float);
    if (n_elem > 0 && (!workspace || workspace_bytes < need))
        return fail(SPMV_ERR_INVALID_VALUE, "workspace of %zu bytes is smaller than %zu", workspace_bytes, need);
    if (n_elem > 0 && !aligned16(workspace)) return fail(SPMV_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
    if (n_dof == 0) return SPMV_OK;
    hipStream_t st = as_stream(stream);
    if (beta != 1.0f) {
        beta_launch(n_dof, beta, y, st);
        SPMV_LAUNCHED("k_fe_beta");
    }
    if (n_elem == 0) return SPMV_OK;
    float *U = static_cast<float *>(workspace);
    float *F = U + (size_t)n_elem * NDOF_E;
    return threestage_launch(n_elem, n_dof, edof, rho, penalty, Ke, alpha, x, y, U, F, st);
}

extern "C" spmv_status fem_matvec_threestage_noalloc(int32_t n_elem, int32_t n_dof, const int32_t *edof,
                                                     const float *rho, int32_t penalty, const float *Ke, float alpha,
                                                     const float *x, float beta, float *y, void *stream) {
    spmv_status s = check_fe(n_elem, n_dof, edof, rho, penalty, Ke, x, y);
    if (s != SPMV_OK) return s;
    if (n_dof == 0) return SPMV_OK;
    float *U = nullptr;
    s = scratch_address(&U);
    if (s != SPMV_OK) return s;
    float *F = U + (size_t)FE_NOALLOC_CHUNK * NDOF_E;
    hipStream_t st = as_stream(stream);
    if (beta != 1.0f) {
        beta_launch(n_dof, beta, y, st);
        SPMV_LAUNCHED("k_fe_beta");
    }
    // chunks of elements one after another on the stream: a chunk's gather
    // overwrites U only after the previous chunk's kernels have used it
    for (int off = 0; off < n_elem; off += FE_NOALLOC_CHUNK) {
        const int m = std::min(FE_NOALLOC_CHUNK, n_elem - off);
        s = threestage_launch(m, n_dof, edof + (size_t)off * NDOF_E, rho + off, penalty, Ke, alpha, x, y, U, F, st);
        if (s != SPMV_OK) return s;
    }
    return SPMV_OK;
}
