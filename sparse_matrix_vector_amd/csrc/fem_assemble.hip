// Assembled stiffness matrix of the FE operator, in CSR, on the GPU.
//
// "Fused GPU SpMV kernel optimisation: from bandwidth bottleneck to BF16
// precision", section 2.1: the conventional route assembles the global
// stiffness matrix K = sum_e rho_e^p P_e^T Ke P_e once and then runs a
// sparse matrix-vector product on it; the fused kernel avoids storing K.
// This builds that K, so that the library's CSR SpMV can be timed on it
// beside the fused matvec.
//
// Rows are DOFs.  Row d of K collects, for every element e and local DOF a
// with edof[e][a] = d, the products rho_e^p Ke[a][b] at columns edof[e][b]
// (constrained entries dropped).  Steps:
//   1. the inverse map: for each DOF its (element, local DOF) entries in
//      increasing entry order (count, scan, fill, per-list sort);
//   2. one wave per row gathers the row's candidates -- (column, candidate
//      number) for every entry of the list and every b -- sorts them in LDS
//      (bitonic, at most FA_CAND of them) and counts the distinct columns
//      (fem_assemble_pattern) or writes each distinct column once with the
//      sum of its candidates, taken in candidate order in fp64 and rounded
//      to fp32 (fem_assemble_values).  Columns come out in increasing order.
#include "common.hpp"

#include <algorithm>

namespace spmv {
namespace {

constexpr int NDOF_E = 24;
constexpr int MAX_PENALTY = 8;
constexpr int FA_CAND = 256;                 // candidates per row (4 per lane)
constexpr int FA_WAVES = 4;                  // rows per workgroup of the row kernels
constexpr int FA_SCAN_WG = 1024;
constexpr int FA_ERR_CAND = 1;               // a row has more than FA_CAND candidates

__global__ void k_fa_count(int64_t n_ent, int n_dof, const int *__restrict__ edof, int *__restrict__ cnt) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n_ent) return;
    const int d = edof[t];
    if ((unsigned)d < (unsigned)n_dof) atomicAdd(cnt + d, 1);
}

// Exclusive scan of n counts into out[0 .. n] (out[n] = total), one
// workgroup; 64-bit total into *total.
__global__ __launch_bounds__(FA_SCAN_WG) void k_fa_scan(int n, const int *__restrict__ in, int *__restrict__ out,
                                                        long long *__restrict__ total) {
    __shared__ long long wsum[FA_SCAN_WG / 64];
    long long carry = 0;
    for (int base = 0; base < n; base += FA_SCAN_WG) {
        const int i = base + (int)threadIdx.x;
        const long long v = i < n ? in[i] : 0;
        long long incl = v;
        for (int off = 1; off < 64; off <<= 1) {
            const long long u = __shfl_up(incl, off, 64);
            if ((threadIdx.x & 63) >= off) incl += u;
        }
        if ((threadIdx.x & 63) == 63) wsum[threadIdx.x >> 6] = incl;
        __syncthreads();
        long long wbase = 0, tot = 0;
        for (int w = 0; w < FA_SCAN_WG / 64; ++w) {
            if (w < (int)(threadIdx.x >> 6)) wbase += wsum[w];
            tot += wsum[w];
        }
        if (i < n) out[i] = (int)(carry + wbase + incl - v);
        carry += tot;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        out[n] = (int)carry;
        *total = carry;
    }
}

__global__ void k_fa_fill(int64_t n_ent, int n_dof, const int *__restrict__ edof, const int *__restrict__ inv_rp,
                          int *__restrict__ cursor, int *__restrict__ inv) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n_ent) return;
    const int d = edof[t];
    if ((unsigned)d < (unsigned)n_dof) inv[inv_rp[d] + atomicAdd(cursor + d, 1)] = (int)t;
}

__global__ void k_fa_sort_lists(int n_dof, const int *__restrict__ inv_rp, int *__restrict__ inv) {
    const int d = blockIdx.x * 256 + threadIdx.x;
    if (d >= n_dof) return;
    const int a = inv_rp[d], b = inv_rp[d + 1];
    for (int i = a + 1; i < b; ++i) {
        const int v = inv[i];
        int j = i - 1;
        while (j >= a && inv[j] > v) {
            inv[j + 1] = inv[j];
            --j;
        }
        inv[j + 1] = v;
    }
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave per row.  FILL = false: row_len[d] = number of distinct columns.
// FILL = true: the row's columns (increasing) and summed values at
// row_ptr[d] ..
template <bool FILL>
__global__ __launch_bounds__(64 * FA_WAVES) void k_fa_rows(int n_dof, const int *__restrict__ edof,
                                                           const int *__restrict__ inv_rp,
                                                           const int *__restrict__ inv, const float *__restrict__ rho,
                                                           int penalty, const float *__restrict__ Ke,
                                                           int *__restrict__ row_len, const int *__restrict__ row_ptr,
                                                           int *__restrict__ col_idx, float *__restrict__ vals,
                                                           int *__restrict__ err) {
    __shared__ unsigned long long keys[FA_WAVES][FA_CAND];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int d = blockIdx.x * FA_WAVES + wv;
    if (d >= n_dof) return;                       // whole waves leave together
    unsigned long long *k = keys[wv];
    const int a0 = inv_rp[d], m = inv_rp[d + 1] - a0;
    if (m * NDOF_E > FA_CAND) {
        if (lane == 0) atomicOr(err, FA_ERR_CAND);
        return;
    }
    // candidate q = 24 j + b: column edof[e_j][b] (constrained: sorts last)
#pragma unroll
    for (int r = 0; r < FA_CAND / 64; ++r) {
        const int q = lane + 64 * r;
        unsigned long long key = ~0ull;
        if (q < m * NDOF_E) {
            const int t = inv[a0 + q / NDOF_E];
            const int e = t / NDOF_E;
            const int c = edof[(size_t)e * NDOF_E + q % NDOF_E];
            const unsigned hi = (unsigned)c < (unsigned)n_dof ? (unsigned)c : 0xFFFFFFFFu;
            key = ((unsigned long long)hi << 32) | (unsigned)q;
        }
        k[q] = key;
    }
    wave_sync();
    for (int size = 2; size <= FA_CAND; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
#pragma unroll
            for (int r = 0; r < FA_CAND / 128; ++r) {
                const int t = lane + 64 * r;
                const int lo = 2 * t - (t & (stride - 1)), hi = lo + stride;
                const bool up = (lo & size) == 0;
                const unsigned long long x = k[lo], y = k[hi];
                if ((x > y) == up) {
                    k[lo] = y;
                    k[hi] = x;
                }
            }
            wave_sync();
        }
    }
    // heads of runs of equal columns; lane l looks at positions 4 l .. 4 l + 3
    int heads = 0;
    bool hd[FA_CAND / 64];
#pragma unroll
    for (int j = 0; j < FA_CAND / 64; ++j) {
        const int p = 4 * lane + j;
        const unsigned c = (unsigned)(k[p] >> 32);
        hd[j] = c != 0xFFFFFFFFu && (p == 0 || (unsigned)(k[p - 1] >> 32) != c);
        heads += hd[j];
    }
    if (!FILL) {
        const int total = __builtin_amdgcn_readlane(wave_inclusive_scan(heads), 63);
        if (lane == 0) row_len[d] = total;
        return;
    }
    int rank = wave_inclusive_scan(heads) - heads;   // heads before position 4 lane
    const int base = row_ptr[d];
#pragma unroll
    for (int j = 0; j < FA_CAND / 64; ++j) {
        if (!hd[j]) continue;
        const int p = 4 * lane + j;
        const unsigned c = (unsigned)(k[p] >> 32);
        double sum = 0.0;
        for (int q = p; q < FA_CAND && (unsigned)(k[q] >> 32) == c; ++q) {
            const int cand = (int)(unsigned)k[q];
            const int t = inv[a0 + cand / NDOF_E];
            const int e = t / NDOF_E, a = t % NDOF_E, b = cand % NDOF_E;
            double s = 1.0;
            for (int i = 0; i < penalty; ++i) s *= (double)rho[e];
            sum += s * (double)Ke[a * NDOF_E + b];
        }
        col_idx[base + rank] = (int)c;
        vals[base + rank] = (float)sum;
        ++rank;
    }
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct AsmLayout {
    size_t meta, inv_rp, cursor, inv, total;
};

AsmLayout asm_layout(int64_t n_elem, int64_t n_dof) {
    AsmLayout L{};
    size_t at = 0;
    auto take = [&](size_t bytes) {
        const size_t o = at;
        at = align256(at + std::max<size_t>(bytes, 4));
        return o;
    };
    L.meta = take(64);
    L.inv_rp = take(4 * (size_t)(n_dof + 1));
    L.cursor = take(4 * (size_t)(n_dof + 1));
    L.inv = take(4 * (size_t)NDOF_E * (size_t)n_elem);
    L.total = at;
    return L;
}

spmv_status check_asm(int32_t n_elem, int32_t n_dof, const int32_t *edof, void *ws, size_t ws_bytes) {
    if (n_elem < 0 || n_dof < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if ((int64_t)n_elem * NDOF_E > INT32_MAX) return fail(SPMV_ERR_OVERFLOW, "n_elem * 24 exceeds int32");
    if (n_elem > 0 && !edof) return fail(SPMV_ERR_INVALID_VALUE, "edof is NULL");
    const AsmLayout L = asm_layout(n_elem, n_dof);
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u))
        return fail(SPMV_ERR_INVALID_VALUE, "workspace must be non-NULL and 256-byte aligned");
    if (ws_bytes < L.total) return fail(SPMV_ERR_INVALID_VALUE, "workspace of %zu bytes is smaller than %zu", ws_bytes, L.total);
    return SPMV_OK;
}

}  // namespace
}  // namespace spmv

using namespace spmv;

extern "C" spmv_status fem_assemble_size(int32_t n_elem, int32_t n_dof, size_t *bytes) {
    if (!bytes) return fail(SPMV_ERR_INVALID_VALUE, "bytes is NULL");
    if (n_elem < 0 || n_dof < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if ((int64_t)n_elem * NDOF_E > INT32_MAX) return fail(SPMV_ERR_OVERFLOW, "n_elem * 24 exceeds int32");
    *bytes = asm_layout(n_elem, n_dof).total;
    return SPMV_OK;
}

extern "C" spmv_status fem_assemble_pattern(int32_t n_elem, int32_t n_dof, const int32_t *edof, int32_t *row_ptr,
                                            int64_t *nnz, void *workspace, size_t workspace_bytes, void *stream) {
    spmv_status s = check_asm(n_elem, n_dof, edof, workspace, workspace_bytes);
    if (s != SPMV_OK) return s;
    if (!row_ptr || !nnz) return fail(SPMV_ERR_INVALID_VALUE, "row_ptr or nnz is NULL");
    hipStream_t st = as_stream(stream);
    const AsmLayout L = asm_layout(n_elem, n_dof);
    char *w = static_cast<char *>(workspace);
    long long *meta = reinterpret_cast<long long *>(w + L.meta);   // [0] total, [1] error flags
    int *err = reinterpret_cast<int *>(meta + 1);
    int *inv_rp = reinterpret_cast<int *>(w + L.inv_rp);
    int *cursor = reinterpret_cast<int *>(w + L.cursor);
    int *inv = reinterpret_cast<int *>(w + L.inv);
    const int64_t n_ent = (int64_t)n_elem * NDOF_E;
    SPMV_HIP(hipMemsetAsync(w + L.meta, 0, 64, st));
    SPMV_HIP(hipMemsetAsync(cursor, 0, sizeof(int) * ((size_t)n_dof + 1), st));
    if (n_ent > 0) {
        k_fa_count<<<(int)ceil_div(n_ent, 256), 256, 0, st>>>(n_ent, n_dof, edof, cursor);
        SPMV_LAUNCHED("k_fa_count");
    }
    k_fa_scan<<<1, FA_SCAN_WG, 0, st>>>(n_dof, cursor, inv_rp, meta);
    SPMV_LAUNCHED("k_fa_scan");
    SPMV_HIP(hipMemsetAsync(cursor, 0, sizeof(int) * ((size_t)n_dof + 1), st));
    if (n_ent > 0) {
        k_fa_fill<<<(int)ceil_div(n_ent, 256), 256, 0, st>>>(n_ent, n_dof, edof, inv_rp, cursor, inv);
        SPMV_LAUNCHED("k_fa_fill");
    }
    if (n_dof > 0) {
        k_fa_sort_lists<<<(int)ceil_div(n_dof, 256), 256, 0, st>>>(n_dof, inv_rp, inv);
        SPMV_LAUNCHED("k_fa_sort_lists");
        // row lengths into the cursor array, then their scan into row_ptr
        k_fa_rows<false><<<(int)ceil_div(n_dof, FA_WAVES), 64 * FA_WAVES, 0, st>>>(
            n_dof, edof, inv_rp, inv, nullptr, 0, nullptr, cursor, nullptr, nullptr, nullptr, err);
        SPMV_LAUNCHED("k_fa_rows");
    }
    k_fa_scan<<<1, FA_SCAN_WG, 0, st>>>(n_dof, cursor, row_ptr, meta);
    SPMV_LAUNCHED("k_fa_scan");
    long long h[2] = {0, 0};
    SPMV_HIP(hipMemcpyAsync(h, meta, sizeof h, hipMemcpyDeviceToHost, st));
    SPMV_HIP(hipStreamSynchronize(st));
    if ((int)h[1] & FA_ERR_CAND)
        return fail(SPMV_ERR_UNSUPPORTED, "a row has more than %d (element, column) candidates", FA_CAND);
    if (h[0] > INT32_MAX) return fail(SPMV_ERR_OVERFLOW, "nnz(K) = %lld exceeds int32", h[0]);
    *nnz = h[0];
    return SPMV_OK;
}

extern "C" spmv_status fem_assemble_values(int32_t n_elem, int32_t n_dof, const int32_t *edof, const float *rho,
                                           int32_t penalty, const float *Ke, const int32_t *row_ptr,
                                           int32_t *col_idx, float *vals, void *workspace, size_t workspace_bytes,
                                           void *stream) {
    spmv_status s = check_asm(n_elem, n_dof, edof, workspace, workspace_bytes);
    if (s != SPMV_OK) return s;
    if (penalty < 0 || penalty > MAX_PENALTY) return fail(SPMV_ERR_INVALID_VALUE, "penalty must be in [0, %d]", MAX_PENALTY);
    if (!row_ptr || (n_elem > 0 && (!rho || !Ke || !col_idx || !vals)))
        return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    if (n_dof == 0) return SPMV_OK;
    hipStream_t st = as_stream(stream);
    const AsmLayout L = asm_layout(n_elem, n_dof);
    char *w = static_cast<char *>(workspace);
    int *err = reinterpret_cast<int *>(reinterpret_cast<long long *>(w + L.meta) + 1);
    k_fa_rows<true><<<(int)ceil_div(n_dof, FA_WAVES), 64 * FA_WAVES, 0, st>>>(
        n_dof, edof, reinterpret_cast<const int *>(w + L.inv_rp), reinterpret_cast<const int *>(w + L.inv), rho,
        penalty, Ke, nullptr, row_ptr, col_idx, vals, err);
    SPMV_LAUNCHED("k_fa_rows");
    SPMV_HIP(hipStreamSynchronize(st));
    return SPMV_OK;
}
