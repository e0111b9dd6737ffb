// HYB on gfx950 and the CV-driven choice between ELL, HYB and binned CSR.
//
// "Why SpMV needs CUDA optimisation": section 2.1 lists HYB as a mixed CSR +
// ELL format beside CSR and ELL; section 2.2 picks ELL for a row-length CV
// below 0.3, HYB between 0.3 and 0.7 and CSR with row reordering above; its
// tuning example (section 5) splits the storage 0.7 ELL to 0.3 COO.
//
// Layout (the pages fix none of it):
//   ELL part   the first min(len_i, W) entries of every row, slot-major like
//              the ELL format: entry k of row i at [k * n_rows + i], padding
//              column -1 / value +0 (skipped);
//   tail       the entries of row i past W, for the rows longer than W only:
//              tail_rows[t] (ascending), tail_rp[t] .. tail_rp[t + 1] into
//              tail_col / tail_val, in the row's storage order.
//   W          the smallest width whose ELL part holds at least the fraction
//              num / den of the nonzeros (0.7 in the page's example):
//              den * sum_i min(len_i, W) >= num * nnz, in exact integers.
//
// Apply: the ELL kernel writes y = alpha * (ELL part) x + beta * y, then one
// group of G lanes per tail row (G a power of two near the mean tail length)
// adds alpha * (tail part) x.  Both sums have a fixed order.
#include "common.hpp"

#include <algorithm>

namespace spmv {
namespace {

constexpr int WG = 256;
constexpr int WAVES = WG / 64;
constexpr int SCAN_WG = 1024;
static_assert(WG == SCRATCH_ROWS_PER_WG, "the HYB split keeps one count pair per 256-row workgroup in the scratch");

// Block sums over rows of min(len, W), [len > W] and max(len - W, 0), added
// into out[0..2] (exact 64-bit integers).
__global__ __launch_bounds__(WG) void k_hyb_count(int n, const int *__restrict__ rp, int W,
                                                  unsigned long long *__restrict__ out) {
    __shared__ unsigned long long part[3][WG];
    unsigned long long a = 0, b = 0, c = 0;
    for (int i = blockIdx.x * WG + threadIdx.x; i < n; i += gridDim.x * WG) {
        const int len = rp[i + 1] - rp[i];
        a += (unsigned long long)min(len, W);
        b += len > W ? 1ull : 0ull;
        c += len > W ? (unsigned long long)(len - W) : 0ull;
    }
    part[0][threadIdx.x] = a;
    part[1][threadIdx.x] = b;
    part[2][threadIdx.x] = c;
    __syncthreads();
    for (int s = WG / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s)
            for (int q = 0; q < 3; ++q) part[q][threadIdx.x] += part[q][threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        for (int q = 0; q < 3; ++q) atomicAdd(out + q, part[q][0]);
}

// ELL part: row i's first min(len, W) entries, padding after.  Columns
// outside [0, n_cols) raise `err`.
__global__ __launch_bounds__(WG) void k_hyb_ell(int n, int n_cols, int W, const int *__restrict__ rp,
                                                const int *__restrict__ ci, const float *__restrict__ v,
                                                int *__restrict__ ec, float *__restrict__ ev,
                                                int *__restrict__ err) {
    const int i = blockIdx.x * WG + threadIdx.x;
    if (i >= n) return;
    const int s = rp[i], len = rp[i + 1] - s;
    bool bad = false;
    for (int k = 0; k < W; ++k) {
        const size_t slot = (size_t)k * (size_t)n + (size_t)i;
        const bool real = k < len;
        const int c = real ? ci[s + k] : -1;
        bad |= real && (unsigned)c >= (unsigned)n_cols;
        ec[slot] = c;
        ev[slot] = real ? v[s + k] : 0.0f;
    }
    if (bad) atomicOr(err, 1);
}

// Exclusive scan within a workgroup of WG threads (wave scans combined
// through LDS); returns the exclusive prefix, `total` gets the block sum.
__device__ __forceinline__ int block_exclusive(int v, int *lds, int &total) {
    const int lane = __lane_id(), w = threadIdx.x / 64;
    const int incl = wave_inclusive_scan(v);
    if (lane == 63) lds[w] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
    for (int q = 0; q < WAVES; ++q) {
        before += q < w ? lds[q] : 0;
        total += lds[q];
    }
    __syncthreads();
    return before + incl - v;
}

// Per workgroup: tail rows and tail entries of its WG rows.
__global__ __launch_bounds__(WG) void k_hyb_tail_count(int n, const int *__restrict__ rp, int W,
                                                       int *__restrict__ brows, int *__restrict__ bents) {
    __shared__ int lds[2][WAVES];
    const int i = blockIdx.x * WG + threadIdx.x;
    const int len = i < n ? rp[i + 1] - rp[i] : 0;
    int tr, te;
    block_exclusive(len > W ? 1 : 0, lds[0], tr);
    block_exclusive(len > W ? len - W : 0, lds[1], te);
    if (threadIdx.x == 0) {
        brows[blockIdx.x] = tr;
        bents[blockIdx.x] = te;
    }
}

// Exclusive scan of two int arrays of length nb in one workgroup (in place).
__global__ __launch_bounds__(SCAN_WG) void k_hyb_scan(int nb, int *__restrict__ a, int *__restrict__ b) {
    __shared__ int lds[2][SCAN_WG / 64];
    const int lane = __lane_id(), w = threadIdx.x / 64;
    int carry_a = 0, carry_b = 0;
    for (int base = 0; base < nb; base += SCAN_WG) {
        const int i = base + threadIdx.x;
        const int va = i < nb ? a[i] : 0, vb = i < nb ? b[i] : 0;
        const int ia = wave_inclusive_scan(va), ib = wave_inclusive_scan(vb);
        if (lane == 63) {
            lds[0][w] = ia;
            lds[1][w] = ib;
        }
        __syncthreads();
        int pa = 0, pb = 0, ta = 0, tb = 0;
        for (int q = 0; q < SCAN_WG / 64; ++q) {
            pa += q < w ? lds[0][q] : 0;
            pb += q < w ? lds[1][q] : 0;
            ta += lds[0][q];
            tb += lds[1][q];
        }
        if (i < nb) {
            a[i] = carry_a + pa + ia - va;
            b[i] = carry_b + pb + ib - vb;
        }
        carry_a += ta;
        carry_b += tb;
        __syncthreads();
    }
}

// Writes the tail in row order: tail_rows, tail_rp and the entries.
// Columns outside [0, n_cols) raise `err`.
__global__ __launch_bounds__(WG) void k_hyb_tail_write(int n, int n_cols, const int *__restrict__ rp,
                                                       const int *__restrict__ ci, const float *__restrict__ v,
                                                       int W, const int *__restrict__ orows,
                                                       const int *__restrict__ oents, int *__restrict__ trows,
                                                       int *__restrict__ trp, int *__restrict__ tcol,
                                                       float *__restrict__ tval, int *__restrict__ err) {
    __shared__ int lds[2][WAVES];
    const int i = blockIdx.x * WG + threadIdx.x;
    const int s = i < n ? rp[i] : 0;
    const int len = i < n ? rp[i + 1] - s : 0;
    const bool has = len > W;
    int tr, te;
    const int xr = block_exclusive(has ? 1 : 0, lds[0], tr);
    const int xe = block_exclusive(has ? len - W : 0, lds[1], te);
    if (!has) return;
    const int t = orows[blockIdx.x] + xr;
    const int pos = oents[blockIdx.x] + xe;
    trows[t] = i;
    trp[t] = pos;
    bool bad = false;
    for (int k = W; k < len; ++k) {
        const int c = ci[s + k];
        bad |= (unsigned)c >= (unsigned)n_cols;
        tcol[pos + k - W] = c;
        tval[pos + k - W] = v[s + k];
    }
    if (bad) atomicOr(err, 1);
}

__global__ void k_set_int(int *p, int v) { *p = v; }

// The tail per row: tfull[r] = first tail entry of row r or of the next tail
// row after it (tail_rp[number of tail rows < r]), r = 0..n.
__global__ __launch_bounds__(WG) void k_hyb_row_tail(int n, int n_tail, const int *__restrict__ trows,
                                                     const int *__restrict__ trp, int *__restrict__ tfull) {
    const int r = blockIdx.x * WG + threadIdx.x;
    if (r > n) return;
    int lo = 0, hi = n_tail;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (trows[mid] < r)
            lo = mid + 1;
        else
            hi = mid;
    }
    tfull[r] = trp[lo];
}

// y[tail_rows[t]] += alpha * (tail row t) . x, G lanes per tail row.
template <int G>
__global__ __launch_bounds__(WG) void k_hyb_tail(int n_tail, const int *__restrict__ trows,
                                                 const int *__restrict__ trp, const int *__restrict__ tcol,
                                                 const float *__restrict__ tval, const float *__restrict__ x,
                                                 float alpha, float *__restrict__ y) {
    const int gid = (int)((blockIdx.x * (unsigned)WG + threadIdx.x) / G);
    const int sub = threadIdx.x % G;
    if (gid >= n_tail) return;   // whole groups leave together
    const int s = trp[gid], e = trp[gid + 1];
    float acc = 0.0f;
    for (int k = s + sub; k < e; k += G) acc = fmaf(tval[k], x[tcol[k]], acc);
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) acc += __shfl_down(acc, off, G);
    if (sub == 0) {
        const int r = trows[gid];
        y[r] = fmaf(alpha, acc, y[r]);
    }
}

spmv_status hyb_counts(int n, const int *rp, int W, hipStream_t st, unsigned long long *d_out,
                       unsigned long long h[3]) {
    SPMV_HIP(hipMemsetAsync(d_out, 0, 3 * sizeof(unsigned long long), st));
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(n, WG), 4 * device_cu_count()));
    k_hyb_count<<<grid, WG, 0, st>>>(n, rp, W, d_out);
    SPMV_LAUNCHED("k_hyb_count");
    SPMV_HIP(hipMemcpyAsync(h, d_out, 3 * sizeof(unsigned long long), hipMemcpyDeviceToHost, st));
    SPMV_HIP(hipStreamSynchronize(st));
    return SPMV_OK;
}

}  // namespace
}  // namespace spmv

using namespace spmv;

extern "C" spmv_status spmv_hyb_width(int32_t n_rows, const int32_t *row_ptr, int32_t num, int32_t den,
                                      int32_t *width, int32_t *n_tail_rows, int64_t *tail_nnz, void *scratch,
                                      size_t scratch_bytes, void *stream) {
    if (n_rows < 0) return fail(SPMV_ERR_INVALID_VALUE, "n_rows < 0");
    if (!width || !n_tail_rows || !tail_nnz) return fail(SPMV_ERR_INVALID_VALUE, "NULL output pointer");
    if (den <= 0 || num < 0 || num > den) return fail(SPMV_ERR_INVALID_VALUE, "need 0 <= num <= den, den > 0");
    spmv_status s = check_scratch(scratch, scratch_bytes, n_rows);
    if (s != SPMV_OK) return s;
    *width = 0;
    *n_tail_rows = 0;
    *tail_nnz = 0;
    if (n_rows == 0) return SPMV_OK;
    if (!row_ptr) return fail(SPMV_ERR_INVALID_VALUE, "row_ptr is NULL");
    int32_t max_len = 0;
    int64_t s1 = 0, s2 = 0;
    s = spmv_csr_row_stats(n_rows, row_ptr, &max_len, &s1, &s2, scratch, scratch_bytes, stream);
    if (s != SPMV_OK) return s;
    hipStream_t st = as_stream(stream);
    auto *d_out = reinterpret_cast<unsigned long long *>(static_cast<char *>(scratch) + SCRATCH_HYB_COUNTS);
    // smallest W in [0, max_len] with den * count(W) >= num * nnz; the
    // condition is monotone in W and holds at W = max_len (count = nnz)
    int lo = 0, hi = max_len;
    unsigned long long h[3] = {0, 0, 0};
    const __int128 need = (__int128)num * s1;
    while (lo < hi && s == SPMV_OK) {
        const int mid = lo + (hi - lo) / 2;
        s = hyb_counts(n_rows, row_ptr, mid, st, d_out, h);
        if (s == SPMV_OK) {
            if ((__int128)den * (__int128)h[0] >= need)
                hi = mid;
            else
                lo = mid + 1;
        }
    }
    if (s == SPMV_OK) s = hyb_counts(n_rows, row_ptr, lo, st, d_out, h);
    if (s != SPMV_OK) return s;
    *width = lo;
    *n_tail_rows = (int32_t)h[1];
    *tail_nnz = (int64_t)h[2];
    return SPMV_OK;
}

extern "C" spmv_status spmv_hyb_tail_size(int32_t n_rows, const int32_t *row_ptr, int32_t width,
                                          int32_t *n_tail_rows, int64_t *tail_nnz, void *scratch,
                                          size_t scratch_bytes, void *stream) {
    if (n_rows < 0 || width < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if (!n_tail_rows || !tail_nnz) return fail(SPMV_ERR_INVALID_VALUE, "NULL output pointer");
    spmv_status s = check_scratch(scratch, scratch_bytes, n_rows);
    if (s != SPMV_OK) return s;
    *n_tail_rows = 0;
    *tail_nnz = 0;
    if (n_rows == 0) return SPMV_OK;
    if (!row_ptr) return fail(SPMV_ERR_INVALID_VALUE, "row_ptr is NULL");
    // row lengths must be non-negative for the counts to mean anything
    int32_t max_len = 0;
    int64_t s1 = 0, s2 = 0;
    s = spmv_csr_row_stats(n_rows, row_ptr, &max_len, &s1, &s2, scratch, scratch_bytes, stream);
    if (s != SPMV_OK) return s;
    unsigned long long h[3] = {0, 0, 0};
    s = hyb_counts(n_rows, row_ptr, width, as_stream(stream),
                   reinterpret_cast<unsigned long long *>(static_cast<char *>(scratch) + SCRATCH_HYB_COUNTS), h);
    if (s != SPMV_OK) return s;
    if (h[1] > (unsigned long long)INT32_MAX) return fail(SPMV_ERR_OVERFLOW, "tail rows exceed int32");
    *n_tail_rows = (int32_t)h[1];
    *tail_nnz = (int64_t)h[2];
    return SPMV_OK;
}

extern "C" spmv_status spmv_hyb_from_csr(int32_t n_rows, int32_t n_cols, int32_t nnz, const int32_t *row_ptr,
                                         const int32_t *col_idx, const float *vals, int32_t width,
                                         int32_t *ell_col, float *ell_val, int32_t n_tail_rows,
                                         int64_t tail_nnz, int32_t *tail_rows, int32_t *tail_rp,
                                         int32_t *tail_col, float *tail_val, void *scratch, size_t scratch_bytes,
                                         void *stream) {
    if (n_rows < 0 || n_cols < 0 || nnz < 0 || width < 0 || n_tail_rows < 0 || tail_nnz < 0)
        return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if ((int64_t)n_rows * width > INT32_MAX) return fail(SPMV_ERR_OVERFLOW, "width * n_rows exceeds int32");
    spmv_status s = check_scratch(scratch, scratch_bytes, n_rows);
    if (s != SPMV_OK) return s;
    if (n_rows == 0) return SPMV_OK;
    if (!row_ptr || !tail_rp || (nnz > 0 && (!col_idx || !vals)) || (width > 0 && (!ell_col || !ell_val)) ||
        (n_tail_rows > 0 && !tail_rows) || (tail_nnz > 0 && (!tail_col || !tail_val)))
        return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    int32_t max_len = 0;
    int64_t s1 = 0, s2 = 0;
    s = spmv_csr_row_stats(n_rows, row_ptr, &max_len, &s1, &s2, scratch, scratch_bytes, stream);
    if (s != SPMV_OK) return s;
    if (s1 != nnz) return fail(SPMV_ERR_INVALID_MATRIX, "row lengths sum to %lld, not nnz = %d", (long long)s1, nnz);
    hipStream_t st = as_stream(stream);
    int rp0 = -1;
    SPMV_HIP(hipMemcpyAsync(&rp0, row_ptr, sizeof(int), hipMemcpyDeviceToHost, st));
    SPMV_HIP(hipStreamSynchronize(st));
    if (rp0 != 0) return fail(SPMV_ERR_INVALID_MATRIX, "row_ptr[0] != 0");
    // the tail sizes the caller allocated for must be those of this width;
    // checked before any kernel writes the caller's arrays
    unsigned long long h[3] = {0, 0, 0};
    s = hyb_counts(n_rows, row_ptr, width, st,
                   reinterpret_cast<unsigned long long *>(static_cast<char *>(scratch) + SCRATCH_HYB_COUNTS), h);
    if (s != SPMV_OK) return s;
    if ((int64_t)h[1] != n_tail_rows || (int64_t)h[2] != tail_nnz)
        return fail(SPMV_ERR_INVALID_VALUE, "width %d gives %llu tail rows / %llu tail entries, not %d / %lld", width,
                    h[1], h[2], n_tail_rows, (long long)tail_nnz);
    char *sc = static_cast<char *>(scratch);
    int *d_err = reinterpret_cast<int *>(sc + SCRATCH_ERR);
    const int nb = (int)ceil_div(n_rows, WG);   // WG == SCRATCH_ROWS_PER_WG rows per count
    int *brows = reinterpret_cast<int *>(sc + SCRATCH_HEAD), *bents = brows + nb;
    SPMV_HIP(hipMemsetAsync(d_err, 0, sizeof(int), st));
    if (width > 0) {
        k_hyb_ell<<<nb, WG, 0, st>>>(n_rows, n_cols, width, row_ptr, col_idx, vals, ell_col, ell_val, d_err);
        SPMV_LAUNCHED("k_hyb_ell");
    }
    k_hyb_tail_count<<<nb, WG, 0, st>>>(n_rows, row_ptr, width, brows, bents);
    SPMV_LAUNCHED("k_hyb_tail_count");
    k_hyb_scan<<<1, SCAN_WG, 0, st>>>(nb, brows, bents);
    SPMV_LAUNCHED("k_hyb_scan");
    k_hyb_tail_write<<<nb, WG, 0, st>>>(n_rows, n_cols, row_ptr, col_idx, vals, width, brows, bents, tail_rows,
                                        tail_rp, tail_col, tail_val, d_err);
    SPMV_LAUNCHED("k_hyb_tail_write");
    k_set_int<<<1, 1, 0, st>>>(tail_rp + n_tail_rows, (int)tail_nnz);
    SPMV_LAUNCHED("k_set_int");
    int err = 0;
    SPMV_HIP(hipMemcpyAsync(&err, d_err, sizeof(int), hipMemcpyDeviceToHost, st));
    SPMV_HIP(hipStreamSynchronize(st));
    if (err) return fail(SPMV_ERR_INVALID_MATRIX, "a column index is outside [0, n_cols)");
    return SPMV_OK;
}

extern "C" spmv_status spmv_hyb_apply(int32_t n_rows, int32_t n_cols, int32_t width, const int32_t *ell_col,
                                      const float *ell_val, int32_t n_tail_rows, int64_t tail_nnz,
                                      const int32_t *tail_rows, const int32_t *tail_rp, const int32_t *tail_col,
                                      const float *tail_val, float alpha, const float *x, float beta, float *y,
                                      void *stream) {
    if (n_tail_rows < 0 || tail_nnz < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if (n_tail_rows > 0 && (!tail_rows || !tail_rp || (tail_nnz > 0 && (!tail_col || !tail_val))))
        return fail(SPMV_ERR_INVALID_VALUE, "NULL tail pointer");
    if (tail_nnz > 0 && (n_cols == 0 || !x)) return fail(SPMV_ERR_INVALID_VALUE, "tail entries need x");
    spmv_status s = spmv_ell_apply(n_rows, n_cols, width, ell_col, ell_val, alpha, x, beta, y, stream);
    if (s != SPMV_OK || n_tail_rows == 0) return s;
    hipStream_t st = as_stream(stream);
    const int64_t mean = (tail_nnz + n_tail_rows - 1) / n_tail_rows;
    int g = 1;
    while (g < 64 && g < mean) g <<= 1;
    const int grid = (int)ceil_div((int64_t)n_tail_rows * g, WG);
    switch (g) {
#define SPMV_TAIL_G(G)                                                                                       \
    case G:                                                                                                  \
        k_hyb_tail<G><<<grid, WG, 0, st>>>(n_tail_rows, tail_rows, tail_rp, tail_col, tail_val, x, alpha, y); \
        break;
        SPMV_TAIL_G(1) SPMV_TAIL_G(2) SPMV_TAIL_G(4) SPMV_TAIL_G(8) SPMV_TAIL_G(16) SPMV_TAIL_G(32) SPMV_TAIL_G(64)
#undef SPMV_TAIL_G
    default:
        return fail(SPMV_ERR_INVALID_VALUE, "bad group size %d", g);
    }
    SPMV_LAUNCHED("k_hyb_tail");
    return SPMV_OK;
}

// ---------------------------------------------------------------------------
// Format chosen by the CV rule
// ---------------------------------------------------------------------------

struct spmv_auto {
    spmv_auto_plan_t plan;
    int32_t n_rows, n_cols, nnz;
    int32_t *ell_col = nullptr;
    float *ell_val = nullptr;
    int32_t *tail_rows = nullptr, *tail_rp = nullptr, *tail_col = nullptr;
    float *tail_val = nullptr;
    int32_t *tail_full = nullptr;   // HYB: the tail's entries per row (n_rows + 1 pointers)
    bool one_launch = false;        // HYB: short tails, ELL and tail in one kernel when x and y allow
    spmv_csr_t csr = nullptr;    // CSR format, or the HYB tail's binned plan
};

namespace {

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// HYB tails of at most this many entries per row run in the ELL kernel
// (each wave then sums at most 256 * HYB_ONE_LAUNCH_TAIL entries); longer
// ones go through the binned CSR plan of the tail.
constexpr int HYB_ONE_LAUNCH_TAIL = 16;

struct AutoLayout {
    size_t ell_col, ell_val, tail_rows, tail_rp, tail_col, tail_val, tail_full, tail_plan, tail_plan_bytes, scratch,
        scratch_bytes, total;
};

AutoLayout auto_layout(const spmv_auto_plan_t &p, int32_t n_rows) {
    AutoLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align256(off + std::max<size_t>(bytes, 4));
        return at;
    };
    const size_t slots = (size_t)p.width * (size_t)n_rows;
    L.ell_col = take(4 * slots);
    L.ell_val = take(4 * slots);
    L.tail_rows = take(4 * (size_t)p.n_tail_rows);
    L.tail_rp = take(4 * ((size_t)p.n_tail_rows + 1));
    L.tail_col = take(4 * (size_t)p.tail_nnz);
    L.tail_val = take(4 * (size_t)p.tail_nnz);
    L.tail_full = take(p.format == SPMV_FORMAT_HYB ? 4 * ((size_t)n_rows + 1) : 0);
    L.tail_plan_bytes = 0;
    if (p.n_tail_rows > 0 && spmv_csr_plan_size(p.n_tail_rows, (int32_t)p.tail_nnz, nullptr, &L.tail_plan_bytes) != SPMV_OK)
        L.tail_plan_bytes = 0;
    L.tail_plan = take(L.tail_plan_bytes);
    // the conversion's own scratch (spmv_scratch_size), used during create only
    L.scratch_bytes = scratch_bytes(n_rows);
    L.scratch = take(L.scratch_bytes);
    L.total = off;
    return L;
}

}  // namespace

extern "C" spmv_status spmv_auto_plan(int32_t n_rows, int32_t n_cols, int32_t nnz, const int32_t *row_ptr,
                                      spmv_auto_plan_t *plan, void *scratch, size_t scratch_bytes, void *stream) {
    if (!plan) return fail(SPMV_ERR_INVALID_VALUE, "plan is NULL");
    if (n_rows < 0 || n_cols < 0 || nnz < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    spmv_status cs = check_scratch(scratch, scratch_bytes, n_rows);
    if (cs != SPMV_OK) return cs;
    spmv_auto_plan_t p{};
    p.format = SPMV_FORMAT_CSR;
    int32_t max_len = 0;
    int64_t s1 = 0, s2 = 0;
    if (n_rows > 0) {
        if (!row_ptr) return fail(SPMV_ERR_INVALID_VALUE, "row_ptr is NULL");
        spmv_status s = spmv_csr_row_stats(n_rows, row_ptr, &max_len, &s1, &s2, scratch, scratch_bytes, stream);
        if (s != SPMV_OK) return s;
        if (s1 != nnz)
            return fail(SPMV_ERR_INVALID_MATRIX, "row lengths sum to %lld, not nnz = %d", (long long)s1, nnz);
        s = spmv_format_recommend(n_rows, s1, s2, &p.format);
        if (s != SPMV_OK) return s;
    }
    // ELL pads every row to the longest one; when that would more than
    // double the storage of max(nnz, n_rows) entries, or overflow int32
    // slot indices, the HYB split is used instead.
    if (p.format == SPMV_FORMAT_ELL &&
        ((int64_t)max_len * n_rows > 2 * std::max<int64_t>(nnz, n_rows) || (int64_t)max_len * n_rows > INT32_MAX))
        p.format = SPMV_FORMAT_HYB;
    if (p.format == SPMV_FORMAT_ELL) {
        p.width = max_len;
    } else if (p.format == SPMV_FORMAT_HYB) {
        spmv_status s = spmv_hyb_width(n_rows, row_ptr, SPMV_HYB_ELL_NUM, SPMV_HYB_ELL_DEN, &p.width,
                                       &p.n_tail_rows, &p.tail_nnz, scratch, scratch_bytes, stream);
        if (s != SPMV_OK) return s;
        if ((int64_t)p.width * n_rows > INT32_MAX) p.format = SPMV_FORMAT_CSR;
    }
    if (p.format == SPMV_FORMAT_CSR) {
        p.width = 0;
        p.n_tail_rows = 0;
        p.tail_nnz = 0;
        spmv_status s = spmv_csr_plan_size(n_rows, nnz, nullptr, &p.workspace_bytes);
        if (s != SPMV_OK) return s;
    } else {
        p.workspace_bytes = auto_layout(p, n_rows).total;
    }
    *plan = p;
    return SPMV_OK;
}

extern "C" spmv_status spmv_auto_create(spmv_auto_t *out, const spmv_auto_plan_t *plan, int32_t n_rows,
                                        int32_t n_cols, int32_t nnz, const int32_t *row_ptr,
                                        const int32_t *col_idx, const float *vals, void *workspace,
                                        size_t workspace_bytes, void *stream) {
    if (!out || !plan) return fail(SPMV_ERR_INVALID_VALUE, "NULL handle or plan pointer");
    *out = nullptr;
    const spmv_auto_plan_t &p = *plan;
    if (p.format < SPMV_FORMAT_ELL || p.format > SPMV_FORMAT_CSR)
        return fail(SPMV_ERR_INVALID_VALUE, "unknown format %d", p.format);
    if (workspace_bytes < p.workspace_bytes)
        return fail(SPMV_ERR_INVALID_VALUE, "workspace of %zu bytes is smaller than %zu", workspace_bytes,
                    p.workspace_bytes);
    if (p.workspace_bytes > 0 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)))
        return fail(SPMV_ERR_INVALID_VALUE, "workspace must be non-NULL and 256-byte aligned");
    spmv_auto *h = new spmv_auto();
    h->plan = p;
    h->n_rows = n_rows;
    h->n_cols = n_cols;
    h->nnz = nnz;
    spmv_status s = SPMV_OK;
    if (p.format == SPMV_FORMAT_CSR) {
        s = spmv_csr_create(&h->csr, n_rows, n_cols, nnz, row_ptr, col_idx, vals, SPMV_CSR_BINNED, nullptr,
                            workspace, workspace_bytes, stream);
    } else {
        const AutoLayout L = auto_layout(p, n_rows);
        char *ws = static_cast<char *>(workspace);
        h->ell_col = reinterpret_cast<int32_t *>(ws + L.ell_col);
        h->ell_val = reinterpret_cast<float *>(ws + L.ell_val);
        h->tail_rows = reinterpret_cast<int32_t *>(ws + L.tail_rows);
        h->tail_rp = reinterpret_cast<int32_t *>(ws + L.tail_rp);
        h->tail_col = reinterpret_cast<int32_t *>(ws + L.tail_col);
        h->tail_val = reinterpret_cast<float *>(ws + L.tail_val);
        if (p.format == SPMV_FORMAT_ELL)
            s = spmv_ell_from_csr(n_rows, n_cols, nnz, row_ptr, col_idx, vals, p.width, h->ell_col, h->ell_val,
                                  ws + L.scratch, L.scratch_bytes, stream);
        else
            s = spmv_hyb_from_csr(n_rows, n_cols, nnz, row_ptr, col_idx, vals, p.width, h->ell_col, h->ell_val,
                                  p.n_tail_rows, p.tail_nnz, h->tail_rows, h->tail_rp, h->tail_col, h->tail_val,
                                  ws + L.scratch, L.scratch_bytes, stream);
        // the tail as a CSR matrix over the tail rows, with its own plan
        if (s == SPMV_OK && p.format == SPMV_FORMAT_HYB && p.n_tail_rows > 0)
            s = spmv_csr_create(&h->csr, p.n_tail_rows, n_cols, (int32_t)p.tail_nnz, h->tail_rp, h->tail_col,
                                h->tail_val, SPMV_CSR_BINNED, nullptr, ws + L.tail_plan, L.tail_plan_bytes, stream);
        // and per row, for the one-launch apply when every tail is short
        if (s == SPMV_OK && p.format == SPMV_FORMAT_HYB) {
            int32_t max_len = 0;
            int64_t s1 = 0, s2 = 0;
            s = spmv_csr_row_stats(n_rows, row_ptr, &max_len, &s1, &s2, ws + L.scratch, L.scratch_bytes, stream);
            if (s == SPMV_OK) {
                h->tail_full = reinterpret_cast<int32_t *>(ws + L.tail_full);
                hipStream_t st = as_stream(stream);
                k_hyb_row_tail<<<(int)ceil_div((int64_t)n_rows + 1, WG), WG, 0, st>>>(n_rows, p.n_tail_rows,
                                                                                      h->tail_rows, h->tail_rp,
                                                                                      h->tail_full);
                SPMV_LAUNCHED("k_hyb_row_tail");
                h->one_launch = max_len - p.width <= HYB_ONE_LAUNCH_TAIL &&
                                ell_tail_fits(n_rows, n_cols, p.width, h->ell_col, h->ell_val, h->tail_full);
                if (hipStreamSynchronize(st) != hipSuccess) s = fail(SPMV_ERR_HIP, "hipStreamSynchronize failed");
            }
        }
    }
    if (s != SPMV_OK) {
        delete h;
        return s;
    }
    *out = h;
    return SPMV_OK;
}

extern "C" spmv_status spmv_auto_apply(spmv_auto_t h, float alpha, const float *x, float beta, float *y,
                                       void *stream) {
    if (!h) return fail(SPMV_ERR_INVALID_VALUE, "handle is NULL");
    switch (h->plan.format) {
    case SPMV_FORMAT_CSR:
        return spmv_csr_apply(h->csr, alpha, x, beta, y, stream);
    case SPMV_FORMAT_ELL:
        return spmv_ell_apply(h->n_rows, h->n_cols, h->plan.width, h->ell_col, h->ell_val, alpha, x, beta, y,
                              stream);
    default: {
        // short tails: ELL part and tail in one kernel, one store per row
        if (h->one_launch && x && y && aligned16(x) && aligned16(y))
            return ell_tail_apply(h->n_rows, h->plan.width, h->ell_col, h->ell_val, h->tail_full, h->tail_col,
                                  h->tail_val, alpha, x, beta, y, as_stream(stream));
        // else the ELL part, then the tail rows added in place (beta = 1)
        // through the binned CSR kernels with the tail's row map
        spmv_status s = spmv_ell_apply(h->n_rows, h->n_cols, h->plan.width, h->ell_col, h->ell_val, alpha, x,
                                       beta, y, stream);
        if (s != SPMV_OK || !h->csr) return s;
        return spmv_csr_apply_rows(h->csr, alpha, x, 1.0f, y, h->tail_rows, stream);
    }
    }
}

extern "C" spmv_status spmv_auto_destroy(spmv_auto_t h) {
    if (h) spmv_csr_destroy(h->csr);
    delete h;
    return SPMV_OK;
}
