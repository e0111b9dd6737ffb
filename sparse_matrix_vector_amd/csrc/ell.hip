// ELL on gfx950: CSR -> ELL conversion and the ELL product.
//
// "Why SpMV needs CUDA optimisation" (section 2.1 table) names ELL as the
// fixed-width, zero-padded format that suits rows of equal length and is
// sensitive to padding.  Layout here: slot-major, entry k of row i at
// [k * n_rows + i], so lane i of a wave reads row i's k-th entry and
// consecutive lanes read consecutive words.  A padding slot holds column -1
// and value +0.0f and is skipped (x is never read for it).
//
// Apply: when n_rows % 4 == 0 and the arrays are 16-byte aligned, each lane
// owns four consecutive rows and reads each slot as one 16-byte load of
// columns and one of values; otherwise one lane per row with 4-byte loads.
// Products are summed in slot order in fp32.
#include "common.hpp"

#include <algorithm>
#include <climits>

namespace spmv {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WG = 256;

// Copies row i's entries into its slots and pads the rest.  Columns outside
// [0, n_cols) and an inconsistent row_ptr raise `err` (the caller reports it).
__global__ __launch_bounds__(WG) void k_ell_from_csr(int n, int n_cols, int nnz, int width,
                                                     const int *__restrict__ rp, const int *__restrict__ ci,
                                                     const float *__restrict__ v, int *__restrict__ ec,
                                                     float *__restrict__ ev, int *__restrict__ err) {
    const int i = blockIdx.x * WG + threadIdx.x;
    if (i >= n) return;
    const int s = rp[i], len = rp[i + 1] - s;
    bool bad = (i == 0 && s != 0) || (i == n - 1 && rp[n] != nnz) || len < 0 || len > width;
    for (int k = 0; k < width; ++k) {
        const size_t slot = (size_t)k * (size_t)n + (size_t)i;
        const bool real = !bad && k < len;
        const int c = real ? ci[s + k] : -1;
        bad |= real && (unsigned)c >= (unsigned)n_cols;
        ec[slot] = c;
        ev[slot] = real ? v[s + k] : 0.0f;
    }
    if (bad) atomicOr(err, 1);
}

// Same XCD grouping as the CSR kernels: the workgroups dispatched to one XCD
// take a contiguous range of rows.
__device__ __forceinline__ int xcd_contiguous(int w, int nw) {
    constexpr int NX = 8;
    const int q = nw / NX, r = nw % NX;
    const int xcd = w % NX, idx = w / NX;
    return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

__device__ __forceinline__ float finish(float acc, float alpha, float beta, float yold) {
    float r = alpha * acc;
    if (beta != 0.0f) r = fmaf(beta, yold, r);
    return r;
}

// Four rows per lane, 16-byte slot loads.  Slots are taken U at a time (U =
// the whole width when it is at most 8, a compile-time constant): all their
// column and value loads are issued first, then all their gathers (padding
// gathers x[0] and is masked after), so one wait covers each batch instead
// of one per slot.  Slots are summed in slot order.
template <int U>
__global__ __launch_bounds__(WG) void k_ell_apply4(int n, int width, const int *__restrict__ ec,
                                                   const float *__restrict__ ev, float alpha,
                                                   const float *__restrict__ x, float beta, float *__restrict__ y) {
    const int w = xcd_contiguous(blockIdx.x, gridDim.x);
    const int quad = w * WG + threadIdx.x;
    const int i0 = 4 * quad;
    if (i0 >= n) return;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = 0; k0 < width; k0 += U) {
        i32x4 c[U];
        f32x4 f[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = min(k0 + u, width - 1);   // only the generic width reaches past the end
            const size_t slot = (size_t)k * (size_t)n + (size_t)i0;
            c[u] = __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(ec + slot));
            f[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(ev + slot));
        }
        float xv[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < 4; ++t) xv[u][t] = x[(k0 + u < width) ? max(c[u][t], 0) : 0];
#pragma unroll
        for (int u = 0; u < U; ++u) issue_together(xv[u][0], xv[u][1], xv[u][2], xv[u][3]);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc[t] = (k0 + u < width && c[u][t] >= 0) ? fmaf(f[u][t], xv[u][t], acc[t]) : acc[t];
    }
    f32x4 yo = {0.0f, 0.0f, 0.0f, 0.0f};
    if (beta != 0.0f) yo = *reinterpret_cast<const f32x4 *>(y + i0);
    f32x4 r;
#pragma unroll
    for (int t = 0; t < 4; ++t) r[t] = finish(acc[t], alpha, beta, yo[t]);
    *reinterpret_cast<f32x4 *>(y + i0) = r;
}

// Four rows per lane with an x tile in LDS (width U <= 8, x 16-byte aligned,
// n_cols % 4 == 0).  The workgroup's 1024 rows usually gather from a narrow
// range of columns (a banded matrix): after loading its slots, the
// workgroup reduces the smallest and largest column it uses, and if that
// window fits XT_ROUNDS * 4 * WG floats it stages x[window] in LDS with
// 16-byte loads and gathers from LDS (a 16-byte load moves four x values
// through the texture addresser, a gather one).  Wider windows gather from
// memory as in k_ell_apply4.  Every thread takes part in the barriers; rows
// past n only load the matrix's first slot vector.
//
// TAIL: the rows also carry the overflow of a HYB split, stored per row
// (entries of row r at [trp[r], trp[r + 1])), and each row is finished here
// in one store.  A wave's 256 rows own one contiguous run of tail entries:
// its 64 lanes load up to TAIL_BATCH * 64 of them together (issued with the
// x-window loads), take x from the window where the column falls in it
// (else from memory), and leave the products in the wave's LDS buffer, from
// which every lane sums its four rows' share; a longer run takes further
// rounds of the same.
constexpr int XT_ROUNDS = 3;
constexpr int TAIL_BATCH = 8;    // tail entries per lane per round: 512 per wave

struct EllTail {
    const int *trp;     // int32[n + 1], 16-byte aligned
    const int *tcol;
    const float *tval;
};

// One round of a wave's tail: the products of entries [base, base +
// TAIL_BATCH * 64) (clipped to te) are in buf; the lane's rows cover entries
// [b[0], b[4]), row t from b[t].
__device__ __forceinline__ void tail_sum(const float *buf, int base, int te, const int (&b)[5], float (&tacc)[4]) {
    const int end = min(te, base + TAIL_BATCH * 64);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int lo = max(b[t], base), hi = min(b[t + 1], end);
        for (int k = lo; k < hi; ++k) tacc[t] += buf[k - base];
    }
}

// TAIL with width <= 5: held to 128 registers, so that four waves per SIMD
// stay resident (the whole grid of a 1M-row matrix at once)
template <int U, bool TAIL>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(TAIL && U <= 5 ? 4 : 1))) void k_ell_apply4t(int n, const int *__restrict__ ec, const float *__restrict__ ev,
                                                    float alpha, const float *__restrict__ x, float beta,
                                                    float *__restrict__ y, EllTail tl) {
    __shared__ __attribute__((aligned(16))) float xt[XT_ROUNDS * 4 * WG];
    __shared__ int red[2][WG / 64];
    __shared__ float tbuf[TAIL ? WG / 64 : 1][TAIL ? TAIL_BATCH * 64 : 1];
    const int w = xcd_contiguous(blockIdx.x, gridDim.x);
    const int i0 = 4 * (w * WG + (int)threadIdx.x);
    const bool live = i0 < n;
    const int ib = live ? i0 : 0;
    i32x4 c[U];
    f32x4 f[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const size_t slot = (size_t)u * (size_t)n + (size_t)ib;
        c[u] = __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(ec + slot));
        f[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(ev + slot));
    }
    // TAIL: the lane's row bounds in the tail, and the wave's run [tb, te)
    int tb_ = 0, te_ = 0;
    int b[5] = {0, 0, 0, 0, 0};
    const int lane = __lane_id();
    if (TAIL) {
        if (live) {
            const i32x4 q = *reinterpret_cast<const i32x4 *>(tl.trp + i0);
            b[0] = q.x;
            b[1] = q.y;
            b[2] = q.z;
            b[3] = q.w;
            b[4] = tl.trp[i0 + 4];
        }
        // live lanes are a prefix of the wave (rows grow with the lane)
        const int nl = __popcll(__ballot(live));
        tb_ = __builtin_amdgcn_readfirstlane(b[0]);
        te_ = nl > 0 ? __builtin_amdgcn_readlane(b[4], max(nl - 1, 0)) : tb_;
    }
    // the workgroup's column window (padding, -1, and dead rows excluded)
    int mn = INT_MAX, mx = -1;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int cc = live ? c[u][t] : -1;
            mn = cc >= 0 ? min(mn, cc) : mn;
            mx = max(mx, cc);
        }
    for (int off = 32; off > 0; off >>= 1) {
        mn = min(mn, __shfl_xor(mn, off));
        mx = max(mx, __shfl_xor(mx, off));
    }
    if (__lane_id() == 0) {
        red[0][threadIdx.x / 64] = mn;
        red[1][threadIdx.x / 64] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < WG / 64; ++q) {
        mn = min(mn, red[0][q]);
        mx = max(mx, red[1][q]);
    }
    const int tb = mx >= 0 ? (mn & ~3) : 0;
    const int nvec = mx >= 0 ? (mx + 4 - tb) >> 2 : 1;
    // TAIL: the first round's entries, loaded with the window (clamped to
    // the run, zero value past its end)
    int tc[TAIL ? TAIL_BATCH : 1];
    float tv_[TAIL ? TAIL_BATCH : 1];
    auto tail_load = [&](int base) {
#pragma unroll
        for (int j = 0; j < TAIL_BATCH; ++j) {
            const int k = base + j * 64 + lane;
            const int kk = min(k, te_ - 1);
            tc[j] = tl.tcol[kk];
            tv_[j] = k < te_ ? tl.tval[kk] : 0.0f;
        }
    };
    if (TAIL && te_ > tb_) tail_load(tb_);
    float xv[U][4];
    const bool win = nvec <= XT_ROUNDS * WG;
    if (win) {   // uniform over the workgroup
        f32x4 tv[XT_ROUNDS];
#pragma unroll
        for (int r = 0; r < XT_ROUNDS; ++r)
            tv[r] = *reinterpret_cast<const f32x4 *>(x + tb + 4 * min((int)threadIdx.x + r * WG, nvec - 1));
#pragma unroll
        for (int r = 0; r < XT_ROUNDS; ++r)
            *reinterpret_cast<f32x4 *>(xt + 4 * min((int)threadIdx.x + r * WG, nvec - 1)) = tv[r];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        const int hi = 4 * nvec - 1;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < 4; ++t) xv[u][t] = xt[min(max(c[u][t] - tb, 0), hi)];
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < 4; ++t) xv[u][t] = x[max(c[u][t], 0)];
#pragma unroll
        for (int u = 0; u < U; ++u) issue_together(xv[u][0], xv[u][1], xv[u][2], xv[u][3]);
    }
    float tacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (TAIL && te_ > tb_) {   // uniform over the wave
        float *buf = tbuf[threadIdx.x / 64];
        for (int base = tb_; base < te_; base += TAIL_BATCH * 64) {
            if (base != tb_) tail_load(base);
            // x from the workgroup's window where the column falls in it
            float g[TAIL_BATCH];
#pragma unroll
            for (int j = 0; j < TAIL_BATCH; ++j) {
                const unsigned o = (unsigned)(tc[j] - tb);
                g[j] = win && o < 4u * (unsigned)nvec ? xt[o] : x[tc[j]];
            }
#pragma unroll
            for (int j = 0; j < TAIL_BATCH; ++j) buf[j * 64 + lane] = tv_[j] * g[j];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            tail_sum(buf, base, te_, b, tacc);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
    if (!live) return;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = c[u][t] >= 0 ? fmaf(f[u][t], xv[u][t], acc[t]) : acc[t];
    if (TAIL) {
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] += tacc[t];
    }
    f32x4 yo = {0.0f, 0.0f, 0.0f, 0.0f};
    if (beta != 0.0f) yo = *reinterpret_cast<const f32x4 *>(y + i0);
    f32x4 r;
#pragma unroll
    for (int t = 0; t < 4; ++t) r[t] = finish(acc[t], alpha, beta, yo[t]);
    *reinterpret_cast<f32x4 *>(y + i0) = r;
}

// One row per lane.
__global__ __launch_bounds__(WG) void k_ell_apply1(int n, int width, const int *__restrict__ ec,
                                                   const float *__restrict__ ev, float alpha,
                                                   const float *__restrict__ x, float beta, float *__restrict__ y) {
    const int w = xcd_contiguous(blockIdx.x, gridDim.x);
    const int i = w * WG + threadIdx.x;
    if (i >= n) return;
    float acc = 0.0f;
    for (int k = 0; k < width; ++k) {
        const size_t slot = (size_t)k * (size_t)n + (size_t)i;
        const int c = ec[slot];
        const float xv = x[max(c, 0)];
        acc = c >= 0 ? fmaf(ev[slot], xv, acc) : acc;
    }
    y[i] = finish(acc, alpha, beta, beta != 0.0f ? y[i] : 0.0f);
}

__global__ void k_scale(int n, float beta, float *__restrict__ y) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) y[i] = beta != 0.0f ? beta * y[i] : 0.0f;
}

}  // namespace

bool ell_tail_fits(int32_t n_rows, int32_t n_cols, int32_t width, const void *ec, const void *ev, const void *trp) {
    return n_rows > 0 && n_rows % 4 == 0 && n_cols > 0 && n_cols % 4 == 0 && width >= 1 && width <= 8 && ec && ev &&
           trp && aligned16(ec) && aligned16(ev) && aligned16(trp);
}

spmv_status ell_tail_apply(int32_t n_rows, int32_t width, const int32_t *ell_col, const float *ell_val,
                           const int32_t *trp, const int32_t *tcol, const float *tval, float alpha, const float *x,
                           float beta, float *y, hipStream_t st) {
    const int grid = (int)ceil_div(n_rows / 4, WG);
    const EllTail tl{trp, tcol, tval};
    switch (width) {
#define SPMV_ELL_TT(W)                                                                               \
    case W:                                                                                          \
        k_ell_apply4t<W, true><<<grid, WG, 0, st>>>(n_rows, ell_col, ell_val, alpha, x, beta, y, tl); \
        break;
        SPMV_ELL_TT(1) SPMV_ELL_TT(2) SPMV_ELL_TT(3) SPMV_ELL_TT(4) SPMV_ELL_TT(5) SPMV_ELL_TT(6) SPMV_ELL_TT(7)
        SPMV_ELL_TT(8)
#undef SPMV_ELL_TT
    default:
        return fail(SPMV_ERR_INVALID_VALUE, "width %d outside 1..8", width);
    }
    SPMV_LAUNCHED("k_ell_apply4t");
    return SPMV_OK;
}

}  // namespace spmv

using namespace spmv;

extern "C" spmv_status spmv_ell_from_csr(int32_t n_rows, int32_t n_cols, int32_t nnz, const int32_t *row_ptr,
                                         const int32_t *col_idx, const float *vals, int32_t width,
                                         int32_t *ell_col, float *ell_val, void *scratch, size_t scratch_bytes,
                                         void *stream) {
    if (n_rows < 0 || n_cols < 0 || nnz < 0 || width < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if ((int64_t)n_rows * width > INT32_MAX)
        return fail(SPMV_ERR_OVERFLOW, "width * n_rows = %lld exceeds int32", (long long)n_rows * width);
    if (n_rows == 0 || width == 0) {
        if (n_rows > 0 && nnz > 0) return fail(SPMV_ERR_INVALID_VALUE, "width 0 cannot hold %d nonzeros", nnz);
        return SPMV_OK;
    }
    if (!row_ptr || !ell_col || !ell_val || (nnz > 0 && (!col_idx || !vals)))
        return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    int32_t max_len = 0;
    int64_t s1 = 0, s2 = 0;
    spmv_status s = spmv_csr_row_stats(n_rows, row_ptr, &max_len, &s1, &s2, scratch, scratch_bytes, stream);
    if (s != SPMV_OK) return s;
    if (s1 != nnz) return fail(SPMV_ERR_INVALID_MATRIX, "row lengths sum to %lld, not nnz = %d", (long long)s1, nnz);
    if (max_len > width) return fail(SPMV_ERR_INVALID_VALUE, "width %d is shorter than the longest row (%d)", width, max_len);
    hipStream_t st = as_stream(stream);
    // with row_ptr[0] == 0, non-decreasing rows and lengths summing to nnz,
    // every entry the conversion reads lies in [0, nnz)
    int rp0 = -1;
    SPMV_HIP(hipMemcpyAsync(&rp0, row_ptr, sizeof(int), hipMemcpyDeviceToHost, st));
    SPMV_HIP(hipStreamSynchronize(st));
    if (rp0 != 0) return fail(SPMV_ERR_INVALID_MATRIX, "row_ptr[0] != 0");
    int *d_err = reinterpret_cast<int *>(static_cast<char *>(scratch) + SCRATCH_ERR);
    SPMV_HIP(hipMemsetAsync(d_err, 0, sizeof(int), st));
    k_ell_from_csr<<<(int)ceil_div(n_rows, WG), WG, 0, st>>>(n_rows, n_cols, nnz, width, row_ptr, col_idx, vals,
                                                             ell_col, ell_val, d_err);
    SPMV_LAUNCHED("k_ell_from_csr");
    int err = 0;
    SPMV_HIP(hipMemcpyAsync(&err, d_err, sizeof(int), hipMemcpyDeviceToHost, st));
    SPMV_HIP(hipStreamSynchronize(st));
    if (err) return fail(SPMV_ERR_INVALID_MATRIX, "row_ptr inconsistent or a column outside [0, n_cols)");
    return SPMV_OK;
}

extern "C" spmv_status spmv_ell_apply(int32_t n_rows, int32_t n_cols, int32_t width, const int32_t *ell_col,
                                      const float *ell_val, float alpha, const float *x, float beta, float *y,
                                      void *stream) {
    if (n_rows < 0 || n_cols < 0 || width < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if ((int64_t)n_rows * width > INT32_MAX) return fail(SPMV_ERR_OVERFLOW, "width * n_rows exceeds int32");
    if (n_rows == 0) return SPMV_OK;
    if (!y) return fail(SPMV_ERR_INVALID_VALUE, "y is NULL");
    hipStream_t st = as_stream(stream);
    if (width == 0 || n_cols == 0) {   // no slot can hold a column: y = beta * y
        k_scale<<<(int)ceil_div(n_rows, WG), WG, 0, st>>>(n_rows, beta, y);
        SPMV_LAUNCHED("k_scale");
        return SPMV_OK;
    }
    if (!ell_col || !ell_val || !x) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    const bool quad = (n_rows % 4 == 0) && aligned16(ell_col) && aligned16(ell_val) && aligned16(y);
    if (quad && width <= 8 && aligned16(x) && n_cols % 4 == 0) {
        const int grid = (int)ceil_div(n_rows / 4, WG);
        switch (width) {
#define SPMV_ELL_T(W)                                                                                   \
    case W:                                                                                             \
        k_ell_apply4t<W, false><<<grid, WG, 0, st>>>(n_rows, ell_col, ell_val, alpha, x, beta, y, EllTail{}); \
        break;
            SPMV_ELL_T(1) SPMV_ELL_T(2) SPMV_ELL_T(3) SPMV_ELL_T(4) SPMV_ELL_T(5) SPMV_ELL_T(6) SPMV_ELL_T(7)
            SPMV_ELL_T(8)
#undef SPMV_ELL_T
        }
        SPMV_LAUNCHED("k_ell_apply4t");
    } else if (quad) {
        const int grid = (int)ceil_div(n_rows / 4, WG);
        switch (width) {
#define SPMV_ELL_W(W)                                                                                    \
    case W:                                                                                              \
        k_ell_apply4<W><<<grid, WG, 0, st>>>(n_rows, width, ell_col, ell_val, alpha, x, beta, y);      \
        break;
            SPMV_ELL_W(1) SPMV_ELL_W(2) SPMV_ELL_W(3) SPMV_ELL_W(4) SPMV_ELL_W(5) SPMV_ELL_W(6) SPMV_ELL_W(7)
            SPMV_ELL_W(8)
#undef SPMV_ELL_W
        default:
            k_ell_apply4<4><<<grid, WG, 0, st>>>(n_rows, width, ell_col, ell_val, alpha, x, beta, y);
        }
        SPMV_LAUNCHED("k_ell_apply4");
    } else {
        k_ell_apply1<<<(int)ceil_div(n_rows, WG), WG, 0, st>>>(n_rows, width, ell_col, ell_val, alpha, x, beta, y);
        SPMV_LAUNCHED("k_ell_apply1");
    }
    return SPMV_OK;
}
