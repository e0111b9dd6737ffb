// CSR SpMV on gfx950: validation, the row-grouping planner and the apply
// kernels (scalar, vector, binned).
//
// The operation is the CSR product of "Why SpMV needs CUDA optimisation"
// (section 2.1 scalar kernel: one thread sums values[k] * x[col_idx[k]] over
// its row; section 4.1: a warp shares a row and reduces).  The binned variant
// follows the row grouping of "Sparse matrix multiplication acceleration"
// (section 2.1.1 table: groups by work per row with bounds 32 / 512 / 8192,
// one thread-to-row mapping per group; section 2.2.1: the rows of a group
// are reached through a Map[] array; section 2.3: the largest group falls
// back to global memory).  For y = A x the work of a row is its nonzero
// count.
//
// gfx950 mapping of the four groups (wave64, 256-thread workgroups):
//   group 0 (short rows)   runs of consecutive short rows are cut into
//                          blocks of <= 512 staged entries / 128 rows; one wave
//                          streams a block's values and columns with 16-byte
//                          loads, multiplies by the gathered x, stages the
//                          products in LDS and then each lane sums whole
//                          rows (a segmented reduction without atomics);
//   group 1 (32..511)      one wave per row, 16-byte loads, DPP reduction;
//   group 2 (512..8191)    one workgroup per row, LDS reduction of 4 waves;
//   group 3 (>= 8192)      a row is split into 8192-nonzero chunks, one
//                          workgroup per chunk writes a partial sum to the
//                          workspace, a second kernel adds the partials of a
//                          row in order (the global-memory fallback).
// All groups run in one launch; the workgroup id selects the group.  Every
// path sums in a fixed order, so results are bit-reproducible run to run.
#include "common.hpp"

#include <algorithm>
#include <vector>

namespace spmv {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Compile-time shape of the short-row blocks (overridable for tuning sweeps).
#ifndef SPMV_SHORT_VPL
#define SPMV_SHORT_VPL 2
#endif

constexpr int WG = 256;                 // threads per workgroup everywhere here
constexpr int WAVES = WG / 64;
constexpr int SHORT_VPL = SPMV_SHORT_VPL;          // 16-byte vectors per lane in a short block
constexpr int SHORT_SLOTS = 64 * 4 * SHORT_VPL;    // entries staged per wave
constexpr int SHORT_RMAX = 64 * SHORT_VPL;         // rows per short block (VPL per lane)
constexpr int LONG_CHUNK = 8192;        // nonzeros per workgroup in group 3
constexpr int MAX_T0 = SHORT_SLOTS / 2 < 256 ? SHORT_SLOTS / 2 : 256;   // largest bound of group 0

// Error bits raised by the validation kernels.
constexpr int ERR_RP0 = 1, ERR_RPN = 2, ERR_MONO = 4, ERR_COL = 8;

// Device-side plan header (int32 words).
struct Meta {
    int bin_offsets[5];
    int head_totals[2];   // {0, number of runs of short rows}
    int block_totals[2];  // {0, number of short blocks}
    int err;
};

__device__ __forceinline__ int row_group(int len, int t0, int t1, int t2) {
    return len < t0 ? 0 : (len < t1 ? 1 : (len < t2 ? 2 : 3));
}

__device__ __forceinline__ void store_y(float *y, int row, float acc, float alpha, float beta) {
    float r = alpha * acc;
    if (beta != 0.0f) r = fmaf(beta, y[row], r);
    y[row] = r;
}

__device__ __forceinline__ unsigned long long lanemask_lt() {
    const int l = __lane_id();
    return l ? (~0ull >> (64 - l)) : 0ull;
}

// ---------------------------------------------------------------------------
// Validation
// ---------------------------------------------------------------------------
__global__ void k_validate_rows(int n, int nnz, const int *__restrict__ rp, int *__restrict__ err) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i > n) return;
    int bad = 0;
    const int a = rp[i];
    if (i == 0 && a != 0) bad |= ERR_RP0;
    if (i == n && a != nnz) bad |= ERR_RPN;
    if (i < n && rp[i + 1] < a) bad |= ERR_MONO;
    if (bad) atomicOr(err, bad);
}

__global__ void k_validate_cols(int nnz, int n_cols, const int *__restrict__ ci, int *__restrict__ err) {
    int bad = 0;
    for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < nnz; k += gridDim.x * blockDim.x)
        bad |= (unsigned)ci[k] >= (unsigned)n_cols;
    if (bad) atomicOr(err, ERR_COL);
}

// ---------------------------------------------------------------------------
// Row statistics (max, sum, sum of squares of lengths)
// ---------------------------------------------------------------------------
__global__ void k_row_stats(int n, const int *__restrict__ rp, int *__restrict__ out_max,
                            unsigned long long *__restrict__ out_sum,
                            unsigned long long *__restrict__ out_sq, int *__restrict__ err) {
    __shared__ int smax[WAVES];
    __shared__ unsigned long long ssum[WAVES], ssq[WAVES];
    int m = 0;
    unsigned long long s = 0, q = 0;
    int bad = 0;
    for (int i = blockIdx.x * WG + threadIdx.x; i < n; i += gridDim.x * WG) {
        const int len = rp[i + 1] - rp[i];
        bad |= len < 0;
        const int l = len < 0 ? 0 : len;
        m = max(m, l);
        s += (unsigned long long)l;
        q += (unsigned long long)l * (unsigned long long)l;
    }
    if (bad) atomicOr(err, ERR_MONO);
    for (int off = 32; off > 0; off >>= 1) {
        m = max(m, __shfl_xor(m, off));
        s += __shfl_xor(s, off);
        q += __shfl_xor(q, off);
    }
    const int w = threadIdx.x / 64;
    if (__lane_id() == 0) {
        smax[w] = m;
        ssum[w] = s;
        ssq[w] = q;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int k = 1; k < WAVES; ++k) {
            m = max(m, smax[k]);
            s += ssum[k];
            q += ssq[k];
        }
        atomicMax(out_max, m);
        atomicAdd(out_sum, s);
        atomicAdd(out_sq, q);
    }
}

// ---------------------------------------------------------------------------
// Planner: stable counting sort of rows by group (bit-exact with a serial
// counting sort), then the short-row blocks.
// ---------------------------------------------------------------------------

// Per-workgroup count of rows in each group.
__global__ __launch_bounds__(WG) void k_plan_count(int n, const int *__restrict__ rp, int t0, int t1,
                                                   int t2, int *__restrict__ counts) {
    __shared__ int wc[WAVES][4];
    const int i = blockIdx.x * WG + threadIdx.x;
    const int g = i < n ? row_group(rp[i + 1] - rp[i], t0, t1, t2) : -1;
    const int w = threadIdx.x / 64;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const unsigned long long m = __ballot(g == b);
        if (__lane_id() == 0) wc[w][b] = __popcll(m);
    }
    __syncthreads();
    if (threadIdx.x < 4) {
        int c = 0;
        for (int k = 0; k < WAVES; ++k) c += wc[k][threadIdx.x];
        counts[blockIdx.x * 4 + threadIdx.x] = c;
    }
}

// Exclusive scan of per-workgroup counts, `ncol` counters per workgroup
// (ncol = 4 for the groups, 1 for the block heads), column by column:
// offsets[w][c] = sum_{c' < c} total[c'] + sum_{w' < w} counts[w'][c].
// One workgroup of 1024 threads.  totals_out[0..ncol] receives the column
// starts and the grand total.
__global__ __launch_bounds__(1024) void k_plan_scan(int nwg, int ncol, const int *__restrict__ counts,
                                                    int *__restrict__ offsets, int *__restrict__ totals_out) {
    __shared__ int sc[4][1024];
    __shared__ int base[5];
    const int t = threadIdx.x;
    const int per = (nwg + 1023) / 1024;
    const int w0 = min(nwg, t * per), w1 = min(nwg, w0 + per);
    int loc[4] = {0, 0, 0, 0};
    for (int w = w0; w < w1; ++w)
        for (int c = 0; c < ncol; ++c) loc[c] += counts[w * ncol + c];
    for (int c = 0; c < 4; ++c) sc[c][t] = loc[c];
    __syncthreads();
    // Hillis-Steele inclusive scan over the 1024 thread sums.
    for (int d = 1; d < 1024; d <<= 1) {
        int v[4];
        for (int c = 0; c < 4; ++c) v[c] = t >= d ? sc[c][t - d] : 0;
        __syncthreads();
        for (int c = 0; c < 4; ++c) sc[c][t] += v[c];
        __syncthreads();
    }
    if (t == 0) {
        int run = 0;
        for (int c = 0; c < ncol; ++c) {
            base[c] = run;
            run += sc[c][1023];
        }
        base[ncol] = run;
        for (int c = 0; c <= ncol; ++c) totals_out[c] = base[c];
    }
    __syncthreads();
    for (int c = 0; c < ncol; ++c) {
        int run = base[c] + sc[c][t] - loc[c];
        for (int w = w0; w < w1; ++w) {
            offsets[w * ncol + c] = run;
            run += counts[w * ncol + c];
        }
    }
}

// perm[offset of (workgroup, group) + rank among same-group rows before it] = row.
__global__ __launch_bounds__(WG) void k_plan_scatter(int n, const int *__restrict__ rp, int t0, int t1,
                                                     int t2, const int *__restrict__ offsets,
                                                     int *__restrict__ perm) {
    __shared__ int wc[WAVES][4];
    const int i = blockIdx.x * WG + threadIdx.x;
    const int g = i < n ? row_group(rp[i + 1] - rp[i], t0, t1, t2) : -1;
    const int w = threadIdx.x / 64;
    unsigned long long mine = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const unsigned long long m = __ballot(g == b);
        if (g == b) mine = m;
        if (__lane_id() == 0) wc[w][b] = __popcll(m);
    }
    __syncthreads();
    if (g < 0) return;
    int rank = __popcll(mine & lanemask_lt());
    for (int k = 0; k < w; ++k) rank += wc[k][g];
    perm[offsets[blockIdx.x * 4 + g] + rank] = i;
}

// A run of short rows starts at perm position p if row perm[p] does not
// follow row perm[p-1], or if the two rows start in different windows of
// `window` nonzeros.  Every run is then a range of consecutive rows whose
// first entries lie in one window, so it spans at most window + t0 + 2
// entries from a 16-byte boundary.  Runs longer than SHORT_RMAX rows are cut
// into pieces of SHORT_RMAX rows afterwards (k_blocks_write).
__device__ __forceinline__ bool short_head(int p, const int *__restrict__ perm, const int *__restrict__ rp,
                                           int window) {
    if (p == 0) return true;
    const int r = perm[p];
    if (perm[p - 1] != r - 1) return true;
    return rp[r] / window != rp[r - 1] / window;
}

__global__ __launch_bounds__(WG) void k_heads_count(const Meta *__restrict__ meta, const int *__restrict__ perm,
                                                    const int *__restrict__ rp, int window,
                                                    int *__restrict__ counts) {
    __shared__ int wc[WAVES];
    const int n0 = meta->bin_offsets[1];
    const int p = blockIdx.x * WG + threadIdx.x;
    const bool h = p < n0 && short_head(p, perm, rp, window);
    const unsigned long long m = __ballot(h);
    if (__lane_id() == 0) wc[threadIdx.x / 64] = __popcll(m);
    __syncthreads();
    if (threadIdx.x == 0) {
        int c = 0;
        for (int k = 0; k < WAVES; ++k) c += wc[k];
        counts[blockIdx.x] = c;
    }
}

__global__ __launch_bounds__(WG) void k_heads_scatter(const Meta *__restrict__ meta, const int *__restrict__ perm,
                                                      const int *__restrict__ rp, int window,
                                                      const int *__restrict__ offsets,
                                                      int *__restrict__ head_pos) {
    __shared__ int wc[WAVES];
    const int n0 = meta->bin_offsets[1];
    const int p = blockIdx.x * WG + threadIdx.x;
    const bool h = p < n0 && short_head(p, perm, rp, window);
    const unsigned long long m = __ballot(h);
    const int w = threadIdx.x / 64;
    if (__lane_id() == 0) wc[w] = __popcll(m);
    __syncthreads();
    if (!h) return;
    int rank = __popcll(m & lanemask_lt());
    for (int k = 0; k < w; ++k) rank += wc[k];
    head_pos[offsets[blockIdx.x] + rank] = p;
}

// Number of blocks run k becomes: ceil(rows / SHORT_RMAX); 0 past the last run.
__device__ __forceinline__ int run_blocks(int k, int nh, int n0, const int *__restrict__ head_pos) {
    if (k >= nh) return 0;
    const int rows = (k + 1 < nh ? head_pos[k + 1] : n0) - head_pos[k];
    return (rows + SHORT_RMAX - 1) / SHORT_RMAX;
}

// Exclusive prefix of v over the workgroup (in thread order) and the total.
__device__ __forceinline__ int workgroup_exclusive(int v, int *total) {
    __shared__ int wsum[WAVES];
    int incl = v;
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (__lane_id() >= d) incl += o;
    }
    const int w = threadIdx.x / 64;
    if (__lane_id() == 63) wsum[w] = incl;
    __syncthreads();
    int before = 0, all = 0;
    for (int k = 0; k < WAVES; ++k) {
        if (k < w) before += wsum[k];
        all += wsum[k];
    }
    *total = all;
    return before + incl - v;
}

__global__ __launch_bounds__(WG) void k_blocks_count(const Meta *__restrict__ meta, const int *__restrict__ head_pos,
                                                     int *__restrict__ counts) {
    const int k = blockIdx.x * WG + threadIdx.x;
    int total;
    workgroup_exclusive(run_blocks(k, meta->head_totals[1], meta->bin_offsets[1], head_pos), &total);
    if (threadIdx.x == 0) counts[blockIdx.x] = total;
}

// Block descriptor: first row, row count, first and one-past-last nonzero.
__global__ __launch_bounds__(WG) void k_blocks_write(const Meta *__restrict__ meta,
                                                     const int *__restrict__ head_pos,
                                                     const int *__restrict__ offsets,
                                                     const int *__restrict__ perm, const int *__restrict__ rp,
                                                     i32x4 *__restrict__ desc) {
    const int nh = meta->head_totals[1];
    const int n0 = meta->bin_offsets[1];
    const int k = blockIdx.x * WG + threadIdx.x;
    int total;
    int at = offsets[blockIdx.x] + workgroup_exclusive(run_blocks(k, nh, n0, head_pos), &total);
    if (k >= nh) return;
    const int p = head_pos[k];
    const int rows = (k + 1 < nh ? head_pos[k + 1] : n0) - p;
    const int r0 = perm[p];
    for (int j = 0; j < rows; j += SHORT_RMAX) {
        const int nr = min(SHORT_RMAX, rows - j);
        i32x4 d;
        d.x = r0 + j;
        d.y = nr;
        d.z = rp[r0 + j];
        d.w = rp[r0 + j + nr];
        desc[at++] = d;
    }
}

// Start and end nonzero of every group-3 row (copied to the host to cut rows
// into chunks).
__global__ void k_long_rows(int n3, const int *__restrict__ perm3, const int *__restrict__ rp,
                            int *__restrict__ out) {
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n3) return;
    const int r = perm3[k];
    out[2 * k] = rp[r];
    out[2 * k + 1] = rp[r + 1];
}

// ---------------------------------------------------------------------------
// Apply kernels
// ---------------------------------------------------------------------------

// Entries [q, q+4) of the column and value streams, q % 4 == 0.
//
// VEC (both arrays 16-byte aligned and nnz >= 4): one 16-byte load per
// stream at min(q, last_vec), last_vec = (nnz & ~3) - 4, so the load is
// always inside the arrays and needs no branch; a lane whose vector lies
// past last_vec (only the array's final partial vector) re-reads its
// entries one by one.  Entries past nnz read as column 0 / value 0; the
// callers mask entries outside their row range.  Keeping the common path
// free of divergent branches matters: a divergent path that writes the
// same registers would make the compiler wait for the 16-byte loads before
// the next ones are issued.
template <bool VEC>
__device__ __forceinline__ void load4(const int *__restrict__ ci, const float *__restrict__ v, int q, int nnz,
                                      int last_vec, i32x4 &c, f32x4 &f) {
    if (VEC) {
        const int qq = min(q, last_vec);
        c = __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(ci + qq));
        f = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(v + qq));
        if (q > last_vec) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bool in = q + t < nnz;
                c[t] = in ? ci[q + t] : 0;
                f[t] = in ? v[q + t] : 0.0f;
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bool in = q + t < nnz;
            c[t] = in ? ci[q + t] : 0;
            f[t] = in ? v[q + t] : 0.0f;
        }
    }
}

// Sum of v[k] * x[ci[k]] over k in [s, e) by the `nthreads` threads of a
// wave or workgroup, `tid` in [0, nthreads); each thread covers aligned
// 4-entry vectors strided by 4 * nthreads, U vectors per step with all
// their loads issued before any is used.  A vector past e is replaced by
// the thread's first vector of the step (its entries are masked), and the
// four gathers of each vector are issued unconditionally (entries outside
// [s, e) hold valid columns of neighbouring rows, or 0 past nnz) and masked
// afterwards.
template <bool VEC, int ROW_UNROLL>
__device__ __forceinline__ float strided_row_sum(const int *__restrict__ ci, const float *__restrict__ v,
                                                 const float *__restrict__ x, int s, int e, int nnz, int last_vec,
                                                 int tid, int nthreads) {
    float acc = 0.0f;
    const int base = s & ~3;
    const int step = 4 * nthreads;
    for (int q0 = base + 4 * tid; q0 < e; q0 += step * ROW_UNROLL) {
        i32x4 c[ROW_UNROLL];
        f32x4 f[ROW_UNROLL];
#pragma unroll
        for (int u = 0; u < ROW_UNROLL; ++u) {
            const int q = q0 + u * step;
            load4<VEC>(ci, v, q < e ? q : q0, nnz, last_vec, c[u], f[u]);
        }
        // masked entries gather x[0] (one shared line) instead of a column of
        // some other row
        float xv[ROW_UNROLL][4];
#pragma unroll
        for (int u = 0; u < ROW_UNROLL; ++u)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int k = q0 + u * step + t;
                xv[u][t] = x[(k >= s && k < e) ? c[u][t] : 0];
            }
#pragma unroll
        for (int u = 0; u < ROW_UNROLL; ++u) issue_together(xv[u][0], xv[u][1], xv[u][2], xv[u][3]);
#pragma unroll
        for (int u = 0; u < ROW_UNROLL; ++u)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int k = q0 + u * step + t;
                acc = (k >= s && k < e) ? fmaf(f[u][t], xv[u][t], acc) : acc;
            }
    }
    return acc;
}

struct BinnedArgs {
    const int *rp;
    const int *ci;
    const float *v;
    const float *x;
    float *y;
    float alpha, beta;
    int nnz;
    int last_vec;          // (nnz & ~3) - 4: start of the last full 16-byte vector
    const int *perm;
    const i32x4 *blocks;   // short-block descriptors
    int n_blocks;
    int g1_begin, n1;      // group-1 rows: perm[g1_begin .. g1_begin + n1)
    int g2_begin, n2;
    const i32x4 *chunks;   // group-3 chunks: (unused, start, end, unused)
    int n_chunks;
    float *partials;
    int seg_g2, seg_g1, seg_short;   // first workgroup of each segment; chunks come first
};

// Workgroup-level sum of one value per thread (fixed order).
__device__ __forceinline__ float workgroup_sum(float acc, float *red) {
    acc = wave_sum(acc);
    if (__lane_id() == 0) red[threadIdx.x / 64] = acc;
    __syncthreads();
    float r = 0.0f;
#pragma unroll
    for (int k = 0; k < WAVES; ++k) r += red[k];
    return r;
}

// Maps workgroup w of an nw-workgroup segment so that the workgroups that
// run on one XCD (dispatch sends workgroup i to XCD i % 8) take one
// contiguous range of blocks: consecutive rows then share that XCD's L2 when
// they gather nearby entries of x.
__device__ __forceinline__ int xcd_contiguous(int w, int nw) {
    constexpr int NX = 8;
    const int q = nw / NX, r = nw % NX;
    const int xcd = w % NX, idx = w / NX;
    return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

template <bool VEC>
__global__ __launch_bounds__(WG) void k_csr_binned(BinnedArgs a) {
    __shared__ __attribute__((aligned(16))) float stage[WAVES][SHORT_SLOTS];
    __shared__ float red[WAVES];
    const int bid = blockIdx.x;
    const int lane = __lane_id();
    const int wv = threadIdx.x / 64;

    if (bid >= a.seg_short) {
        // ---- group 0: one short block per wave ----
        const int nw = gridDim.x - a.seg_short;
        const int blk = xcd_contiguous(bid - a.seg_short, nw) * WAVES + wv;
        if (blk >= a.n_blocks) return;
        const i32x4 d = a.blocks[blk];
        const int r0 = d.x, nr = d.y, s = d.z, e = d.w;
        const int base = s & ~3;
        // Row starts for the second phase, issued before the streams so that
        // waiting for the streams (memory counters drain in issue order)
        // also covers them.
        int rs[SHORT_RMAX / 64 + 1];
#pragma unroll
        for (int j = 0; j <= SHORT_RMAX / 64; ++j) rs[j] = a.rp[r0 + min(lane + 64 * j, nr)];
        // Idle lanes (vector past e) re-read the block's first vector, which
        // keeps every load unconditional and inside the arrays.
        i32x4 c[SHORT_VPL];
        f32x4 f[SHORT_VPL];
#pragma unroll
        for (int j = 0; j < SHORT_VPL; ++j) {
            const int q = base + 4 * (lane + 64 * j);
            load4<VEC>(a.ci, a.v, q < e ? q : base, a.nnz, a.last_vec, c[j], f[j]);
        }
        float *st = stage[wv];
        if (e > s) {
            // Gathers for every lane and entry, unconditionally, so all
            // 4 * VPL gathers are in flight together; an entry outside the
            // block gathers x[0] and its product is masked after.
            float xv[SHORT_VPL][4];
#pragma unroll
            for (int j = 0; j < SHORT_VPL; ++j)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int k = base + 4 * (lane + 64 * j) + t;
                    xv[j][t] = a.x[(k >= s && k < e) ? c[j][t] : 0];
                }
#pragma unroll
            for (int j = 0; j < SHORT_VPL; ++j) issue_together(xv[j][0], xv[j][1], xv[j][2], xv[j][3]);
#pragma unroll
            for (int j = 0; j < SHORT_VPL; ++j) {
                const int q = base + 4 * (lane + 64 * j);
                f32x4 p;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int k = q + t;
                    p[t] = (k >= s && k < e) ? f[j][t] * xv[j][t] : 0.0f;
                }
                *reinterpret_cast<f32x4 *>(st + 4 * (lane + 64 * j)) = p;
            }
        }
        // The staged products are private to this wave: a wave-level barrier
        // (LDS operations of one wave complete in order) replaces a
        // workgroup barrier, so the four waves of a workgroup never wait for
        // each other.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // Each lane sums whole rows from the staged products in storage
        // order, reading 8 staged entries per step so their LDS latencies
        // overlap.  Row i's end is row i+1's start: lane l holds the start of
        // row l + 64 j; the next row's start comes from lane l + 1 (or from
        // lane 0 of the next j for lane 63).
#pragma unroll
        for (int j = 0; j < SHORT_RMAX / 64; ++j) {
            const int nxt_same = __shfl_down(rs[j], 1);
            const int nxt_wrap = __shfl(rs[j + 1], 0);
            const int end = (lane < 63 ? nxt_same : nxt_wrap) - base;
            const int i = lane + 64 * j;
            if (i < nr) {
                float acc = 0.0f;
                for (int k = rs[j] - base; k < end; k += 8) {
                    float v[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) v[u] = st[min(k + u, SHORT_SLOTS - 1)];
#pragma unroll
                    for (int u = 0; u < 8; ++u) acc += k + u < end ? v[u] : 0.0f;
                }
                store_y(a.y, r0 + i, acc, a.alpha, a.beta);
            }
        }
        return;
    }

    if (bid >= a.seg_g1) {
        // ---- group 1: one wave per row ----
        const int idx = (bid - a.seg_g1) * WAVES + wv;
        if (idx >= a.n1) return;
        const int row = a.perm[a.g1_begin + idx];
        const int s = a.rp[row], e = a.rp[row + 1];
        float acc = strided_row_sum<VEC, 1>(a.ci, a.v, a.x, s, e, a.nnz, a.last_vec, lane, 64);
        acc = wave_sum(acc);
        if (lane == 0) store_y(a.y, row, acc, a.alpha, a.beta);
        return;
    }

    if (bid >= a.seg_g2) {
        // ---- group 2: one workgroup per row ----
        const int row = a.perm[a.g2_begin + (bid - a.seg_g2)];
        const int s = a.rp[row], e = a.rp[row + 1];
        float acc = strided_row_sum<VEC, 4>(a.ci, a.v, a.x, s, e, a.nnz, a.last_vec, threadIdx.x, WG);
        acc = workgroup_sum(acc, red);
        if (threadIdx.x == 0) store_y(a.y, row, acc, a.alpha, a.beta);
        return;
    }

    // ---- group 3: one workgroup per chunk of a long row ----
    const i32x4 ch = a.chunks[bid];
    float acc = strided_row_sum<VEC, 4>(a.ci, a.v, a.x, ch.y, ch.z, a.nnz, a.last_vec, threadIdx.x, WG);
    acc = workgroup_sum(acc, red);
    if (threadIdx.x == 0) a.partials[bid] = acc;
}

// Adds the chunk partial sums of each group-3 row in chunk order.
__global__ void k_csr_long_finish(int n3, const int *__restrict__ perm3, const int *__restrict__ row_chunks,
                                  const float *__restrict__ partials, float alpha, float beta,
                                  float *__restrict__ y) {
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= n3) return;
    float acc = 0.0f;
    for (int c = row_chunks[k]; c < row_chunks[k + 1]; ++c) acc += partials[c];
    store_y(y, perm3[k], acc, alpha, beta);
}

__global__ __launch_bounds__(WG) void k_csr_scalar(int n, const int *__restrict__ rp, const int *__restrict__ ci,
                                                   const float *__restrict__ v, const float *__restrict__ x,
                                                   float alpha, float beta, float *__restrict__ y) {
    const int i = blockIdx.x * WG + threadIdx.x;
    if (i >= n) return;
    float acc = 0.0f;
    for (int k = rp[i]; k < rp[i + 1]; ++k) acc = fmaf(v[k], x[ci[k]], acc);
    store_y(y, i, acc, alpha, beta);
}

// G lanes per row, lanes strided by G, butterfly reduction inside the group.
template <int G>
__global__ __launch_bounds__(WG) void k_csr_vector(int n, const int *__restrict__ rp, const int *__restrict__ ci,
                                                   const float *__restrict__ v, const float *__restrict__ x,
                                                   float alpha, float beta, float *__restrict__ y) {
    const int gid = blockIdx.x * WG + threadIdx.x;
    const int row = gid / G;
    const int sub = gid % G;
    float acc = 0.0f;
    if (row < n) {
        const int e = rp[row + 1];
        for (int k = rp[row] + sub; k < e; k += G) acc = fmaf(v[k], x[ci[k]], acc);
    }
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, G);
    if (row < n && sub == 0) store_y(y, row, acc, alpha, beta);
}

// ---------------------------------------------------------------------------
// Workspace layout of a BINNED plan
// ---------------------------------------------------------------------------
struct Layout {
    size_t meta, perm, counts, offsets, hcounts, hoffsets, heads, blocks, long_rows, chunks, row_chunks,
        partials, total;
    int64_t max_long_rows, max_chunks;
};

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

Layout make_layout(int n, int nnz, int t2) {
    Layout L{};
    const int64_t nwg = ceil_div(std::max(n, 1), WG);
    L.max_long_rows = std::min<int64_t>(n, nnz / std::max(t2, 1));
    L.max_chunks = ceil_div(nnz, LONG_CHUNK) + L.max_long_rows;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    L.meta = take(sizeof(Meta));
    L.perm = take(sizeof(int) * (size_t)std::max(n, 1));
    L.counts = take(sizeof(int) * 4 * nwg);
    L.offsets = take(sizeof(int) * 4 * nwg);
    L.hcounts = take(sizeof(int) * nwg);
    L.hoffsets = take(sizeof(int) * nwg);
    L.heads = take(sizeof(int) * ((size_t)n + 1));
    L.blocks = take(sizeof(i32x4) * ((size_t)n + 1));
    L.long_rows = take(sizeof(int) * 2 * (size_t)(L.max_long_rows + 1));
    L.chunks = take(sizeof(i32x4) * (size_t)(L.max_chunks + 1));
    L.row_chunks = take(sizeof(int) * (size_t)(L.max_long_rows + 1));
    L.partials = take(sizeof(float) * (size_t)(L.max_chunks + 1));
    L.total = off;
    return L;
}

spmv_status check_thresholds(const int32_t *thr, int t[3]) {
    const int def[3] = {32, 512, 8192};
    for (int k = 0; k < 3; ++k) t[k] = thr ? thr[k] : def[k];
    if (!(t[0] >= 1 && t[0] < t[1] && t[1] < t[2]))
        return fail(SPMV_ERR_INVALID_VALUE, "thresholds must satisfy 1 <= t0 < t1 < t2 (got %d %d %d)", t[0],
                    t[1], t[2]);
    if (t[0] > MAX_T0) return fail(SPMV_ERR_UNSUPPORTED, "threshold t0 = %d exceeds %d", t[0], MAX_T0);
    return SPMV_OK;
}

}  // namespace
}  // namespace spmv

using namespace spmv;

struct spmv_csr_plan {
    int n_rows, n_cols, nnz;
    const int *rp, *ci;
    const float *v;
    int variant;
    int group_lanes;
    int t[3];
    bool vec_ok;
    // BINNED plan (pointers into the caller's workspace)
    int *perm = nullptr;
    const i32x4 *blocks = nullptr;
    int n_blocks = 0;
    int bin_off[5] = {0, 0, 0, 0, 0};
    const i32x4 *chunks = nullptr;
    const int *row_chunks = nullptr;
    float *partials = nullptr;
    int n_chunks = 0;
};

extern "C" spmv_status spmv_csr_row_stats(int32_t n_rows, const int32_t *row_ptr, int32_t *max_len,
                                          int64_t *sum_len, int64_t *sum_len_sq, void *stream) {
    if (n_rows < 0) return fail(SPMV_ERR_INVALID_VALUE, "n_rows < 0");
    if (!row_ptr || !max_len || !sum_len || !sum_len_sq) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    if (n_rows == 0) {
        *max_len = 0;
        *sum_len = 0;
        *sum_len_sq = 0;
        return SPMV_OK;
    }
    hipStream_t st = as_stream(stream);
    struct Out {
        unsigned long long sum, sq;
        int mx, err;
    };
    Out *d = nullptr;
    SPMV_HIP(hipMallocAsync(reinterpret_cast<void **>(&d), sizeof(Out), st));
    SPMV_HIP(hipMemsetAsync(d, 0, sizeof(Out), st));
    const int grid = (int)std::min<int64_t>(ceil_div(n_rows, WG), 4 * device_cu_count());
    k_row_stats<<<grid, WG, 0, st>>>(n_rows, row_ptr, &d->mx, &d->sum, &d->sq, &d->err);
    SPMV_LAUNCHED("k_row_stats");
    Out h{};
    SPMV_HIP(hipMemcpyAsync(&h, d, sizeof(Out), hipMemcpyDeviceToHost, st));
    SPMV_HIP(hipFreeAsync(d, st));
    SPMV_HIP(hipStreamSynchronize(st));
    if (h.err) return fail(SPMV_ERR_INVALID_MATRIX, "row_ptr decreases somewhere");
    *max_len = h.mx;
    *sum_len = (int64_t)h.sum;
    *sum_len_sq = (int64_t)h.sq;
    return SPMV_OK;
}

extern "C" spmv_status spmv_csr_plan_size(int32_t n_rows, int32_t nnz, const int32_t *thresholds, size_t *bytes) {
    if (!bytes) return fail(SPMV_ERR_INVALID_VALUE, "bytes is NULL");
    if (n_rows < 0 || nnz < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    int t[3];
    spmv_status s = check_thresholds(thresholds, t);
    if (s != SPMV_OK) return s;
    *bytes = make_layout(n_rows, nnz, t[2]).total;
    return SPMV_OK;
}

namespace {

spmv_status validate_matrix(spmv_csr_plan *h, hipStream_t st, int *d_err) {
    k_validate_rows<<<(int)ceil_div((int64_t)h->n_rows + 1, WG), WG, 0, st>>>(h->n_rows, h->nnz, h->rp, d_err);
    SPMV_LAUNCHED("k_validate_rows");
    if (h->nnz > 0) {
        const int grid = (int)std::min<int64_t>(ceil_div(h->nnz, WG), 8 * device_cu_count());
        k_validate_cols<<<grid, WG, 0, st>>>(h->nnz, h->n_cols, h->ci, d_err);
        SPMV_LAUNCHED("k_validate_cols");
    }
    int err = 0;
    SPMV_HIP(hipMemcpyAsync(&err, d_err, sizeof(int), hipMemcpyDeviceToHost, st));
    SPMV_HIP(hipStreamSynchronize(st));
    if (err & ERR_RP0) return fail(SPMV_ERR_INVALID_MATRIX, "row_ptr[0] != 0");
    if (err & ERR_RPN) return fail(SPMV_ERR_INVALID_MATRIX, "row_ptr[n_rows] != nnz");
    if (err & ERR_MONO) return fail(SPMV_ERR_INVALID_MATRIX, "row_ptr decreases somewhere");
    if (err & ERR_COL) return fail(SPMV_ERR_INVALID_MATRIX, "a column index is outside [0, n_cols)");
    return SPMV_OK;
}

spmv_status build_binned_plan(spmv_csr_plan *h, char *ws, const Layout &L, hipStream_t st) {
    const int n = h->n_rows;
    Meta *meta = reinterpret_cast<Meta *>(ws + L.meta);
    int *perm = reinterpret_cast<int *>(ws + L.perm);
    int *counts = reinterpret_cast<int *>(ws + L.counts);
    int *offsets = reinterpret_cast<int *>(ws + L.offsets);
    int *hcounts = reinterpret_cast<int *>(ws + L.hcounts);
    int *hoffsets = reinterpret_cast<int *>(ws + L.hoffsets);
    int *heads = reinterpret_cast<int *>(ws + L.heads);
    i32x4 *blocks = reinterpret_cast<i32x4 *>(ws + L.blocks);
    const int nwg = (int)ceil_div(std::max(n, 1), WG);
    const int window = SHORT_SLOTS - h->t[0] - 1;

    k_plan_count<<<nwg, WG, 0, st>>>(n, h->rp, h->t[0], h->t[1], h->t[2], counts);
    SPMV_LAUNCHED("k_plan_count");
    k_plan_scan<<<1, 1024, 0, st>>>(nwg, 4, counts, offsets, meta->bin_offsets);
    SPMV_LAUNCHED("k_plan_scan");
    k_plan_scatter<<<nwg, WG, 0, st>>>(n, h->rp, h->t[0], h->t[1], h->t[2], offsets, perm);
    SPMV_LAUNCHED("k_plan_scatter");
    k_heads_count<<<nwg, WG, 0, st>>>(meta, perm, h->rp, window, hcounts);
    SPMV_LAUNCHED("k_heads_count");
    k_plan_scan<<<1, 1024, 0, st>>>(nwg, 1, hcounts, hoffsets, meta->head_totals);
    SPMV_LAUNCHED("k_plan_scan(heads)");
    k_heads_scatter<<<nwg, WG, 0, st>>>(meta, perm, h->rp, window, hoffsets, heads);
    SPMV_LAUNCHED("k_heads_scatter");
    k_blocks_count<<<nwg, WG, 0, st>>>(meta, heads, hcounts);
    SPMV_LAUNCHED("k_blocks_count");
    k_plan_scan<<<1, 1024, 0, st>>>(nwg, 1, hcounts, hoffsets, meta->block_totals);
    SPMV_LAUNCHED("k_plan_scan(blocks)");
    k_blocks_write<<<nwg, WG, 0, st>>>(meta, heads, hoffsets, perm, h->rp, blocks);
    SPMV_LAUNCHED("k_blocks_write");
    Meta hm{};
    SPMV_HIP(hipMemcpyAsync(&hm, meta, sizeof(Meta), hipMemcpyDeviceToHost, st));
    SPMV_HIP(hipStreamSynchronize(st));
    for (int g = 0; g < 5; ++g) h->bin_off[g] = hm.bin_offsets[g];
    h->n_blocks = hm.block_totals[1];
    h->perm = perm;
    h->blocks = blocks;

    // group 3: cut rows into chunks on the host
    const int n3 = h->bin_off[4] - h->bin_off[3];
    h->n_chunks = 0;
    if (n3 > 0) {
        if (n3 > L.max_long_rows) return fail(SPMV_ERR_INVALID_MATRIX, "more long rows than nnz allows");
        int *long_rows = reinterpret_cast<int *>(ws + L.long_rows);
        k_long_rows<<<(int)ceil_div(n3, WG), WG, 0, st>>>(n3, perm + h->bin_off[3], h->rp, long_rows);
        SPMV_LAUNCHED("k_long_rows");
        std::vector<int> se(2 * (size_t)n3);
        SPMV_HIP(hipMemcpyAsync(se.data(), long_rows, sizeof(int) * se.size(), hipMemcpyDeviceToHost, st));
        SPMV_HIP(hipStreamSynchronize(st));
        std::vector<i32x4> ch;
        std::vector<int> rc(n3 + 1, 0);
        for (int k = 0; k < n3; ++k) {
            rc[k] = (int)ch.size();
            for (int64_t a = se[2 * k]; a < se[2 * k + 1]; a += LONG_CHUNK) {
                i32x4 c;
                c.x = k;
                c.y = (int)a;
                c.z = (int)std::min<int64_t>(a + LONG_CHUNK, se[2 * k + 1]);
                c.w = 0;
                ch.push_back(c);
            }
        }
        rc[n3] = (int)ch.size();
        if ((int64_t)ch.size() > L.max_chunks) return fail(SPMV_ERR_INVALID_MATRIX, "chunk count exceeds bound");
        i32x4 *d_ch = reinterpret_cast<i32x4 *>(ws + L.chunks);
        int *d_rc = reinterpret_cast<int *>(ws + L.row_chunks);
        SPMV_HIP(hipMemcpyAsync(d_ch, ch.data(), sizeof(i32x4) * ch.size(), hipMemcpyHostToDevice, st));
        SPMV_HIP(hipMemcpyAsync(d_rc, rc.data(), sizeof(int) * rc.size(), hipMemcpyHostToDevice, st));
        SPMV_HIP(hipStreamSynchronize(st));
        h->chunks = d_ch;
        h->row_chunks = d_rc;
        h->partials = reinterpret_cast<float *>(ws + L.partials);
        h->n_chunks = (int)ch.size();
    }
    return SPMV_OK;
}

}  // namespace

extern "C" spmv_status spmv_csr_create(spmv_csr_t *out, int32_t n_rows, int32_t n_cols, int32_t nnz,
                                       const int32_t *row_ptr, const int32_t *col_idx, const float *vals,
                                       int32_t variant, const int32_t *thresholds, void *workspace,
                                       size_t workspace_bytes, void *stream) {
    if (!out) return fail(SPMV_ERR_INVALID_VALUE, "handle pointer is NULL");
    *out = nullptr;
    if (n_rows < 0 || n_cols < 0 || nnz < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if (!row_ptr) return fail(SPMV_ERR_INVALID_VALUE, "row_ptr is NULL");
    if (nnz > 0 && (!col_idx || !vals)) return fail(SPMV_ERR_INVALID_VALUE, "col_idx or vals is NULL");
    if (variant < SPMV_CSR_AUTO || variant > SPMV_CSR_BINNED)
        return fail(SPMV_ERR_INVALID_VALUE, "unknown variant %d", variant);
    int t[3];
    spmv_status s = check_thresholds(thresholds, t);
    if (s != SPMV_OK) return s;
    const int var = variant == SPMV_CSR_AUTO ? SPMV_CSR_BINNED : variant;
    Layout L = make_layout(n_rows, nnz, t[2]);
    if (var == SPMV_CSR_BINNED) {
        if (!workspace) return fail(SPMV_ERR_INVALID_VALUE, "workspace is NULL");
        if (workspace_bytes < L.total)
            return fail(SPMV_ERR_INVALID_VALUE, "workspace of %zu bytes is smaller than %zu", workspace_bytes,
                        L.total);
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(SPMV_ERR_INVALID_VALUE, "workspace must be 256-byte aligned");
    }
    spmv_csr_plan *h = new spmv_csr_plan();
    h->n_rows = n_rows;
    h->n_cols = n_cols;
    h->nnz = nnz;
    h->rp = row_ptr;
    h->ci = col_idx;
    h->v = vals;
    h->variant = var;
    h->t[0] = t[0];
    h->t[1] = t[1];
    h->t[2] = t[2];
    h->vec_ok = aligned16(col_idx) && aligned16(vals) && nnz >= 4;
    h->group_lanes = 0;
    if (var == SPMV_CSR_VECTOR) {
        const double mean = n_rows ? double(nnz) / n_rows : 1.0;
        int g = 2;
        while (g < 64 && g < mean) g <<= 1;
        h->group_lanes = g;
    }
    hipStream_t st = as_stream(stream);
    // validation needs 4 bytes of device scratch: the workspace if there is
    // one, otherwise a short-lived allocation
    int *d_err = nullptr;
    bool own = false;
    if (var == SPMV_CSR_BINNED) {
        d_err = &reinterpret_cast<Meta *>(static_cast<char *>(workspace) + L.meta)->err;
    } else {
        if (hipMallocAsync(reinterpret_cast<void **>(&d_err), sizeof(int), st) != hipSuccess) {
            delete h;
            return fail(SPMV_ERR_HIP, "hipMallocAsync failed");
        }
        own = true;
    }
    spmv_status r = SPMV_OK;
    if (hipMemsetAsync(d_err, 0, sizeof(int), st) != hipSuccess) r = fail(SPMV_ERR_HIP, "hipMemsetAsync failed");
    if (r == SPMV_OK) r = validate_matrix(h, st, d_err);
    if (own) (void)hipFreeAsync(d_err, st);
    if (r == SPMV_OK && var == SPMV_CSR_BINNED) r = build_binned_plan(h, static_cast<char *>(workspace), L, st);
    if (r != SPMV_OK) {
        (void)hipStreamSynchronize(st);
        delete h;
        return r;
    }
    *out = h;
    return SPMV_OK;
}

extern "C" spmv_status spmv_csr_apply(spmv_csr_t h, float alpha, const float *x, float beta, float *y,
                                      void *stream) {
    if (!h) return fail(SPMV_ERR_INVALID_VALUE, "handle is NULL");
    if (h->n_rows == 0) return SPMV_OK;
    if (!y || (h->n_cols > 0 && !x)) return fail(SPMV_ERR_INVALID_VALUE, "x or y is NULL");
    hipStream_t st = as_stream(stream);
    const int n = h->n_rows;
    switch (h->variant) {
    case SPMV_CSR_SCALAR:
        k_csr_scalar<<<(int)ceil_div(n, WG), WG, 0, st>>>(n, h->rp, h->ci, h->v, x, alpha, beta, y);
        SPMV_LAUNCHED("k_csr_scalar");
        return SPMV_OK;
    case SPMV_CSR_VECTOR: {
        const int g = h->group_lanes;
        const int grid = (int)ceil_div((int64_t)n * g, WG);
#define SPMV_VEC_CASE(G)                                                                   \
    case G:                                                                                \
        k_csr_vector<G><<<grid, WG, 0, st>>>(n, h->rp, h->ci, h->v, x, alpha, beta, y); \
        break;
        switch (g) {
            SPMV_VEC_CASE(2)
            SPMV_VEC_CASE(4)
            SPMV_VEC_CASE(8)
            SPMV_VEC_CASE(16)
            SPMV_VEC_CASE(32)
            SPMV_VEC_CASE(64)
        default:
            return fail(SPMV_ERR_INVALID_VALUE, "bad group size %d", g);
        }
#undef SPMV_VEC_CASE
        SPMV_LAUNCHED("k_csr_vector");
        return SPMV_OK;
    }
    default:
        break;
    }
    BinnedArgs a{};
    a.rp = h->rp;
    a.ci = h->ci;
    a.v = h->v;
    a.x = x;
    a.y = y;
    a.alpha = alpha;
    a.beta = beta;
    a.nnz = h->nnz;
    a.last_vec = (h->nnz & ~3) - 4;
    a.perm = h->perm;
    a.blocks = h->blocks;
    a.n_blocks = h->n_blocks;
    a.g1_begin = h->bin_off[1];
    a.n1 = h->bin_off[2] - h->bin_off[1];
    a.g2_begin = h->bin_off[2];
    a.n2 = h->bin_off[3] - h->bin_off[2];
    a.chunks = h->chunks;
    a.n_chunks = h->n_chunks;
    a.partials = h->partials;
    a.seg_g2 = h->n_chunks;
    a.seg_g1 = a.seg_g2 + a.n2;
    a.seg_short = a.seg_g1 + (int)ceil_div(a.n1, WAVES);
    const int grid = a.seg_short + (int)ceil_div(a.n_blocks, WAVES);
    if (grid > 0) {
        if (h->vec_ok)
            k_csr_binned<true><<<grid, WG, 0, st>>>(a);
        else
            k_csr_binned<false><<<grid, WG, 0, st>>>(a);
        SPMV_LAUNCHED("k_csr_binned");
    }
    const int n3 = h->bin_off[4] - h->bin_off[3];
    if (n3 > 0) {
        k_csr_long_finish<<<(int)ceil_div(n3, WG), WG, 0, st>>>(n3, h->perm + h->bin_off[3], h->row_chunks,
                                                                h->partials, alpha, beta, y);
        SPMV_LAUNCHED("k_csr_long_finish");
    }
    return SPMV_OK;
}

extern "C" spmv_status spmv_csr_get_plan(spmv_csr_t h, int32_t *h_bin_offsets, int32_t *d_perm, void *stream) {
    if (!h) return fail(SPMV_ERR_INVALID_VALUE, "handle is NULL");
    if (h->variant != SPMV_CSR_BINNED) return fail(SPMV_ERR_INVALID_VALUE, "handle has no grouping plan");
    if (h_bin_offsets)
        for (int g = 0; g < 5; ++g) h_bin_offsets[g] = h->bin_off[g];
    if (d_perm && h->n_rows > 0) {
        hipStream_t st = as_stream(stream);
        SPMV_HIP(hipMemcpyAsync(d_perm, h->perm, sizeof(int) * (size_t)h->n_rows, hipMemcpyDeviceToDevice, st));
        SPMV_HIP(hipStreamSynchronize(st));
    }
    return SPMV_OK;
}

extern "C" spmv_status spmv_csr_info(spmv_csr_t h, int32_t *variant, int32_t *group_lanes,
                                     int32_t *n_short_blocks) {
    if (!h) return fail(SPMV_ERR_INVALID_VALUE, "handle is NULL");
    if (variant) *variant = h->variant;
    if (group_lanes) *group_lanes = h->group_lanes;
    if (n_short_blocks) *n_short_blocks = h->n_blocks;
    return SPMV_OK;
}

extern "C" spmv_status spmv_csr_destroy(spmv_csr_t h) {
    delete h;
    return SPMV_OK;
}
