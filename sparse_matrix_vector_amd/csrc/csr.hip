// CSR SpMV on gfx950: validation, the row-grouping planner and the apply
// kernels (scalar, vector, binned).
//
// The operation is the CSR product of "Why SpMV needs CUDA optimisation"
// (section 2.1 scalar kernel: one thread sums values[k] * x[col_idx[k]] over
// its row; section 4.1: a warp shares a row and reduces).  The binned variant
// follows the row grouping of "Sparse matrix multiplication acceleration"
// (section 2.1.1 table: groups by work per row with bounds 32 / 512 / 8192,
// a different thread-to-row mapping per group; section 2.2.1: the rows of a
// group are reached through a Map[] array; section 2.3: the largest rows
// fall back to global memory).  For y = A x the work of a row is its nonzero
// count.
//
// gfx950 mapping of the groups.  The planner builds a list of tasks, each
// covering at most SLOTS = 512 consecutive entries (two 16-byte vectors of
// columns and of values per lane of a wave64):
//   group 0 (short rows)   runs of consecutive short rows cut into blocks of
//                          <= 512 staged entries / 128 rows; the products
//                          are staged in LDS and each lane sums whole rows
//                          (a segmented reduction without atomics);
//   group 1 (32..511)      one task per row (a wave per row, DPP reduction);
//   rows of 2..16 chunks   one workgroup per row: its waves take every
//                          fourth 512-entry chunk and add their sums in LDS;
//   longer rows            one task per 512-entry chunk, so such a row gets
//                          as many waves as it needs; chunk sums go to a
//                          partial slot and a small second kernel adds them
//                          in chunk order.
// One launch runs the workgroup rows, then one wave per task.  Every sum has
// a fixed order, so results are bit-reproducible run to run.
#include "common.hpp"

#include <algorithm>
#include <climits>
#include <vector>

namespace spmv {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WG = 256;                 // threads per workgroup everywhere here
constexpr int WAVES = WG / 64;
#ifndef SPMV_TASK_VPL
#define SPMV_TASK_VPL 2
#endif
#ifndef SPMV_SHORT_RMAX
#define SPMV_SHORT_RMAX (64 * SPMV_TASK_VPL)
#endif
constexpr int TASK_VPL = SPMV_TASK_VPL;   // 16-byte vectors per lane and stream in a task
constexpr int SLOTS = 64 * 4 * TASK_VPL;   // entries a task stages: 512
constexpr int SHORT_RMAX = SPMV_SHORT_RMAX;   // rows per short block (2 per lane)
constexpr int MAX_T0 = 256;             // largest supported bound of group 0
#ifndef SPMV_TASK_WAVES
#define SPMV_TASK_WAVES 4
#endif
constexpr int TWAVES = SPMV_TASK_WAVES;  // waves per workgroup of the task kernel
constexpr int TWG = 64 * TWAVES;
constexpr int X_TILE_MAX = 6144;        // largest x window staged in LDS per block workgroup (floats)
constexpr int X_SEG = 32;               // floats per segment of an x window (one 128-byte line)
constexpr int X_SEG_WORDS = X_TILE_MAX / X_SEG / 32;
static_assert(X_TILE_MAX % (32 * X_SEG) == 0, "whole mask words");

// Column window of one block workgroup: the smallest and largest column of
// its entries and, over the window from the X_SEG-float boundary below the
// smallest column, one bit per X_SEG-float segment holding a column of its
// entries (all ones when the window is wider than X_TILE_MAX).
struct __attribute__((aligned(16))) XWindow {
    int lo, hi;
    unsigned seg[X_SEG_WORDS];
};

// Error bits raised by the validation kernels.
constexpr int ERR_RP0 = 1, ERR_RPN = 2, ERR_MONO = 4, ERR_COL = 8;

// Device-side plan header (int32 words).
struct Meta {
    int bin_offsets[5];
    int head_totals[2];   // {0, number of runs of short rows}
    int block_totals[2];  // {0, number of short blocks}
    int row_task_totals[2];   // {0, number of one-wave tasks of rows in groups 1-3}
    int wgrow_totals[2];      // {0, number of rows in groups 1-3 applied by one workgroup each}
    int err;
    int max_window;       // largest column span (from a 16-byte boundary) of a block workgroup
    int max_short;        // longest row of group 0
};

__device__ __forceinline__ int row_group(int len, int t0, int t1, int t2) {
    return len < t0 ? 0 : (len < t1 ? 1 : (len < t2 ? 2 : 3));
}

// y[row] = alpha * acc + beta * y[row], where y's element for `row` is
// ymap[row] when an output row map is given (the scatter form), else row.
__device__ __forceinline__ void store_y(float *y, const int *ymap, int row, float acc, float alpha, float beta) {
    if (ymap) row = ymap[row];
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
                                                   int t2, int *__restrict__ counts, int *__restrict__ max_short) {
    __shared__ int wc[WAVES][4];
    const int i = blockIdx.x * WG + threadIdx.x;
    const int len = i < n ? rp[i + 1] - rp[i] : 0;
    const int g = i < n ? row_group(len, t0, t1, t2) : -1;
    const int w = threadIdx.x / 64;
    int ms = g == 0 ? len : 0;
    for (int off = 32; off > 0; off >>= 1) ms = max(ms, __shfl_xor(ms, off));
    if (__lane_id() == 0 && ms > 0) atomicMax(max_short, ms);
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
// first entries lie in one window, so it spans at most window + L + 2
// entries from a 16-byte boundary, L the longest short row; the window is
// SLOTS - L - 2 (run_window), so a run always fits one task.  Sizing it by
// the matrix's L rather than the group bound keeps runs long when short rows
// are much shorter than the bound.  Runs longer than SHORT_RMAX rows are cut
// into pieces of SHORT_RMAX rows afterwards (k_blocks_write).
__device__ __forceinline__ int run_window(const Meta *__restrict__ meta) { return SLOTS - meta->max_short - 2; }

__device__ __forceinline__ bool short_head(int p, const int *__restrict__ perm, const int *__restrict__ rp,
                                           int window) {
    if (p == 0) return true;
    const int r = perm[p];
    if (perm[p - 1] != r - 1) return true;
    return rp[r] / window != rp[r - 1] / window;
}

__global__ __launch_bounds__(WG) void k_heads_count(const Meta *__restrict__ meta, const int *__restrict__ perm,
                                                    const int *__restrict__ rp, int *__restrict__ counts) {
    __shared__ int wc[WAVES];
    const int n0 = meta->bin_offsets[1];
    const int window = run_window(meta);
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
                                                      const int *__restrict__ rp, const int *__restrict__ offsets,
                                                      int *__restrict__ head_pos) {
    __shared__ int wc[WAVES];
    const int n0 = meta->bin_offsets[1];
    const int window = run_window(meta);
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

// A short block as a task: rows r0 .. r0 + nr - 1, entries [s, e).
__global__ __launch_bounds__(WG) void k_blocks_write(const Meta *__restrict__ meta,
                                                     const int *__restrict__ head_pos,
                                                     const int *__restrict__ offsets,
                                                     const int *__restrict__ perm, const int *__restrict__ rp,
                                                     i32x4 *__restrict__ tasks) {
    const int nh = meta->head_totals[1];
    const int n0 = meta->bin_offsets[1];
    const int k = blockIdx.x * WG + threadIdx.x;
    int total;
    int at = meta->wgrow_totals[1] + meta->row_task_totals[1] + offsets[blockIdx.x] +
             workgroup_exclusive(run_blocks(k, nh, n0, head_pos), &total);
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
        tasks[at++] = d;
    }
}

// Rows of groups 1-3 are cut into SLOTS-entry chunks, counted from the row's
// 16-byte-aligned start: chunk c covers [max(s, A + c SLOTS),
// min(e, A + (c + 1) SLOTS)) with A = s & ~3, so every chunk fits the
// staging area.  A row with one chunk is a one-wave task with nr = 1.  A row
// of 2 .. WG_ROW_MAX_CHUNKS chunks is one workgroup task {row, chunks, s, e}
// (its waves take every TWAVES-th chunk and add their sums in LDS, so no
// second kernel is needed).  Chunk c of a longer row is a one-wave task with
// nr = -(c + 1) whose sum goes to a partial slot.
__device__ __forceinline__ int row_chunk_count(int s, int e) { return (e - (s & ~3) + SLOTS - 1) / SLOTS; }

constexpr int WG_ROW_MAX_CHUNKS = 4 * TWAVES;   // at most 4 chunks per wave

__device__ __forceinline__ bool is_wg_row(int nch) { return nch >= 2 && nch <= WG_ROW_MAX_CHUNKS; }

__global__ __launch_bounds__(WG) void k_rowtasks_count(const Meta *__restrict__ meta, int n,
                                                       const int *__restrict__ perm, const int *__restrict__ rp,
                                                       int *__restrict__ counts, int *__restrict__ wcounts) {
    const int p = meta->bin_offsets[1] + blockIdx.x * WG + threadIdx.x;
    int nch = 0;
    if (p < n) {
        const int r = perm[p];
        nch = row_chunk_count(rp[r], rp[r + 1]);
    }
    const bool wgr = is_wg_row(nch);
    int total, wtotal;
    workgroup_exclusive(wgr ? 0 : nch, &total);
    __syncthreads();   // the scan's LDS is reused
    workgroup_exclusive(wgr ? 1 : 0, &wtotal);
    if (threadIdx.x == 0) {
        counts[blockIdx.x] = total;
        wcounts[blockIdx.x] = wtotal;
    }
}

// Task order: the workgroup rows, then the one-wave tasks of rows in groups
// 1-3 (both in perm order), then the short-row blocks.
__global__ __launch_bounds__(WG) void k_rowtasks_write(const Meta *__restrict__ meta, int n,
                                                       const int *__restrict__ perm, const int *__restrict__ rp,
                                                       const int *__restrict__ offsets,
                                                       const int *__restrict__ woffsets, i32x4 *__restrict__ tasks) {
    const int p = meta->bin_offsets[1] + blockIdx.x * WG + threadIdx.x;
    int r = 0, s = 0, e = 0, nch = 0;
    if (p < n) {
        r = perm[p];
        s = rp[r];
        e = rp[r + 1];
        nch = row_chunk_count(s, e);
    }
    const bool wgr = is_wg_row(nch);
    int total, wtotal;
    const int first = meta->wgrow_totals[1] + offsets[blockIdx.x] + workgroup_exclusive(wgr ? 0 : nch, &total);
    __syncthreads();   // the scan's LDS is reused
    const int wfirst = woffsets[blockIdx.x] + workgroup_exclusive(wgr ? 1 : 0, &wtotal);
    if (wgr) {
        tasks[wfirst] = i32x4{r, nch, s, e};
        nch = 0;
    }
    const int A = s & ~3;
    for (int c = 0; c < nch; ++c) {
        i32x4 d;
        d.x = r;
        d.y = nch == 1 ? 1 : -(c + 1);
        d.z = max(s, A + c * SLOTS);
        d.w = min(e, A + (c + 1) * SLOTS);
        tasks[first + c] = d;
    }
}

// Column window of each block workgroup (blocks TWAVES q .. TWAVES q + TWAVES - 1
// of the short-row blocks, the blocks one workgroup of the task kernel
// applies): its smallest and largest column, and which X_SEG-float segments
// of the window its entries touch.  max_window gets the largest span counted
// from the X_SEG-float boundary below the smallest column.
__global__ __launch_bounds__(TWG) void k_block_spans(Meta *__restrict__ meta, const i32x4 *__restrict__ tasks,
                                                     const int *__restrict__ ci, XWindow *__restrict__ spans) {
    __shared__ int lo[TWAVES], hi[TWAVES];
    __shared__ unsigned segs[X_SEG_WORDS];
    const int nb = meta->block_totals[1];
    const int first = meta->wgrow_totals[1] + meta->row_task_totals[1];
    const int lane = __lane_id(), wv = threadIdx.x / 64;
    const int b = blockIdx.x * TWAVES + wv;
    const i32x4 d = b < nb ? tasks[first + b] : i32x4{0, 0, 0, 0};
    int mn = INT_MAX, mx = -1;
    for (int k = d.z + lane; k < d.w; k += 64) {
        const int c = ci[k];
        mn = min(mn, c);
        mx = max(mx, c);
    }
    for (int off = 32; off > 0; off >>= 1) {
        mn = min(mn, __shfl_xor(mn, off));
        mx = max(mx, __shfl_xor(mx, off));
    }
    if (lane == 0) {
        lo[wv] = mn;
        hi[wv] = mx;
    }
    if ((int)threadIdx.x < X_SEG_WORDS) segs[threadIdx.x] = 0u;
    __syncthreads();
    for (int w = 0; w < TWAVES; ++w) {
        mn = min(mn, lo[w]);
        mx = max(mx, hi[w]);
    }
    const int tb = mn & ~(X_SEG - 1);
    const bool fits = mx >= 0 && mx + 1 - tb <= X_TILE_MAX;
    if (fits)
        for (int k = d.z + lane; k < d.w; k += 64) {
            const int sg = (ci[k] - tb) / X_SEG;
            atomicOr(&segs[sg >> 5], 1u << (sg & 31));
        }
    __syncthreads();
    if (threadIdx.x == 0) {
        XWindow w;
        w.lo = mn;
        w.hi = mx;
        for (int i = 0; i < X_SEG_WORDS; ++i) w.seg[i] = fits ? segs[i] : ~0u;
        spans[blockIdx.x] = w;
        if (mx >= 0) atomicMax(&meta->max_window, mx + 1 - tb);
    }
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
// callers mask entries outside their range.  Keeping the common path free
// of divergent branches matters: a divergent path that writes the same
// registers would make the compiler wait for the 16-byte loads before the
// next ones are issued.
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

// Maps workgroup w of an nw-workgroup grid so that the workgroups that run
// on one XCD (dispatch sends workgroup i to XCD i % 8) take one contiguous
// range: consecutive rows then share that XCD's L2 when they gather nearby
// entries of x.
__device__ __forceinline__ int xcd_contiguous(int w, int nw) {
    constexpr int NX = 8;
    const int q = nw / NX, r = nw % NX;
    const int xcd = w % NX, idx = w / NX;
    return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

// Scalars of the task kernel; its arrays are separate __restrict__ kernel
// parameters, which lets the compiler read task descriptors with scalar
// loads even after the kernel has stored to y (a struct member pointer
// could alias y, and the scalar cache does not see vector stores).
struct TaskArgs {
    float alpha, beta;
    int nnz;
    int last_vec;          // (nnz & ~3) - 4: start of the last full 16-byte vector
    int n_row_tasks;       // tasks [0, n_row_tasks): rows of groups 1-3; then n_blocks short blocks
    int n_wg_rows;         // the first n_wg_rows of them: one workgroup each
    int n_blocks;
    int n_rows, n_cols;
};

struct Arrays {
    const int *__restrict__ rp;
    const int *__restrict__ ci;
    const float *__restrict__ v;
    const float *__restrict__ x;
};

// Stage-1 data of one task: the streams of its (at most SLOTS) entries.
struct Staged {
    i32x4 c[TASK_VPL];
    f32x4 f[TASK_VPL];
};

template <bool VEC>
__device__ __forceinline__ void stage_streams(const TaskArgs &a, const Arrays &m, i32x4 d, int lane, Staged &g) {
    const int base = d.z & ~3;
    // Idle lanes (vector past e) re-read the task's first vector, which
    // keeps every load unconditional and inside the arrays.
#pragma unroll
    for (int j = 0; j < TASK_VPL; ++j) {
        const int q = base + 4 * (lane + 64 * j);
        load4<VEC>(m.ci, m.v, q < d.w ? q : base, a.nnz, a.last_vec, g.c[j], g.f[j]);
    }
}

// x[c] (and rp[i]) through a buffer resource when the array is below 4 GiB:
// a 32-bit byte offset per lane instead of 64-bit address arithmetic.
constexpr int BUF_DWORD3 = 0x00020000;   // gfx9-family buffer resource word 3 (raw 32-bit data)
// A buffer offset that is out of range for every x below 2 GiB (a load there
// returns zeros and touches no memory) and inside any larger x.
constexpr int X_OOB = 0x7FFFFFF0;

template <bool BUF>
struct Gather {
    const float *__restrict__ p;
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ Gather(const float *ptr, int n) : p(ptr) {
        if (BUF) r = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(ptr), 0, (int)(4u * (unsigned)n), BUF_DWORD3);
    }
    __device__ __forceinline__ float operator[](int i) const {
        // the builtin returns the loaded bits as an unsigned integer
        return BUF ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, 0)) : p[i];
    }
};

// Cache-policy operand of a buffer load: non-temporal, for data a pass reads
// once (the row starts of short blocks, like the column and value streams).
constexpr int CPOL_NT = 2;

template <bool BUF>
struct GatherI {
    const int *__restrict__ p;
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ GatherI(const int *ptr, int n) : p(ptr) {
        if (BUF) r = __builtin_amdgcn_make_buffer_rsrc(const_cast<int *>(ptr), 0, (int)(4u * (unsigned)n), BUF_DWORD3);
    }
    __device__ __forceinline__ int operator[](int i) const {
        return BUF ? __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, CPOL_NT))
                   : __builtin_nontemporal_load(p + i);
    }
};

// Block of short rows r0 .. r0 + nr - 1 (nr = d.y > 1), given its streams,
// row starts and gathered x: products are staged in the wave's LDS area and
// lane l sums rows l + 64 j in storage order (or, for at most 32 rows, a
// group of lanes sums each row).  Entries of the staged vectors
// outside the block (neighbouring rows, re-read vectors) are multiplied too
// but never read back.
__device__ __forceinline__ void finish_block(const TaskArgs &a, i32x4 d, const Staged &cur,
                                             const int (&rs)[SHORT_RMAX / 64], const float (&xv)[TASK_VPL][4],
                                             float *st, int lane, float *__restrict__ y, const int *__restrict__ ymap) {
    const int nr = d.y, base = d.z & ~3;
#pragma unroll
    for (int j = 0; j < TASK_VPL; ++j) {
        f32x4 p;
#pragma unroll
        for (int q = 0; q < 4; ++q) p[q] = cur.f[j][q] * xv[j][q];
        *reinterpret_cast<f32x4 *>(st + 4 * (lane + 64 * j)) = p;
    }
    // The staged products are private to this wave: a wave-level barrier
    // (LDS operations of one wave complete in order) is enough.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (nr <= 32) {   // uniform
        // Few, longer rows (e.g. ~80 entries of an assembled stiffness row):
        // G = 64 / 2^ceil(log2 nr) lanes per row, lane j of a row's group
        // summing entries j, j + G, ... four at a time, then a butterfly
        // within the group (fixed order, so results stay reproducible).
        // One lane per row would leave most of the wave idle through a
        // long serial sum.
        const int G = 64 >> (32 - __builtin_clz((unsigned)(nr - 1)));
        const int i_row = lane / G, sub = lane % G;
        const int start = __shfl(rs[0], i_row < nr ? i_row : 0) - base;
        const int nxt = __shfl(rs[0], i_row + 1 < nr ? i_row + 1 : 0);
        const int end = (i_row + 1 < nr ? nxt : d.w) - base;
        float acc = 0.0f;
        if (i_row < nr) {
            for (int k = start + sub; k < end; k += 4 * G) {
                float vv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) vv[u] = st[min(k + u * G, end - 1)];   // stays inside the row
#pragma unroll
                for (int u = 0; u < 4; ++u) acc += k + u * G < end ? vv[u] : 0.0f;
            }
        }
        for (int off = G >> 1; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        if (i_row < nr && sub == 0) store_y(y, ymap, d.x + i_row, acc, a.alpha, a.beta);
        return;
    }
    // Lane l sums row l + 64 j, reading 8 staged entries per step so their
    // LDS latencies overlap.  Row i's end is row i+1's start: from lane l + 1,
    // or for lane 63 from lane 0 of the next j, or the block's end entry.
#pragma unroll
    for (int j = 0; j < SHORT_RMAX / 64; ++j) {
        const int nxt_same = __shfl_down(rs[j], 1);
        const int nxt_wrap = j + 1 < SHORT_RMAX / 64 ? __shfl(rs[j + 1 < SHORT_RMAX / 64 ? j + 1 : j], 0) : d.w;
        const int end = (lane < 63 ? nxt_same : nxt_wrap) - base;
        const int i_row = lane + 64 * j;
        if (i_row < nr) {
            float acc = 0.0f;
            for (int k = rs[j] - base; k < end; k += 8) {
                float vv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) vv[u] = st[k + u];
                const int left = end - k;
#pragma unroll
                for (int u = 0; u < 8; ++u) acc += u < left ? vv[u] : 0.0f;
            }
            store_y(y, ymap, d.x + i_row, acc, a.alpha, a.beta);
        }
    }
}

// One row (d.y == 1) or one chunk of a long row (d.y < 0): masked lane sums,
// DPP wave sum, then y or the task's partial slot.
__device__ __forceinline__ void finish_row(const TaskArgs &a, i32x4 d, int t, const Staged &cur,
                                           const float (&xv)[TASK_VPL][4], int lane, float *__restrict__ y,
                                           const int *__restrict__ ymap, float *__restrict__ partials) {
    const int s = d.z, e = d.w, base = s & ~3;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < TASK_VPL; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int k = base + 4 * (lane + 64 * j) + q;
            acc += (k >= s && k < e) ? cur.f[j][q] * xv[j][q] : 0.0f;
        }
    acc = wave_sum(acc);
    if (d.y == 1) {
        if (lane == 0) store_y(y, ymap, d.x, acc, a.alpha, a.beta);
    } else {
        if (lane == 0) partials[t] = acc;
    }
}

// The grid is [workgroup rows][row tasks][short blocks].  A workgroup row
// (a row of 2 .. WG_ROW_MAX_CHUNKS chunks) takes a whole workgroup: its
// waves walk every TWAVES-th chunk and their sums meet in LDS, so such rows
// need no second kernel and start first.  Otherwise one wave per task: row
// tasks in natural order, blocks through the XCD-contiguous map
// (neighbouring blocks on one XCD share its L2 for nearby x entries; for the
// scattered gathers of long rows the plain order measured faster).  The
// wave loads the task's streams, issues all gathers at once, then reduces by
// task kind:
//   nr > 1   a block of short rows (finish_block): every staged entry is
//            gathered and multiplied without masks, since every staged
//            column is a valid column of A;
//   nr == 1  one row: masked lane sums (entries outside [s, e) gather x[0]),
//            then a DPP wave reduction;
//   nr < 0   chunk c = -nr - 1 of a long row: as one row, but the wave sum
//            goes to the task's partial slot; k_csr_chunks_finish adds a
//            row's partials in chunk order afterwards.  (Combining here
//            would need device-scope release/acquire fences, which write
//            back and invalidate the whole L2 of an XCD on this part.)
// BUF: x and row_ptr are below 4 GiB and gathered with buffer loads.
// XTR > 0: the TWAVES blocks of a block workgroup span at most
// XTR * 4 * TWG columns (spans[q], from the plan).  The workgroup stages the
// segments of that window of x that its entries touch into LDS with 16-byte
// loads, issued after each wave's own stream loads, and the gathers read
// LDS: a 16-byte load moves four x values through the texture addresser
// where a gather moves one.  The section "x caching in shared memory" of
// "Why SpMV needs CUDA optimisation" (section 3.1) suggests this; here it
// is used whenever the plan finds narrow windows.
template <bool VEC, bool BUF, int XTR>
__global__ __launch_bounds__(TWG) void k_csr_tasks(TaskArgs a, const i32x4 *__restrict__ tasks,
                                                  const int *__restrict__ rp, const int *__restrict__ ci,
                                                  const float *__restrict__ v, const float *__restrict__ x,
                                                  float *__restrict__ y, const int *__restrict__ ymap,
                                                  float *__restrict__ partials, const XWindow *__restrict__ spans) {
    constexpr bool XT = XTR > 0;
    // 8 slack entries: a row's 8-entry reads never need clamping
    __shared__ __attribute__((aligned(16))) float stage[TWAVES][SLOTS + 8];
    extern __shared__ __attribute__((aligned(16))) float xtile[];
    const Arrays m{rp, ci, v, x};
    const Gather<BUF> xg(x, a.n_cols);
    const GatherI<BUF> rg(rp, a.n_rows + 1);
    const int lane = __lane_id();
    // wave-uniform, stated so that task indices and descriptors are scalar
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int nwgr = a.n_wg_rows;
    const int seg_rows = (a.n_row_tasks - nwgr + TWAVES - 1) / TWAVES;
    float *st = stage[wv];
    Staged cur;
    float xv[TASK_VPL][4];

    if ((int)blockIdx.x < nwgr) {
        // ---- a row of 2 .. WG_ROW_MAX_CHUNKS chunks: wave wv takes chunks
        // wv, wv + TWAVES, ... in order; the wave sums are added in wave
        // order ----
        const i32x4 d = tasks[blockIdx.x];
        const int s = d.z, e = d.w, A = s & ~3;
        float acc = 0.0f;
        for (int c = wv; c < d.y; c += TWAVES) {
            const int cs = max(s, A + c * SLOTS), ce = min(e, A + (c + 1) * SLOTS), cb = cs & ~3;
            stage_streams<VEC>(a, m, i32x4{d.x, 1, cs, ce}, lane, cur);
#pragma unroll
            for (int j = 0; j < TASK_VPL; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int k = cb + 4 * (lane + 64 * j) + q;
                    xv[j][q] = xg[(k >= cs && k < ce) ? cur.c[j][q] : 0];
                }
#pragma unroll
            for (int j = 0; j < TASK_VPL; ++j) issue_together(xv[j][0], xv[j][1], xv[j][2], xv[j][3]);
#pragma unroll
            for (int j = 0; j < TASK_VPL; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int k = cb + 4 * (lane + 64 * j) + q;
                    acc += (k >= cs && k < ce) ? cur.f[j][q] * xv[j][q] : 0.0f;
                }
        }
        acc = wave_sum(acc);
        if (lane == 0) st[0] = acc;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        if (wv == 0 && lane == 0) {
            float sum = stage[0][0];
            for (int w = 1; w < TWAVES; ++w) sum += stage[w][0];
            store_y(y, ymap, d.x, sum, a.alpha, a.beta);
        }
        return;
    }
    const int bx = (int)blockIdx.x - nwgr;
    if (bx < seg_rows) {
        // ---- one-wave tasks of rows in groups 1-3 ----
        const int t = nwgr + bx * TWAVES + wv;
        if (t >= a.n_row_tasks) return;
        const i32x4 d = tasks[t];
        stage_streams<VEC>(a, m, d, lane, cur);
        const int s = d.z, e = d.w, base = s & ~3;
#pragma unroll
        for (int j = 0; j < TASK_VPL; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = base + 4 * (lane + 64 * j) + q;
                xv[j][q] = xg[(k >= s && k < e) ? cur.c[j][q] : 0];
            }
#pragma unroll
        for (int j = 0; j < TASK_VPL; ++j) issue_together(xv[j][0], xv[j][1], xv[j][2], xv[j][3]);
        finish_row(a, d, t, cur, xv, lane, y, ymap, partials);
        return;
    }

    // ---- short-row blocks ----
    const int qw = xcd_contiguous(bx - seg_rows, (int)gridDim.x - nwgr - seg_rows);
    const int wb = qw * TWAVES + wv;
    const bool have = wb < a.n_blocks;
    if (!XT && !have) return;
    const int t = a.n_row_tasks + wb;
    // the workgroup's column window (XT), read together with the descriptor
    const XWindow sp = XT ? spans[qw] : XWindow{0, -1, {}};
    // a wave without a block (XT only) still helps stage the tile: it loads
    // a dummy task (the first entries of the arrays)
    const i32x4 d = have ? tasks[t] : i32x4{0, 0, 0, 0};
    // the window of x (XT) from the X_SEG-float boundary below the
    // workgroup's smallest column (a workgroup without entries stages
    // x[0..3]); its loads depend only on the plan, so they are issued
    // before the row starts and streams: the in-order load counter then
    // lets the LDS stores and the barrier below complete while the streams
    // are still in flight.
    // XTR rounds of 16-byte loads: enough for the widest window of the
    // matrix; threads past a window's end load and store its last vector
    // again.  Only segments holding a column of the workgroup's entries are
    // read (a banded matrix touches a few bands of its window): the other
    // lanes get a buffer offset past the end of x, which the hardware
    // answers with zeros and no memory access, so the loads need no branch.
    // Round u of wave wv covers vectors 64 wv + u TWG .. + 63, i.e. the 8
    // segments from 8 wv + 32 u TWAVES / 4: one mask word for the wave,
    // picked without per-lane selects, and one bit per 8 lanes.  Threads
    // past the window's end re-load its last vector, which holds the
    // largest column and must be read.
    static_assert(X_SEG == 32 && TWAVES % 4 == 0, "segment word layout");
    __builtin_assume(wv >= 0 && wv < TWAVES);
    const int tb = XT && sp.hi >= 0 ? (sp.lo & ~(X_SEG - 1)) : 0;
    const int nvec = XT && sp.hi >= 0 ? (sp.hi + 4 - tb) >> 2 : 1;
    f32x4 tv[XTR > 0 ? XTR : 1];
    if (XT) {
#pragma unroll
        for (int u = 0; u < XTR; ++u) {
            const int iu = (int)threadIdx.x + u * TWG;
            const int i = min(iu, nvec - 1);
            const unsigned word = sp.seg[u * (TWAVES / 4) + (wv >> 2)];
            const bool need = iu >= nvec || ((word >> ((8 * wv + lane / 8) & 31)) & 1u);
            const int off = need ? (int)(4u * (unsigned)(tb + 4 * i)) : X_OOB;
            tv[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xg.r, off, 0, 0));
        }
    }
    // start of each row (lane l: rows l + 64 j; entry nr is the block's end),
    // loaded together with the streams, ahead of the gathers
    int rs[SHORT_RMAX / 64];
    const int nr = max(d.y, 0);
#pragma unroll
    for (int j = 0; j < SHORT_RMAX / 64; ++j) rs[j] = rg[d.x + min(lane + 64 * j, nr)];
    stage_streams<VEC>(a, m, d, lane, cur);
    __builtin_amdgcn_sched_barrier(0);
    if (XT) {
#pragma unroll
        for (int u = 0; u < XTR; ++u)
            *reinterpret_cast<f32x4 *>(xtile + 4 * min((int)threadIdx.x + u * TWG, nvec - 1)) = tv[u];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        if (!have) return;
        // entries of this block lie in the window; others (never used) are
        // clamped into it
        const int hi = 4 * nvec - 1;
        if (d.y > 1) {
#pragma unroll
            for (int j = 0; j < TASK_VPL; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) xv[j][q] = xtile[min(max(cur.c[j][q] - tb, 0), hi)];
            finish_block(a, d, cur, rs, xv, st, lane, y, ymap);
        } else {
            const int s = d.z, e = d.w, base = s & ~3;
#pragma unroll
            for (int j = 0; j < TASK_VPL; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int k = base + 4 * (lane + 64 * j) + q;
                    xv[j][q] = xtile[(k >= s && k < e) ? min(max(cur.c[j][q] - tb, 0), hi) : 0];
                }
            finish_row(a, d, t, cur, xv, lane, y, ymap, partials);
        }
        return;
    }
    if (d.y > 1) {
#pragma unroll
        for (int j = 0; j < TASK_VPL; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) xv[j][q] = xg[cur.c[j][q]];
#pragma unroll
        for (int j = 0; j < TASK_VPL; ++j) issue_together(xv[j][0], xv[j][1], xv[j][2], xv[j][3]);
        finish_block(a, d, cur, rs, xv, st, lane, y, ymap);
    } else {
        const int s = d.z, e = d.w, base = s & ~3;
#pragma unroll
        for (int j = 0; j < TASK_VPL; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = base + 4 * (lane + 64 * j) + q;
                xv[j][q] = xg[(k >= s && k < e) ? cur.c[j][q] : 0];
            }
#pragma unroll
        for (int j = 0; j < TASK_VPL; ++j) issue_together(xv[j][0], xv[j][1], xv[j][2], xv[j][3]);
        finish_row(a, d, t, cur, xv, lane, y, ymap, partials);
    }
}

// One thread per row task; the thread of a long row's first chunk adds the
// row's chunk partials in chunk order and writes y.
__global__ void k_csr_chunks_finish(int n_row_tasks, const i32x4 *__restrict__ tasks, const int *__restrict__ rp,
                                    const float *__restrict__ partials, float alpha, float beta,
                                    float *__restrict__ y, const int *__restrict__ ymap) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_row_tasks) return;
    const i32x4 d = tasks[t];
    if (d.y != -1) return;
    const int nch = row_chunk_count(rp[d.x], rp[d.x + 1]);
    float acc = 0.0f;
    for (int c = 0; c < nch; ++c) acc += partials[t + c];
    store_y(y, ymap, d.x, acc, alpha, beta);
}

// y = beta * y (no read when beta == 0): the whole product when A has no
// nonzeros.  The task kernel is never launched then, because its masked
// gathers read x[0], which exists only when n_cols >= 1 (guaranteed by the
// column validation once nnz > 0).
__global__ void k_csr_scale(int n, float beta, float *__restrict__ y, const int *__restrict__ ymap) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int r = ymap ? ymap[i] : i;
    y[r] = beta != 0.0f ? beta * y[r] : 0.0f;
}

__global__ __launch_bounds__(WG) void k_csr_scalar(int n, const int *__restrict__ rp, const int *__restrict__ ci,
                                                   const float *__restrict__ v, const float *__restrict__ x,
                                                   float alpha, float beta, float *__restrict__ y,
                                                   const int *__restrict__ ymap) {
    const int i = blockIdx.x * WG + threadIdx.x;
    if (i >= n) return;
    float acc = 0.0f;
    for (int k = rp[i]; k < rp[i + 1]; ++k) acc = fmaf(v[k], x[ci[k]], acc);
    store_y(y, ymap, i, acc, alpha, beta);
}

// G lanes per row, lanes strided by G, butterfly reduction inside the group.
template <int G>
__global__ __launch_bounds__(WG) void k_csr_vector(int n, const int *__restrict__ rp, const int *__restrict__ ci,
                                                   const float *__restrict__ v, const float *__restrict__ x,
                                                   float alpha, float beta, float *__restrict__ y,
                                                   const int *__restrict__ ymap) {
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
    if (row < n && sub == 0) store_y(y, ymap, row, acc, alpha, beta);
}

// ---------------------------------------------------------------------------
// Workspace layout of a BINNED plan
// ---------------------------------------------------------------------------
struct Layout {
    size_t meta, perm, counts, offsets, hcounts, hoffsets, heads, tasks, partials, spans, total;
    int64_t max_row_tasks, max_tasks;
};

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Bounds: a row of groups 1-3 (>= t0 entries) has at most len / SLOTS + 2
// chunks, and there are at most min(n, nnz / t0) such rows; blocks are at
// most one per short row.
Layout make_layout(int n, int nnz, int t0) {
    Layout L{};
    const int64_t nwg = ceil_div(std::max(n, 1), WG);
    L.max_row_tasks = (int64_t)nnz / SLOTS + 2 * std::min<int64_t>(n, nnz / std::max(t0, 1)) + 1;
    L.max_tasks = L.max_row_tasks + n + 1;
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
    L.tasks = take(sizeof(i32x4) * (size_t)L.max_tasks);
    L.partials = take(sizeof(float) * (size_t)L.max_row_tasks);
    L.spans = take(sizeof(XWindow) * (size_t)(ceil_div((int64_t)n + 1, TWAVES) + 1));
    L.total = off;
    return L;
}

spmv_status check_thresholds(const int32_t *thr, int t[3]) {
    // The first bound is 128, not the page's 32: a task stages 512 entries,
    // so rows up to 127 entries still pack several to a wave, and a wave per
    // 32..127-entry row left most of its lanes idle (power-law: 38.4 ->
    // 36.3 us).  The other bounds are the page's.
    const int def[3] = {128, 512, 8192};
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
    int bin_off[5] = {0, 0, 0, 0, 0};
    const i32x4 *tasks = nullptr;
    int n_row_tasks = 0;   // tasks of rows in groups 1-3 (workgroup rows included)
    int n_wg_rows = 0;     // rows applied by one workgroup each (the first tasks)
    int n_blocks = 0;
    float *partials = nullptr;
    bool has_chunked_rows = false;   // some row is split into several tasks
    int grid = 0;          // workgroups of the task kernel
    const XWindow *spans = nullptr;  // column window of each block workgroup
    int x_tile = 0;        // floats of x staged in LDS per block workgroup (0: gathers from memory)
};

extern "C" spmv_status spmv_csr_row_stats(int32_t n_rows, const int32_t *row_ptr, int32_t *max_len,
                                          int64_t *sum_len, int64_t *sum_len_sq, void *scratch,
                                          size_t scratch_bytes, void *stream) {
    if (n_rows < 0) return fail(SPMV_ERR_INVALID_VALUE, "n_rows < 0");
    if (!row_ptr || !max_len || !sum_len || !sum_len_sq) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    spmv_status cs = check_scratch(scratch, scratch_bytes, n_rows);
    if (cs != SPMV_OK) return cs;
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
    Out *d = reinterpret_cast<Out *>(static_cast<char *>(scratch) + SCRATCH_ROW_STATS);
    SPMV_HIP(hipMemsetAsync(d, 0, sizeof(Out), st));
    const int grid = (int)std::min<int64_t>(ceil_div(n_rows, WG), 4 * device_cu_count());
    k_row_stats<<<grid, WG, 0, st>>>(n_rows, row_ptr, &d->mx, &d->sum, &d->sq, &d->err);
    SPMV_LAUNCHED("k_row_stats");
    Out h{};
    SPMV_HIP(hipMemcpyAsync(&h, d, sizeof(Out), hipMemcpyDeviceToHost, st));
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
    *bytes = make_layout(n_rows, nnz, t[0]).total;
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
    i32x4 *tasks = reinterpret_cast<i32x4 *>(ws + L.tasks);
    const int nwg = (int)ceil_div(std::max(n, 1), WG);

    // 1. rows grouped by length: bin_offsets and perm (a stable counting sort)
    SPMV_HIP(hipMemsetAsync(&meta->max_short, 0, sizeof(int), st));
    k_plan_count<<<nwg, WG, 0, st>>>(n, h->rp, h->t[0], h->t[1], h->t[2], counts, &meta->max_short);
    SPMV_LAUNCHED("k_plan_count");
    k_plan_scan<<<1, 1024, 0, st>>>(nwg, 4, counts, offsets, meta->bin_offsets);
    SPMV_LAUNCHED("k_plan_scan");
    k_plan_scatter<<<nwg, WG, 0, st>>>(n, h->rp, h->t[0], h->t[1], h->t[2], offsets, perm);
    SPMV_LAUNCHED("k_plan_scatter");
    // 2. tasks of the rows in groups 1-3 (perm order)
    //    (counts / offsets of step 1 are free again and hold the workgroup rows)
    k_rowtasks_count<<<nwg, WG, 0, st>>>(meta, n, perm, h->rp, hcounts, counts);
    SPMV_LAUNCHED("k_rowtasks_count");
    k_plan_scan<<<1, 1024, 0, st>>>(nwg, 1, hcounts, hoffsets, meta->row_task_totals);
    SPMV_LAUNCHED("k_plan_scan(row tasks)");
    k_plan_scan<<<1, 1024, 0, st>>>(nwg, 1, counts, offsets, meta->wgrow_totals);
    SPMV_LAUNCHED("k_plan_scan(workgroup rows)");
    k_rowtasks_write<<<nwg, WG, 0, st>>>(meta, n, perm, h->rp, hoffsets, offsets, tasks);
    SPMV_LAUNCHED("k_rowtasks_write");
    // 3. blocks of short rows, after the row tasks
    k_heads_count<<<nwg, WG, 0, st>>>(meta, perm, h->rp, hcounts);
    SPMV_LAUNCHED("k_heads_count");
    k_plan_scan<<<1, 1024, 0, st>>>(nwg, 1, hcounts, hoffsets, meta->head_totals);
    SPMV_LAUNCHED("k_plan_scan(heads)");
    k_heads_scatter<<<nwg, WG, 0, st>>>(meta, perm, h->rp, hoffsets, heads);
    SPMV_LAUNCHED("k_heads_scatter");
    k_blocks_count<<<nwg, WG, 0, st>>>(meta, heads, hcounts);
    SPMV_LAUNCHED("k_blocks_count");
    k_plan_scan<<<1, 1024, 0, st>>>(nwg, 1, hcounts, hoffsets, meta->block_totals);
    SPMV_LAUNCHED("k_plan_scan(blocks)");
    k_blocks_write<<<nwg, WG, 0, st>>>(meta, heads, hoffsets, perm, h->rp, tasks);
    SPMV_LAUNCHED("k_blocks_write");
    Meta hm{};
    SPMV_HIP(hipMemcpyAsync(&hm, meta, sizeof(Meta), hipMemcpyDeviceToHost, st));
    SPMV_HIP(hipStreamSynchronize(st));
    for (int g = 0; g < 5; ++g) h->bin_off[g] = hm.bin_offsets[g];
    h->n_wg_rows = hm.wgrow_totals[1];
    h->n_row_tasks = hm.wgrow_totals[1] + hm.row_task_totals[1];
    h->n_blocks = hm.block_totals[1];
    if (h->n_row_tasks > L.max_row_tasks || (int64_t)h->n_row_tasks + h->n_blocks > L.max_tasks)
        return fail(SPMV_ERR_INVALID_MATRIX, "task count exceeds its bound");
    h->perm = perm;
    h->tasks = tasks;
    h->partials = reinterpret_cast<float *>(ws + L.partials);
    // rows of groups 1-3 each give one task unless some row was split into
    // chunk tasks
    h->has_chunked_rows = h->n_row_tasks > h->bin_off[4] - h->bin_off[1];
    // a workgroup per workgroup row, then one wave per task: row-task
    // workgroups, then block workgroups
    h->grid = (int)(h->n_wg_rows + ceil_div(h->n_row_tasks - h->n_wg_rows, TWAVES) + ceil_div(h->n_blocks, TWAVES));
    // column windows of the block workgroups: narrow ones let the apply stage
    // x in LDS
    if (h->n_blocks > 0) {
        XWindow *spans = reinterpret_cast<XWindow *>(ws + L.spans);
        SPMV_HIP(hipMemsetAsync(&meta->max_window, 0, sizeof(int), st));
        k_block_spans<<<(int)ceil_div(h->n_blocks, TWAVES), TWG, 0, st>>>(meta, tasks, h->ci, spans);
        SPMV_LAUNCHED("k_block_spans");
        int mw = 0;
        SPMV_HIP(hipMemcpyAsync(&mw, &meta->max_window, sizeof(int), hipMemcpyDeviceToHost, st));
        SPMV_HIP(hipStreamSynchronize(st));
        h->spans = spans;
        h->x_tile = mw > 0 && mw <= X_TILE_MAX ? 4 * (int)ceil_div(mw, 4) : 0;
    }
    SPMV_HIP(hipStreamSynchronize(st));
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
    Layout L = make_layout(n_rows, nnz, t[0]);
    // BINNED keeps its plan in the workspace; SCALAR and VECTOR use only its
    // first 256 bytes, for the validation flags, during this call
    const size_t need = var == SPMV_CSR_BINNED ? L.total : SCRATCH_HEAD;
    if (!workspace) return fail(SPMV_ERR_INVALID_VALUE, "workspace is NULL");
    if (workspace_bytes < need)
        return fail(SPMV_ERR_INVALID_VALUE, "workspace of %zu bytes is smaller than %zu", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(SPMV_ERR_INVALID_VALUE, "workspace must be 256-byte aligned");
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
    // validation flags: in the plan's header (BINNED) or the workspace's
    // first bytes (SCALAR, VECTOR)
    int *d_err = var == SPMV_CSR_BINNED
                     ? &reinterpret_cast<Meta *>(static_cast<char *>(workspace) + L.meta)->err
                     : reinterpret_cast<int *>(static_cast<char *>(workspace) + SCRATCH_ERR);
    spmv_status r = SPMV_OK;
    if (hipMemsetAsync(d_err, 0, sizeof(int), st) != hipSuccess) r = fail(SPMV_ERR_HIP, "hipMemsetAsync failed");
    if (r == SPMV_OK) r = validate_matrix(h, st, d_err);
    if (r == SPMV_OK && var == SPMV_CSR_BINNED) r = build_binned_plan(h, static_cast<char *>(workspace), L, st);
    if (r != SPMV_OK) {
        (void)hipStreamSynchronize(st);
        delete h;
        return r;
    }
    *out = h;
    return SPMV_OK;
}

namespace {

spmv_status csr_apply(spmv_csr_t h, float alpha, const float *x, float beta, float *y, const int *ymap,
                      void *stream) {
    if (!h) return fail(SPMV_ERR_INVALID_VALUE, "handle is NULL");
    if (h->n_rows == 0) return SPMV_OK;
    if (!y || (h->n_cols > 0 && !x)) return fail(SPMV_ERR_INVALID_VALUE, "x or y is NULL");
    hipStream_t st = as_stream(stream);
    const int n = h->n_rows;
    switch (h->variant) {
    case SPMV_CSR_SCALAR:
        k_csr_scalar<<<(int)ceil_div(n, WG), WG, 0, st>>>(n, h->rp, h->ci, h->v, x, alpha, beta, y, ymap);
        SPMV_LAUNCHED("k_csr_scalar");
        return SPMV_OK;
    case SPMV_CSR_VECTOR: {
        const int g = h->group_lanes;
        const int grid = (int)ceil_div((int64_t)n * g, WG);
#define SPMV_VEC_CASE(G)                                                                   \
    case G:                                                                                \
        k_csr_vector<G><<<grid, WG, 0, st>>>(n, h->rp, h->ci, h->v, x, alpha, beta, y, ymap); \
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
    if (h->nnz == 0) {
        k_csr_scale<<<(int)ceil_div(n, WG), WG, 0, st>>>(n, beta, y, ymap);
        SPMV_LAUNCHED("k_csr_scale");
        return SPMV_OK;
    }
    if (h->grid == 0) return SPMV_OK;
    TaskArgs a{};
    a.alpha = alpha;
    a.beta = beta;
    a.nnz = h->nnz;
    a.last_vec = (h->nnz & ~3) - 4;
    a.n_row_tasks = h->n_row_tasks;
    a.n_wg_rows = h->n_wg_rows;
    a.n_blocks = h->n_blocks;
    a.n_rows = n;
    a.n_cols = h->n_cols;
    // buffer gathers address at most 4 GiB with 32-bit byte offsets
    const bool buf = h->n_cols < (1 << 30) && n < (1 << 30) - 1;
    // x tile in LDS: narrow block windows, aligned arrays, x 16-byte aligned
    // and a multiple of 4 long (the window's 16-byte loads stay inside x)
    const bool xt = h->x_tile > 0 && h->vec_ok && buf && aligned16(x) && h->n_cols % 4 == 0;
    if (xt) {
        // rounds of 16-byte loads per thread that the widest window needs
        const int rounds = (int)ceil_div(h->x_tile / 4, TWG);
        const size_t lds = sizeof(float) * (size_t)h->x_tile;
        switch (rounds) {
#define SPMV_XT_CASE(R)                                                                                  \
    case R:                                                                                              \
        k_csr_tasks<true, true, R><<<h->grid, TWG, lds, st>>>(a, h->tasks, h->rp, h->ci, h->v, x, y, ymap, \
                                                             h->partials, h->spans);                      \
        break;
            SPMV_XT_CASE(1) SPMV_XT_CASE(2) SPMV_XT_CASE(3) SPMV_XT_CASE(4) SPMV_XT_CASE(5) SPMV_XT_CASE(6)
#undef SPMV_XT_CASE
        default:
            return fail(SPMV_ERR_INVALID_VALUE, "x window of %d floats exceeds the tile", h->x_tile);
        }
    } else if (h->vec_ok && buf)
        k_csr_tasks<true, true, 0><<<h->grid, TWG, 0, st>>>(a, h->tasks, h->rp, h->ci, h->v, x, y, ymap,
                                                            h->partials, h->spans);
    else if (h->vec_ok)
        k_csr_tasks<true, false, 0><<<h->grid, TWG, 0, st>>>(a, h->tasks, h->rp, h->ci, h->v, x, y, ymap,
                                                             h->partials, h->spans);
    else if (buf)
        k_csr_tasks<false, true, 0><<<h->grid, TWG, 0, st>>>(a, h->tasks, h->rp, h->ci, h->v, x, y, ymap,
                                                             h->partials, h->spans);
    else
        k_csr_tasks<false, false, 0><<<h->grid, TWG, 0, st>>>(a, h->tasks, h->rp, h->ci, h->v, x, y, ymap,
                                                              h->partials, h->spans);
    SPMV_LAUNCHED("k_csr_tasks");
    if (h->has_chunked_rows) {
        k_csr_chunks_finish<<<(int)ceil_div(h->n_row_tasks, WG), WG, 0, st>>>(h->n_row_tasks, h->tasks, h->rp,
                                                                               h->partials, alpha, beta, y, ymap);
        SPMV_LAUNCHED("k_csr_chunks_finish");
    }
    return SPMV_OK;
}

}  // namespace

extern "C" spmv_status spmv_csr_apply(spmv_csr_t h, float alpha, const float *x, float beta, float *y,
                                      void *stream) {
    return csr_apply(h, alpha, x, beta, y, nullptr, stream);
}

extern "C" spmv_status spmv_csr_apply_rows(spmv_csr_t h, float alpha, const float *x, float beta, float *y,
                                           const int32_t *row_map, void *stream) {
    if (h && h->n_rows > 0 && !row_map) return fail(SPMV_ERR_INVALID_VALUE, "row_map is NULL");
    return csr_apply(h, alpha, x, beta, y, row_map, stream);
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
