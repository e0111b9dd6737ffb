// MACKO SpMV and column decoding on gfx950.
//
// "MACKO-SpMV: GPU acceleration and storage optimisation at low sparsity",
// section 2.2: a warp owns a row and walks it in chunks; the lanes load the
// chunk's packed 4-bit gaps and fp16 values cooperatively with wide loads
// (2.2.1), rebuild absolute columns with a lane-local sum of the gaps
// followed by a warp-wide prefix sum (2.2.2), and multiply by the gathered
// vector (2.2.3).
//
// gfx950 shape: one wave64 per row, 512 entries per chunk, lane l owns
// entries 8l..8l+7 of the chunk: one 4-byte load of its code word and one
// 16-byte load of its eight fp16 values (256 B + 1 KB per wave, fully
// coalesced).  Columns: lane-local inclusive prefix of (code + 1) over its 8
// nibbles, a 6-step DPP scan of the lane totals (row shifts + row
// broadcasts), plus the carry of the row so far (the last column of the
// previous chunk, starting at -1).  x (fp16) is staged once per workgroup
// in LDS; products are fp16 x fp16 -> fp32 with v_dot2_f32_f16 (exact
// products, fp32 accumulate).  Trailing alignment entries can decode past
// the last column; their LDS index is clamped and their value is +0.
// Workgroups are persistent: each wave takes rows gridDim * waves apart, so
// x is staged into LDS once per workgroup instead of once per row.
#include "common.hpp"

#include <algorithm>

namespace spmv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int MK_WAVES = 12;          // waves per workgroup (2 workgroups per CU: 24 waves)
constexpr int MK_WG = 64 * MK_WAVES;
constexpr int MK_CHUNK = 512;         // entries per wave per step (64 lanes x 8)
constexpr int MK_UNROLL = 4;          // chunks whose loads are issued together
constexpr int MK_LDS_MAX_COLS = 32768;   // x in LDS up to 64 KB
constexpr int MK_XPAD = 512;          // zero halfs after x in LDS (> 255 + 128)

__device__ __forceinline__ f16x2 as_h2(unsigned int w) { return __builtin_bit_cast(f16x2, w); }

// Lane-local inclusive prefix of (code + 1) over the 8 nibbles of `word`.
__device__ __forceinline__ void nibble_prefix(unsigned int word, int (&p)[8]) {
    int run = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        run += (int)((word >> (4 * t)) & 15u) + 1;
        p[t] = run;
    }
}

// The first MK_UNROLL chunks (up to MK_UNROLL * 512 entries) of [c0, e1):
// lane l holds entries c0 + 512 u + 8 l .. + 7 of chunk u (its code word and
// its eight fp16 values).  Entries at or past e1 are not valid; apply_group
// masks them by position.
//   UNCOND: every load is issued, at a valid address: lanes past e1 re-read
//   the row's last 8 entries, and an empty range reads 16 bytes at `dummy`
//   (which must be readable and 16-byte aligned).  With no branches around
//   the loads the compiler can keep them in flight across later waits.
//   Otherwise lanes past e1 load nothing and hold zeros.
struct Group {
    unsigned int word[MK_UNROLL];
    u32x4 val[MK_UNROLL];
};

template <bool UNCOND>
__device__ __forceinline__ void load_group(Group &g, const unsigned int *__restrict__ codes,
                                           const unsigned short *__restrict__ mvals, int c0, int e1, int lane,
                                           const void *dummy) {
    if (UNCOND) {
        const bool any = e1 > c0;   // uniform
        const unsigned int *wp = any ? codes : static_cast<const unsigned int *>(dummy);
        const u32x4 *vp = any ? reinterpret_cast<const u32x4 *>(mvals) : static_cast<const u32x4 *>(dummy);
#pragma unroll
        for (int u = 0; u < MK_UNROLL; ++u) {
            const int ent = any ? min(c0 + u * MK_CHUNK + 8 * lane, e1 - 8) : 0;
            g.word[u] = __builtin_nontemporal_load(wp + (ent >> 3));
            g.val[u] = __builtin_nontemporal_load(vp + (ent >> 3));
        }
    } else {
#pragma unroll
        for (int u = 0; u < MK_UNROLL; ++u) {
            const int ent = c0 + u * MK_CHUNK + 8 * lane;
            const bool valid = ent < e1;
            g.word[u] = valid ? __builtin_nontemporal_load(codes + (ent >> 3)) : 0u;
            g.val[u] = valid ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(mvals + ent))
                             : u32x4{0u, 0u, 0u, 0u};
        }
    }
}

// One chunk of 512 entries: lane-local prefix of (code + 1), wave scan of
// the lane totals plus the running carry, then 8 reads of x and 4
// v_dot2_f32_f16.  MASKED: some lanes lie past the row's end (the row's last
// chunk); their totals count 0 and their values are masked.  CLAMP: x is
// read from memory, so columns are clamped to the last column; with x in
// LDS they are not, because the LDS copy is followed by MK_XPAD zeros and
// no decoded column goes further (see k_macko_spmv).
template <bool MASKED, bool CLAMP>
__device__ __forceinline__ void apply_chunk(unsigned int word, u32x4 val, bool valid, int last_col,
                                            const unsigned short *xv, int &carry, float &acc) {
    int p[8];
    nibble_prefix(word, p);
    const int tot = (!MASKED || valid) ? p[7] : 0;
    const int incl = wave_inclusive_scan(tot);
    const int base = carry + incl - tot;
    carry += __builtin_amdgcn_readlane(incl, 63);
    // No branch on `valid`: an idle lane's columns stay inside x or its
    // padding (they are >= 0: base >= carry >= -1 and p[t] >= 1), so all 8
    // reads of every lane are issued together; its values are masked.
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
        const int ca = CLAMP ? min(base + p[t], last_col) : base + p[t];
        const int cb = CLAMP ? min(base + p[t + 1], last_col) : base + p[t + 1];
        const unsigned int xp = (unsigned int)xv[ca] | ((unsigned int)xv[cb] << 16);
        const unsigned int vp = (!MASKED || valid) ? val[t >> 1] : 0u;
        acc = __builtin_amdgcn_fdot2(as_h2(vp), as_h2(xp), acc, false);
    }
}

// Decodes the columns of a loaded group (continuing from `carry`, the last
// column decoded so far in the row) and accumulates value * x[column].
template <bool CLAMP>
__device__ __forceinline__ void apply_group(const Group &g, int c0, int e1, int lane, int last_col,
                                            const unsigned short *xv, int &carry, float &acc) {
#pragma unroll
    for (int u = 0; u < MK_UNROLL; ++u) {
        const int cs = c0 + u * MK_CHUNK;
        if (cs >= e1) break;   // uniform: rows end on 256-entry units
        if (cs + MK_CHUNK <= e1)   // uniform: the whole chunk is inside the row
            apply_chunk<false, CLAMP>(g.word[u], g.val[u], true, last_col, xv, carry, acc);
        else
            apply_chunk<true, CLAMP>(g.word[u], g.val[u], cs + 8 * lane < e1, last_col, xv, carry, acc);
    }
    // Consume every register of the group, also of chunks past the row's
    // end, so that no load into them is still outstanding when they are
    // reloaded (that would make the compiler wait for every younger load,
    // the prefetched group included).
#pragma unroll
    for (int u = 0; u < MK_UNROLL; ++u) asm volatile("" ::"v"(g.word[u]), "v"(g.val[u]));
}

// Wave w of the grid owns rows w, w + W, w + 2W, ... (W waves in all).  Its
// row bounds are read up front, one row per lane (64 rows at a time), so
// the stream loads of a row never wait for a row_ptr load; the first group
// of the first row is in flight while x is staged into LDS, and the next
// group (of the same row, or of the wave's next row) is in flight while the
// current one is decoded and multiplied.
// XM: 0 = x read from global memory; 1 = x staged into LDS with 16-byte
// copies (x 16-byte aligned, n_cols >= 8); 2 = x staged element by element.
template <int XM>
__global__ __launch_bounds__(MK_WG) void k_macko_spmv(int n_rows, int n_cols, const int *__restrict__ mrp,
                                                      const unsigned int *__restrict__ codes,
                                                      const unsigned short *__restrict__ mvals, float alpha,
                                                      const unsigned short *__restrict__ x, float beta,
                                                      float *__restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) unsigned short xs_dyn[];
    const int lane = __lane_id();
    // wave-uniform, stated so that row indices and bounds are scalar
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int stride = gridDim.x * MK_WAVES;
    const int first = blockIdx.x * MK_WAVES + wv;
    const int nk = first < n_rows ? (n_rows - 1 - first) / stride + 1 : 0;   // rows of this wave

    // bounds of the wave's rows 0..63, one per lane
    int bs = 0, be = 0;
    if (lane < nk) {
        const int r = first + lane * stride;
        bs = mrp[r];
        be = mrp[r + 1];
    }
    // x: the first pass of the LDS copy is loaded now and stored later
    // (loads at clamped addresses, so they need no branch)
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    constexpr int XU = 4;
    const int n8 = XM == 1 ? (n_cols & ~7) : 0;
    const int xstride = 8 * MK_WG;
    u32x4_t xr[XU];
    if (XM == 1) {
#pragma unroll
        for (int u = 0; u < XU; ++u)
            xr[u] = *reinterpret_cast<const u32x4_t *>(x + min(8 * (int)threadIdx.x + u * xstride, n8 - 8));
    }
    int b0 = __builtin_amdgcn_readlane(bs, 0), b1 = __builtin_amdgcn_readlane(be, 0);
    Group g;
    load_group<XM == 1>(g, codes, mvals, b0, nk > 0 ? b1 : 0, lane, x);
    if (XM != 0) {
        if (XM == 1) {
            // clamped like the loads: threads past the end store the last
            // vector again, with the same data
#pragma unroll
            for (int u = 0; u < XU; ++u)
                *reinterpret_cast<u32x4_t *>(xs_dyn + min(8 * (int)threadIdx.x + u * xstride, n8 - 8)) = xr[u];
            for (int k = 8 * (int)threadIdx.x + XU * xstride; k < n8; k += xstride)
                *reinterpret_cast<u32x4_t *>(xs_dyn + k) = *reinterpret_cast<const u32x4_t *>(x + k);
        }
        for (int k = n8 + (int)threadIdx.x; k < n_cols; k += MK_WG) xs_dyn[k] = x[k];
        // MK_XPAD zeros after x: decoded columns of trailing alignment
        // entries (at most 255 past the last real column) and of idle lanes
        // (at most 128 further) read zeros instead of being clamped
        for (int k = n_cols + (int)threadIdx.x; k < n_cols + MK_XPAD; k += MK_WG) xs_dyn[k] = 0;
        // an LDS-only barrier: the stream loads issued above stay in flight
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
    const unsigned short *xv = XM != 0 ? xs_dyn : x;
    const int last_col = n_cols - 1;

    // Rows are taken in batches of 64 (one per lane for bounds and sums).
    // Within a batch there is one step per group; two Group buffers take
    // turns as current and prefetched, so no loaded data is ever copied
    // between registers (a copy would have to wait for its load), and the
    // loop has no stores (with a store in the loop the compiler waits for
    // every outstanding load at the loop head).  Row sums are collected in
    // `res` (lane l: row l of the batch) and stored after the batch.
    Group g2;
    for (int kb = 0; kb < nk; kb += 64) {
        const int cnt = min(64, nk - kb);
        if (kb > 0) {
            // bounds of the batch's rows, then its first group
            bs = be = 0;
            if (lane < cnt) {
                const int r = first + (kb + lane) * stride;
                bs = mrp[r];
                be = mrp[r + 1];
            }
            b0 = __builtin_amdgcn_readlane(bs, 0);
            b1 = __builtin_amdgcn_readlane(be, 0);
            load_group<XM == 1>(g, codes, mvals, b0, b1, lane, x);
        }
        int k = 0;               // row of the batch being reduced
        int c0 = b0, e1 = b1;    // current group start, current row end
        int nb0 = 0, nb1 = 0;    // bounds of row k + 1
        if (cnt > 1) {
            nb0 = __builtin_amdgcn_readlane(bs, 1);
            nb1 = __builtin_amdgcn_readlane(be, 1);
        }
        int carry = -1;
        float acc = 0.0f, res = 0.0f;
        // steps of the batch: one per group of each row, one for an empty row
        const int len = be - bs;
        const int nsteps = wave_sum_int(lane < cnt ? max(1, (len + MK_CHUNK * MK_UNROLL - 1) / (MK_CHUNK * MK_UNROLL)) : 0);
        auto step = [&](const Group &cur, Group &nxt) {
            const int c1 = c0 + MK_CHUNK * MK_UNROLL;
            const bool row_done = c1 >= e1;
            load_group<XM == 1>(nxt, codes, mvals, row_done ? nb0 : c1, row_done ? nb1 : e1, lane, x);
            apply_group<XM == 0>(cur, c0, e1, lane, last_col, xv, carry, acc);
            if (!row_done) {
                c0 = c1;
            } else {
                const float sum = wave_sum(acc);
                if (lane == k) res = sum;
                acc = 0.0f;
                carry = -1;
                ++k;
                c0 = nb0;
                e1 = nb1;
                nb0 = nb1 = 0;
                if (k + 1 < cnt) {
                    nb0 = __builtin_amdgcn_readlane(bs, k + 1);
                    nb1 = __builtin_amdgcn_readlane(be, k + 1);
                }
            }
        };
        // no exit inside the loop body: an early exit there would give the
        // compiler a path on which the prefetched loads reach the loop head
        // unwaited, and it would then wait for them on every iteration
        int i = 0;
        for (; i + 1 < nsteps; i += 2) {
            step(g, g2);
            step(g2, g);
        }
        if (i < nsteps) step(g, g2);
        if (lane < cnt) {
            const int row = first + (kb + lane) * stride;
            float r = alpha * res;
            if (beta != 0.0f) r = fmaf(beta, y[row], r);
            y[row] = r;
        }
        // s_waitcnt vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt left at their
        // maxima): the store is complete before the next batch, so the
        // compiler sees no outstanding store at the head of the step loop
        __builtin_amdgcn_s_waitcnt(0x0F70);
    }
}

// Writes the column of every stored entry, with the same decoder.
__global__ __launch_bounds__(MK_WG) void k_macko_decode(int n_rows, const int *__restrict__ mrp,
                                                        const unsigned int *__restrict__ codes,
                                                        int *__restrict__ cols) {
    const int lane = __lane_id();
    const int wv = threadIdx.x / 64;
    for (int row = blockIdx.x * MK_WAVES + wv; row < n_rows; row += gridDim.x * MK_WAVES) {
        const int e0 = mrp[row], e1 = mrp[row + 1];
        int carry = -1;
        for (int c0 = e0; c0 < e1; c0 += MK_CHUNK) {
            const int ent = c0 + 8 * lane;
            const bool valid = ent < e1;
            int p[8];
            nibble_prefix(valid ? codes[ent >> 3] : 0u, p);
            const int tot = valid ? p[7] : 0;
            const int incl = wave_inclusive_scan(tot);
            const int base = carry + incl - tot;
            carry += __builtin_amdgcn_readlane(incl, 63);
            if (valid) {
#pragma unroll
                for (int t = 0; t < 8; ++t) cols[ent + t] = base + p[t];
            }
        }
    }
}

int persistent_grid(int n_rows, int per_cu) {
    const int want = (int)ceil_div(n_rows, MK_WAVES);
    return std::max(1, std::min(want, per_cu * device_cu_count()));
}

}  // namespace
}  // namespace spmv

using namespace spmv;

extern "C" spmv_status macko_spmv(int32_t n_rows, int32_t n_cols, const int32_t *mrow_ptr, const uint32_t *codes,
                                  const uint16_t *mvals, float alpha, const uint16_t *x_f16, float beta, float *y,
                                  void *stream) {
    if (n_rows < 0 || n_cols < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if (n_rows == 0) return SPMV_OK;
    if (!mrow_ptr || !y) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    if (n_cols == 0) return fail(SPMV_ERR_INVALID_VALUE, "n_cols must be positive when there are rows");
    if (!codes || !mvals || !x_f16) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    if (!aligned16(mvals) || (reinterpret_cast<uintptr_t>(codes) & 3u))
        return fail(SPMV_ERR_UNSUPPORTED, "mvals must be 16-byte aligned and codes 4-byte aligned");
    hipStream_t st = as_stream(stream);
    if (n_cols <= MK_LDS_MAX_COLS) {
        const size_t lds = (size_t)((n_cols + MK_XPAD + 7) & ~7) * sizeof(uint16_t);
        // as many workgroups per CU as the LDS allows, at most 2
        const int per_cu = lds <= 48 * 1024 ? 2 : 1;
        const int grid = persistent_grid(n_rows, per_cu);
        if (aligned16(x_f16) && n_cols >= 8)
            k_macko_spmv<1><<<grid, MK_WG, lds, st>>>(n_rows, n_cols, mrow_ptr, codes, mvals, alpha, x_f16, beta, y);
        else
            k_macko_spmv<2><<<grid, MK_WG, lds, st>>>(n_rows, n_cols, mrow_ptr, codes, mvals, alpha, x_f16, beta, y);
    } else {
        k_macko_spmv<0><<<persistent_grid(n_rows, 2), MK_WG, 0, st>>>(n_rows, n_cols, mrow_ptr, codes, mvals, alpha,
                                                                       x_f16, beta, y);
    }
    SPMV_LAUNCHED("k_macko_spmv");
    return SPMV_OK;
}

extern "C" spmv_status macko_decode_columns(int32_t n_rows, const int32_t *mrow_ptr, const uint32_t *codes,
                                            int32_t *cols_out, void *stream) {
    if (n_rows < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if (n_rows == 0) return SPMV_OK;
    if (!mrow_ptr || !codes || !cols_out) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    hipStream_t st = as_stream(stream);
    k_macko_decode<<<persistent_grid(n_rows, 4), MK_WG, 0, st>>>(n_rows, mrow_ptr, codes, cols_out);
    SPMV_LAUNCHED("k_macko_decode");
    return SPMV_OK;
}
