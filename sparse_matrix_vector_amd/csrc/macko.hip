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

template <bool X_LDS>
__global__ __launch_bounds__(MK_WG) void k_macko_spmv(int n_rows, int n_cols, const int *__restrict__ mrp,
                                                      const unsigned int *__restrict__ codes,
                                                      const unsigned short *__restrict__ mvals, float alpha,
                                                      const unsigned short *__restrict__ x, float beta,
                                                      float *__restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) unsigned short xs_dyn[];
    if (X_LDS) {
        stage_halfs(xs_dyn, x, n_cols);
        __syncthreads();
    }
    const unsigned short *xv = X_LDS ? xs_dyn : x;
    const int lane = __lane_id();
    const int wv = threadIdx.x / 64;
    const int last_col = n_cols - 1;
    for (int row = blockIdx.x * MK_WAVES + wv; row < n_rows; row += gridDim.x * MK_WAVES) {
        const int e0 = mrp[row], e1 = mrp[row + 1];
        int carry = -1;
        float acc = 0.0f;
        for (int c0 = e0; c0 < e1; c0 += MK_CHUNK * MK_UNROLL) {
            unsigned int word[MK_UNROLL];
            u32x4 val[MK_UNROLL];
#pragma unroll
            for (int u = 0; u < MK_UNROLL; ++u) {
                const int ent = c0 + u * MK_CHUNK + 8 * lane;
                const bool valid = ent < e1;
                word[u] = valid ? __builtin_nontemporal_load(codes + (ent >> 3)) : 0u;
                val[u] = valid ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(mvals + ent))
                               : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < MK_UNROLL; ++u) {
                if (c0 + u * MK_CHUNK >= e1) break;   // uniform: rows end on 256-entry units
                const bool valid = c0 + u * MK_CHUNK + 8 * lane < e1;
                int p[8];
                nibble_prefix(word[u], p);
                const int tot = valid ? p[7] : 0;
                const int incl = wave_inclusive_scan(tot);
                const int base = carry + incl - tot;
                carry += __builtin_amdgcn_readlane(incl, 63);
                // No branch on `valid`: an idle lane holds zero values and its
                // clamped columns stay inside x, so all 8 LDS reads of every
                // lane are issued together.
                (void)valid;
#pragma unroll
                for (int t = 0; t < 8; t += 2) {
                    const int ca = min(base + p[t], last_col);
                    const int cb = min(base + p[t + 1], last_col);
                    const unsigned int xp = (unsigned int)xv[ca] | ((unsigned int)xv[cb] << 16);
                    acc = __builtin_amdgcn_fdot2(as_h2(val[u][t >> 1]), as_h2(xp), acc, false);
                }
            }
        }
        acc = wave_sum(acc);
        if (lane == 0) {
            float r = alpha * acc;
            if (beta != 0.0f) r = fmaf(beta, y[row], r);
            y[row] = r;
        }
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
        const size_t lds = (size_t)((n_cols + 7) & ~7) * sizeof(uint16_t);
        // as many workgroups per CU as the LDS allows, at most 2
        const int per_cu = lds <= 48 * 1024 ? 2 : 1;
        k_macko_spmv<true><<<persistent_grid(n_rows, per_cu), MK_WG, lds, st>>>(n_rows, n_cols, mrow_ptr, codes, mvals,
                                                                                 alpha, x_f16, beta, y);
    } else {
        k_macko_spmv<false><<<persistent_grid(n_rows, 2), MK_WG, 0, st>>>(n_rows, n_cols, mrow_ptr, codes, mvals,
                                                                           alpha, x_f16, beta, y);
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
