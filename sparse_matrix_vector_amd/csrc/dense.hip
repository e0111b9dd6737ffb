// Dense fp16 GEMV on gfx950: the dense comparator of the MACKO page's
// section 3.1 table ("MACKO-SpMV: GPU acceleration and storage optimisation
// at low sparsity"), y = alpha * W x + beta * y with W fp16 row-major.
//
// One wave per row, persistent workgroups: x is staged in LDS once per
// workgroup; each lane streams 16 bytes (8 fp16) of the row per step with
// several steps' loads in flight, reads the matching 8 entries of x from LDS
// as one 16-byte read, and accumulates with v_dot2_f32_f16 (fp16 products,
// fp32 sums).  Rows whose byte length is not a multiple of 16 use a 2-byte
// path.  No matrix cores: a matrix-vector product has one flop per byte
// loaded, far below what MFMA tiles need.
#include "common.hpp"

#include <algorithm>

namespace spmv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int DW_WAVES = 8;
constexpr int DW_WG = 64 * DW_WAVES;
constexpr int DW_UNROLL = 4;
constexpr int DW_LDS_MAX_COLS = 32768;

__device__ __forceinline__ f16x2 as_h2(unsigned int w) { return __builtin_bit_cast(f16x2, w); }

__device__ __forceinline__ float h2f(unsigned short h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

template <bool VEC, bool X_LDS>
__global__ __launch_bounds__(DW_WG) void k_gemv_f16(int m, int n, const unsigned short *__restrict__ W,
                                                    const unsigned short *__restrict__ x, float alpha, float beta,
                                                    float *__restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) unsigned short xs_dyn[];
    if (X_LDS) {
        stage_halfs(xs_dyn, x, n);
        __syncthreads();
    }
    const unsigned short *xv = X_LDS ? xs_dyn : x;
    const int lane = __lane_id();
    const int wv = threadIdx.x / 64;
    for (int row = blockIdx.x * DW_WAVES + wv; row < m; row += gridDim.x * DW_WAVES) {
        const unsigned short *wr = W + (size_t)row * (size_t)n;
        float acc = 0.0f;
        if (VEC) {
            for (int j0 = 8 * lane; j0 < n; j0 += 512 * DW_UNROLL) {
                u32x4 w[DW_UNROLL];
#pragma unroll
                for (int u = 0; u < DW_UNROLL; ++u) {
                    const int j = j0 + 512 * u;
                    w[u] = j < n ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wr + j))
                                 : u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int u = 0; u < DW_UNROLL; ++u) {
                    const int j = j0 + 512 * u;
                    if (j < n) {
                        const u32x4 xq = *reinterpret_cast<const u32x4 *>(xv + j);
#pragma unroll
                        for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_fdot2(as_h2(w[u][t]), as_h2(xq[t]), acc, false);
                    }
                }
            }
        } else {
            for (int j = lane; j < n; j += 64) acc = fmaf(h2f(wr[j]), h2f(xv[j]), acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) {
            float r = alpha * acc;
            if (beta != 0.0f) r = fmaf(beta, y[row], r);
            y[row] = r;
        }
    }
}

}  // namespace
}  // namespace spmv

using namespace spmv;

extern "C" spmv_status dense_gemv_f16(int32_t m, int32_t n, const uint16_t *W, const uint16_t *x_f16, float alpha,
                                      float beta, float *y, void *stream) {
    if (m < 0 || n < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if (m == 0) return SPMV_OK;
    if (!y || (n > 0 && (!W || !x_f16))) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    hipStream_t st = as_stream(stream);
    const bool vec = (n % 8 == 0) && aligned16(W) && aligned16(x_f16);
    const bool lds = n <= DW_LDS_MAX_COLS;
    const size_t lds_bytes = lds ? (size_t)((n + 7) & ~7) * sizeof(uint16_t) : 0;
    const int per_cu = (!lds || lds_bytes <= 48 * 1024) ? 2 : 1;
    const int grid = std::max(1, (int)std::min<int64_t>(ceil_div(m, DW_WAVES), (int64_t)per_cu * device_cu_count()));
    if (vec && lds)
        k_gemv_f16<true, true><<<grid, DW_WG, lds_bytes, st>>>(m, n, W, x_f16, alpha, beta, y);
    else if (vec)
        k_gemv_f16<true, false><<<grid, DW_WG, 0, st>>>(m, n, W, x_f16, alpha, beta, y);
    else if (lds)
        k_gemv_f16<false, true><<<grid, DW_WG, lds_bytes, st>>>(m, n, W, x_f16, alpha, beta, y);
    else
        k_gemv_f16<false, false><<<grid, DW_WG, 0, st>>>(m, n, W, x_f16, alpha, beta, y);
    SPMV_LAUNCHED("k_gemv_f16");
    return SPMV_OK;
}
