// Reference streaming kernels: the measured bandwidth denominator beside the
// 8 TB/s HBM peak.  Every SpMV path here is bound by HBM bandwidth, so the
// best a kernel of a given size can do on this GPU is what a plain stream of
// the same bytes reaches.  Two shapes: a copy (n bytes read, n written) and a
// read-only pass (n bytes read, one partial per workgroup written).  Both use
// non-temporal 16-byte accesses, like the matrix streams of the SpMV
// kernels, one per thread per grid-stride step, over a grid of 8 workgroups
// per CU: 32 waves per CU keep enough loads in flight.  Of the shapes
// measured (1, 2, 4 or 8 loads per thread per step; 1 to 64 workgroups per
// CU; grid-stride or one contiguous chunk per workgroup), this one was the
// fastest or within 2% of it at 48 MB, 52 MB and 200 MB, where four loads
// per thread over 4 workgroups per CU took 15-25% longer.
#include "common.hpp"

#include <algorithm>

namespace spmv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int ST_WG = 256;
__global__ __launch_bounds__(ST_WG) void k_stream_copy(int64_t n16, const f32x4 *__restrict__ src,
                                                       f32x4 *__restrict__ dst) {
    const int64_t stride = (int64_t)gridDim.x * ST_WG;
    for (int64_t i = (int64_t)blockIdx.x * ST_WG + threadIdx.x; i < n16; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(ST_WG) void k_stream_read(int64_t n16, const f32x4 *__restrict__ src,
                                                       float *__restrict__ partial) {
    __shared__ float red[ST_WG / 64];
    const int64_t stride = (int64_t)gridDim.x * ST_WG;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t i = (int64_t)blockIdx.x * ST_WG + threadIdx.x; i < n16; i += stride)
        acc += __builtin_nontemporal_load(src + i);
    float s = wave_sum(acc.x + acc.y + acc.z + acc.w);
    if (lane_id() == 0) red[threadIdx.x / 64] = s;
    __syncthreads();
    if (threadIdx.x == 0) partial[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

int stream_grid(int64_t n16) {
    return (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(n16, ST_WG), 8 * (int64_t)device_cu_count()));
}

spmv_status check_stream(const void *p, size_t bytes) {
    if (bytes % 16) return fail(SPMV_ERR_INVALID_VALUE, "bytes must be a multiple of 16");
    if (bytes > 0 && (!p || !aligned16(p))) return fail(SPMV_ERR_INVALID_VALUE, "buffer NULL or not 16-byte aligned");
    return SPMV_OK;
}

}  // namespace
}  // namespace spmv

using namespace spmv;

extern "C" spmv_status spmv_stream_copy(const void *src, void *dst, size_t bytes, void *stream) {
    spmv_status s = check_stream(src, bytes);
    if (s == SPMV_OK) s = check_stream(dst, bytes);
    if (s != SPMV_OK || bytes == 0) return s;
    const int64_t n16 = (int64_t)(bytes / 16);
    k_stream_copy<<<stream_grid(n16), ST_WG, 0, as_stream(stream)>>>(n16, static_cast<const f32x4 *>(src),
                                                                        static_cast<f32x4 *>(dst));
    SPMV_LAUNCHED("k_stream_copy");
    return SPMV_OK;
}

extern "C" spmv_status spmv_stream_read(const void *src, size_t bytes, float *partial, size_t partial_count,
                                        void *stream) {
    spmv_status s = check_stream(src, bytes);
    if (s != SPMV_OK || bytes == 0) return s;
    if (!partial) return fail(SPMV_ERR_INVALID_VALUE, "partial is NULL");
    const int64_t n16 = (int64_t)(bytes / 16);
    const int grid = stream_grid(n16);
    if (partial_count < (size_t)grid) return fail(SPMV_ERR_INVALID_VALUE, "partial holds fewer floats than workgroups");
    k_stream_read<<<grid, ST_WG, 0, as_stream(stream)>>>(n16, static_cast<const f32x4 *>(src), partial);
    SPMV_LAUNCHED("k_stream_read");
    return SPMV_OK;
}
