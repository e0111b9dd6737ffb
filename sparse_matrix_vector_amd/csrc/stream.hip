// Reference streaming kernels: the measured bandwidth denominator beside the
// 8 TB/s HBM peak.  Every SpMV path here is bound by HBM bandwidth, so the
// best a kernel of a given size can do on this GPU is what a plain stream of
// the same bytes reaches.  Two shapes: a copy (n bytes read, n written) and a
// read-only pass (n bytes read, one partial per workgroup written).  Both use
// 16-byte accesses, four per thread in flight, non-temporal like the matrix
// streams of the SpMV kernels, over a grid of 4 workgroups per CU.
#include "common.hpp"

#include <algorithm>

namespace spmv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int ST_WG = 256;
constexpr int ST_UNROLL = 4;

__global__ __launch_bounds__(ST_WG) void k_stream_copy(int64_t n16, const f32x4 *__restrict__ src,
                                                       f32x4 *__restrict__ dst) {
    const int64_t stride = (int64_t)gridDim.x * ST_WG;
    int64_t i = (int64_t)blockIdx.x * ST_WG + threadIdx.x;
    for (; i + (ST_UNROLL - 1) * stride < n16; i += ST_UNROLL * stride) {
        f32x4 v[ST_UNROLL];
#pragma unroll
        for (int u = 0; u < ST_UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < ST_UNROLL; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
    }
    for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(ST_WG) void k_stream_read(int64_t n16, const f32x4 *__restrict__ src,
                                                       float *__restrict__ partial) {
    __shared__ float red[ST_WG / 64];
    const int64_t stride = (int64_t)gridDim.x * ST_WG;
    int64_t i = (int64_t)blockIdx.x * ST_WG + threadIdx.x;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (; i + (ST_UNROLL - 1) * stride < n16; i += ST_UNROLL * stride) {
        f32x4 v[ST_UNROLL];
#pragma unroll
        for (int u = 0; u < ST_UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < ST_UNROLL; ++u) acc += v[u];
    }
    for (; i < n16; i += stride) acc += __builtin_nontemporal_load(src + i);
    float s = wave_sum(acc.x + acc.y + acc.z + acc.w);
    if (lane_id() == 0) red[threadIdx.x / 64] = s;
    __syncthreads();
    if (threadIdx.x == 0) partial[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

int stream_grid(int64_t n16) {
    return (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(n16, ST_WG), 4 * (int64_t)device_cu_count()));
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

extern "C" spmv_status spmv_stream_read(const void *src, size_t bytes, float *partial, void *stream) {
    spmv_status s = check_stream(src, bytes);
    if (s != SPMV_OK || bytes == 0) return s;
    if (!partial) return fail(SPMV_ERR_INVALID_VALUE, "partial is NULL");
    const int64_t n16 = (int64_t)(bytes / 16);
    k_stream_read<<<stream_grid(n16), ST_WG, 0, as_stream(stream)>>>(n16, static_cast<const f32x4 *>(src), partial);
    SPMV_LAUNCHED("k_stream_read");
    return SPMV_OK;
}
