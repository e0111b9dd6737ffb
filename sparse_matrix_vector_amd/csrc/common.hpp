// Shared host helpers (status / error text / launch checks) and wave64
// device primitives for the gfx950 SpMV kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "spmv.h"

namespace spmv {

// ---------------------------------------------------------------------------
// Host: thread-local error message and status helpers.
// ---------------------------------------------------------------------------
void set_error(const char *fmt, ...);
void clear_error();

inline spmv_status fail(spmv_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    set_error("%s", buf);
    return s;
}

#define SPMV_HIP(call)                                                          \
    do {                                                                        \
        hipError_t e_ = (call);                                                 \
        if (e_ != hipSuccess)                                                   \
            return ::spmv::fail(SPMV_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
    } while (0)

#define SPMV_LAUNCHED(name)                                                     \
    do {                                                                        \
        hipError_t e_ = hipGetLastError();                                      \
        if (e_ != hipSuccess)                                                   \
            return ::spmv::fail(SPMV_ERR_HIP, "launch of %s: %s", name, hipGetErrorString(e_)); \
    } while (0)

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Number of compute units of the current device (cached per device id).
int device_cu_count();

// ---------------------------------------------------------------------------
// Host: the caller's device scratch of the synchronous statistics, planning
// and conversion calls (spmv_scratch_size).  A 256-byte head of counters,
// each call using its own fixed offset, then two int32 counts per
// 256-row workgroup (the HYB split's compaction).
// ---------------------------------------------------------------------------
constexpr size_t SCRATCH_ROW_STATS = 0;     // {u64 sum, u64 sum_sq, i32 max, i32 err}
constexpr size_t SCRATCH_HYB_COUNTS = 32;   // u64[3]: sum min(len, W), rows > W, entries past W
constexpr size_t SCRATCH_ERR = 64;          // i32 error flags of a conversion or validation
constexpr size_t SCRATCH_SG_ERR = 96;       // i32 error flags of the SpGEMM validation
constexpr size_t SCRATCH_SG_TOTALS = 128;   // SpGEMM intermediate-product totals (<= 128 bytes)
constexpr size_t SCRATCH_HEAD = 256;
constexpr int SCRATCH_ROWS_PER_WG = 256;

inline size_t scratch_bytes(int64_t n_rows) {
    const int64_t nb = (n_rows + SCRATCH_ROWS_PER_WG - 1) / SCRATCH_ROWS_PER_WG;
    const size_t counts = (size_t)8 * (size_t)(nb > 0 ? nb : 1);
    return SCRATCH_HEAD + ((counts + 255) & ~size_t(255));
}

// Checks a caller scratch buffer for a matrix of n_rows rows.
spmv_status check_scratch(const void *scratch, size_t bytes, int64_t n_rows);

// HYB in one launch (ell.hip): the ELL part and a tail stored per row (entries
// of row r at [trp[r], trp[r + 1]) of tcol / tval) summed into one store per
// row.  ell_tail_fits: the shape and alignments the kernel needs of the
// matrix (width 1..8, n_rows and n_cols multiples of 4, 16-byte aligned
// arrays); x and y must be 16-byte aligned too.
bool ell_tail_fits(int32_t n_rows, int32_t n_cols, int32_t width, const void *ec, const void *ev, const void *trp);
spmv_status ell_tail_apply(int32_t n_rows, int32_t width, const int32_t *ell_col, const float *ell_val,
                           const int32_t *trp, const int32_t *tcol, const float *tval, float alpha, const float *x,
                           float beta, float *y, hipStream_t st);

// ---------------------------------------------------------------------------
// Device: wave64 primitives.
//
// DPP controls of the GFX9-family data-parallel-primitives encoding (CDNA
// keeps the row broadcasts that RDNA dropped).
// ---------------------------------------------------------------------------
constexpr int DPP_ROW_SHR1 = 0x111;
constexpr int DPP_ROW_SHR2 = 0x112;
constexpr int DPP_ROW_SHR4 = 0x114;
constexpr int DPP_ROW_SHR8 = 0x118;
constexpr int DPP_ROW_BCAST15 = 0x142;
constexpr int DPP_ROW_BCAST31 = 0x143;

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active).
// Rows of 16 lanes are scanned with shifted adds, then row totals are
// propagated with the two row broadcasts.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, DPP_ROW_SHR1, 0xf, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, DPP_ROW_SHR2, 0xf, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, DPP_ROW_SHR4, 0xf, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, DPP_ROW_SHR8, 0xf, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, DPP_ROW_BCAST15, 0xa, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, DPP_ROW_BCAST31, 0xc, 0xf, false);
    return v;
}

// Sum over the 64 lanes (all lanes active), as a wave-uniform value.
__device__ __forceinline__ int wave_sum_int(int v) {
    return __builtin_amdgcn_readlane(wave_inclusive_scan(v), 63);
}

// One scan step on floats: v += (v of the lane selected by `ctrl`), lanes
// without a source (or outside `row_mask`) add +0.
#define SPMV_DPP_FADD(v, ctrl, row_mask)                                              \
    (v) += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), (ctrl),     \
                                                      (row_mask), 0xf, false))

// Sum over the 64 lanes (all lanes active); the total is returned in every
// lane.  Fixed order, so the result is bit-reproducible.
__device__ __forceinline__ float wave_sum(float v) {
    SPMV_DPP_FADD(v, DPP_ROW_SHR1, 0xf);
    SPMV_DPP_FADD(v, DPP_ROW_SHR2, 0xf);
    SPMV_DPP_FADD(v, DPP_ROW_SHR4, 0xf);
    SPMV_DPP_FADD(v, DPP_ROW_SHR8, 0xf);
    SPMV_DPP_FADD(v, DPP_ROW_BCAST15, 0xa);
    SPMV_DPP_FADD(v, DPP_ROW_BCAST31, 0xc);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Marks loaded values as used at this point.  Without it the compiler may
// move a load whose result is only consumed under a condition into that
// conditional block, issuing it after the others and waiting for it there;
// with it all gathers are issued together and waited for once.
__device__ __forceinline__ void pin_value(float &v) { asm volatile("" : "+v"(v)); }

template <typename... T>
__device__ __forceinline__ void issue_together(T &...v) {
    (pin_value(v), ...);
}

// Copies n 2-byte elements from global memory into LDS, cooperatively by
// the whole workgroup.  Each thread issues up to 4 loads (16 bytes each
// when `src` is 16-byte aligned) before storing any, so the copy costs about
// one memory round trip per 4 * 8 * blockDim elements instead of one per
// loop iteration.
__device__ __forceinline__ void stage_halfs(unsigned short *dst, const unsigned short *__restrict__ src, int n) {
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    const int n8 = (reinterpret_cast<uintptr_t>(src) & 15u) == 0 ? (n & ~7) : 0;
    const int stride = 8 * blockDim.x;
    for (int k0 = 8 * threadIdx.x; k0 < n8; k0 += 4 * stride) {
        u32x4_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int k = min(k0 + u * stride, n8 - 8);
            v[u] = *reinterpret_cast<const u32x4_t *>(src + k);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (k0 + u * stride < n8) *reinterpret_cast<u32x4_t *>(dst + k0 + u * stride) = v[u];
    }
    for (int k = n8 + threadIdx.x; k < n; k += blockDim.x) dst[k] = src[k];
}

// Non-temporal loads for streamed matrix data: read once, so keep them from
// evicting the gathered vector from the caches.
template <typename T>
__device__ __forceinline__ T stream_load(const T *p) {
    return __builtin_nontemporal_load(p);
}

}  // namespace spmv
