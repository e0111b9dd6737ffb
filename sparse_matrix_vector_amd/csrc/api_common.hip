// Error reporting, device queries and the host-only format rule.
#include "common.hpp"

#include <string>

namespace spmv {

namespace {
thread_local std::string g_last_error;
}

void set_error(const char *fmt, ...) {
    char buf[1024];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
}

void clear_error() { g_last_error.clear(); }

int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

spmv_status check_scratch(const void *scratch, size_t bytes, int64_t n_rows) {
    const size_t need = scratch_bytes(n_rows);
    if (!scratch) return fail(SPMV_ERR_INVALID_VALUE, "scratch is NULL (spmv_scratch_size gives its size)");
    if (reinterpret_cast<uintptr_t>(scratch) & 255u) return fail(SPMV_ERR_INVALID_VALUE, "scratch must be 256-byte aligned");
    if (bytes < need) return fail(SPMV_ERR_INVALID_VALUE, "scratch of %zu bytes is smaller than %zu", bytes, need);
    return SPMV_OK;
}

}  // namespace spmv

extern "C" const char *spmv_last_error(void) { return spmv::g_last_error.c_str(); }

extern "C" spmv_status spmv_scratch_size(int32_t n_rows, size_t *bytes) {
    if (!bytes) return spmv::fail(SPMV_ERR_INVALID_VALUE, "bytes is NULL");
    if (n_rows < 0) return spmv::fail(SPMV_ERR_INVALID_VALUE, "n_rows < 0");
    *bytes = spmv::scratch_bytes(n_rows);
    return SPMV_OK;
}

// Coefficient-of-variation rule ("Why SpMV needs CUDA optimisation", section
// 2.2) in exact integer arithmetic: with S1 = sum of lengths, S2 = sum of
// squares, CV^2 = (n S2 - S1^2) / S1^2, so CV < 0.3 <=> 100 (n S2 - S1^2) <
// 9 S1^2 and CV <= 0.7 <=> 100 (n S2 - S1^2) <= 49 S1^2.
extern "C" spmv_status spmv_format_recommend(int64_t n_rows, int64_t sum_len,
                                             int64_t sum_len_sq, int32_t *format) {
    if (!format) return spmv::fail(SPMV_ERR_INVALID_VALUE, "format is NULL");
    if (n_rows < 0 || sum_len < 0 || sum_len_sq < 0)
        return spmv::fail(SPMV_ERR_INVALID_VALUE, "negative statistics");
    if (n_rows == 0 || sum_len == 0) {
        *format = SPMV_FORMAT_CSR;
        return SPMV_OK;
    }
    __int128 spread = (__int128)n_rows * sum_len_sq - (__int128)sum_len * sum_len;
    __int128 mean_sq = (__int128)sum_len * sum_len;
    if (spread < 0) return spmv::fail(SPMV_ERR_INVALID_VALUE, "inconsistent statistics");
    if (100 * spread < 9 * mean_sq)
        *format = SPMV_FORMAT_ELL;
    else if (100 * spread <= 49 * mean_sq)
        *format = SPMV_FORMAT_HYB;
    else
        *format = SPMV_FORMAT_CSR;
    return SPMV_OK;
}
