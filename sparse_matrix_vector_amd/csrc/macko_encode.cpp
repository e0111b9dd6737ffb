// MACKO encoder (host side, like the page's offline conversion step).
//
// "MACKO-SpMV: GPU acceleration and storage optimisation at low sparsity",
// section 2.1: column indices become gaps to the previous column (delta
// coding), a gap wider than the code's span is bridged by zero values
// (dynamic padding), codes are packed into 32-bit words, and rows are
// aligned so that every load is a full aligned transaction.  Section 3.3
// makes the code width b one of 1, 2, 4, 8 bits (4 by default) and names
// int8 values as an alternative to fp16.
//
// Format written here (the library's reading of the page), for width b:
//   - per row the previous column starts at -1; an entry with gap g in
//     1..2^b stores code g - 1;
//   - a gap g > 2^b first emits (g - 1) / 2^b padding entries, each code
//     2^b - 1 (gap 2^b) with value +0, so the real entry's gap becomes
//     1..2^b;
//   - each row ends with (code 0, value +0) entries up to a multiple of
//     1024 / b entries: one 128-byte block of codes (with 2048 / b bytes of
//     fp16 values, or 1024 / b bytes of int8 values), so every row begins on
//     a 128-byte code boundary;
//   - entry e's code occupies bits [b (e % (32/b)), b (e % (32/b)) + b - 1]
//     of word e / (32/b).
// 8-bit values (macko_quantize_i8): per row s = max |v| / 127 as an fp32
// division (1 for a row of zeros), q = v / s in double, rounded to nearest
// with ties to even and clamped to [-127, 127]; the value is s * q.
#include "common.hpp"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <thread>
#include <vector>

namespace spmv {
namespace {

bool width_ok(int32_t b) { return b == 1 || b == 2 || b == 4 || b == 8; }

// Entry count of one row after alignment, or -1 with *err set.
int64_t row_entries(const int32_t *col, int32_t len, int32_t n_cols, int32_t bits, spmv_status *err) {
    const int64_t SPAN = int64_t(1) << bits, ROW_ALIGN = 1024 / bits;
    int64_t prev = -1, count = 0;
    for (int32_t k = 0; k < len; ++k) {
        const int64_t c = col[k];
        if (c < 0 || c >= n_cols) {
            *err = SPMV_ERR_INVALID_MATRIX;
            return -1;
        }
        if (c <= prev) {
            *err = SPMV_ERR_UNSORTED;
            return -1;
        }
        count += 1 + (c - prev - 1) / SPAN;   // the entry plus its bridging pads
        prev = c;
    }
    return (count + ROW_ALIGN - 1) / ROW_ALIGN * ROW_ALIGN;
}

int worker_count(int64_t work) {
    unsigned hw = std::thread::hardware_concurrency();
    int64_t w = std::min<int64_t>(hw ? hw : 1, 16);
    return (int)std::max<int64_t>(1, std::min<int64_t>(w, work / 65536 + 1));
}

// Runs f(row_begin, row_end) over [0, n) on a few threads.
template <typename F>
void parallel_rows(int32_t n, int64_t work, F f) {
    const int nt = worker_count(work);
    if (nt == 1 || n < 2 * nt) {
        f(0, n);
        return;
    }
    std::vector<std::thread> th;
    for (int t = 0; t < nt; ++t) {
        const int32_t a = (int32_t)((int64_t)n * t / nt), b = (int32_t)((int64_t)n * (t + 1) / nt);
        th.emplace_back([=] { f(a, b); });
    }
    for (auto &x : th) x.join();
}

spmv_status count_rows(int32_t n_rows, int32_t n_cols, int32_t bits, const int32_t *rp, const int32_t *col,
                       std::vector<int64_t> &counts, int64_t *total) {
    if (rp[0] != 0) return fail(SPMV_ERR_INVALID_MATRIX, "row_ptr[0] != 0");
    for (int32_t i = 0; i < n_rows; ++i)
        if (rp[i + 1] < rp[i]) return fail(SPMV_ERR_INVALID_MATRIX, "row_ptr decreases at row %d", i);
    counts.assign(n_rows, 0);
    std::atomic<int> bad{0};
    std::atomic<int32_t> bad_row{-1};
    parallel_rows(n_rows, rp[n_rows], [&](int32_t a, int32_t b) {
        for (int32_t i = a; i < b && !bad.load(std::memory_order_relaxed); ++i) {
            spmv_status e = SPMV_OK;
            const int64_t c = row_entries(col + rp[i], rp[i + 1] - rp[i], n_cols, bits, &e);
            if (c < 0) {
                int expected = 0;
                if (bad.compare_exchange_strong(expected, (int)e)) bad_row.store(i);
                return;
            }
            counts[i] = c;
        }
    });
    if (bad.load()) {
        const int r = bad_row.load();
        if (bad.load() == SPMV_ERR_UNSORTED)
            return fail(SPMV_ERR_UNSORTED, "row %d: columns are not strictly increasing", r);
        return fail(SPMV_ERR_INVALID_MATRIX, "row %d: a column is outside [0, %d)", r, n_cols);
    }
    int64_t t = 0;
    for (int32_t i = 0; i < n_rows; ++i) t += counts[i];
    if (t > INT32_MAX) return fail(SPMV_ERR_OVERFLOW, "%lld encoded entries exceed int32", (long long)t);
    *total = t;
    return SPMV_OK;
}

}  // namespace
}  // namespace spmv

using namespace spmv;

extern "C" spmv_status macko_encode_size(int32_t n_rows, int32_t n_cols, int32_t bdelta, const int32_t *h_row_ptr,
                                         const int32_t *h_col, int64_t *n_entries) {
    if (!n_entries) return fail(SPMV_ERR_INVALID_VALUE, "n_entries is NULL");
    if (n_rows < 0 || n_cols < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if (!width_ok(bdelta)) return fail(SPMV_ERR_INVALID_VALUE, "code width %d is not 1, 2, 4 or 8", bdelta);
    if (!h_row_ptr) return fail(SPMV_ERR_INVALID_VALUE, "row_ptr is NULL");
    if (n_rows > 0 && h_row_ptr[n_rows] > 0 && !h_col) return fail(SPMV_ERR_INVALID_VALUE, "col is NULL");
    std::vector<int64_t> counts;
    int64_t total = 0;
    spmv_status s = count_rows(n_rows, n_cols, bdelta, h_row_ptr, h_col, counts, &total);
    if (s != SPMV_OK) return s;
    *n_entries = total;
    return SPMV_OK;
}

extern "C" spmv_status macko_encode(int32_t n_rows, int32_t n_cols, int32_t bdelta, const int32_t *h_row_ptr,
                                    const int32_t *h_col, const uint16_t *h_vals_f16, int32_t *h_mrow_ptr,
                                    uint32_t *h_codes, uint16_t *h_mvals) {
    if (n_rows < 0 || n_cols < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if (!width_ok(bdelta)) return fail(SPMV_ERR_INVALID_VALUE, "code width %d is not 1, 2, 4 or 8", bdelta);
    if (!h_row_ptr || !h_mrow_ptr) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    const int32_t nnz = n_rows > 0 ? h_row_ptr[n_rows] : 0;
    if (nnz > 0 && (!h_col || !h_vals_f16)) return fail(SPMV_ERR_INVALID_VALUE, "col or vals is NULL");
    std::vector<int64_t> counts;
    int64_t total = 0;
    spmv_status s = count_rows(n_rows, n_cols, bdelta, h_row_ptr, h_col, counts, &total);
    if (s != SPMV_OK) return s;
    if (total > 0 && (!h_codes || !h_mvals)) return fail(SPMV_ERR_INVALID_VALUE, "codes or mvals is NULL");
    int64_t at = 0;
    for (int32_t i = 0; i < n_rows; ++i) {
        h_mrow_ptr[i] = (int32_t)at;
        at += counts[i];
    }
    h_mrow_ptr[n_rows] = (int32_t)at;
    const int bits = bdelta, per_word = 32 / bdelta;
    const int64_t span = int64_t(1) << bits;
    // Each row starts on a 128-byte code boundary, so rows own disjoint code
    // words and can be filled independently.
    parallel_rows(n_rows, total, [&](int32_t a, int32_t b) {
        for (int32_t i = a; i < b; ++i) {
            const int64_t e_begin = h_mrow_ptr[i], e_end = h_mrow_ptr[i + 1];
            std::fill(h_codes + e_begin / per_word, h_codes + e_end / per_word, 0u);
            int64_t e = e_begin, prev = -1;
            auto emit = [&](uint32_t code, uint16_t val) {
                h_codes[e / per_word] |= code << (bits * (int)(e % per_word));
                h_mvals[e] = val;
                ++e;
            };
            for (int32_t k = h_row_ptr[i]; k < h_row_ptr[i + 1]; ++k) {
                const int64_t gap = (int64_t)h_col[k] - prev;
                const int64_t pads = (gap - 1) / span;
                for (int64_t p = 0; p < pads; ++p) emit((uint32_t)(span - 1), 0);
                emit((uint32_t)(gap - 1 - pads * span), h_vals_f16[k]);
                prev = h_col[k];
            }
            while (e < e_end) emit(0u, 0);
        }
    });
    return SPMV_OK;
}

extern "C" spmv_status macko_quantize_i8(int32_t n_rows, const int32_t *h_mrow_ptr, const uint16_t *h_mvals,
                                         int8_t *h_q, float *h_row_scale) {
    if (n_rows < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if (n_rows == 0) return SPMV_OK;
    if (!h_mrow_ptr || !h_row_scale) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    if (h_mrow_ptr[0] != 0) return fail(SPMV_ERR_INVALID_MATRIX, "mrow_ptr[0] != 0");
    for (int32_t i = 0; i < n_rows; ++i)
        if (h_mrow_ptr[i + 1] < h_mrow_ptr[i]) return fail(SPMV_ERR_INVALID_MATRIX, "mrow_ptr decreases at row %d", i);
    const int64_t total = h_mrow_ptr[n_rows];
    if (total > 0 && (!h_mvals || !h_q)) return fail(SPMV_ERR_INVALID_VALUE, "mvals or q is NULL");
    parallel_rows(n_rows, total, [&](int32_t a, int32_t b) {
        for (int32_t i = a; i < b; ++i) {
            const int32_t e0 = h_mrow_ptr[i], e1 = h_mrow_ptr[i + 1];
            float m = 0.0f;   // fp16 -> fp32 is exact
            for (int32_t e = e0; e < e1; ++e)
                m = std::max(m, std::fabs((float)__builtin_bit_cast(_Float16, h_mvals[e])));
            const float s = m > 0.0f ? m / 127.0f : 1.0f;
            h_row_scale[i] = s;
            for (int32_t e = e0; e < e1; ++e) {
                const double r = std::nearbyint((double)__builtin_bit_cast(_Float16, h_mvals[e]) / (double)s);
                h_q[e] = (int8_t)std::min(127.0, std::max(-127.0, r));
            }
        }
    });
    return SPMV_OK;
}
