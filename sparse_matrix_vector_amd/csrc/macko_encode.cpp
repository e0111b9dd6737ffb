// MACKO encoder (host side, like the page's offline conversion step).
//
// "MACKO-SpMV: GPU acceleration and storage optimisation at low sparsity",
// section 2.1: column indices become gaps to the previous column (delta
// coding), a gap wider than the 4-bit code's span of 16 is bridged by zero
// values (dynamic padding), codes are packed eight to a 32-bit word, and
// rows are aligned so that every load is a full aligned transaction.
//
// Format written here (the library's reading of the page):
//   - per row the previous column starts at -1; an entry with gap g in 1..16
//     stores code g - 1;
//   - a gap g > 16 first emits (g - 1) / 16 padding entries, each code 15
//     (gap 16) with value +0, so the real entry's gap becomes 1..16;
//   - each row ends with (code 0, value +0) entries up to a multiple of 256
//     entries: 128 bytes of codes and 512 bytes of values per 256 entries,
//     so every row begins on a 128-byte code boundary and a 512-byte value
//     boundary, and a wave's 512-entry chunk is two such units;
//   - entry e's code occupies bits [4 (e % 8), 4 (e % 8) + 3] of word e / 8.
#include "common.hpp"

#include <algorithm>
#include <atomic>
#include <thread>
#include <vector>

namespace spmv {
namespace {

constexpr int64_t ROW_ALIGN = 256;
constexpr int64_t SPAN = 16;

// Entry count of one row before alignment, or a negative status.
int64_t row_entries(const int32_t *col, int32_t len, int32_t n_cols, spmv_status *err) {
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

spmv_status count_rows(int32_t n_rows, int32_t n_cols, const int32_t *rp, const int32_t *col,
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
            const int64_t c = row_entries(col + rp[i], rp[i + 1] - rp[i], n_cols, &e);
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

extern "C" spmv_status macko_encode_size(int32_t n_rows, int32_t n_cols, const int32_t *h_row_ptr,
                                         const int32_t *h_col, int64_t *n_entries) {
    if (!n_entries) return fail(SPMV_ERR_INVALID_VALUE, "n_entries is NULL");
    if (n_rows < 0 || n_cols < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if (!h_row_ptr) return fail(SPMV_ERR_INVALID_VALUE, "row_ptr is NULL");
    if (n_rows > 0 && h_row_ptr[n_rows] > 0 && !h_col) return fail(SPMV_ERR_INVALID_VALUE, "col is NULL");
    std::vector<int64_t> counts;
    int64_t total = 0;
    spmv_status s = count_rows(n_rows, n_cols, h_row_ptr, h_col, counts, &total);
    if (s != SPMV_OK) return s;
    *n_entries = total;
    return SPMV_OK;
}

extern "C" spmv_status macko_encode(int32_t n_rows, int32_t n_cols, const int32_t *h_row_ptr,
                                    const int32_t *h_col, const uint16_t *h_vals_f16, int32_t *h_mrow_ptr,
                                    uint32_t *h_codes, uint16_t *h_mvals) {
    if (n_rows < 0 || n_cols < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if (!h_row_ptr || !h_mrow_ptr) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    const int32_t nnz = n_rows > 0 ? h_row_ptr[n_rows] : 0;
    if (nnz > 0 && (!h_col || !h_vals_f16)) return fail(SPMV_ERR_INVALID_VALUE, "col or vals is NULL");
    std::vector<int64_t> counts;
    int64_t total = 0;
    spmv_status s = count_rows(n_rows, n_cols, h_row_ptr, h_col, counts, &total);
    if (s != SPMV_OK) return s;
    if (total > 0 && (!h_codes || !h_mvals)) return fail(SPMV_ERR_INVALID_VALUE, "codes or mvals is NULL");
    int64_t at = 0;
    for (int32_t i = 0; i < n_rows; ++i) {
        h_mrow_ptr[i] = (int32_t)at;
        at += counts[i];
    }
    h_mrow_ptr[n_rows] = (int32_t)at;
    // Each row starts on a 256-entry boundary, so rows own disjoint code
    // words and can be filled independently.
    parallel_rows(n_rows, total, [&](int32_t a, int32_t b) {
        for (int32_t i = a; i < b; ++i) {
            const int64_t e_begin = h_mrow_ptr[i], e_end = h_mrow_ptr[i + 1];
            std::fill(h_codes + e_begin / 8, h_codes + e_end / 8, 0u);
            int64_t e = e_begin, prev = -1;
            auto emit = [&](uint32_t code, uint16_t val) {
                h_codes[e >> 3] |= code << (4 * (e & 7));
                h_mvals[e] = val;
                ++e;
            };
            for (int32_t k = h_row_ptr[i]; k < h_row_ptr[i + 1]; ++k) {
                const int64_t gap = (int64_t)h_col[k] - prev;
                const int64_t pads = (gap - 1) / SPAN;
                for (int64_t p = 0; p < pads; ++p) emit((uint32_t)(SPAN - 1), 0);
                emit((uint32_t)(gap - 1 - pads * SPAN), h_vals_f16[k]);
                prev = h_col[k];
            }
            while (e < e_end) emit(0u, 0);
        }
    });
    return SPMV_OK;
}
