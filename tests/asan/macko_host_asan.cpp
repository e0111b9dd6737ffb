// Host-side memory check of the library's MACKO encoder and 8-bit
// quantiser, built with AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_asan_host.py compiles and runs it).  Every output buffer is
// allocated with exactly the size the size query reports, so a write one
// element past it is caught.  Inputs: seeded random rows (empty rows,
// entries at the first and last column, gaps far wider than any code span,
// single-entry rows) and the error paths (unsorted, duplicate or
// out-of-range columns, a bad width, negative sizes, a decreasing row
// pointer); outputs are compared bit for bit with the oracle's encoder,
// which is linked in from oracle.c under the same sanitizers.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "spmv.h"

extern "C" {
int64_t oracle_macko_size(int n_rows, int n_cols, int b, const int32_t *rp, const int32_t *ci);
int oracle_macko_encode(int n_rows, int n_cols, int b, const int32_t *rp, const int32_t *ci, const uint16_t *vals,
                        int32_t *mrow_ptr, uint32_t *codes, uint16_t *mvals);
void oracle_macko_quantize_i8(int n_rows, const int32_t *mrow_ptr, const uint16_t *mvals, int8_t *q,
                              float *row_scale);
}

static int failures = 0;
#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            std::fprintf(stderr, "FAIL %s:%d ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);            \
            std::fprintf(stderr, "\n");                   \
            ++failures;                                   \
        }                                                 \
    } while (0)

struct Csr {
    int n_rows, n_cols;
    std::vector<int32_t> rp, ci;
    std::vector<uint16_t> v;
};

static Csr random_csr(std::mt19937_64 &g, int n_rows, int n_cols) {
    Csr A{n_rows, n_cols, {0}, {}, {}};
    std::uniform_int_distribution<int> len_kind(0, 9);
    for (int i = 0; i < n_rows; ++i) {
        std::vector<int32_t> cols;
        const int kind = len_kind(g);
        if (kind == 0) {
            // empty row
        } else if (kind == 1) {
            cols = {0, n_cols - 1};           // first and last column: one huge gap
            if (n_cols == 1) cols = {0};
        } else if (kind == 2) {
            cols = {n_cols - 1};
        } else {
            std::uniform_int_distribution<int> c(0, n_cols - 1);
            const int k = std::min(n_cols, (int)(g() % 40));
            std::vector<char> used(n_cols, 0);
            while ((int)cols.size() < k) {
                const int x = c(g);
                if (!used[x]) used[x] = 1, cols.push_back(x);
            }
            std::sort(cols.begin(), cols.end());
        }
        for (int32_t x : cols) {
            A.ci.push_back(x);
            uint16_t h = (uint16_t)(g() & 0xFFFF);
            if ((h & 0x7C00) == 0x7C00) h &= 0xBFFF;   // no inf / nan
            if ((h & 0x7FFF) == 0) h |= 0x3C00;        // stored values are nonzero
            A.v.push_back(h);
        }
        A.rp.push_back((int32_t)A.ci.size());
    }
    return A;
}

static void check_one(const Csr &A, int b) {
    int64_t E = -1;
    spmv_status s = macko_encode_size(A.n_rows, A.n_cols, b, A.rp.data(), A.ci.data(), &E);
    CHECK(s == SPMV_OK, "size status %d", s);
    const int64_t Eo = oracle_macko_size(A.n_rows, A.n_cols, b, A.rp.data(), A.ci.data());
    CHECK(E == Eo, "entries %lld vs oracle %lld", (long long)E, (long long)Eo);
    if (s != SPMV_OK || E != Eo) return;
    // exact sizes, heap-allocated, so ASan sees any overrun
    std::vector<int32_t> mrp(A.n_rows + 1), omrp(A.n_rows + 1);
    std::vector<uint32_t> codes(E * b / 32), ocodes(E * b / 32);
    std::vector<uint16_t> mv(E), omv(E);
    s = macko_encode(A.n_rows, A.n_cols, b, A.rp.data(), A.ci.data(), A.v.data(), mrp.data(), codes.data(), mv.data());
    CHECK(s == SPMV_OK, "encode status %d", s);
    CHECK(oracle_macko_encode(A.n_rows, A.n_cols, b, A.rp.data(), A.ci.data(), A.v.data(), omrp.data(),
                              ocodes.data(), omv.data()) == 0, "oracle encode failed");
    CHECK(mrp == omrp, "mrow_ptr differs (b=%d)", b);
    CHECK(codes == ocodes, "codes differ (b=%d)", b);
    CHECK(mv == omv, "values differ (b=%d)", b);
    std::vector<int8_t> q(E), oq(E);
    std::vector<float> sc(A.n_rows), osc(A.n_rows);
    s = macko_quantize_i8(A.n_rows, mrp.data(), mv.data(), q.data(), sc.data());
    CHECK(s == SPMV_OK, "quantise status %d", s);
    oracle_macko_quantize_i8(A.n_rows, omrp.data(), omv.data(), oq.data(), osc.data());
    CHECK(q == oq, "int8 values differ (b=%d)", b);
    CHECK(sc.empty() || std::memcmp(sc.data(), osc.data(), sizeof(float) * sc.size()) == 0,
          "row scales differ (b=%d)", b);
}

static void error_paths() {
    const int32_t rp[3] = {0, 2, 3};
    const uint16_t v[3] = {0x3C00, 0x3C00, 0x3C00};
    int64_t E = 0;
    const int32_t unsorted[3] = {5, 2, 1}, dup[3] = {2, 2, 1}, range[3] = {1, 64, 0};
    CHECK(macko_encode_size(2, 64, 4, rp, unsorted, &E) == SPMV_ERR_UNSORTED, "unsorted");
    CHECK(macko_encode_size(2, 64, 4, rp, dup, &E) == SPMV_ERR_UNSORTED, "duplicate");
    CHECK(macko_encode_size(2, 64, 4, rp, range, &E) == SPMV_ERR_INVALID_MATRIX, "out of range");
    CHECK(macko_encode_size(2, 64, 3, rp, range, &E) == SPMV_ERR_INVALID_VALUE, "bad width");
    CHECK(macko_encode_size(-1, 64, 4, rp, range, &E) == SPMV_ERR_INVALID_VALUE, "negative rows");
    const int32_t bad_rp[3] = {0, 3, 2};
    const int32_t ok_cols[3] = {1, 2, 3};
    CHECK(macko_encode_size(2, 64, 4, bad_rp, ok_cols, &E) == SPMV_ERR_INVALID_MATRIX, "decreasing row_ptr");
    int32_t mrp[3];
    uint32_t codes[64];
    uint16_t mv[512];
    CHECK(macko_encode(2, 64, 4, rp, unsorted, v, mrp, codes, mv) == SPMV_ERR_UNSORTED, "encode unsorted");
    const int32_t mrp_bad[3] = {0, 256, 128};
    int8_t q[256];
    float sc[2];
    CHECK(macko_quantize_i8(2, mrp_bad, mv, q, sc) == SPMV_ERR_INVALID_MATRIX, "quantise decreasing mrow_ptr");
    CHECK(std::strlen(spmv_last_error()) > 0, "no error message");
}

int main() {
    std::mt19937_64 g(20261202);
    int cases = 0;
    for (int trial = 0; trial < 60; ++trial) {
        const int n_rows = (int)(g() % 70);              // includes 0 rows
        const int n_cols = 1 + (int)(g() % (trial % 3 == 0 ? 40000 : 600));
        const Csr A = random_csr(g, n_rows, n_cols);
        for (int b : {1, 2, 4, 8}) {
            check_one(A, b);
            ++cases;
        }
    }
    error_paths();
    std::printf("%d encoder cases, %d failures\n", cases, failures);
    return failures ? 1 : 0;
}
