/*
 * CPU oracle for the SpMV library -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, serial, obviously-correct C with fp64 accumulation.  It is called
 * only by the tests, by the smoke check and by the bench's CPU-baseline leg;
 * the library (HIP kernels + C-ABI) never links, includes or calls it, and it
 * shares no source with the library.
 *
 * Each function follows one passage of the source pages (cited by page title
 * and section) or the plain mathematical definition of the operation.  Where
 * a page is silent or garbled, the reading taken is stated at the function.
 *
 * Value outputs come with a per-row error scale
 *     scale_i = |alpha| * sum_k |a_ik * x_k| + |beta * y_in_i|
 * so that a tolerance of the form |y_gpu - y_ref| <= tau * scale_i can be
 * checked by the caller.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16 -> binary64, decoded field by field (exact).           */
/* ------------------------------------------------------------------------ */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int mant = h & 0x3ff;
    double v;
    if (expo == 0)            /* zero or subnormal: mant * 2^-24 */
        v = ldexp((double)mant, -24);
    else if (expo == 31)      /* inf or nan */
        v = mant ? NAN : INFINITY;
    else                      /* normal: (1024 + mant) * 2^(expo - 25) */
        v = ldexp((double)(1024 + mant), expo - 25);
    return sign ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* CSR SpMV.  "Why SpMV needs CUDA optimisation", section 2.1 (scalar CSR   */
/* kernel: dot += values[i] * x[col_idx[i]] over the row's range) and       */
/* section 4.1 (warp-per-row form computes the same sum).  The product is   */
/* y = alpha*A*x + beta*y; y_in is not read when beta == 0.                 */
/* Duplicate columns are summed; the sum runs in storage order.             */
/* ------------------------------------------------------------------------ */
void oracle_csr_spmv(int n_rows, const int32_t *rp, const int32_t *ci,
                     const float *v, const float *x, double alpha, double beta,
                     const float *y_in, double *y_out, double *scale)
{
    for (int i = 0; i < n_rows; ++i) {
        double s = 0.0, a = 0.0;
        for (int32_t k = rp[i]; k < rp[i + 1]; ++k) {
            double p = (double)v[k] * (double)x[ci[k]];
            s += p;
            a += fabs(p);
        }
        double yi = alpha * s;
        double sc = fabs(alpha) * a;
        if (beta != 0.0) {
            yi += beta * (double)y_in[i];
            sc += fabs(beta * (double)y_in[i]);
        }
        y_out[i] = yi;
        if (scale) scale[i] = sc;
    }
}

/* Same definition with fp64 matrix values (used for the assembled FE form). */
void oracle_csr_spmv_f64(int n_rows, const int32_t *rp, const int32_t *ci,
                         const double *v, const float *x, double alpha, double beta,
                         const float *y_in, double *y_out, double *scale)
{
    for (int i = 0; i < n_rows; ++i) {
        double s = 0.0, a = 0.0;
        for (int32_t k = rp[i]; k < rp[i + 1]; ++k) {
            double p = v[k] * (double)x[ci[k]];
            s += p;
            a += fabs(p);
        }
        double yi = alpha * s, sc = fabs(alpha) * a;
        if (beta != 0.0) {
            yi += beta * (double)y_in[i];
            sc += fabs(beta * (double)y_in[i]);
        }
        y_out[i] = yi;
        if (scale) scale[i] = sc;
    }
}

/* The same definition with fp64 values and an fp64 vector, alpha = 1 and
 * beta = 0: y = A x, each row summed in storage order (the matvec of the
 * fp64 reference solver on the assembled FE operator). */
void oracle_csr_spmv_f64v(int n_rows, const int32_t *rp, const int32_t *ci,
                          const double *v, const double *x, double *y_out)
{
    for (int i = 0; i < n_rows; ++i) {
        double s = 0.0;
        for (int32_t k = rp[i]; k < rp[i + 1]; ++k) s += v[k] * x[ci[k]];
        y_out[i] = s;
    }
}

/* ------------------------------------------------------------------------ */
/* Row statistics: max row length, sum and sum of squares (int64).          */
/* ------------------------------------------------------------------------ */
void oracle_row_stats(int n_rows, const int32_t *rp, int32_t *max_len,
                      int64_t *sum_len, int64_t *sum_len_sq)
{
    int32_t m = 0;
    int64_t s = 0, q = 0;
    for (int i = 0; i < n_rows; ++i) {
        int32_t len = rp[i + 1] - rp[i];
        if (len > m) m = len;
        s += len;
        q += (int64_t)len * len;
    }
    *max_len = m;
    *sum_len = s;
    *sum_len_sq = q;
}

/* ------------------------------------------------------------------------ */
/* Row grouping ("Sparse matrix multiplication acceleration", section 2.1.1 */
/* grouping table and the Map[] indirection of section 2.2.1).  For SpMV    */
/* the dense operand is an n x 1 vector, so a row's count of intermediate   */
/* products equals its nonzero count.  Group g holds rows with             */
/* t[g-1] <= len < t[g] (t[-1] = 0, t[3] = infinity); the page's table      */
/* gives t = {32, 512, 8192}.  perm lists rows group by group, ascending     */
/* row id inside a group (a stable counting sort); bin_offsets[g] is the    */
/* position of group g's first row in perm, bin_offsets[4] = n_rows.        */
/* ------------------------------------------------------------------------ */
int oracle_row_bin(int32_t len, const int32_t *t)
{
    if (len < t[0]) return 0;
    if (len < t[1]) return 1;
    if (len < t[2]) return 2;
    return 3;
}

void oracle_bins(int n_rows, const int32_t *rp, const int32_t *t,
                 int32_t *bin_offsets, int32_t *perm)
{
    int32_t count[4] = {0, 0, 0, 0};
    for (int i = 0; i < n_rows; ++i)
        count[oracle_row_bin(rp[i + 1] - rp[i], t)]++;
    bin_offsets[0] = 0;
    for (int g = 0; g < 4; ++g)
        bin_offsets[g + 1] = bin_offsets[g] + count[g];
    int32_t next[4];
    for (int g = 0; g < 4; ++g) next[g] = bin_offsets[g];
    for (int i = 0; i < n_rows; ++i) {
        int g = oracle_row_bin(rp[i + 1] - rp[i], t);
        perm[next[g]++] = i;
    }
}

/* ------------------------------------------------------------------------ */
/* Format choice by coefficient of variation of row lengths ("Why SpMV     */
/* needs CUDA optimisation", section 2.2): CV < 0.3 -> ELL,                 */
/* 0.3 <= CV <= 0.7 -> HYB, CV > 0.7 -> CSR with row reordering.            */
/* Reading: population standard deviation; the comparisons are done         */
/* exactly in integers, CV^2 = (n*S2 - S1^2) / S1^2; an undefined CV        */
/* (n == 0 or S1 == 0) picks CSR.  Returns 0 = ELL, 1 = HYB, 2 = CSR.       */
/* ------------------------------------------------------------------------ */
int oracle_format_choice(int64_t n, int64_t s1, int64_t s2)
{
    if (n <= 0 || s1 <= 0) return 2;
    __int128 num = (__int128)n * s2 - (__int128)s1 * s1;
    __int128 den = (__int128)s1 * s1;
    if (100 * num < 9 * den) return 0;
    if (100 * num <= 49 * den) return 1;
    return 2;
}

/* ------------------------------------------------------------------------ */
/* ELL ("Why SpMV needs CUDA optimisation", section 2.1 table: fixed width, */
/* zero padding).  Reading: width W >= the longest row, slot-major layout   */
/* ell[k*n + i]; a padding slot holds column -1 and value +0.0f and is       */
/* skipped by the product.  Returns 0, or -1 when a row is longer than W.   */
/* ------------------------------------------------------------------------ */
int oracle_ell_from_csr(int n_rows, const int32_t *rp, const int32_t *ci,
                        const float *v, int W, int32_t *ell_col, float *ell_val)
{
    for (int i = 0; i < n_rows; ++i)
        if (rp[i + 1] - rp[i] > W) return -1;
    for (int k = 0; k < W; ++k) {
        for (int i = 0; i < n_rows; ++i) {
            int32_t len = rp[i + 1] - rp[i];
            size_t slot = (size_t)k * (size_t)n_rows + (size_t)i;
            if (k < len) {
                ell_col[slot] = ci[rp[i] + k];
                ell_val[slot] = v[rp[i] + k];
            } else {
                ell_col[slot] = -1;
                ell_val[slot] = 0.0f;
            }
        }
    }
    return 0;
}

void oracle_ell_spmv(int n_rows, int W, const int32_t *ell_col, const float *ell_val,
                     const float *x, double alpha, double beta, const float *y_in,
                     double *y_out, double *scale)
{
    for (int i = 0; i < n_rows; ++i) {
        double s = 0.0, a = 0.0;
        for (int k = 0; k < W; ++k) {
            size_t slot = (size_t)k * (size_t)n_rows + (size_t)i;
            if (ell_col[slot] < 0) continue;
            double p = (double)ell_val[slot] * (double)x[ell_col[slot]];
            s += p;
            a += fabs(p);
        }
        double yi = alpha * s, sc = fabs(alpha) * a;
        if (beta != 0.0) {
            yi += beta * (double)y_in[i];
            sc += fabs(beta * (double)y_in[i]);
        }
        y_out[i] = yi;
        if (scale) scale[i] = sc;
    }
}

/* ------------------------------------------------------------------------ */
/* HYB ("Why SpMV needs CUDA optimisation", section 2.1 table: a mixed       */
/* CSR + ELL format; section 2.2: used when the row-length CV is between    */
/* 0.3 and 0.7; section 5: a tuned example splits the storage 0.7 ELL to    */
/* 0.3 COO).  Readings taken where the page is silent:                      */
/*  - the ELL part holds the first min(len_i, W) entries of every row, in    */
/*    the slot-major ELL layout above (-1 / +0 padding);                     */
/*  - the remaining entries of each row form the tail, a CSR over only the  */
/*    rows that have one: tail_rows[t] (ascending row ids), tail_rp[t] ..    */
/*    tail_rp[t+1] into tail_col / tail_val, in the row's storage order;    */
/*  - W is the smallest width whose ELL part holds at least the fraction    */
/*    num/den of the nonzeros: den * sum_i min(len_i, W) >= num * nnz        */
/*    (exact integers; W = 0 when nnz == 0).                                 */
/* ------------------------------------------------------------------------ */
static long long hyb_ell_count(int n_rows, const int32_t *rp, int W)
{
    long long c = 0;
    for (int i = 0; i < n_rows; ++i) {
        int32_t len = rp[i + 1] - rp[i];
        c += len < W ? len : W;
    }
    return c;
}

int oracle_hyb_width(int n_rows, const int32_t *rp, int num, int den)
{
    long long nnz = n_rows > 0 ? (long long)rp[n_rows] - rp[0] : 0;
    int W = 0;
    /* the smallest W that satisfies the rule, by counting upwards */
    while ((long long)den * hyb_ell_count(n_rows, rp, W) < (long long)num * nnz) ++W;
    return W;
}

/* Sizes of the tail for width W: rows with len > W and their entries past W. */
void oracle_hyb_tail_size(int n_rows, const int32_t *rp, int W, int *n_tail_rows, long long *tail_nnz)
{
    int r = 0;
    long long t = 0;
    for (int i = 0; i < n_rows; ++i) {
        int32_t len = rp[i + 1] - rp[i];
        if (len > W) {
            ++r;
            t += len - W;
        }
    }
    *n_tail_rows = r;
    *tail_nnz = t;
}

void oracle_hyb_from_csr(int n_rows, const int32_t *rp, const int32_t *ci, const float *v, int W,
                         int32_t *ell_col, float *ell_val, int32_t *tail_rows, int32_t *tail_rp,
                         int32_t *tail_col, float *tail_val)
{
    for (int k = 0; k < W; ++k) {
        for (int i = 0; i < n_rows; ++i) {
            int32_t len = rp[i + 1] - rp[i];
            size_t slot = (size_t)k * (size_t)n_rows + (size_t)i;
            if (k < len) {
                ell_col[slot] = ci[rp[i] + k];
                ell_val[slot] = v[rp[i] + k];
            } else {
                ell_col[slot] = -1;
                ell_val[slot] = 0.0f;
            }
        }
    }
    int t = 0;
    int32_t pos = 0;
    tail_rp[0] = 0;
    for (int i = 0; i < n_rows; ++i) {
        int32_t len = rp[i + 1] - rp[i];
        if (len <= W) continue;
        tail_rows[t] = i;
        for (int32_t k = W; k < len; ++k) {
            tail_col[pos] = ci[rp[i] + k];
            tail_val[pos] = v[rp[i] + k];
            ++pos;
        }
        ++t;
        tail_rp[t] = pos;
    }
}

/* Row i's ELL slots in slot order, then its tail entries: the row's storage
   order, so the sum equals the CSR definition term by term. */
void oracle_hyb_spmv(int n_rows, int W, const int32_t *ell_col, const float *ell_val,
                     int n_tail_rows, const int32_t *tail_rows, const int32_t *tail_rp,
                     const int32_t *tail_col, const float *tail_val, const float *x,
                     double alpha, double beta, const float *y_in, double *y_out, double *scale)
{
    int t = 0;
    for (int i = 0; i < n_rows; ++i) {
        double s = 0.0, a = 0.0;
        for (int k = 0; k < W; ++k) {
            size_t slot = (size_t)k * (size_t)n_rows + (size_t)i;
            if (ell_col[slot] < 0) continue;
            double p = (double)ell_val[slot] * (double)x[ell_col[slot]];
            s += p;
            a += fabs(p);
        }
        if (t < n_tail_rows && tail_rows[t] == i) {
            for (int32_t k = tail_rp[t]; k < tail_rp[t + 1]; ++k) {
                double p = (double)tail_val[k] * (double)x[tail_col[k]];
                s += p;
                a += fabs(p);
            }
            ++t;
        }
        double yi = alpha * s, sc = fabs(alpha) * a;
        if (beta != 0.0) {
            yi += beta * (double)y_in[i];
            sc += fabs(beta * (double)y_in[i]);
        }
        y_out[i] = yi;
        if (scale) scale[i] = sc;
    }
}

/* ------------------------------------------------------------------------ */
/* MACKO format ("MACKO-SpMV: GPU acceleration and storage optimisation at  */
/* low sparsity", section 2.1: delta coding, dynamic zero padding, packing   */
/* of the codes into 32-bit words, aligned loads; section 3.3: the code      */
/* width b (the page's b-delta) is one of 1, 2, 4, 8, default 4).  Readings  */
/* taken where the page is silent or self-contradictory:                     */
/*  - a row starts at previous column -1, every stored entry has a column    */
/*    gap g = col - prev in 1..2^b and code g-1 in 0..2^b-1 (the page: a     */
/*    4-bit delta spans at most 16);                                         */
/*  - a gap larger than 2^b is bridged by zero-valued padding entries placed */
/*    2^b columns after the previous entry (code 2^b-1, value +0);           */
/*  - each row is then padded with (code 0, value +0) entries to a multiple  */
/*    of 1024/b entries, i.e. whole 128-byte blocks of codes (256 entries at */
/*    b = 4, where 128 B of codes go with 512 B of fp16 values);             */
/*  - entry e's code is field (e % (32/b)) of word e / (32/b), fields of b   */
/*    bits, least significant field first.                                   */
/* Columns must be strictly increasing in each row and lie in [0, n_cols).  */
/* ------------------------------------------------------------------------ */
static int oracle_macko_bits_ok(int b)
{
    return b == 1 || b == 2 || b == 4 || b == 8;
}

static int64_t oracle_macko_row_entries(const int32_t *cols, int32_t len, int b)
{
    const int64_t span = (int64_t)1 << b, align = 1024 / b;
    int64_t count = 0;
    int64_t prev = -1;
    for (int32_t k = 0; k < len; ++k) {
        int64_t g = (int64_t)cols[k] - prev;
        while (g > span) {                    /* one padding entry per span */
            count++;
            prev += span;
            g -= span;
        }
        count++;
        prev = cols[k];
    }
    int64_t rem = count % align;
    if (rem) count += align - rem;
    return count;
}

/* Total encoded entries, -1 for unsorted/duplicate/out-of-range columns, -2
 * for a code width other than 1, 2, 4, 8. */
int64_t oracle_macko_size(int n_rows, int n_cols, int b, const int32_t *rp, const int32_t *ci)
{
    if (!oracle_macko_bits_ok(b)) return -2;
    int64_t total = 0;
    for (int i = 0; i < n_rows; ++i) {
        for (int32_t k = rp[i]; k < rp[i + 1]; ++k) {
            if (ci[k] < 0 || ci[k] >= n_cols) return -1;
            if (k > rp[i] && ci[k] <= ci[k - 1]) return -1;
        }
        total += oracle_macko_row_entries(ci + rp[i], rp[i + 1] - rp[i], b);
    }
    return total;
}

static uint32_t oracle_macko_code(const uint32_t *codes, int64_t e, int b)
{
    const int per_word = 32 / b;
    return (codes[e / per_word] >> (b * (e % per_word))) & (((uint32_t)1 << b) - 1u);
}

static void oracle_macko_put(uint32_t *codes, uint16_t *mvals, int64_t e, int b,
                             uint32_t code, uint16_t val)
{
    const int per_word = 32 / b;
    codes[e / per_word] |= code << (b * (e % per_word));
    mvals[e] = val;
}

/* Fills mrow_ptr[n_rows+1] (entry offsets), codes[E*b/32] and mvals[E]
 * (fp16 bits).  Returns 0, or -1 on invalid columns or code width. */
int oracle_macko_encode(int n_rows, int n_cols, int b, const int32_t *rp, const int32_t *ci,
                        const uint16_t *vals, int32_t *mrow_ptr, uint32_t *codes,
                        uint16_t *mvals)
{
    int64_t total = oracle_macko_size(n_rows, n_cols, b, rp, ci);
    if (total < 0 || total > INT32_MAX) return -1;
    const int64_t span = (int64_t)1 << b, align = 1024 / b;
    if (total > 0) memset(codes, 0, (size_t)(total * b / 32) * sizeof(uint32_t));
    int64_t e = 0;
    for (int i = 0; i < n_rows; ++i) {
        mrow_ptr[i] = (int32_t)e;
        int64_t row_begin = e;
        int64_t prev = -1;
        for (int32_t k = rp[i]; k < rp[i + 1]; ++k) {
            int64_t g = (int64_t)ci[k] - prev;
            while (g > span) {
                oracle_macko_put(codes, mvals, e++, b, (uint32_t)(span - 1), 0);
                prev += span;
                g -= span;
            }
            oracle_macko_put(codes, mvals, e++, b, (uint32_t)(g - 1), vals[k]);
            prev = ci[k];
        }
        while ((e - row_begin) % align)
            oracle_macko_put(codes, mvals, e++, b, 0, 0);
    }
    mrow_ptr[n_rows] = (int32_t)e;
    return 0;
}

/* Column of every stored entry: restart at -1 per row, col = prev + code + 1. */
void oracle_macko_decode(int n_rows, int b, const int32_t *mrow_ptr, const uint32_t *codes,
                         int32_t *cols)
{
    for (int i = 0; i < n_rows; ++i) {
        int64_t prev = -1;
        for (int64_t e = mrow_ptr[i]; e < mrow_ptr[i + 1]; ++e) {
            prev = prev + (int64_t)oracle_macko_code(codes, e, b) + 1;
            cols[e] = (int32_t)prev;
        }
    }
}

/* MACKO SpMV (section 2.2): y_i = alpha * sum over the row's stored entries
 * of value * x[col] + beta * y_i, with fp16 values and fp16 x taken exactly
 * into fp64.  Trailing alignment entries may decode to a column >= n_cols;
 * they hold +0 and are skipped. */
void oracle_macko_spmv(int n_rows, int n_cols, int b, const int32_t *mrow_ptr,
                       const uint32_t *codes, const uint16_t *mvals,
                       const uint16_t *x, double alpha, double beta,
                       const float *y_in, double *y_out, double *scale)
{
    for (int i = 0; i < n_rows; ++i) {
        double s = 0.0, a = 0.0;
        int64_t prev = -1;
        for (int64_t e = mrow_ptr[i]; e < mrow_ptr[i + 1]; ++e) {
            prev = prev + (int64_t)oracle_macko_code(codes, e, b) + 1;
            if (prev >= n_cols) continue;
            double p = oracle_half_to_double(mvals[e]) * oracle_half_to_double(x[prev]);
            s += p;
            a += fabs(p);
        }
        double yi = alpha * s, sc = fabs(alpha) * a;
        if (beta != 0.0) {
            yi += beta * (double)y_in[i];
            sc += fabs(beta * (double)y_in[i]);
        }
        y_out[i] = yi;
        if (scale) scale[i] = sc;
    }
}

/* ------------------------------------------------------------------------ */
/* MACKO 8-bit value mode (the MACKO-SpMV page, section 3.3 names int8      */
/* values for some layers; section 5 lists an 8-bit mode).  The page does   */
/* not say how the int8 values are scaled.  Reading: symmetric per-row      */
/* scaling, the plainest form of int8 weight quantisation:                   */
/*   m_i     = max |v| over the row's stored fp16 values (exact);            */
/*   s_i     = m_i / 127 as a correctly rounded fp32 division (1 if m_i = 0);*/
/*   q_e     = v_e / s_i in fp64, rounded to the nearest integer with ties   */
/*             to even, clamped to [-127, 127];                              */
/* the value of entry e is then s_i * q_e.  Pads stay 0.                     */
/* ------------------------------------------------------------------------ */
void oracle_macko_quantize_i8(int n_rows, const int32_t *mrow_ptr, const uint16_t *mvals,
                              int8_t *q, float *row_scale)
{
    for (int i = 0; i < n_rows; ++i) {
        double m = 0.0;
        for (int64_t e = mrow_ptr[i]; e < mrow_ptr[i + 1]; ++e) {
            double v = fabs(oracle_half_to_double(mvals[e]));
            if (v > m) m = v;
        }
        /* (float)m is exact: m is an fp16 value */
        float s = m > 0.0 ? (float)m / 127.0f : 1.0f;
        row_scale[i] = s;
        for (int64_t e = mrow_ptr[i]; e < mrow_ptr[i + 1]; ++e) {
            double r = nearbyint(oracle_half_to_double(mvals[e]) / (double)s);
            if (r > 127.0) r = 127.0;
            if (r < -127.0) r = -127.0;
            q[e] = (int8_t)r;
        }
    }
}

/* y_i = alpha * sum over stored entries of (s_i * q_e) * x[col] + beta * y_i,
 * everything exact in fp64 up to the sum's rounding. */
void oracle_macko_spmv_i8(int n_rows, int n_cols, int b, const int32_t *mrow_ptr,
                          const uint32_t *codes, const int8_t *q, const float *row_scale,
                          const uint16_t *x, double alpha, double beta,
                          const float *y_in, double *y_out, double *scale)
{
    for (int i = 0; i < n_rows; ++i) {
        double s = 0.0, a = 0.0;
        int64_t prev = -1;
        for (int64_t e = mrow_ptr[i]; e < mrow_ptr[i + 1]; ++e) {
            prev = prev + (int64_t)oracle_macko_code(codes, e, b) + 1;
            if (prev >= n_cols) continue;
            double p = (double)row_scale[i] * (double)q[e] * oracle_half_to_double(x[prev]);
            s += p;
            a += fabs(p);
        }
        double yi = alpha * s, sc = fabs(alpha) * a;
        if (beta != 0.0) {
            yi += beta * (double)y_in[i];
            sc += fabs(beta * (double)y_in[i]);
        }
        y_out[i] = yi;
        if (scale) scale[i] = sc;
    }
}

/* ------------------------------------------------------------------------ */
/* Dense fp16 GEMV, the dense comparator of the MACKO-SpMV page's section    */
/* 3.1 table: y = alpha * W x + beta * y, W row-major m x n fp16.            */
/* ------------------------------------------------------------------------ */
void oracle_gemv_f16(int m, int n, const uint16_t *W, const uint16_t *x,
                     double alpha, double beta, const float *y_in,
                     double *y_out, double *scale)
{
    for (int i = 0; i < m; ++i) {
        double s = 0.0, a = 0.0;
        for (int j = 0; j < n; ++j) {
            double p = oracle_half_to_double(W[(size_t)i * n + j]) * oracle_half_to_double(x[j]);
            s += p;
            a += fabs(p);
        }
        double yi = alpha * s, sc = fabs(alpha) * a;
        if (beta != 0.0) {
            yi += beta * (double)y_in[i];
            sc += fabs(beta * (double)y_in[i]);
        }
        y_out[i] = yi;
        if (scale) scale[i] = sc;
    }
}

/* ------------------------------------------------------------------------ */
/* Finite-element stiffness matvec ("Fused GPU SpMV kernel optimisation:     */
/* from bandwidth bottleneck to BF16 precision", sections 2.1-2.2 and 5.1):  */
/* for every element gather the 24 local DOFs through edof, multiply by the  */
/* element matrix, and add the result into the global vector.  Readings:     */
/* one shared Ke scaled by rho_e^p (the SIMP interpolation the page's         */
/* topology-optimisation setting uses; section 5.2 notes a shared Ke), and   */
/* edof = -1 marks a constrained DOF that is neither gathered nor written.   */
/* y = alpha * sum_e rho_e^p P_e^T Ke P_e x + beta * y.                      */
/* scale_a = |alpha| sum_e sum_b |rho_e^p Ke_ab x_b| + |beta y_a|.           */
/* ------------------------------------------------------------------------ */
static double oracle_ipow(double r, int p)
{
    double s = 1.0;
    for (int k = 0; k < p; ++k) s *= r;
    return s;
}

void oracle_fe_matvec(int n_elem, int n_dof, const int32_t *edof, const float *rho,
                      int penalty, const float *Ke, const float *x, double alpha,
                      double beta, const float *y_in, double *y_out, double *scale)
{
    for (int d = 0; d < n_dof; ++d) {
        y_out[d] = (beta != 0.0) ? beta * (double)y_in[d] : 0.0;
        if (scale) scale[d] = (beta != 0.0) ? fabs(beta * (double)y_in[d]) : 0.0;
    }
    for (int e = 0; e < n_elem; ++e) {
        const int32_t *dof = edof + (size_t)e * 24;
        double s = oracle_ipow((double)rho[e], penalty);
        double u[24];
        for (int b = 0; b < 24; ++b)
            u[b] = dof[b] >= 0 ? (double)x[dof[b]] : 0.0;
        for (int a = 0; a < 24; ++a) {
            if (dof[a] < 0) continue;
            double f = 0.0, fa = 0.0;
            for (int b = 0; b < 24; ++b) {
                double p = s * (double)Ke[a * 24 + b] * u[b];
                f += p;
                fa += fabs(p);
            }
            y_out[dof[a]] += alpha * f;
            if (scale) scale[dof[a]] += fabs(alpha) * fa;
        }
    }
}

/* Assembled form of the same operator: every element contributes
 * (edof[a], edof[b], rho^p Ke_ab) for unconstrained a, b; entries are sorted
 * by (row, column) and equal positions are summed in fp64, giving CSR.
 * Two calls: with rp_out == NULL it returns the number of distinct entries;
 * otherwise it fills rp_out[n_dof+1], ci_out[nnz], v_out[nnz] and returns
 * nnz.  Returns -1 on allocation failure. */
typedef struct { int32_t r, c; int64_t order; double v; } oracle_coo_t;

static int oracle_coo_cmp(const void *pa, const void *pb)
{
    const oracle_coo_t *a = (const oracle_coo_t *)pa, *b = (const oracle_coo_t *)pb;
    if (a->r != b->r) return a->r < b->r ? -1 : 1;
    if (a->c != b->c) return a->c < b->c ? -1 : 1;
    if (a->order != b->order) return a->order < b->order ? -1 : 1;
    return 0;
}

int64_t oracle_fe_assemble(int n_elem, int n_dof, const int32_t *edof, const float *rho,
                           int penalty, const float *Ke, int32_t *rp_out,
                           int32_t *ci_out, double *v_out)
{
    size_t cap = (size_t)n_elem * 576;
    oracle_coo_t *coo = (oracle_coo_t *)malloc(cap * sizeof(oracle_coo_t) + 1);
    if (!coo) return -1;
    size_t m = 0;
    for (int e = 0; e < n_elem; ++e) {
        const int32_t *dof = edof + (size_t)e * 24;
        double s = oracle_ipow((double)rho[e], penalty);
        for (int a = 0; a < 24; ++a) {
            if (dof[a] < 0) continue;
            for (int b = 0; b < 24; ++b) {
                if (dof[b] < 0) continue;
                coo[m].r = dof[a];
                coo[m].c = dof[b];
                coo[m].order = (int64_t)m;
                coo[m].v = s * (double)Ke[a * 24 + b];
                m++;
            }
        }
    }
    qsort(coo, m, sizeof(oracle_coo_t), oracle_coo_cmp);
    int64_t nnz = 0;
    for (size_t k = 0; k < m; ++k) {
        int fresh = (k == 0) || coo[k].r != coo[k - 1].r || coo[k].c != coo[k - 1].c;
        if (fresh) {
            if (rp_out) {
                ci_out[nnz] = coo[k].c;
                v_out[nnz] = coo[k].v;
            }
            nnz++;
        } else if (rp_out) {
            v_out[nnz - 1] += coo[k].v;
        }
    }
    if (rp_out) {
        for (int d = 0; d <= n_dof; ++d) rp_out[d] = 0;
        for (size_t k = 0; k < m; ++k) {
            int fresh = (k == 0) || coo[k].r != coo[k - 1].r || coo[k].c != coo[k - 1].c;
            if (fresh) rp_out[coo[k].r + 1]++;
        }
        for (int d = 0; d < n_dof; ++d) rp_out[d + 1] += rp_out[d];
    }
    free(coo);
    return nnz;
}

/* ------------------------------------------------------------------------ */
/* SpGEMM C = A * B ("Sparse matrix multiplication acceleration techniques", */
/* the hash-based multi-phase SpGEMM page, sections 1.1 and 2.1).           */
/* The product's definition: C_ij = sum_k A_ik B_kj.  Row i of C needs, for */
/* each stored A_ik, row k of B: its intermediate products (IP) number      */
/* sum over k in row i of A of nnz(B row k) (section 2.1.1 bins rows by     */
/* this count).  The oracle is Gustavson's row-by-row form with a dense    */
/* fp64 accumulator over the columns of B and a marker per column; each    */
/* row of C lists its distinct columns in increasing order (the method     */
/* leaves the order open; sorted is the canonical CSR).  Entries that sum  */
/* to zero are kept: the pattern is the set of columns reached.            */
/* ------------------------------------------------------------------------ */
void oracle_spgemm_ip(int m, const int32_t *rpa, const int32_t *cia, const int32_t *rpb, int64_t *ip)
{
    for (int i = 0; i < m; ++i) {
        int64_t s = 0;
        for (int32_t j = rpa[i]; j < rpa[i + 1]; ++j) s += rpb[cia[j] + 1] - rpb[cia[j]];
        ip[i] = s;
    }
}

static int oracle_cmp_i32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Row counts of C into rpc (rpc[0] = 0, rpc[i+1] = rpc[i] + distinct columns
 * of row i); returns nnz(C), or -1 if n < 1 with a nonempty product. */
int64_t oracle_spgemm_rows(int m, int n, const int32_t *rpa, const int32_t *cia,
                           const int32_t *rpb, const int32_t *cib, int64_t *rpc)
{
    int32_t *mark = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    if (!mark) return -1;
    for (int c = 0; c < n; ++c) mark[c] = -1;
    rpc[0] = 0;
    for (int i = 0; i < m; ++i) {
        int64_t cnt = 0;
        for (int32_t j = rpa[i]; j < rpa[i + 1]; ++j) {
            int32_t k = cia[j];
            for (int32_t t = rpb[k]; t < rpb[k + 1]; ++t)
                if (mark[cib[t]] != i) {
                    mark[cib[t]] = i;
                    cnt++;
                }
        }
        rpc[i + 1] = rpc[i] + cnt;
    }
    free(mark);
    return rpc[m];
}

/* Fills cic[nnz(C)] (sorted per row) and vc[nnz(C)] = sum_k A_ik B_kj in fp64,
 * and scale[nnz(C)] = sum_k |A_ik B_kj| (the error scale of each entry);
 * rpc from oracle_spgemm_rows.  Returns 0, or -1 on allocation failure. */
int oracle_spgemm_fill(int m, int n, const int32_t *rpa, const int32_t *cia, const float *va,
                       const int32_t *rpb, const int32_t *cib, const float *vb,
                       const int64_t *rpc, int32_t *cic, double *vc, double *scale)
{
    double *acc = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
    double *mag = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
    int32_t *mark = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    if (!acc || !mag || !mark) {
        free(acc); free(mag); free(mark);
        return -1;
    }
    for (int c = 0; c < n; ++c) mark[c] = -1;
    for (int i = 0; i < m; ++i) {
        int64_t at = rpc[i];
        for (int32_t j = rpa[i]; j < rpa[i + 1]; ++j) {
            int32_t k = cia[j];
            double a = va[j];
            for (int32_t t = rpb[k]; t < rpb[k + 1]; ++t) {
                int32_t c = cib[t];
                if (mark[c] != i) {
                    mark[c] = i;
                    cic[at++] = c;
                    acc[c] = 0.0;
                    mag[c] = 0.0;
                }
                double p = a * (double)vb[t];
                acc[c] += p;
                mag[c] += fabs(p);
            }
        }
        qsort(cic + rpc[i], (size_t)(rpc[i + 1] - rpc[i]), sizeof(int32_t), oracle_cmp_i32);
        for (int64_t e = rpc[i]; e < rpc[i + 1]; ++e) {
            vc[e] = acc[cic[e]];
            if (scale) scale[e] = mag[cic[e]];
        }
    }
    free(acc); free(mag); free(mark);
    return 0;
}
