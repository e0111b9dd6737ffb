/*
 * spmv.h -- C ABI of the MI355X (gfx950) sparse matrix-vector library.
 *
 * Every entry point computes (a step of) y = alpha * A * x + beta * y, the
 * operation all four source pages turn on:
 *   - "Why SpMV needs CUDA optimisation" (codechina.net): CSR scalar and
 *     warp-per-row kernels (sections 2.1, 4.1), ELL and the CV-based format
 *     rule (sections 2.1-2.2);
 *   - "Sparse matrix multiplication acceleration" (mlqm.cn, hash-based
 *     multi-phase SpGEMM): row grouping by work per row (section 2.1.1) and
 *     the group-ordered row map (section 2.2.1);
 *   - "MACKO-SpMV: GPU acceleration and storage optimisation at low sparsity"
 *     (maplevalley.com.cn): the MACKO format and its kernel (section 2);
 *   - "Fused GPU SpMV kernel optimisation: from bandwidth bottleneck to BF16
 *     precision" (bbs.csdn.net): the fused gather / element product / atomic
 *     scatter finite-element matvec (sections 2 and 5.1).
 *
 * Conventions shared by all calls
 *   - Indices are int32, as on the pages.  Counts that do not fit int32 return
 *     SPMV_ERR_OVERFLOW.
 *   - "device" pointers point to GPU memory (hipMalloc / torch CUDA tensors),
 *     "host" pointers to CPU memory.  All memory is owned by the caller; the
 *     library never allocates device memory and never frees what it is
 *     given.  Device scratch and plan storage come in as workspace or
 *     scratch arguments sized by the *_size queries.  A CSR handle *borrows* the
 *     matrix arrays: they must stay allocated and structurally unchanged until
 *     spmv_csr_destroy (values may be rewritten in place between applies).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls that launch kernels are asynchronous on that stream unless their
 *     comment says "synchronises".
 *   - beta == 0 means y is write-only: it is not read, so it may hold NaN.
 *   - Every call returns an spmv_status.  On failure nothing was launched
 *     (validation runs first, on the host) unless the status is SPMV_ERR_HIP,
 *     and spmv_last_error() gives a message (per calling thread).
 *   - fp16 data is passed as its IEEE binary16 bit pattern (uint16_t).
 */
#ifndef SPMV_AMD_H
#define SPMV_AMD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPMV_OK = 0,
    SPMV_ERR_INVALID_VALUE = 1,   /* bad size, null pointer, workspace too small */
    SPMV_ERR_INVALID_MATRIX = 2,  /* row_ptr not monotone / inconsistent, column out of range */
    SPMV_ERR_UNSORTED = 3,        /* MACKO input: columns not strictly increasing in a row */
    SPMV_ERR_OVERFLOW = 4,        /* a count does not fit int32 */
    SPMV_ERR_UNSUPPORTED = 5,     /* valid request the library does not support */
    SPMV_ERR_HIP = 6              /* a HIP runtime call failed */
} spmv_status;

/* Message of the last failing call on this thread ("" if none). */
const char *spmv_last_error(void);

/* Device scratch of the synchronous statistics, planning and conversion
 * calls: spmv_csr_row_stats, spmv_hyb_width, spmv_hyb_tail_size,
 * spmv_ell_from_csr, spmv_hyb_from_csr, spmv_auto_plan and
 * spgemm_workspace_size.  They keep reduction counters and per-workgroup
 * counts there, so that the library itself allocates no device memory.
 * *bytes receives the size for a matrix of n_rows rows (for SpGEMM: the rows
 * of A): 256 bytes plus 8 bytes per 256 rows, rounded up to 256.  The caller
 * allocates it (device memory, 256-byte aligned) and keeps ownership; its
 * contents on entry do not matter and on return are unspecified.  Those
 * calls synchronise, so one scratch buffer may serve call after call on one
 * stream.  Host only.  SPMV_ERR_INVALID_VALUE for n_rows < 0. */
spmv_status spmv_scratch_size(int32_t n_rows, size_t *bytes);

/* ======================================================================== */
/* Row statistics and format choice                                         */
/* ======================================================================== */

/* Longest row, sum and sum of squares of the row lengths of a CSR row_ptr
 * (the statistics of the CV rule below).
 * row_ptr: device int32[n_rows+1].  Outputs: host.  scratch: device, at
 * least spmv_scratch_size(n_rows) bytes.  Synchronises `stream`.
 * SPMV_ERR_INVALID_MATRIX if some row has negative length. */
spmv_status spmv_csr_row_stats(int32_t n_rows, const int32_t *row_ptr,
                               int32_t *max_len, int64_t *sum_len,
                               int64_t *sum_len_sq, void *scratch,
                               size_t scratch_bytes, void *stream);

/* Format recommendation by the coefficient of variation (CV) of the row
 * lengths ("Why SpMV needs CUDA optimisation", section 2.2): CV < 0.3 -> ELL,
 * 0.3 <= CV <= 0.7 -> HYB, CV > 0.7 -> CSR with row reordering (the binned
 * CSR path).  CV uses the population standard deviation; the comparison is
 * exact integer arithmetic on (n, sum_len, sum_len_sq).  No rows or no
 * nonzeros -> CSR.  Host only, no GPU call. */
typedef enum { SPMV_FORMAT_ELL = 0, SPMV_FORMAT_HYB = 1, SPMV_FORMAT_CSR = 2 } spmv_format;
spmv_status spmv_format_recommend(int64_t n_rows, int64_t sum_len, int64_t sum_len_sq,
                                  int32_t *format);

/* ======================================================================== */
/* CSR: y = alpha * A * x + beta * y                                        */
/* ("Why SpMV needs CUDA optimisation", sections 2.1 and 4.1; row grouping  */
/*  from "Sparse matrix multiplication acceleration", section 2.1.1)        */
/* ======================================================================== */

typedef enum {
    SPMV_CSR_AUTO = 0,     /* = BINNED */
    SPMV_CSR_SCALAR = 1,   /* one lane per row, rows in natural order */
    SPMV_CSR_VECTOR = 2,   /* G lanes per row (G = power of two >= mean row length, 2..64) */
    SPMV_CSR_BINNED = 3    /* rows grouped by length, one kernel shape per group */
} spmv_csr_variant;

typedef struct spmv_csr_plan *spmv_csr_t;

/* Bytes of device workspace spmv_csr_create needs for a matrix of this size.
 * thresholds: host int32[3] or NULL for {128, 512, 8192} (the grouping
 * page's table starts at 32; a wave task stages 512 entries, so rows up to
 * 127 entries still share a wave here); valid thresholds satisfy
 * 1 <= t0 < t1 < t2 and t0 <= 256. */
spmv_status spmv_csr_plan_size(int32_t n_rows, int32_t nnz, const int32_t *thresholds,
                               size_t *bytes);

/* Validates the matrix on the GPU (row_ptr[0] == 0, row_ptr[n_rows] == nnz,
 * non-decreasing row_ptr, 0 <= col < n_cols) and, for BINNED/AUTO, builds
 * the row-grouping plan in `workspace` (device, 256-byte aligned, >=
 * spmv_csr_plan_size bytes, owned by the caller, kept until destroy).
 * SCALAR and VECTOR need only 256 bytes of workspace, used for the
 * validation flags during this call and free again afterwards.  The grouping: group g holds rows
 * with t[g-1] <= length < t[g]; `perm` lists rows group by group in
 * ascending row order.  row_ptr, col_idx: device int32; vals: device fp32.
 * Column order inside a row is free (duplicates are summed).  Synchronises
 * `stream`.  *h receives a handle (host memory owned by the library until
 * spmv_csr_destroy). */
spmv_status spmv_csr_create(spmv_csr_t *h, int32_t n_rows, int32_t n_cols, int32_t nnz,
                            const int32_t *row_ptr, const int32_t *col_idx,
                            const float *vals, int32_t variant,
                            const int32_t *thresholds, void *workspace,
                            size_t workspace_bytes, void *stream);

/* y = alpha * A * x + beta * y with fp32 products summed in fp32.
 * x: device fp32[n_cols]; y: device fp32[n_rows].  x and y must not overlap.
 * Asynchronous; no synchronisation and no allocation. */
spmv_status spmv_csr_apply(spmv_csr_t h, float alpha, const float *x, float beta,
                           float *y, void *stream);

/* Test hook: copies the grouping plan.  h_bin_offsets: host int32[5] (group
 * g occupies perm[bin_offsets[g] .. bin_offsets[g+1]-1]); d_perm: device
 * int32[n_rows] or NULL.  Synchronises `stream`.  SPMV_ERR_INVALID_VALUE for
 * a handle without a plan (SCALAR / VECTOR). */
spmv_status spmv_csr_get_plan(spmv_csr_t h, int32_t *h_bin_offsets, int32_t *d_perm,
                              void *stream);

/* Resolved variant, lanes per row of the VECTOR variant (0 otherwise) and the
 * number of short-row blocks of the BINNED plan (0 otherwise).  Host only. */
spmv_status spmv_csr_info(spmv_csr_t h, int32_t *variant, int32_t *group_lanes,
                          int32_t *n_short_blocks);

/* Scatter form of spmv_csr_apply: for i < n_rows,
 *   y[row_map[i]] = alpha * (A x)_i + beta * y[row_map[i]],
 * with the same kernels and sum order.  row_map: device int32[n_rows]; its
 * entries must be distinct valid indices of y (not checked).  With
 * beta = 1 it adds A x into selected rows of a longer y (the HYB tail uses
 * it).  Asynchronous. */
spmv_status spmv_csr_apply_rows(spmv_csr_t h, float alpha, const float *x, float beta, float *y,
                                const int32_t *row_map, void *stream);

/* Releases the handle (not the borrowed arrays or the workspace). */
spmv_status spmv_csr_destroy(spmv_csr_t h);

/* ======================================================================== */
/* ELL ("Why SpMV needs CUDA optimisation", section 2.1 table)               */
/* Layout: slot-major, entry k of row i at [k * n_rows + i]; a padding slot */
/* holds column -1 and value +0.0f and is skipped.                          */
/* ======================================================================== */

/* Converts CSR (device arrays) to ELL of the given width (device outputs
 * int32 / fp32 [width * n_rows]).  width must be >= the longest row
 * (SPMV_ERR_INVALID_VALUE otherwise).  Row order of entries is kept.
 * scratch: device, >= spmv_scratch_size(n_rows) bytes.
 * Synchronises `stream` (it checks the width and the matrix first). */
spmv_status spmv_ell_from_csr(int32_t n_rows, int32_t n_cols, int32_t nnz,
                              const int32_t *row_ptr, const int32_t *col_idx,
                              const float *vals, int32_t width, int32_t *ell_col,
                              float *ell_val, void *scratch, size_t scratch_bytes,
                              void *stream);

/* y = alpha * A * x + beta * y for an ELL matrix; slots are summed in slot
 * order in fp32.  ell_col entries must be -1 or in [0, n_cols) (as written
 * by spmv_ell_from_csr).  Asynchronous. */
spmv_status spmv_ell_apply(int32_t n_rows, int32_t n_cols, int32_t width,
                           const int32_t *ell_col, const float *ell_val, float alpha,
                           const float *x, float beta, float *y, void *stream);

/* ======================================================================== */
/* HYB: ELL part + CSR tail ("Why SpMV needs CUDA optimisation", section    */
/* 2.1 table: a mixed CSR + ELL format; section 2.2: the format for a       */
/* row-length CV between 0.3 and 0.7; section 5: a tuned split of 0.7 ELL   */
/* to 0.3 COO).                                                             */
/* Layout: the ELL part holds the first min(len_i, W) entries of each row   */
/* (ELL layout above); the tail holds the rest, for the rows longer than W  */
/* only: tail_rows[t] (ascending row ids), tail_rp[t] .. tail_rp[t+1]       */
/* indexing tail_col / tail_val, in each row's storage order.               */
/* ======================================================================== */

/* Default ELL share of the nonzeros (the page's 0.7 : 0.3 example). */
#define SPMV_HYB_ELL_NUM 7
#define SPMV_HYB_ELL_DEN 10

/* Width rule: the smallest W with den * sum_i min(len_i, W) >= num * nnz
 * (exact integers; needs 0 <= num <= den, den > 0), and the tail sizes for
 * that W: n_tail_rows = #rows longer than W, tail_nnz = their entries past
 * W.  row_ptr: device int32[n_rows+1].  Outputs: host.  scratch: device,
 * >= spmv_scratch_size(n_rows) bytes.  Synchronises. */
spmv_status spmv_hyb_width(int32_t n_rows, const int32_t *row_ptr, int32_t num, int32_t den,
                           int32_t *width, int32_t *n_tail_rows, int64_t *tail_nnz, void *scratch,
                           size_t scratch_bytes, void *stream);

/* Tail sizes of the HYB split at an explicit width W >= 0 (the sizes the
 * tail arrays of spmv_hyb_from_csr need): n_tail_rows = #rows longer than
 * W, tail_nnz = the sum of (len_i - W) over those rows.  row_ptr: device
 * int32[n_rows+1]; outputs: host; scratch as above.  SPMV_ERR_INVALID_MATRIX
 * if some row has negative length.  Synchronises. */
spmv_status spmv_hyb_tail_size(int32_t n_rows, const int32_t *row_ptr, int32_t width,
                               int32_t *n_tail_rows, int64_t *tail_nnz, void *scratch,
                               size_t scratch_bytes, void *stream);

/* Splits a CSR matrix (device arrays) into HYB of width `width`.  Outputs
 * (device, caller-allocated): ell_col / ell_val [width * n_rows],
 * tail_rows [n_tail_rows], tail_rp [n_tail_rows + 1], tail_col / tail_val
 * [tail_nnz].  n_tail_rows / tail_nnz must be the sizes this width gives
 * (spmv_hyb_width or spmv_hyb_tail_size; SPMV_ERR_INVALID_VALUE otherwise,
 * before anything is written).  scratch: device, >=
 * spmv_scratch_size(n_rows) bytes.  Checks the matrix
 * (SPMV_ERR_INVALID_MATRIX).  Synchronises. */
spmv_status spmv_hyb_from_csr(int32_t n_rows, int32_t n_cols, int32_t nnz, const int32_t *row_ptr,
                              const int32_t *col_idx, const float *vals, int32_t width,
                              int32_t *ell_col, float *ell_val, int32_t n_tail_rows,
                              int64_t tail_nnz, int32_t *tail_rows, int32_t *tail_rp,
                              int32_t *tail_col, float *tail_val, void *scratch,
                              size_t scratch_bytes, void *stream);

/* y = alpha * A * x + beta * y for a HYB matrix: the ELL part writes
 * alpha * (ELL part) x + beta * y, then each tail row adds alpha * its tail
 * sum (fp32, fixed order).  All arrays device.  Asynchronous. */
spmv_status spmv_hyb_apply(int32_t n_rows, int32_t n_cols, int32_t width, const int32_t *ell_col,
                           const float *ell_val, int32_t n_tail_rows, int64_t tail_nnz,
                           const int32_t *tail_rows, const int32_t *tail_rp,
                           const int32_t *tail_col, const float *tail_val, float alpha,
                           const float *x, float beta, float *y, void *stream);

/* ======================================================================== */
/* Format chosen by the CV rule (spmv_format_recommend): ELL, HYB or binned */
/* CSR, built in a caller workspace and applied through one handle.         */
/* ELL is replaced by HYB when padding to the longest row would more than   */
/* double the storage of max(nnz, n_rows) entries or overflow int32.        */
/* ======================================================================== */
typedef struct {
    int32_t format;          /* SPMV_FORMAT_ELL / _HYB / _CSR */
    int32_t width;           /* ELL width (ELL: the longest row; HYB: the width rule) */
    int32_t n_tail_rows;     /* HYB tail rows (0 otherwise) */
    int64_t tail_nnz;        /* HYB tail entries (0 otherwise) */
    size_t workspace_bytes;  /* device workspace spmv_auto_create needs */
} spmv_auto_plan_t;

typedef struct spmv_auto *spmv_auto_t;

/* Row statistics and the choice (device row_ptr; plan: host; scratch:
 * device, >= spmv_scratch_size(n_rows) bytes).  Synchronises. */
spmv_status spmv_auto_plan(int32_t n_rows, int32_t n_cols, int32_t nnz, const int32_t *row_ptr,
                           spmv_auto_plan_t *plan, void *scratch, size_t scratch_bytes, void *stream);

/* Builds the planned format in `workspace` (device, 256-byte aligned, at
 * least plan->workspace_bytes).  The handle borrows the CSR arrays when the
 * format is CSR; ELL and HYB keep their own copy in the workspace, and the
 * conversion's scratch is part of it.  For HYB the tail is kept per tail
 * row with a binned CSR plan, and per row (one pointer per row): when no
 * row has more than 16 entries past the width, n_rows and n_cols are
 * multiples of 4 and x, y are 16-byte aligned, spmv_auto_apply runs the ELL
 * part and the tail in one kernel; otherwise the ELL kernel, then the tail
 * through spmv_csr_apply_rows.  Synchronises. */
spmv_status spmv_auto_create(spmv_auto_t *h, const spmv_auto_plan_t *plan, int32_t n_rows,
                             int32_t n_cols, int32_t nnz, const int32_t *row_ptr,
                             const int32_t *col_idx, const float *vals, void *workspace,
                             size_t workspace_bytes, void *stream);

/* y = alpha * A * x + beta * y with the planned format.  Asynchronous. */
spmv_status spmv_auto_apply(spmv_auto_t h, float alpha, const float *x, float beta, float *y,
                            void *stream);

/* Releases the handle (not the workspace or the borrowed arrays). */
spmv_status spmv_auto_destroy(spmv_auto_t h);

/* ======================================================================== */
/* MACKO ("MACKO-SpMV: GPU acceleration and storage optimisation at low      */
/* sparsity", section 2; code widths and int8 values: section 3.3)          */
/* Format for code width b in {1, 2, 4, 8} (the page's b-delta, 4 by        */
/* default): per row, entries in column order; each entry has a b-bit code  */
/* c meaning "column = previous column + c + 1" (the previous column starts */
/* at -1 in each row) and a value.  A gap larger than 2^b is bridged by     */
/* padding entries (code 2^b - 1, value +0) placed 2^b columns after the    */
/* previous entry; each row is padded with (code 0, value +0) to a multiple */
/* of 1024 / b entries (one 128-byte block of codes).  codes: entry e in    */
/* bits [b (e % (32/b)), b (e % (32/b)) + b - 1] of word e / (32/b); the    */
/* array holds n_entries * b / 32 words.  mrow_ptr[i] is the first entry of */
/* row i; mrow_ptr[n_rows] = total.  The device entry points expect         */
/* mrow_ptr, codes and values exactly as the encoder wrote them.             */
/* A code width other than 1, 2, 4, 8 gives SPMV_ERR_INVALID_VALUE.         */
/* ======================================================================== */

/* Number of encoded entries (host inputs).  SPMV_ERR_UNSORTED if a row's
 * columns are not strictly increasing, SPMV_ERR_INVALID_MATRIX for a column
 * outside [0, n_cols) or a bad row_ptr, SPMV_ERR_OVERFLOW past int32. */
spmv_status macko_encode_size(int32_t n_rows, int32_t n_cols, int32_t bdelta, const int32_t *h_row_ptr,
                              const int32_t *h_col, int64_t *n_entries);

/* Encodes on the host into caller buffers: h_mrow_ptr int32[n_rows+1],
 * h_codes uint32[n_entries*bdelta/32], h_mvals uint16[n_entries] (fp16
 * bits).  Same errors as macko_encode_size. */
spmv_status macko_encode(int32_t n_rows, int32_t n_cols, int32_t bdelta, const int32_t *h_row_ptr,
                         const int32_t *h_col, const uint16_t *h_vals_f16,
                         int32_t *h_mrow_ptr, uint32_t *h_codes, uint16_t *h_mvals);

/* The 8-bit value mode (section 3.3 names int8 values; the scaling is this
 * library's reading): for each row, s = max |v| / 127 over its stored fp16
 * values as an fp32 division (1 for a row of zeros), and every value becomes
 * q = v / s computed in double, rounded to nearest with ties to even and
 * clamped to [-127, 127]; the entry's value is then s * q.  Host inputs
 * h_mrow_ptr int32[n_rows+1] and h_mvals uint16[total] as written by
 * macko_encode (values must be finite); outputs h_q int8[total] and
 * h_row_scale fp32[n_rows].  SPMV_ERR_INVALID_MATRIX for a decreasing
 * mrow_ptr. */
spmv_status macko_quantize_i8(int32_t n_rows, const int32_t *h_mrow_ptr, const uint16_t *h_mvals,
                              int8_t *h_q, float *h_row_scale);

/* y = alpha * A * x + beta * y: fp16 values times fp16 x, fp32 accumulate,
 * fp32 y.  Columns are rebuilt on the GPU from the codes by a wave-wide
 * prefix sum (section 2.2.2).  All pointers are device; mvals must be
 * 16-byte aligned and codes 4-byte aligned (8-byte for bdelta 8), else
 * SPMV_ERR_UNSUPPORTED.  Asynchronous. */
spmv_status macko_spmv(int32_t n_rows, int32_t n_cols, int32_t bdelta, const int32_t *mrow_ptr,
                       const uint32_t *codes, const uint16_t *mvals, float alpha,
                       const uint16_t *x_f16, float beta, float *y, void *stream);

/* The same product with int8 values: y_i = alpha * s_i * sum q * x + beta * y_i
 * (q int8[total] 8-byte aligned, row_scale fp32[n_rows], both device; the
 * products q * x are exact in fp32, the sum is fp32).  Asynchronous. */
spmv_status macko_spmv_i8(int32_t n_rows, int32_t n_cols, int32_t bdelta, const int32_t *mrow_ptr,
                          const uint32_t *codes, const int8_t *q, const float *row_scale, float alpha,
                          const uint16_t *x_f16, float beta, float *y, void *stream);

/* Test hook: the column of every stored entry (device int32[total entries]),
 * rebuilt by the same on-GPU decoder.  Asynchronous. */
spmv_status macko_decode_columns(int32_t n_rows, int32_t bdelta, const int32_t *mrow_ptr,
                                 const uint32_t *codes, int32_t *cols_out, void *stream);

/* ======================================================================== */
/* Dense fp16 GEMV, the dense comparator of the MACKO page's section 3.1    */
/* y = alpha * W x + beta * y; W device fp16[m * n] row-major, x fp16[n],   */
/* y fp32[m]; fp32 accumulation.  Asynchronous.                             */
/* ======================================================================== */
spmv_status dense_gemv_f16(int32_t m, int32_t n, const uint16_t *W, const uint16_t *x_f16,
                           float alpha, float beta, float *y, void *stream);

/* ======================================================================== */
/* Finite-element stiffness matvec ("Fused GPU SpMV kernel optimisation",   */
/* sections 2.1-2.2 and 5.1-5.2)                                             */
/* y = alpha * sum_e rho_e^penalty * P_e^T Ke P_e x + beta * y               */
/* edof: device int32[n_elem * 24], element e's 24 global DOFs; -1 (or any   */
/* value outside [0, n_dof)) marks a constrained DOF, neither gathered nor   */
/* written.  rho: device fp32[n_elem]; Ke: device fp32[24 * 24] row-major,   */
/* shared by all elements; x, y: device fp32[n_dof]; 0 <= penalty <= 8.      */
/* The scatter uses fp32 atomics, so the order of additions (and the last   */
/* bits of y) may differ from call to call.                                 */
/* ======================================================================== */

/* One fused kernel (after a y = beta * y pass): gather, 24x24 product,
 * atomic scatter.  Asynchronous. */
spmv_status fem_matvec_apply(int32_t n_elem, int32_t n_dof, const int32_t *edof,
                             const float *rho, int32_t penalty, const float *Ke,
                             float alpha, const float *x, float beta, float *y,
                             void *stream);

/* Element blocks ("Fused GPU SpMV kernel optimisation", sections 2.2 and
 * 5.2: the fused pass, with what the elements share held in on-chip memory).
 * A plan built once from edof cuts the elements into compact blocks of at
 * most 512 (256 where a 512-element block's workgroup would need more than
 * 64 KB of LDS; one workgroup each).  It works on units of G DOFs: a node's
 * three DOFs (G = 3) when every element corner is either three constrained
 * DOFs or the DOFs 3i, 3i+1, 3i+2 of one node, else single DOFs (G = 1).
 * Each block numbers its units locally, stores each element's 24 / G units
 * as 16-bit local indices and gives each entry a 16-bit position in the
 * block's product buffer, so that the entries of one local unit form a run.
 * The apply stages x of a block's units in LDS, writes the element products
 * to their positions there, sums each run in order and writes every DOF of
 * y once: a unit private to one block with plain stores (y = beta * y +
 * sum), any other unit (shared by blocks, or touched by none) in a second
 * kernel that adds the blocks' partial sums in increasing block order.  No
 * atomics and no separate beta pass; any numbering is valid; the order of
 * every addition is fixed by the plan, so repeated calls give the same bits.
 * Same operator and arguments as fem_matvec_apply; the result agrees with it
 * up to the order of additions.
 *   fem_blocks_size: device workspace bytes for the shape (an upper bound,
 *     about 500 bytes per element + 44 per DOF).
 *   fem_blocks_create: copies edof (device) to the host, builds the plan and
 *     uploads it into `workspace` (device, 256-byte aligned, >= the size,
 *     kept until destroy).  group: 0 picks 3 when the numbering allows it,
 *     else 1; 1 or 3 forces it (3 on a numbering without the node structure
 *     is SPMV_ERR_INVALID_VALUE).  Synchronises.
 *   fem_blocks_apply: y = alpha * K x + beta * y with rho, penalty (0..8),
 *     Ke as for fem_matvec_apply.  Two launches.  Asynchronous; calls that
 *     overlap on one plan race on its partial sums.
 *   fem_blocks_info: counts[0] blocks, [1] most local units of a block, [2]
 *     units finished by the second kernel, [3] largest product buffer of a
 *     block (products and padding words),
 *     [4] G, [5] rank planes of the partial sums, [6] most elements per
 *     block (512 or 256).
 *   fem_blocks_plan_host: the same plan from a host edof into host buffers
 *     (NULL buffers are skipped).  Upper-bound sizes: blk_elem_off,
 *     blk_dof_off n_elem + 1; perm n_elem; ldof, ldst, crun, lidx, lpos
 *     24 n_elem; shr_ptr n_dof + 1; shr_dof, shr_cnt n_dof.  Per block b:
 *     elements perm[blk_elem_off[b] ..], local units at blk_dof_off[b] + l
 *     with first DOF ldof (increasing), destination ldst of the first
 *     component (the DOF itself if private, else ~slot; component c at that
 *     + c) and its run crun = start | end << 16 in the block's product
 *     buffer (runs in local-unit order, a run of even length followed by
 *     one unused word); lidx / lpos [k * (24 / G) + j]: local unit and product position
 *     of entry j of the block list's k-th element (0xFFFF where constrained;
 *     component c of the entry at lpos + c).  Second-kernel units shr_dof
 *     (first DOF, increasing), each touched by shr_cnt blocks; the partial
 *     sum of the r-th of them sits, for r < planes, at slot
 *     (r * n_shared + i) * G, else at planes * n_shared * G + shr_ptr[i] +
 *     (r - planes) * G.  counts = {blocks, local units in all, second-kernel
 *     units, slots, most local units of a block, largest product buffer of a
 *     block, G, planes, most elements per block} (counts holds 9).  For inspection and tests. */
typedef struct fem_blocks *fem_blocks_t;
spmv_status fem_blocks_size(int32_t n_elem, int32_t n_dof, size_t *bytes);
spmv_status fem_blocks_create(fem_blocks_t *plan, int32_t n_elem, int32_t n_dof, const int32_t *edof,
                              int32_t group, void *workspace, size_t workspace_bytes, void *stream);
spmv_status fem_blocks_apply(fem_blocks_t plan, const float *rho, int32_t penalty, const float *Ke,
                             float alpha, const float *x, float beta, float *y, void *stream);
spmv_status fem_blocks_info(fem_blocks_t plan, int32_t *counts);
spmv_status fem_blocks_destroy(fem_blocks_t plan);
spmv_status fem_blocks_plan_host(int32_t n_elem, int32_t n_dof, const int32_t *edof, int32_t group,
                                 int32_t *counts,
                                 int32_t *blk_elem_off, int32_t *perm, int32_t *blk_dof_off, int32_t *ldof,
                                 int32_t *ldst, uint32_t *crun, uint16_t *lidx, uint16_t *lpos,
                                 int32_t *shr_ptr, int32_t *shr_dof, int32_t *shr_cnt);

/* Workspace bytes of the three-stage comparator (2 * n_elem * 24 floats). */
spmv_status fem_threestage_size(int32_t n_elem, size_t *bytes);

/* The unfused comparator the page measures against (section 2.1): a gather
 * kernel writing per-element vectors to the workspace, an element-product
 * kernel, and an atomic scatter kernel.  Same result as fem_matvec_apply up
 * to rounding order.  Asynchronous. */
spmv_status fem_matvec_threestage(int32_t n_elem, int32_t n_dof, const int32_t *edof,
                                  const float *rho, int32_t penalty, const float *Ke,
                                  float alpha, const float *x, float beta, float *y,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* The assembled stiffness matrix K = sum_e rho_e^penalty P_e^T Ke P_e in CSR
 * (section 2.1: the conventional route the fused kernel is measured
 * against: assemble K once, then run a CSR SpMV on it).  Row and column d
 * are DOF d; each row lists its distinct columns in increasing order; an
 * entry is the sum of its element terms rho_e^penalty Ke[a][b], taken in a
 * fixed order in fp64 and rounded to fp32.  Constrained edof entries (-1 or
 * outside [0, n_dof)) are dropped.  Two synchronous calls that share a
 * device workspace (256-byte aligned, >= fem_assemble_size bytes, about
 * 100 bytes per element; keep it between the calls):
 * fem_assemble_pattern writes row_ptr (device int32[n_dof + 1]) and *nnz
 * (host); fem_assemble_values then writes col_idx (device int32[nnz]) and
 * vals (device fp32[nnz]) for the given rho, penalty and Ke (the layout of
 * fem_matvec_apply).  A row may collect at most 256 (element, column)
 * candidates (24 per element reaching the DOF: 10 elements per node),
 * else SPMV_ERR_UNSUPPORTED; nnz beyond int32 gives SPMV_ERR_OVERFLOW. */
spmv_status fem_assemble_size(int32_t n_elem, int32_t n_dof, size_t *bytes);
spmv_status fem_assemble_pattern(int32_t n_elem, int32_t n_dof, const int32_t *edof, int32_t *row_ptr,
                                 int64_t *nnz, void *workspace, size_t workspace_bytes, void *stream);
spmv_status fem_assemble_values(int32_t n_elem, int32_t n_dof, const int32_t *edof, const float *rho,
                                int32_t penalty, const float *Ke, const int32_t *row_ptr,
                                int32_t *col_idx, float *vals, void *workspace, size_t workspace_bytes,
                                void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * three-stage comparator with its per-element vectors in a library-owned
 * static device array instead of a workspace.  The array holds 65,536
 * elements' U and F (12 MiB per GPU, kept until the process ends); larger
 * meshes run as consecutive chunks of 65,536 elements on `stream`, so no
 * size is rejected.  Same arguments, validation and result as
 * fem_matvec_threestage (up to the order of the atomic adds).  Every call
 * on one GPU uses that GPU's one array: calls that overlap on one GPU (on
 * different streams or threads) race and give wrong results.  The stream
 * must belong to the current device.  Nothing is allocated, no memset is
 * issued; only kernels are launched.  Asynchronous. */
spmv_status fem_matvec_threestage_noalloc(int32_t n_elem, int32_t n_dof, const int32_t *edof,
                                          const float *rho, int32_t penalty, const float *Ke,
                                          float alpha, const float *x, float beta, float *y,
                                          void *stream);

/* ======================================================================== */
/* FE solver ("Fused GPU SpMV kernel optimisation", section 6.1: Jacobi-     */
/* preconditioned CG around the fused matvec, with an iteration cap;        */
/* section 4.1: the condition number of K by power iteration).  The        */
/* operator arguments (n_elem, n_dof, edof, rho, penalty, Ke) are those of  */
/* fem_matvec_apply, with the same validation.  The caller's vectors (f, u, */
/* v0) are fp32 device arrays of n_dof entries; the iteration keeps its     */
/* vectors in fp64 in the workspace, accumulates inner products in fp64,    */
/* and sums each matvec in 64-bit fixed point (element products in fp64,    */
/* integer atomic adds, scale set per product from max|x|), so that results */
/* and iteration counts are the same bit for bit from run to run.  The      */
/* workspace is device memory, 256-byte aligned, of at least the size       */
/* fem_solver_workspace_size returns; it is not freed by these calls.       */
/* ======================================================================== */

/* diag[d] = sum of rho_e^penalty * Ke[a][a] over the elements e and local
 * DOFs a with edof[e][a] = d: the Jacobi preconditioner, summed with fp32
 * atomic adds (the solver computes its own copy in fixed point).
 * Asynchronous. */
spmv_status fem_jacobi_diagonal(int32_t n_elem, int32_t n_dof, const int32_t *edof, const float *rho,
                                int32_t penalty, const float *Ke, float *diag, void *stream);

/* Workspace bytes for the calls below (about 64 bytes per DOF plus 64 KB);
 * max_history >= the `iterations` of fem_lambda_max / fem_lambda_min (0 for
 * fem_pcg_solve alone). */
spmv_status fem_solver_workspace_size(int32_t n_dof, int32_t max_history, size_t *bytes);

/* Solves K u = f by Jacobi-PCG from the initial guess in u (device, fp32,
 * overwritten with the solution).  Stops when the recursively updated
 * residual satisfies ||r|| <= rtol * ||f|| or after max_iter iterations.
 * *iterations (host, optional) receives the iterations done and
 * *rel_residual (host, optional) ||r|| / ||f|| (||r|| if f = 0).
 * SPMV_ERR_INVALID_MATRIX if a diagonal entry is not positive or p.Kp <= 0
 * (the operator is not SPD).  Synchronises the stream. */
spmv_status fem_pcg_solve(int32_t n_elem, int32_t n_dof, const int32_t *edof, const float *rho,
                          int32_t penalty, const float *Ke, const float *f, float *u, float rtol,
                          int32_t max_iter, void *workspace, size_t workspace_bytes, int32_t *iterations,
                          double *rel_residual, void *stream);

/* Largest eigenvalue of K by power iteration from v0 (device, nonzero):
 * v <- K v / ||K v||; h_lambda (host, `iterations` entries) receives the
 * Rayleigh quotient v.Kv of every normalised iterate; the last one is the
 * estimate.  Synchronises the stream. */
spmv_status fem_lambda_max(int32_t n_elem, int32_t n_dof, const int32_t *edof, const float *rho,
                           int32_t penalty, const float *Ke, const float *v0, int32_t iterations,
                           void *workspace, size_t workspace_bytes, double *h_lambda, void *stream);

/* Smallest eigenvalue of K by the same iteration on K^-1: each step solves
 * K w = v by Jacobi-PCG from zero (inner_rtol, inner_max_iter), then
 * v <- w / ||w||; h_lambda (host) receives the Rayleigh quotients v.Kv,
 * h_inner_iterations (host, optional) the PCG iterations of each step.
 * kappa(K) = lambda_max / lambda_min.  Synchronises the stream. */
spmv_status fem_lambda_min(int32_t n_elem, int32_t n_dof, const int32_t *edof, const float *rho,
                           int32_t penalty, const float *Ke, const float *v0, int32_t iterations,
                           float inner_rtol, int32_t inner_max_iter, void *workspace, size_t workspace_bytes,
                           double *h_lambda, int32_t *h_inner_iterations, void *stream);

/* ======================================================================== */
/* SpGEMM C = A * B ("Sparse matrix multiplication acceleration techniques", */
/* the hash-based multi-phase SpGEMM page, section 2): rows grouped by their */
/* intermediate products (IP = the total length of the rows of B that a row */
/* of A reaches; groups 0-31, 32-511, 512-8191, >= 8192, section 2.1.1), an */
/* allocation phase that counts each row's distinct columns with hash       */
/* tables (section 2.2), and an accumulation phase that adds the products   */
/* (section 2.3).  A is m x k, B is k x n, both CSR with int32 indices and  */
/* fp32 values on the device; columns in a row may come in any order and   */
/* repeat.  C is CSR with each row's distinct columns in increasing order;  */
/* a column that is reached is stored even when its products cancel to 0.   */
/* ======================================================================== */
typedef struct spgemm *spgemm_t;

/* Workspace bytes for spgemm_create on these A and B (device arrays).
 * Validates both (SPMV_ERR_INVALID_MATRIX for a row_ptr that is not
 * monotone from 0 to nnz or a column out of range).  scratch: device, >=
 * spmv_scratch_size(m) bytes.  Synchronises. */
spmv_status spgemm_workspace_size(int32_t m, int32_t k, int32_t n, int32_t nnz_a, const int32_t *rp_a,
                                  const int32_t *ci_a, int32_t nnz_b, const int32_t *rp_b,
                                  const int32_t *ci_b, size_t *bytes, void *scratch,
                                  size_t scratch_bytes, void *stream);

/* Grouping and allocation phase: validates, counts the distinct columns of
 * every row of C and their offsets.  The handle borrows A, B and the
 * workspace (device, 256-byte aligned, at least spgemm_workspace_size
 * bytes) until spgemm_destroy.  SPMV_ERR_OVERFLOW if nnz(C) exceeds int32.
 * Synchronises. */
spmv_status spgemm_create(spgemm_t *h, int32_t m, int32_t k, int32_t n, int32_t nnz_a, const int32_t *rp_a,
                          const int32_t *ci_a, const float *v_a, int32_t nnz_b, const int32_t *rp_b,
                          const int32_t *ci_b, const float *v_b, void *workspace, size_t workspace_bytes,
                          void *stream);

/* nnz(C), the total intermediate products, and the rows per IP group
 * (group_rows: int32[4]); any output may be NULL.  Host only. */
spmv_status spgemm_info(spgemm_t h, int64_t *nnz_c, int64_t *intermediate_products, int32_t *group_rows);

/* Accumulation phase: rp_c int32[m+1], ci_c int32[nnz(C)], v_c fp32[nnz(C)]
 * (device, caller-owned).  Uses the current values of A and B, so it may be
 * repeated after they change with the same patterns.  fp32 products summed
 * by atomic adds: values agree with the exact sum to rounding, in an order
 * that varies.  Asynchronous; allocates nothing.  The row groups run
 * concurrently on the handle's own streams, forked from and joined back into
 * `stream`; calls on one handle must not overlap. */
spmv_status spgemm_compute(spgemm_t h, int32_t *rp_c, int32_t *ci_c, float *v_c, void *stream);

/* Releases the handle (not the workspace or the borrowed arrays). */
spmv_status spgemm_destroy(spgemm_t h);

/* ======================================================================== */
/* Reference streams: the measured bandwidth a plain kernel reaches, beside  */
/* the HBM peak, as the second denominator of the roofline figures.          */
/* ======================================================================== */

/* dst[0 .. bytes) = src[0 .. bytes) with 16-byte non-temporal loads and
 * stores (bytes read + bytes written).  bytes: a multiple of 16; src and
 * dst device, 16-byte aligned, not overlapping.  Asynchronous. */
spmv_status spmv_stream_copy(const void *src, void *dst, size_t bytes, void *stream);

/* Reads src[0 .. bytes) once with 16-byte non-temporal loads and writes one
 * fp32 sum per workgroup to partial (device, partial_count floats).  The
 * kernel runs min(ceil(bytes / 4096), 8 * CUs) workgroups (at most 2048 on
 * MI355X); a partial_count below that is rejected (SPMV_ERR_INVALID_VALUE)
 * before anything is launched, and entries past it are not written.  Same
 * size and alignment rules as the copy.  Asynchronous. */
spmv_status spmv_stream_read(const void *src, size_t bytes, float *partial, size_t partial_count, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPMV_AMD_H */
