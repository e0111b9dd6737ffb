// MACKO SpMV and column decoding on gfx950.
//
// "MACKO-SpMV: GPU acceleration and storage optimisation at low sparsity",
// section 2.2: a warp owns a row and walks it in chunks; the lanes load the
// chunk's packed gap codes and values cooperatively with wide loads (2.2.1),
// rebuild absolute columns with a lane-local sum of the gaps followed by a
// warp-wide prefix sum (2.2.2), and multiply by the gathered vector (2.2.3).
// Section 3.3: the code width b is 1, 2, 4 or 8 bits, and values may be
// int8 instead of fp16.
//
// gfx950 shape: one wave64 per row, 512 entries per chunk, lane l owns
// entries 8l..8l+7 of the chunk: its 8 b-bit codes (one 4-byte load, shared
// with 4/b - 1 neighbours for b < 4, or one 8-byte load for b = 8) and its
// eight values (one 16-byte load of fp16, or one 8-byte load of int8), all
// fully coalesced.  Columns: lane-local inclusive prefix of (code + 1) over
// its 8 fields, a 6-step DPP scan of the lane totals (row shifts + row
// broadcasts), plus the carry of the row so far (the last column of the
// previous chunk, starting at -1).  x (fp16) is staged once per workgroup
// in LDS; products are fp16 x fp16 -> fp32 with v_dot2_f32_f16 (exact
// products, fp32 accumulate).  int8 values become fp16 exactly on the way:
// byte q ^ 0x80 = q + 128 placed under the fp16 exponent of 1024 is
// 1024 + q + 128, and subtracting 1152 leaves q; the row's scale multiplies
// the finished sum.  Trailing alignment entries can decode past the last
// column; they read zeros placed after x in LDS (or a clamped column when x
// stays in global memory) and their value is +0.  Workgroups are
// persistent: each wave takes rows gridDim * waves apart, so x is staged
// into LDS once per workgroup instead of once per row.
#include "common.hpp"

#include <algorithm>
#include <type_traits>

namespace spmv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

#ifndef SPMV_MK_WAVES
#define SPMV_MK_WAVES 8
#endif
constexpr int MK_WAVES = SPMV_MK_WAVES;   // waves per workgroup (2 workgroups per CU: 16 waves)
constexpr int MK_WG = 64 * MK_WAVES;
#ifndef SPMV_MK_PER_CU
#define SPMV_MK_PER_CU 2
#endif
constexpr int MK_PER_CU = SPMV_MK_PER_CU;   // workgroups per CU when x fits in 48 KB of LDS
constexpr int MK_CHUNK = 512;         // entries per wave per step (64 lanes x 8)
#ifndef SPMV_MK_UNROLL
#define SPMV_MK_UNROLL 3
#endif
constexpr int MK_UNROLL = SPMV_MK_UNROLL;   // chunks whose loads are issued together
constexpr int MK_LDS_MAX_HALFS = 32768;  // x and its zero padding in LDS: up to 64 KB

// Code layout of width BD bits.
template <int BD>
struct Fmt {
    static constexpr unsigned MASK = (1u << BD) - 1u;
    static constexpr int ALIGN = 1024 / BD;   // row alignment in entries (128 B of codes)
    // zero halfs after x in LDS: trailing alignment entries decode at most
    // ALIGN - 1 columns past the last column, and idle lanes of a row's last
    // chunk (codes zeroed) at most 8 more
    static constexpr int XPAD = ALIGN + 64;
    // a lane's 8 codes (8 BD bits): the word that holds them, or two words
    typedef typename std::conditional<BD == 8, u32x2, unsigned int>::type lane_t;
};

// a lane's 8 values: 16 bytes of fp16 or 8 bytes of int8
template <bool I8>
using vals_t = typename std::conditional<I8, u32x2, u32x4>::type;

__device__ __forceinline__ f16x2 as_h2(unsigned int w) { return __builtin_bit_cast(f16x2, w); }

__device__ __forceinline__ unsigned int zero_unless(bool keep, unsigned int w) { return keep ? w : 0u; }
__device__ __forceinline__ u32x2 zero_unless(bool keep, u32x2 w) {
    return u32x2{keep ? w.x : 0u, keep ? w.y : 0u};
}

// The codes of the 8 entries from `ent` (a multiple of 8) on.
template <int BD>
__device__ __forceinline__ typename Fmt<BD>::lane_t load_codes(const unsigned int *__restrict__ codes, int ent) {
    if constexpr (BD == 8)
        return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(codes) + (ent >> 3));
    else
        return __builtin_nontemporal_load(codes + ((ent * BD) >> 5));
}

// Lane-local inclusive prefix of (code + 1) over the lane's 8 fields.
// `shift` is the bit offset of the lane's first field in its word (b < 4).
template <int BD>
__device__ __forceinline__ void code_prefix(typename Fmt<BD>::lane_t w, int shift, int (&p)[8]) {
    int run = 0;
    if constexpr (BD == 8) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            run += (int)(((t < 4 ? w.x : w.y) >> (8 * (t & 3))) & 255u) + 1;
            p[t] = run;
        }
    } else {
        const unsigned int ws = BD < 4 ? w >> shift : w;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            run += (int)((ws >> (BD * t)) & Fmt<BD>::MASK) + 1;
            p[t] = run;
        }
    }
}

// Values of entries t, t + 1 (t even) as two fp16; zeros unless `keep`.
template <bool I8>
__device__ __forceinline__ f16x2 value_pair(const vals_t<I8> &v, int t, bool keep) {
    if constexpr (!I8) {
        return as_h2(keep ? v[t >> 1] : 0u);
    } else {
        // bytes q ^ 0x80 under the exponent byte 0x64: 1024 + (q + 128);
        // a masked word of zero bytes gives q = 0
        const unsigned int w = (keep ? v[t >> 2] : 0u) ^ 0x80808080u;
        const unsigned int h = __builtin_amdgcn_perm(0x64646464u, w, (t & 2) ? 0x04030402u : 0x04010400u);
        return as_h2(h) - f16x2{(_Float16)1152.0f, (_Float16)1152.0f};
    }
}

// The first MK_UNROLL chunks (up to MK_UNROLL * 512 entries) of [c0, e1):
// lane l holds the codes and values of entries c0 + 512 u + 8 l .. + 7 of
// chunk u.  Entries at or past e1 are not valid; apply_group masks them by
// position.
//   UNCOND: every load is issued, at a valid address: lanes past e1 re-read
//   the row's last 8 entries, and an empty range reads at `dummy` (which
//   must be readable and 16-byte aligned).  With no branches around the
//   loads the compiler can keep them in flight across later waits.
//   Otherwise lanes past e1 load nothing and hold zeros.
template <int BD, bool I8>
struct Group {
    typename Fmt<BD>::lane_t word[MK_UNROLL];
    vals_t<I8> val[MK_UNROLL];
};

template <bool UNCOND, int BD, bool I8>
__device__ __forceinline__ void load_group(Group<BD, I8> &g, const unsigned int *__restrict__ codes,
                                           const void *__restrict__ vals, int c0, int e1, int lane,
                                           const void *dummy) {
    typedef vals_t<I8> V;
    if (UNCOND) {
        const bool any = e1 > c0;   // uniform
        const unsigned int *wp = any ? codes : static_cast<const unsigned int *>(dummy);
        const V *vp = static_cast<const V *>(any ? vals : dummy);
#pragma unroll
        for (int u = 0; u < MK_UNROLL; ++u) {
            const int ent = any ? min(c0 + u * MK_CHUNK + 8 * lane, e1 - 8) : 0;
            g.word[u] = load_codes<BD>(wp, ent);
            g.val[u] = __builtin_nontemporal_load(vp + (ent >> 3));
        }
    } else {
#pragma unroll
        for (int u = 0; u < MK_UNROLL; ++u) {
            const int ent = c0 + u * MK_CHUNK + 8 * lane;
            const bool valid = ent < e1;
            g.word[u] = valid ? load_codes<BD>(codes, ent) : typename Fmt<BD>::lane_t{};
            g.val[u] = valid ? __builtin_nontemporal_load(static_cast<const V *>(vals) + (ent >> 3)) : V{};
        }
    }
}

// The 4-bit case with x in LDS, in SWAR form: the lane's 8 nibbles are
// split into even and odd fields (one per byte), the pair sums get an
// inclusive byte-wise prefix with two shifted adds, and from it the byte
// offsets 2 * (column - base) of all 8 entries come out as bytes of two
// words (at most 240 and 210: no carries between bytes).  Each LDS address
// is then one byte-select add onto 2 * base, with the constant part in the
// instruction's offset.
template <bool I8, bool MASKED>
__device__ __forceinline__ void apply_chunk_swar(unsigned int w, const vals_t<I8> &val, bool valid,
                                                 const unsigned short *xv, int &carry, float &acc) {
    // All byte sums below are doubled (2-byte x elements): at most 240.
    // The opaque steps keep the compiler from folding the shifted adds into
    // quarter-rate multiplies.
    const unsigned int lo2 = (w << 1) & 0x1E1E1E1Eu;  // 2 f0, 2 f2, 2 f4, 2 f6
    const unsigned int hi2 = (w >> 3) & 0x1E1E1E1Eu;  // 2 f1, 2 f3, 2 f5, 2 f7
    unsigned int P2 = lo2 + hi2;
    asm volatile("" : "+v"(P2));
    P2 += P2 << 8;
    asm volatile("" : "+v"(P2));
    P2 += P2 << 16;                                   // byte k: 2 (f0 + ... + f(2k+1))
    asm volatile("" : "+v"(P2));
    const unsigned int E2 = (P2 << 8) + lo2;          // byte k: 2 (f0 + ... + f(2k))
    const int tot = (!MASKED || valid) ? (int)(P2 >> 25) + 8 : 0;
    int incl = wave_inclusive_scan(tot);
    asm volatile("" : "+v"(incl));
    // byte offset in x of column base = carry + incl - tot
    const int base2 = 2 * (carry + incl - tot);
    carry += __builtin_amdgcn_readlane(incl, 63);
    const char *xb = reinterpret_cast<const char *>(xv);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        // entries 2k (column base + E_k + 2k + 1) and 2k + 1 (base + P_k + 2k + 2)
        const unsigned int xa =
            *reinterpret_cast<const unsigned short *>(xb + base2 + ((E2 >> (8 * k)) & 255u) + 2 * (2 * k + 1));
        const unsigned int xc =
            *reinterpret_cast<const unsigned short *>(xb + base2 + ((P2 >> (8 * k)) & 255u) + 2 * (2 * k + 2));
        acc = __builtin_amdgcn_fdot2(value_pair<I8>(val, 2 * k, !MASKED || valid), as_h2(xa | (xc << 16)), acc,
                                     false);
    }
}

// One chunk of 512 entries: lane-local prefix of (code + 1), wave scan of
// the lane totals plus the running carry, then 8 reads of x and 4
// v_dot2_f32_f16.  MASKED: some lanes lie past the row's end (the row's last
// chunk); their codes are taken as 0, their totals count 0 and their values
// are masked.  CLAMP: x is read from memory, so columns are clamped to the
// last column; with x in LDS they are not, because the LDS copy is followed
// by Fmt<BD>::XPAD zeros and no decoded column goes further.
template <int BD, bool I8, bool MASKED, bool CLAMP>
__device__ __forceinline__ void apply_chunk(typename Fmt<BD>::lane_t word, const vals_t<I8> &val, bool valid,
                                            int shift, int last_col, const unsigned short *xv, int &carry,
                                            float &acc) {
    if constexpr (BD == 4 && !CLAMP) {
        apply_chunk_swar<I8, MASKED>(MASKED ? zero_unless(valid, word) : word, val, valid, xv, carry, acc);
        return;
    }
    int p[8];
    code_prefix<BD>(MASKED ? zero_unless(valid, word) : word, shift, p);
    const int tot = (!MASKED || valid) ? p[7] : 0;
    int incl = wave_inclusive_scan(tot);
    // opaque, so that incl - tot is not rebuilt from the scan's partial sums
    // (that keeps every DPP step fused into its add)
    asm volatile("" : "+v"(incl));
    const int base = carry + incl - tot;
    carry += __builtin_amdgcn_readlane(incl, 63);
    // No branch on `valid`: an idle lane's columns stay inside x or its
    // padding (they are >= 0: base >= carry >= -1 and p[t] >= 1), so all 8
    // reads of every lane are issued together; its values are zero.
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
        const int ca = CLAMP ? min(base + p[t], last_col) : base + p[t];
        const int cb = CLAMP ? min(base + p[t + 1], last_col) : base + p[t + 1];
        const unsigned int xp = (unsigned int)xv[ca] | ((unsigned int)xv[cb] << 16);
        acc = __builtin_amdgcn_fdot2(value_pair<I8>(val, t, !MASKED || valid), as_h2(xp), acc, false);
    }
}

// Decodes the columns of a loaded group (continuing from `carry`, the last
// column decoded so far in the row) and accumulates value * x[column].
template <bool CLAMP, int BD, bool I8>
__device__ __forceinline__ void apply_group(const Group<BD, I8> &g, int c0, int e1, int lane, int shift,
                                            int last_col, const unsigned short *xv, int &carry, float &acc) {
#pragma unroll
    for (int u = 0; u < MK_UNROLL; ++u) {
        const int cs = c0 + u * MK_CHUNK;
        if (cs >= e1) break;   // uniform
        if (cs + MK_CHUNK <= e1)   // uniform: the whole chunk is inside the row
            apply_chunk<BD, I8, false, CLAMP>(g.word[u], g.val[u], true, shift, last_col, xv, carry, acc);
        else
            apply_chunk<BD, I8, true, CLAMP>(g.word[u], g.val[u], cs + 8 * lane < e1, shift, last_col, xv, carry,
                                             acc);
    }
    // Consume every register of the group, also of chunks past the row's
    // end, so that no load into them is still outstanding when they are
    // reloaded (that would make the compiler wait for every younger load,
    // the prefetched group included).
#pragma unroll
    for (int u = 0; u < MK_UNROLL; ++u) asm volatile("" ::"v"(g.word[u]), "v"(g.val[u]));
}

// Wave w of the grid owns rows w, w + W, w + 2W, ... (W waves in all).  Its
// row bounds (and, for int8 values, row scales) are read up front, one row
// per lane (64 rows at a time), so the stream loads of a row never wait for
// a row_ptr load; the first group of the first row is in flight while x is
// staged into LDS, and the next group (of the same row, or of the wave's
// next row) is in flight while the current one is decoded and multiplied.
// XM: 0 = x read from global memory; 1 = x staged into LDS with 16-byte
// copies (x 16-byte aligned, n_cols >= 8); 2 = x staged element by element.
template <int XM, int BD, bool I8>
__global__ __launch_bounds__(MK_WG) void k_macko_spmv(int n_rows, int n_cols, const int *__restrict__ mrp,
                                                      const unsigned int *__restrict__ codes,
                                                      const void *__restrict__ vals,
                                                      const float *__restrict__ row_scale, float alpha,
                                                      const unsigned short *__restrict__ x, float beta,
                                                      float *__restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) unsigned short xs_dyn[];
    const int lane = __lane_id();
    // bit offset of the lane's first code in its word: rows start on
    // 1024-bit boundaries and chunks are 512 entries, so it depends on the
    // lane alone
    const int shift = BD < 4 ? (8 * BD * lane) & 31 : 0;
    // wave-uniform, stated so that row indices and bounds are scalar
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int stride = gridDim.x * MK_WAVES;
    const int first = blockIdx.x * MK_WAVES + wv;
    const int nk = first < n_rows ? (n_rows - 1 - first) / stride + 1 : 0;   // rows of this wave

    // bounds (and scales) of the wave's rows 0..63, one per lane
    int bs = 0, be = 0;
    float rs = 1.0f;
    if (lane < nk) {
        const int r = first + lane * stride;
        bs = mrp[r];
        be = mrp[r + 1];
        if (I8) rs = row_scale[r];
    }
    // x: the first pass of the LDS copy is loaded now and stored later
    // (loads at clamped addresses, so they need no branch)
    constexpr int XU = 4;
    const int n8 = XM == 1 ? (n_cols & ~7) : 0;
    const int xstride = 8 * MK_WG;
    u32x4 xr[XU];
    if (XM == 1) {
#pragma unroll
        for (int u = 0; u < XU; ++u)
            xr[u] = *reinterpret_cast<const u32x4 *>(x + min(8 * (int)threadIdx.x + u * xstride, n8 - 8));
    }
    int b0 = __builtin_amdgcn_readlane(bs, 0), b1 = __builtin_amdgcn_readlane(be, 0);
    Group<BD, I8> g;
    load_group<XM == 1>(g, codes, vals, b0, nk > 0 ? b1 : 0, lane, x);
    if (XM != 0) {
        if (XM == 1) {
            // clamped like the loads: threads past the end store the last
            // vector again, with the same data
#pragma unroll
            for (int u = 0; u < XU; ++u)
                *reinterpret_cast<u32x4 *>(xs_dyn + min(8 * (int)threadIdx.x + u * xstride, n8 - 8)) = xr[u];
            for (int k = 8 * (int)threadIdx.x + XU * xstride; k < n8; k += xstride)
                *reinterpret_cast<u32x4 *>(xs_dyn + k) = *reinterpret_cast<const u32x4 *>(x + k);
        }
        for (int k = n8 + (int)threadIdx.x; k < n_cols; k += MK_WG) xs_dyn[k] = x[k];
        // zeros after x for the decoded columns of trailing alignment
        // entries and of idle lanes, which are not clamped
        for (int k = n_cols + (int)threadIdx.x; k < n_cols + Fmt<BD>::XPAD; k += MK_WG) xs_dyn[k] = 0;
        // an LDS-only barrier: the stream loads issued above stay in flight
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
    const unsigned short *xv = XM != 0 ? xs_dyn : x;
    const int last_col = n_cols - 1;

    // Rows are taken in batches of 64 (one per lane for bounds and sums).
    // Within a batch there is one step per group; two Group buffers take
    // turns as current and prefetched, so no loaded data is ever copied
    // between registers (a copy would have to wait for its load), and the
    // loop has no stores (with a store in the loop the compiler waits for
    // every outstanding load at the loop head).  Row sums are collected in
    // `res` (lane l: row l of the batch) and stored after the batch.
    Group<BD, I8> g2;
    for (int kb = 0; kb < nk; kb += 64) {
        const int cnt = min(64, nk - kb);
        if (kb > 0) {
            // bounds of the batch's rows, then its first group
            bs = be = 0;
            if (lane < cnt) {
                const int r = first + (kb + lane) * stride;
                bs = mrp[r];
                be = mrp[r + 1];
                if (I8) rs = row_scale[r];
            }
            b0 = __builtin_amdgcn_readlane(bs, 0);
            b1 = __builtin_amdgcn_readlane(be, 0);
            load_group<XM == 1>(g, codes, vals, b0, b1, lane, x);
        }
        int k = 0;               // row of the batch being reduced
        int c0 = b0, e1 = b1;    // current group start, current row end
        int nb0 = 0, nb1 = 0;    // bounds of row k + 1
        if (cnt > 1) {
            nb0 = __builtin_amdgcn_readlane(bs, 1);
            nb1 = __builtin_amdgcn_readlane(be, 1);
        }
        int carry = -1;
        float acc = 0.0f, res = 0.0f;
        // steps of the batch: one per group of each row, one for an empty row
        const int len = be - bs;
        const int nsteps = wave_sum_int(lane < cnt ? max(1, (len + MK_CHUNK * MK_UNROLL - 1) / (MK_CHUNK * MK_UNROLL)) : 0);
        auto step = [&](const Group<BD, I8> &cur, Group<BD, I8> &nxt) {
            const int c1 = c0 + MK_CHUNK * MK_UNROLL;
            const bool row_done = c1 >= e1;
            load_group<XM == 1>(nxt, codes, vals, row_done ? nb0 : c1, row_done ? nb1 : e1, lane, x);
            apply_group<XM == 0>(cur, c0, e1, lane, shift, last_col, xv, carry, acc);
            if (!row_done) {
                c0 = c1;
            } else {
                const float sum = wave_sum(acc);
                if (lane == k) res = sum;
                acc = 0.0f;
                carry = -1;
                ++k;
                c0 = nb0;
                e1 = nb1;
                nb0 = nb1 = 0;
                if (k + 1 < cnt) {
                    nb0 = __builtin_amdgcn_readlane(bs, k + 1);
                    nb1 = __builtin_amdgcn_readlane(be, k + 1);
                }
            }
        };
        // no exit inside the loop body: an early exit there would give the
        // compiler a path on which the prefetched loads reach the loop head
        // unwaited, and it would then wait for them on every iteration
        int i = 0;
        for (; i + 1 < nsteps; i += 2) {
            step(g, g2);
            step(g2, g);
        }
        if (i < nsteps) step(g, g2);
        if (lane < cnt) {
            const int row = first + (kb + lane) * stride;
            float r = alpha * (I8 ? res * rs : res);
            if (beta != 0.0f) r = fmaf(beta, y[row], r);
            y[row] = r;
        }
        // s_waitcnt vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt left at their
        // maxima): the store is complete before the next batch, so the
        // compiler sees no outstanding store at the head of the step loop
        __builtin_amdgcn_s_waitcnt(0x0F70);
    }
}

// Writes the column of every stored entry, with the same decoder.
template <int BD>
__global__ __launch_bounds__(MK_WG) void k_macko_decode(int n_rows, const int *__restrict__ mrp,
                                                        const unsigned int *__restrict__ codes,
                                                        int *__restrict__ cols) {
    const int lane = __lane_id();
    const int shift = BD < 4 ? (8 * BD * lane) & 31 : 0;
    const int wv = threadIdx.x / 64;
    for (int row = blockIdx.x * MK_WAVES + wv; row < n_rows; row += gridDim.x * MK_WAVES) {
        const int e0 = mrp[row], e1 = mrp[row + 1];
        int carry = -1;
        for (int c0 = e0; c0 < e1; c0 += MK_CHUNK) {
            const int ent = c0 + 8 * lane;
            const bool valid = ent < e1;
            int p[8];
            code_prefix<BD>(valid ? load_codes<BD>(codes, ent) : typename Fmt<BD>::lane_t{}, shift, p);
            const int tot = valid ? p[7] : 0;
            const int incl = wave_inclusive_scan(tot);
            const int base = carry + incl - tot;
            carry += __builtin_amdgcn_readlane(incl, 63);
            if (valid) {
#pragma unroll
                for (int t = 0; t < 8; ++t) cols[ent + t] = base + p[t];
            }
        }
    }
}

int persistent_grid(int n_rows, int per_cu) {
    const int want = (int)ceil_div(n_rows, MK_WAVES);
    return std::max(1, std::min(want, per_cu * device_cu_count()));
}

bool width_ok(int32_t b) { return b == 1 || b == 2 || b == 4 || b == 8; }

template <int BD, bool I8>
void launch_spmv(int32_t n_rows, int32_t n_cols, const int32_t *mrow_ptr, const uint32_t *codes, const void *vals,
                 const float *row_scale, float alpha, const uint16_t *x, float beta, float *y, hipStream_t st) {
    const int64_t halfs = ((int64_t)n_cols + Fmt<BD>::XPAD + 7) & ~int64_t(7);
    if (halfs <= MK_LDS_MAX_HALFS) {
        const size_t lds = (size_t)halfs * sizeof(uint16_t);
        // as many workgroups per CU as the LDS allows, at most 2
        const int per_cu = lds <= 48 * 1024 ? MK_PER_CU : 1;
        const int grid = persistent_grid(n_rows, per_cu);
        if (aligned16(x) && n_cols >= 8)
            k_macko_spmv<1, BD, I8><<<grid, MK_WG, lds, st>>>(n_rows, n_cols, mrow_ptr, codes, vals, row_scale,
                                                              alpha, x, beta, y);
        else
            k_macko_spmv<2, BD, I8><<<grid, MK_WG, lds, st>>>(n_rows, n_cols, mrow_ptr, codes, vals, row_scale,
                                                              alpha, x, beta, y);
    } else {
        k_macko_spmv<0, BD, I8><<<persistent_grid(n_rows, 2), MK_WG, 0, st>>>(n_rows, n_cols, mrow_ptr, codes, vals,
                                                                              row_scale, alpha, x, beta, y);
    }
}

template <bool I8>
spmv_status macko_apply(int32_t n_rows, int32_t n_cols, int32_t bdelta, const int32_t *mrow_ptr,
                        const uint32_t *codes, const void *vals, const float *row_scale, float alpha,
                        const uint16_t *x_f16, float beta, float *y, void *stream) {
    if (n_rows < 0 || n_cols < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if (!width_ok(bdelta)) return fail(SPMV_ERR_INVALID_VALUE, "code width %d is not 1, 2, 4 or 8", bdelta);
    if (n_rows == 0) return SPMV_OK;
    if (!mrow_ptr || !y) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    if (n_cols == 0) return fail(SPMV_ERR_INVALID_VALUE, "n_cols must be positive when there are rows");
    if (!codes || !vals || !x_f16 || (I8 && !row_scale)) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    const uintptr_t va = reinterpret_cast<uintptr_t>(vals), ca = reinterpret_cast<uintptr_t>(codes);
    if ((va & (I8 ? 7u : 15u)) || (ca & (bdelta == 8 ? 7u : 3u)))
        return fail(SPMV_ERR_UNSUPPORTED, I8 ? "q must be 8-byte aligned and codes %d-byte aligned"
                                             : "mvals must be 16-byte aligned and codes %d-byte aligned",
                    bdelta == 8 ? 8 : 4);
    hipStream_t st = as_stream(stream);
    switch (bdelta) {
        case 1: launch_spmv<1, I8>(n_rows, n_cols, mrow_ptr, codes, vals, row_scale, alpha, x_f16, beta, y, st); break;
        case 2: launch_spmv<2, I8>(n_rows, n_cols, mrow_ptr, codes, vals, row_scale, alpha, x_f16, beta, y, st); break;
        case 4: launch_spmv<4, I8>(n_rows, n_cols, mrow_ptr, codes, vals, row_scale, alpha, x_f16, beta, y, st); break;
        default: launch_spmv<8, I8>(n_rows, n_cols, mrow_ptr, codes, vals, row_scale, alpha, x_f16, beta, y, st); break;
    }
    SPMV_LAUNCHED("k_macko_spmv");
    return SPMV_OK;
}

}  // namespace
}  // namespace spmv

using namespace spmv;

extern "C" spmv_status macko_spmv(int32_t n_rows, int32_t n_cols, int32_t bdelta, const int32_t *mrow_ptr,
                                  const uint32_t *codes, const uint16_t *mvals, float alpha, const uint16_t *x_f16,
                                  float beta, float *y, void *stream) {
    return macko_apply<false>(n_rows, n_cols, bdelta, mrow_ptr, codes, mvals, nullptr, alpha, x_f16, beta, y, stream);
}

extern "C" spmv_status macko_spmv_i8(int32_t n_rows, int32_t n_cols, int32_t bdelta, const int32_t *mrow_ptr,
                                     const uint32_t *codes, const int8_t *q, const float *row_scale, float alpha,
                                     const uint16_t *x_f16, float beta, float *y, void *stream) {
    return macko_apply<true>(n_rows, n_cols, bdelta, mrow_ptr, codes, q, row_scale, alpha, x_f16, beta, y, stream);
}

extern "C" spmv_status macko_decode_columns(int32_t n_rows, int32_t bdelta, const int32_t *mrow_ptr,
                                            const uint32_t *codes, int32_t *cols_out, void *stream) {
    if (n_rows < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if (!width_ok(bdelta)) return fail(SPMV_ERR_INVALID_VALUE, "code width %d is not 1, 2, 4 or 8", bdelta);
    if (n_rows == 0) return SPMV_OK;
    if (!mrow_ptr || !codes || !cols_out) return fail(SPMV_ERR_INVALID_VALUE, "NULL pointer");
    if (bdelta == 8 && (reinterpret_cast<uintptr_t>(codes) & 7u))
        return fail(SPMV_ERR_UNSUPPORTED, "codes must be 8-byte aligned");
    hipStream_t st = as_stream(stream);
    const int grid = persistent_grid(n_rows, 4);
    switch (bdelta) {
        case 1: k_macko_decode<1><<<grid, MK_WG, 0, st>>>(n_rows, mrow_ptr, codes, cols_out); break;
        case 2: k_macko_decode<2><<<grid, MK_WG, 0, st>>>(n_rows, mrow_ptr, codes, cols_out); break;
        case 4: k_macko_decode<4><<<grid, MK_WG, 0, st>>>(n_rows, mrow_ptr, codes, cols_out); break;
        default: k_macko_decode<8><<<grid, MK_WG, 0, st>>>(n_rows, mrow_ptr, codes, cols_out); break;
    }
    SPMV_LAUNCHED("k_macko_decode");
    return SPMV_OK;
}
