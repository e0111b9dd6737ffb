// Hash-based multi-phase SpGEMM, C = A * B (CSR, fp32), on gfx950.
//
// "Sparse matrix multiplication acceleration techniques" (the hash-based
// multi-phase SpGEMM page), section 2: rows of A are first grouped by their
// intermediate products (IP: the total length of the rows of B they reach,
// section 2.1.1: 0-31, 32-511, 512-8191, >= 8192); an allocation phase
// counts each row's distinct output columns with a hash table (section 2.2),
// and an accumulation phase inserts the products again, adding values
// (section 2.3: linear probing, -1 for an empty slot, compare-and-swap to
// claim a slot, atomic add of the product).  Light rows share a wave, a few
// lanes per row (PWPR, section 2.2.1); heavier rows get a workgroup each
// (TBPR, section 2.2.2) with its table in LDS; the heaviest fall back to a
// table in global memory (section 2.3).
//
// gfx950 shape (the page's group 2 is split into four bins by table size,
// so that lighter rows take smaller workgroups and less LDS, and more of
// them fit on a CU):
//   bin 0 = group 0 (IP < 32): 4 lanes per row, 128 rows per 512-thread
//     workgroup, a 64-slot table per row in LDS (keys and values: 64 KB);
//   bin 1 = group 1 (IP < 512): a 256-thread workgroup per row, <= 1024 slots;
//   bins 2-5 = group 2 (IP < 1024 / 2048 / 4096 / 8192): 256 / 512 / 1024 /
//     1024 threads per row and 2048 / 4096 / 8192 / 16384 slots (16 to 128
//     KB of LDS with the values; gfx950 has 160 KB per CU);
//   bin 6 = group 3: a 1024-thread workgroup per row, its table in the
//     caller's workspace.
// Rows are binned by a stable counting sort (per-workgroup counts, one scan,
// a scatter with ranks from wave ballots), which gives the page's Map[]
// without contended atomics.
// Every table has the smallest power of two >= 2 IP slots (at least 64), so
// it is at most half full: the page's 8192-slot table for group 2 could be
// filled to the last slot, where linear probing takes thousands of steps
// (measured: 10 ms of the 18 ms accumulation phase on the power-law square),
// so group 2 gets 16384 slots at most.  Sizing each table to its row also
// keeps the clearing and the sort proportional to the row.
// In the workgroup mappings each thread walks the B rows of short reach (at
// most SG_SHORT_B entries) of its entries of A's row, and whole waves walk
// the longer ones, lanes over the B row.  Tables are powers of two, the
// hash of column c is (c * 2654435761) mod size, and no table can fill
// (distinct columns <= IP < size), so every probe sequence ends; each is
// still bounded by the table size.  The accumulation phase then writes the
// row in increasing column order: group 0 ranks each key against its table;
// the LDS-table bins move the table's entries to its front and sort those
// (bitonic); a global-table row compacts its table into C's row, sorts runs
// of G3_CH entries in LDS and merges them along merge paths.  The bins of a
// phase run concurrently on side streams.  Values add up in fp32 through
// atomics, so their low bits vary from run to run; the pattern does not.
#include "common.hpp"

#include <algorithm>
#include <array>
#include <climits>
#include <map>
#include <mutex>
#include <vector>

namespace spmv {
namespace {

constexpr int SG_B1 = 32, SG_B2 = 512, SG_B3 = 8192;   // IP group bounds (page)
constexpr int SG_NBIN = 7;                             // bins (above)
constexpr int SG_ROWS_PER_WG = 1024;                   // rows per workgroup in the binning passes
constexpr int G0_LANES = 4;                            // PWPR lanes per row
constexpr int G0_WG = 512;
constexpr int G0_ROWS = G0_WG / G0_LANES;              // rows per workgroup
constexpr int G0_T = 64;                               // slots per row (IP <= 31)
constexpr int G3_WG = 1024;
constexpr int G3_CH = 16384;                           // LDS chunk of the global-table sort (128 KB)
constexpr unsigned SG_EMPTY = 0xFFFFFFFFu;
constexpr unsigned SG_MUL = 2654435761u;
constexpr int SG_SCAN_WG = 1024;

enum { SG_ERR_ROWS = 1, SG_ERR_COLS_A = 2, SG_ERR_COLS_B = 4, SG_ERR_PROBE = 8 };

__device__ __forceinline__ unsigned sg_slot(int key, unsigned mask) { return ((unsigned)key * SG_MUL) & mask; }

// Table slots for a row: the smallest power of two >= 2 * ip, at least 64.
__host__ __device__ __forceinline__ int64_t g3_table(int64_t ip) {
    int64_t t = 64;
    while (t < 2 * ip) t <<= 1;
    return t;
}

// ---- validation and intermediate products ----

// row_ptr: rp[0] = 0, non-decreasing, rp[m] = nnz.
__global__ void k_sg_check_rows(int m, int nnz, const int *__restrict__ rp, int *err) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i > m) return;
    bool ok = true;
    if (i == 0) ok = rp[0] == 0;
    else ok = rp[i] >= rp[i - 1];
    if (i == m) ok = ok && rp[m] == nnz;
    if (!ok) atomicOr(err, SG_ERR_ROWS);
}

__global__ void k_sg_check_cols(int nnz, const int *__restrict__ ci, int n_cols, int flag, int *err) {
    bool ok = true;
    for (int j = blockIdx.x * 256 + threadIdx.x; j < nnz; j += gridDim.x * 256)
        ok = ok && (unsigned)ci[j] < (unsigned)n_cols;
    if (!ok) atomicOr(err, flag);
}

struct IpTotals {
    unsigned long long g3_slots;   // sum of the global tables' slots
    unsigned long long ip;         // total intermediate products
    int counts[SG_NBIN];           // rows per bin
};

__device__ __forceinline__ unsigned long long sg_wave_sum(unsigned long long v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__host__ __device__ __forceinline__ int sg_bin(long long ip) {
    return ip < SG_B1 ? 0 : ip < SG_B2 ? 1 : ip < 1024 ? 2 : ip < 2048 ? 3 : ip < 4096 ? 4 : ip < SG_B3 ? 5 : 6;
}

// IP of every row (optional output); per workgroup, the rows of each bin
// (bcnt[bin * nwg + wg], when given); totals by one set of atomic adds per
// workgroup.  Workgroup wg covers rows [wg, wg + 1) * SG_ROWS_PER_WG; 16
// lanes per row stride over it, so a long row does not hold up its wave.
constexpr int IP_LANES = 16;
__global__ __launch_bounds__(256) void k_sg_ip(int m, const int *__restrict__ rpa, const int *__restrict__ cia,
                                               const int *__restrict__ rpb, long long *__restrict__ ip,
                                               int *__restrict__ bcnt, IpTotals *tot) {
    __shared__ unsigned long long red[2][4];
    __shared__ int cnt_s[SG_NBIN];
    if (threadIdx.x < SG_NBIN) cnt_s[threadIdx.x] = 0;
    __syncthreads();
    const int sub = threadIdx.x % IP_LANES;
    const int r0 = blockIdx.x * SG_ROWS_PER_WG;
    const int r1 = min(m, r0 + SG_ROWS_PER_WG);
    unsigned long long ips = 0, slots = 0;
    for (int i = r0 + (int)threadIdx.x / IP_LANES; i < r1; i += 256 / IP_LANES) {
        long long s = 0;
        for (int j = rpa[i] + sub; j < rpa[i + 1]; j += IP_LANES) {
            const int k = cia[j];
            s += rpb[k + 1] - rpb[k];
        }
        for (int off = IP_LANES / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, IP_LANES);
        if (sub == 0) {
            if (ip) ip[i] = s;
            const int b = sg_bin(s);
            atomicAdd(&cnt_s[b], 1);   // LDS
            ips += (unsigned long long)s;
            if (b == SG_NBIN - 1) slots += (unsigned long long)g3_table(s);
        }
    }
    ips = sg_wave_sum(ips);
    slots = sg_wave_sum(slots);
    if (__lane_id() == 0) {
        red[0][threadIdx.x / 64] = ips;
        red[1][threadIdx.x / 64] = slots;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned long long a = red[0][0] + red[0][1] + red[0][2] + red[0][3];
        const unsigned long long b = red[1][0] + red[1][1] + red[1][2] + red[1][3];
        if (a) atomicAdd(&tot->ip, a);
        if (b) atomicAdd(&tot->g3_slots, b);
        for (int q = 0; q < SG_NBIN; ++q) {
            if (cnt_s[q]) atomicAdd(&tot->counts[q], cnt_s[q]);
            if (bcnt) bcnt[q * gridDim.x + blockIdx.x] = cnt_s[q];
        }
    }
}

// Exclusive scan of the per-workgroup counts of every bin, in place
// (one workgroup).
__global__ __launch_bounds__(SG_SCAN_WG) void k_sg_bin_offsets(int nwg, int *__restrict__ bcnt) {
    __shared__ int part[SG_SCAN_WG];
    for (int q = 0; q < SG_NBIN; ++q) {
        int *c = bcnt + (size_t)q * nwg;
        int carry = 0;
        for (int c0 = 0; c0 < nwg; c0 += SG_SCAN_WG) {
            const int r = c0 + (int)threadIdx.x;
            const int t = r < nwg ? c[r] : 0;
            part[threadIdx.x] = t;
            __syncthreads();
            for (int d = 1; d < SG_SCAN_WG; d <<= 1) {
                const int v = threadIdx.x >= (unsigned)d ? part[threadIdx.x - d] : 0;
                __syncthreads();
                part[threadIdx.x] += v;
                __syncthreads();
            }
            if (r < nwg) c[r] = carry + part[threadIdx.x] - t;
            const int last = part[SG_SCAN_WG - 1];
            __syncthreads();
            carry += last;
        }
    }
}

// The page's Map[]: the rows of every bin, bin after bin, in row order
// inside a bin.  Workgroup wg scatters its rows (as in k_sg_ip) to
// base[bin] + boff[bin * nwg + wg] + their rank among its rows of that bin.
__global__ __launch_bounds__(256) void k_sg_map(int m, const long long *__restrict__ ip, const int *__restrict__ base,
                                                const int *__restrict__ boff, int *__restrict__ map) {
    __shared__ int wcnt[4][SG_NBIN];
    __shared__ int carry[SG_NBIN];
    if (threadIdx.x < SG_NBIN) carry[threadIdx.x] = 0;
    const int lane = __lane_id(), wv = threadIdx.x / 64;
    const unsigned long long below = (1ull << lane) - 1ull;
    const int r0 = blockIdx.x * SG_ROWS_PER_WG;
    const int r1 = min(m, r0 + SG_ROWS_PER_WG);
    for (int p0 = r0; p0 < r1; p0 += 256) {
        const int i = p0 + (int)threadIdx.x;
        const int b = i < r1 ? sg_bin(ip[i]) : -1;
        int rank = 0;
        __syncthreads();   // carry of the previous pass is complete
#pragma unroll
        for (int q = 0; q < SG_NBIN; ++q) {
            const unsigned long long mask = __ballot(b == q);
            if (b == q) rank = __popcll(mask & below);
            if (lane == 0) wcnt[wv][q] = __popcll(mask);
        }
        __syncthreads();
        if (b >= 0) {
            int before = carry[b];
            for (int w = 0; w < wv; ++w) before += wcnt[w][b];
            map[base[b] + boff[b * gridDim.x + blockIdx.x] + before + rank] = i;
        }
        __syncthreads();
        if (threadIdx.x < SG_NBIN)
            carry[threadIdx.x] += wcnt[0][threadIdx.x] + wcnt[1][threadIdx.x] + wcnt[2][threadIdx.x] +
                                  wcnt[3][threadIdx.x];
    }
}

// Table offsets (in slots) of the n3 group-3 rows, in list order: one
// workgroup, an exclusive scan in chunks of SG_SCAN_WG.
__global__ __launch_bounds__(SG_SCAN_WG) void k_sg_g3_offsets(int n3, const int *__restrict__ map3,
                                                              const long long *__restrict__ ip,
                                                              long long *__restrict__ off) {
    __shared__ long long part[SG_SCAN_WG];
    long long carry = 0;
    for (int c0 = 0; c0 < n3; c0 += SG_SCAN_WG) {
        const int r = c0 + (int)threadIdx.x;
        const long long t = r < n3 ? g3_table(ip[map3[r]]) : 0;
        part[threadIdx.x] = t;
        __syncthreads();
        for (int d = 1; d < SG_SCAN_WG; d <<= 1) {
            const long long v = threadIdx.x >= (unsigned)d ? part[threadIdx.x - d] : 0;
            __syncthreads();
            part[threadIdx.x] += v;
            __syncthreads();
        }
        if (r < n3) off[r] = carry + part[threadIdx.x] - t;
        const long long last = part[SG_SCAN_WG - 1];
        __syncthreads();
        carry += last;
    }
    if (threadIdx.x == 0) off[n3] = carry;
}

// ---- hash tables ----

// Inserts key (symbolic: counts a new key in *count).  Returns false only if
// the bounded probe sequence found no slot (cannot happen for the table
// sizes used).
template <typename KeyPtr>
__device__ __forceinline__ bool sg_insert_key(KeyPtr keys, unsigned mask, int key, int *count) {
    unsigned s = sg_slot(key, mask);
    for (unsigned p = 0; p <= mask; ++p) {
        const unsigned cur = keys[s];
        if (cur == (unsigned)key) return true;
        if (cur == SG_EMPTY) {
            const unsigned old = atomicCAS(&keys[s], SG_EMPTY, (unsigned)key);
            if (old == SG_EMPTY) {
                atomicAdd(count, 1);
                return true;
            }
            if (old == (unsigned)key) return true;
        }
        s = (s + 1) & mask;
    }
    return false;
}

// Inserts key and adds v to its value.
template <typename KeyPtr, typename ValPtr>
__device__ __forceinline__ bool sg_insert_add(KeyPtr keys, ValPtr vals, unsigned mask, int key, float v) {
    unsigned s = sg_slot(key, mask);
    for (unsigned p = 0; p <= mask; ++p) {
        const unsigned cur = keys[s];
        if (cur == (unsigned)key) {
            atomicAdd(&vals[s], v);
            return true;
        }
        if (cur == SG_EMPTY) {
            const unsigned old = atomicCAS(&keys[s], SG_EMPTY, (unsigned)key);
            if (old == SG_EMPTY || old == (unsigned)key) {
                atomicAdd(&vals[s], v);
                return true;
            }
        }
        s = (s + 1) & mask;
    }
    return false;
}

// Bitonic sort of T (a power of two) key/value pairs by unsigned key, by
// the whole workgroup (WG threads); empty slots (all ones) end up last.
template <int WG, typename KeyPtr, typename ValPtr>
__device__ void sg_bitonic(KeyPtr keys, ValPtr vals, unsigned T) {
    for (unsigned k = 2; k <= T; k <<= 1) {
        for (unsigned j = k >> 1; j > 0; j >>= 1) {
            for (unsigned i = threadIdx.x; i < T; i += WG) {
                const unsigned l = i ^ j;
                if (l > i) {
                    const unsigned a = keys[i], b = keys[l];
                    const bool up = (i & k) == 0;
                    if ((a > b) == up) {
                        keys[i] = b;
                        keys[l] = a;
                        const float va = vals[i];
                        vals[i] = vals[l];
                        vals[l] = va;
                    }
                }
            }
            __syncthreads();
        }
    }
}

// Calls f(j, t) for every intermediate product a_j * b_t of row `row` of A
// (j: entry of A's row, t: entry of the row of B it reaches), by a whole
// workgroup of WG threads.  Each thread first takes whole entries of A's row
// and walks their B rows itself when they are short (at most SG_SHORT_B
// entries), so a row of many short B rows costs one round of dependent
// loads instead of one per entry; entries with longer B rows go to an LDS
// list (`defer`, SG_DEFER slots, `ndefer` zeroed by the caller before a
// barrier) and are then walked by whole waves, lanes over the B row.  An
// entry that finds the list full is walked by its thread.
constexpr int SG_SHORT_B = 4;
constexpr int SG_DEFER = 1024;

template <int WG, typename F>
__device__ __forceinline__ void sg_walk(int row, const int *__restrict__ rpa, const int *__restrict__ cia,
                                        const int *__restrict__ rpb, int *defer, int *ndefer, F &&f) {
    const int a0 = rpa[row], a1 = rpa[row + 1];
    for (int j = a0 + (int)threadIdx.x; j < a1; j += WG) {
        const int k = cia[j];
        const int t0 = rpb[k], t1 = rpb[k + 1];
        if (t1 - t0 > SG_SHORT_B) {
            const int at = atomicAdd(ndefer, 1);
            if (at < SG_DEFER) {
                defer[at] = j;
                continue;
            }
        }
        for (int t = t0; t < t1; ++t) f(j, t);
    }
    __syncthreads();
    const int nd = min(*ndefer, SG_DEFER);
    const int wv = threadIdx.x / 64, lane = threadIdx.x % 64;
    for (int q = wv; q < nd; q += WG / 64) {
        const int j = defer[q];
        const int k = cia[j];
        for (int t = rpb[k] + lane; t < rpb[k + 1]; t += 64) f(j, t);
    }
}

// Moves the non-empty slots of an LDS hash table of T <= PER * WG slots to
// its front (in any order), pads them with empty slots up to P, the
// smallest power of two >= their count (at least 64), and returns P: the
// sort then works on P slots instead of the whole, at most half-full, table.
template <int WG, int PER>
__device__ unsigned sg_compact(unsigned *keys, float *vals, unsigned T, int *counter) {
    const int lane = __lane_id();
    const unsigned long long below = (1ull << lane) - 1ull;
    unsigned k[PER];
    float v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const unsigned s = threadIdx.x + i * WG;
        k[i] = s < T ? keys[s] : SG_EMPTY;
        v[i] = s < T ? vals[s] : 0.0f;
    }
    if (threadIdx.x == 0) *counter = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const bool has = k[i] != SG_EMPTY;
        const unsigned long long bal = __ballot(has);
        int at = 0;
        if (lane == 0 && bal) at = atomicAdd(counter, __popcll(bal));
        at = __shfl(at, 0) + __popcll(bal & below);
        if (has) {
            keys[at] = k[i];
            vals[at] = v[i];
        }
    }
    __syncthreads();
    const unsigned n = (unsigned)*counter;
    unsigned P = 64;
    while (P < n) P <<= 1;
    for (unsigned s = n + threadIdx.x; s < P; s += WG) {
        keys[s] = SG_EMPTY;
        vals[s] = 0.0f;
    }
    __syncthreads();
    return P;
}

// Merges the sorted runs a[0, la) and b[0, lb) (distinct keys) into
// out[0, la + lb) with the whole workgroup: thread t writes the outputs
// t * per .. (t + 1) * per - 1, starting where the merge path crosses that
// diagonal (found by binary search), so no thread waits for another.
template <int WG>
__device__ void sg_merge(const unsigned *ak, const float *av, int la, const unsigned *bk, const float *bv, int lb,
                         unsigned *ok, float *ov) {
    const int n = la + lb;
    const int per = (n + WG - 1) / WG;
    const int d0 = min(n, (int)threadIdx.x * per), d1 = min(n, d0 + per);
    if (d0 >= d1) return;
    // i = how many of the first d0 outputs come from a
    int lo = max(0, d0 - lb), hi = min(d0, la);
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (ak[mid] < bk[d0 - 1 - mid]) lo = mid + 1;
        else hi = mid;
    }
    int i = lo, j = d0 - lo;
    for (int d = d0; d < d1; ++d) {
        const bool from_a = j >= lb || (i < la && ak[i] < bk[j]);
        if (from_a) {
            ok[d] = ak[i];
            ov[d] = av[i];
            ++i;
        } else {
            ok[d] = bk[j];
            ov[d] = bv[j];
            ++j;
        }
    }
}

// ---- group 0: PWPR, 4 lanes per row ----

// Allocation phase: distinct columns of each row into cnt[row].
__global__ __launch_bounds__(G0_WG) void k_sg_g0_count(int n0, const int *__restrict__ map0,
                                                       const int *__restrict__ rpa, const int *__restrict__ cia,
                                                       const int *__restrict__ rpb, const int *__restrict__ cib,
                                                       int *__restrict__ cnt, int *err) {
    __shared__ unsigned keys[G0_ROWS][G0_T];
    __shared__ int counts[G0_ROWS];
    const int r = threadIdx.x / G0_LANES, lane = threadIdx.x % G0_LANES;
    for (int s = lane; s < G0_T; s += G0_LANES) keys[r][s] = SG_EMPTY;
    if (lane == 0) counts[r] = 0;
    __syncthreads();
    const int li = blockIdx.x * G0_ROWS + r;
    const int row = li < n0 ? map0[li] : -1;
    bool ok = true;
    if (row >= 0) {
        for (int j = rpa[row] + lane; j < rpa[row + 1]; j += G0_LANES) {
            const int k = cia[j];
            for (int t = rpb[k]; t < rpb[k + 1]; ++t) ok = ok && sg_insert_key(&keys[r][0], G0_T - 1, cib[t], &counts[r]);
        }
    }
    if (!ok) atomicOr(err, SG_ERR_PROBE);
    __syncthreads();
    if (row >= 0 && lane == 0) cnt[row] = counts[r];
}

// Accumulation phase: products added per column, then each key written at
// its rank among the row's keys (increasing columns) from rpc[row] on.
__global__ __launch_bounds__(G0_WG) void k_sg_g0_fill(int n0, const int *__restrict__ map0,
                                                      const int *__restrict__ rpa, const int *__restrict__ cia,
                                                      const float *__restrict__ va, const int *__restrict__ rpb,
                                                      const int *__restrict__ cib, const float *__restrict__ vb,
                                                      const int *__restrict__ rpc, int *__restrict__ cic,
                                                      float *__restrict__ vc, int *err) {
    __shared__ unsigned keys[G0_ROWS][G0_T];
    __shared__ float vals[G0_ROWS][G0_T];
    const int r = threadIdx.x / G0_LANES, lane = threadIdx.x % G0_LANES;
    for (int s = lane; s < G0_T; s += G0_LANES) {
        keys[r][s] = SG_EMPTY;
        vals[r][s] = 0.0f;
    }
    __syncthreads();
    const int li = blockIdx.x * G0_ROWS + r;
    const int row = li < n0 ? map0[li] : -1;
    bool ok = true;
    if (row >= 0) {
        for (int j = rpa[row] + lane; j < rpa[row + 1]; j += G0_LANES) {
            const int k = cia[j];
            const float a = va[j];
            for (int t = rpb[k]; t < rpb[k + 1]; ++t)
                ok = ok && sg_insert_add(&keys[r][0], &vals[r][0], G0_T - 1, cib[t], a * vb[t]);
        }
    }
    if (!ok) atomicOr(err, SG_ERR_PROBE);
    __syncthreads();
    if (row < 0) return;
    const int base = rpc[row], len = rpc[row + 1] - base;
    for (int s = lane; s < G0_T; s += G0_LANES) {
        const unsigned key = keys[r][s];
        if (key == SG_EMPTY) continue;
        int rank = 0;
        for (int q = 0; q < G0_T; ++q) rank += keys[r][q] < key;
        if (rank < len) {
            cic[base + rank] = (int)key;
            vc[base + rank] = vals[r][s];
        }
    }
}

// ---- groups 1 and 2: TBPR with the table in LDS ----

template <int WG, int TMAX>
__global__ __launch_bounds__(WG) void k_sg_tb_count(const int *__restrict__ list, const long long *__restrict__ ip,
                                                    const int *__restrict__ rpa, const int *__restrict__ cia,
                                                    const int *__restrict__ rpb, const int *__restrict__ cib,
                                                    int *__restrict__ cnt, int *err) {
    __shared__ unsigned keys[TMAX];
    __shared__ int count, ndefer;
    __shared__ int defer[SG_DEFER];
    const int row = list[blockIdx.x];
    const unsigned T = (unsigned)min((long long)TMAX, (long long)g3_table(ip[row]));
    for (unsigned s = threadIdx.x; s < T; s += WG) keys[s] = SG_EMPTY;
    if (threadIdx.x == 0) count = ndefer = 0;
    __syncthreads();
    bool ok = true;
    sg_walk<WG>(row, rpa, cia, rpb, defer, &ndefer,
                [&](int, int t) { ok = ok && sg_insert_key(keys, T - 1, cib[t], &count); });
    if (!ok) atomicOr(err, SG_ERR_PROBE);
    __syncthreads();
    if (threadIdx.x == 0) cnt[row] = count;
}

template <int WG, int TMAX>
__global__ __launch_bounds__(WG) void k_sg_tb_fill(const int *__restrict__ list, const long long *__restrict__ ip,
                                                   const int *__restrict__ rpa, const int *__restrict__ cia,
                                                   const float *__restrict__ va, const int *__restrict__ rpb,
                                                   const int *__restrict__ cib, const float *__restrict__ vb,
                                                   const int *__restrict__ rpc, int *__restrict__ cic,
                                                   float *__restrict__ vc, int *err) {
    __shared__ unsigned keys[TMAX];
    __shared__ float vals[TMAX];
    __shared__ int used, ndefer;
    __shared__ int defer[SG_DEFER];
    const int row = list[blockIdx.x];
    const unsigned T = (unsigned)min((long long)TMAX, (long long)g3_table(ip[row]));
    for (unsigned s = threadIdx.x; s < T; s += WG) {
        keys[s] = SG_EMPTY;
        vals[s] = 0.0f;
    }
    if (threadIdx.x == 0) ndefer = 0;
    __syncthreads();
    bool ok = true;
    sg_walk<WG>(row, rpa, cia, rpb, defer, &ndefer,
                [&](int j, int t) { ok = ok && sg_insert_add(keys, vals, T - 1, cib[t], va[j] * vb[t]); });
    if (!ok) atomicOr(err, SG_ERR_PROBE);
    __syncthreads();
    static_assert(TMAX % WG == 0, "whole slots per thread");
    const unsigned P = sg_compact<WG, TMAX / WG>(keys, vals, T, &used);
    sg_bitonic<WG>(keys, vals, P);
    const int base = rpc[row], len = rpc[row + 1] - base;
    for (int s = threadIdx.x; s < len && (unsigned)s < T; s += WG) {
        cic[base + s] = (int)keys[s];
        vc[base + s] = vals[s];
    }
}

// ---- group 3: TBPR with the table in global memory (slots off[r]..off[r+1]) ----

__global__ __launch_bounds__(G3_WG) void k_sg_g3_count(const int *__restrict__ list, const long long *__restrict__ off,
                                                       unsigned *__restrict__ tkeys, const int *__restrict__ rpa,
                                                       const int *__restrict__ cia, const int *__restrict__ rpb,
                                                       const int *__restrict__ cib, int *__restrict__ cnt, int *err) {
    __shared__ int count, ndefer;
    __shared__ int defer[SG_DEFER];
    const int r = blockIdx.x;
    const int row = list[r];
    const unsigned T = (unsigned)(off[r + 1] - off[r]);
    unsigned *keys = tkeys + off[r];
    for (unsigned s = threadIdx.x; s < T; s += G3_WG) keys[s] = SG_EMPTY;
    if (threadIdx.x == 0) count = ndefer = 0;
    __syncthreads();
    bool ok = true;
    sg_walk<G3_WG>(row, rpa, cia, rpb, defer, &ndefer,
                   [&](int, int t) { ok = ok && sg_insert_key(keys, T - 1, cib[t], &count); });
    if (!ok) atomicOr(err, SG_ERR_PROBE);
    __syncthreads();
    if (threadIdx.x == 0) cnt[row] = count;
}

__global__ __launch_bounds__(G3_WG) void k_sg_g3_fill(const int *__restrict__ list, const long long *__restrict__ off,
                                                      unsigned *__restrict__ tkeys, float *__restrict__ tvals,
                                                      const int *__restrict__ rpa, const int *__restrict__ cia,
                                                      const float *__restrict__ va, const int *__restrict__ rpb,
                                                      const int *__restrict__ cib, const float *__restrict__ vb,
                                                      const int *__restrict__ rpc, int *__restrict__ cic,
                                                      float *__restrict__ vc, int *err) {
    __shared__ unsigned lk[G3_CH];
    __shared__ float lv[G3_CH];
    __shared__ int ndefer;
    __shared__ int defer[SG_DEFER];
    const int r = blockIdx.x;
    const int row = list[r];
    const unsigned T = (unsigned)(off[r + 1] - off[r]);
    unsigned *keys = tkeys + off[r];
    float *vals = tvals + off[r];
    for (unsigned s = threadIdx.x; s < T; s += G3_WG) {
        keys[s] = SG_EMPTY;
        vals[s] = 0.0f;
    }
    if (threadIdx.x == 0) ndefer = 0;
    __syncthreads();
    const int lane = threadIdx.x % 64;
    bool ok = true;
    sg_walk<G3_WG>(row, rpa, cia, rpb, defer, &ndefer,
                   [&](int j, int t) { ok = ok && sg_insert_add(keys, vals, T - 1, cib[t], va[j] * vb[t]); });
    if (!ok) atomicOr(err, SG_ERR_PROBE);
    // Compact the table's len entries into C's row (in any order): the table
    // is at least half empty, so sorting it whole would sort mostly padding.
    __shared__ int fill;
    if (threadIdx.x == 0) fill = 0;
    __syncthreads();
    const int base = rpc[row], len = rpc[row + 1] - base;
    unsigned *ck = reinterpret_cast<unsigned *>(cic + base);
    float *cv = vc + base;
    const unsigned long long below = (1ull << lane) - 1ull;
    for (unsigned s0 = 0; s0 < T; s0 += G3_WG) {
        const unsigned s = s0 + threadIdx.x;
        const unsigned key = s < T ? keys[s] : SG_EMPTY;
        const bool has = key != SG_EMPTY;
        const unsigned long long bal = __ballot(has);
        int at = 0;
        if (lane == 0 && bal) at = atomicAdd(&fill, __popcll(bal));
        at = __shfl(at, 0) + __popcll(bal & below);
        if (has && at < len) {
            ck[at] = key;
            cv[at] = vals[s];
        }
    }
    __syncthreads();
    // Sort: runs of up to G3_CH entries in LDS, then pairwise merges between
    // C's row and the (now free) table, which holds at least 2 * len slots.
    for (int c0 = 0; c0 < len; c0 += G3_CH) {
        const int cl = min(G3_CH, len - c0);
        unsigned P = 64;
        while ((int)P < cl) P <<= 1;
        for (unsigned i = threadIdx.x; i < P; i += G3_WG) {
            const bool in = (int)i < cl;
            lk[i] = in ? ck[c0 + i] : SG_EMPTY;
            lv[i] = in ? cv[c0 + i] : 0.0f;
        }
        __syncthreads();
        sg_bitonic<G3_WG>(lk, lv, P);
        for (int i = threadIdx.x; i < cl; i += G3_WG) {
            ck[c0 + i] = lk[i];
            cv[c0 + i] = lv[i];
        }
        __syncthreads();
    }
    unsigned *sk = ck, *dk = keys;
    float *sv = cv, *dv = vals;
    for (int run = G3_CH; run < len; run *= 2) {
        for (int a0 = 0; a0 < len; a0 += 2 * run) {
            const int la = min(run, len - a0), lb = min(run, max(0, len - a0 - run));
            sg_merge<G3_WG>(sk + a0, sv + a0, la, sk + a0 + la, sv + a0 + la, lb, dk + a0, dv + a0);
        }
        __syncthreads();
        unsigned *tk = sk;
        sk = dk;
        dk = tk;
        float *tv = sv;
        sv = dv;
        dv = tv;
    }
    if (sk != ck)
        for (int i = threadIdx.x; i < len; i += G3_WG) {
            ck[i] = sk[i];
            cv[i] = sv[i];
        }
}

// ---- row pointers of C: exclusive scan of the counts ----

// Per-workgroup sums of SG_SCAN_WG counts.
__global__ __launch_bounds__(SG_SCAN_WG) void k_sg_scan_sums(int m, const int *__restrict__ cnt,
                                                             long long *__restrict__ sums) {
    __shared__ long long part[SG_SCAN_WG / 64];
    const int i = blockIdx.x * SG_SCAN_WG + threadIdx.x;
    long long v = i < m ? cnt[i] : 0;
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        long long s = 0;
        for (int k = 0; k < SG_SCAN_WG / 64; ++k) s += part[k];
        sums[blockIdx.x] = s;
    }
}

// Exclusive scan of the nb workgroup sums (one workgroup; total in sums[nb]).
__global__ __launch_bounds__(SG_SCAN_WG) void k_sg_scan_top(int nb, long long *__restrict__ sums) {
    __shared__ long long part[SG_SCAN_WG];
    long long carry = 0;
    for (int c0 = 0; c0 < nb; c0 += SG_SCAN_WG) {
        const int r = c0 + (int)threadIdx.x;
        const long long t = r < nb ? sums[r] : 0;
        part[threadIdx.x] = t;
        __syncthreads();
        for (int d = 1; d < SG_SCAN_WG; d <<= 1) {
            const long long v = threadIdx.x >= (unsigned)d ? part[threadIdx.x - d] : 0;
            __syncthreads();
            part[threadIdx.x] += v;
            __syncthreads();
        }
        if (r < nb) sums[r] = carry + part[threadIdx.x] - t;
        const long long last = part[SG_SCAN_WG - 1];
        __syncthreads();
        carry += last;
    }
    if (threadIdx.x == 0) sums[nb] = carry;
}

// rp[i] = offset of row i (int32; totals past INT32_MAX are caught on the
// host before this runs), rp[m] = total.
__global__ __launch_bounds__(SG_SCAN_WG) void k_sg_scan_rows(int m, const int *__restrict__ cnt,
                                                             const long long *__restrict__ sums,
                                                             int *__restrict__ rp) {
    __shared__ long long part[SG_SCAN_WG];
    const int i = blockIdx.x * SG_SCAN_WG + threadIdx.x;
    const long long t = i < m ? cnt[i] : 0;
    part[threadIdx.x] = t;
    __syncthreads();
    for (int d = 1; d < SG_SCAN_WG; d <<= 1) {
        const long long v = threadIdx.x >= (unsigned)d ? part[threadIdx.x - d] : 0;
        __syncthreads();
        part[threadIdx.x] += v;
        __syncthreads();
    }
    if (i < m) rp[i] = (int)(sums[blockIdx.x] + part[threadIdx.x] - t);
    if (i == m - 1) rp[m] = (int)(sums[blockIdx.x] + part[threadIdx.x]);
}

}  // namespace
}  // namespace spmv

// ---- handle ----

struct spgemm {
    int32_t m, k, n, nnz_a, nnz_b;
    const int32_t *rpa, *cia, *rpb, *cib;
    const float *va, *vb;
    int counts[spmv::SG_NBIN], base[spmv::SG_NBIN + 1];
    int64_t nnz_c, total_ip;
    long long *ip, *g3off, *sums;
    int *map, *cnt, *rp, *err, *bcnt, *dbase;
    unsigned *tkeys;
    float *tvals;
    spmv::IpTotals *tot;
    // Side streams (the device's shared pool, default priority) and this
    // handle's events: the bins of a phase run concurrently, forked from and
    // joined back into the caller's stream.
    hipStream_t side[3] = {};
    hipEvent_t fork = nullptr, join[3] = {};
    ~spgemm() {
        for (hipEvent_t e : join)
            if (e) (void)hipEventDestroy(e);
        if (fork) (void)hipEventDestroy(fork);
    }
};

namespace spmv {
namespace {

size_t r256(size_t b) { return (b + 255) & ~size_t(255); }

// Three non-blocking streams per device, created on first use and kept for
// the life of the process (creating streams per handle costs more than a
// small product).  Handles on one device share them, which only orders
// their bins, never their results.
bool side_streams(hipStream_t (&out)[3]) {
    static std::mutex mu;
    static std::map<int, std::array<hipStream_t, 3>> pool;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    std::lock_guard<std::mutex> lock(mu);
    auto it = pool.find(dev);
    if (it == pool.end()) {
        std::array<hipStream_t, 3> q{};
        for (auto &x : q)
            if (hipStreamCreateWithFlags(&x, hipStreamNonBlocking) != hipSuccess) return false;
        it = pool.emplace(dev, q).first;
    }
    for (int i = 0; i < 3; ++i) out[i] = it->second[i];
    return true;
}

struct SgLayout {
    size_t ip, map, cnt, rp, sums, bcnt, dbase, g3off, tot, err, tkeys, tvals, total;
};

int sg_nwg(int64_t m) { return (int)std::max<int64_t>(1, ceil_div(m, SG_ROWS_PER_WG)); }

SgLayout sg_layout(int64_t m, int64_t n3, int64_t g3_slots) {
    SgLayout L;
    size_t at = 0;
    auto take = [&](size_t bytes) {
        const size_t here = at;
        at += r256(std::max<size_t>(bytes, 1));
        return here;
    };
    const int64_t nb = ceil_div(std::max<int64_t>(m, 1), SG_SCAN_WG);
    L.ip = take(sizeof(long long) * m);
    L.map = take(sizeof(int) * m);
    L.cnt = take(sizeof(int) * m);
    L.rp = take(sizeof(int) * (m + 1));
    L.sums = take(sizeof(long long) * (nb + 1));
    L.bcnt = take(sizeof(int) * SG_NBIN * (size_t)sg_nwg(m));
    L.dbase = take(sizeof(int) * SG_NBIN);
    L.g3off = take(sizeof(long long) * (n3 + 1));
    L.tot = take(sizeof(IpTotals));
    L.err = take(sizeof(int));
    L.tkeys = take(sizeof(unsigned) * g3_slots);
    L.tvals = take(sizeof(float) * g3_slots);
    L.total = at;
    return L;
}

spmv_status sg_check_args(int32_t m, int32_t k, int32_t n, int32_t nnz_a, const int32_t *rpa, const int32_t *cia,
                          int32_t nnz_b, const int32_t *rpb, const int32_t *cib) {
    if (m < 0 || k < 0 || n < 0 || nnz_a < 0 || nnz_b < 0) return fail(SPMV_ERR_INVALID_VALUE, "negative size");
    if (!rpa || !rpb) return fail(SPMV_ERR_INVALID_VALUE, "row_ptr is NULL");
    if ((nnz_a > 0 && !cia) || (nnz_b > 0 && !cib)) return fail(SPMV_ERR_INVALID_VALUE, "col_idx is NULL");
    return SPMV_OK;
}

// Validates A and B on the GPU (err: device int, zeroed here).  Synchronises.
spmv_status sg_validate(int32_t m, int32_t k, int32_t n, int32_t nnz_a, const int32_t *rpa, const int32_t *cia,
                        int32_t nnz_b, const int32_t *rpb, const int32_t *cib, int *err, hipStream_t st) {
    SPMV_HIP(hipMemsetAsync(err, 0, sizeof(int), st));
    k_sg_check_rows<<<(int)ceil_div((int64_t)m + 1, 256), 256, 0, st>>>(m, nnz_a, rpa, err);
    SPMV_LAUNCHED("k_sg_check_rows");
    k_sg_check_rows<<<(int)ceil_div((int64_t)k + 1, 256), 256, 0, st>>>(k, nnz_b, rpb, err);
    SPMV_LAUNCHED("k_sg_check_rows");
    const int ga = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(nnz_a, 256), 4096));
    const int gb = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(nnz_b, 256), 4096));
    k_sg_check_cols<<<ga, 256, 0, st>>>(nnz_a, cia, k, SG_ERR_COLS_A, err);
    SPMV_LAUNCHED("k_sg_check_cols");
    k_sg_check_cols<<<gb, 256, 0, st>>>(nnz_b, cib, n, SG_ERR_COLS_B, err);
    SPMV_LAUNCHED("k_sg_check_cols");
    int h = 0;
    SPMV_HIP(hipMemcpyAsync(&h, err, sizeof(int), hipMemcpyDeviceToHost, st));
    SPMV_HIP(hipStreamSynchronize(st));
    if (h & SG_ERR_ROWS) return fail(SPMV_ERR_INVALID_MATRIX, "a row_ptr is not monotone from 0 to nnz");
    if (h & SG_ERR_COLS_A) return fail(SPMV_ERR_INVALID_MATRIX, "a column of A is outside [0, k)");
    if (h & SG_ERR_COLS_B) return fail(SPMV_ERR_INVALID_MATRIX, "a column of B is outside [0, n)");
    return SPMV_OK;
}

// IP totals into *tot (device), per-row IP and per-workgroup bin counts
// when given.  Synchronises and returns the host copy.
spmv_status sg_ip(int32_t m, const int32_t *rpa, const int32_t *cia, const int32_t *rpb, long long *ip, int *bcnt,
                  IpTotals *tot, IpTotals *h, hipStream_t st) {
    SPMV_HIP(hipMemsetAsync(tot, 0, sizeof(IpTotals), st));
    if (m > 0) {
        k_sg_ip<<<sg_nwg(m), 256, 0, st>>>(m, rpa, cia, rpb, ip, bcnt, tot);
        SPMV_LAUNCHED("k_sg_ip");
    }
    SPMV_HIP(hipMemcpyAsync(h, tot, sizeof(IpTotals), hipMemcpyDeviceToHost, st));
    SPMV_HIP(hipStreamSynchronize(st));
    return SPMV_OK;
}

// Allocation (SYM) or accumulation phase over every bin.
// The bins are independent, so they run concurrently: the global-table rows
// (the longest-running, with the fewest workgroups) start first on one side
// stream, bins 5 and 4 on a second, bins 3 and 2 on a third, and bins 1 and
// 0 on the caller's stream, which then waits for the side streams.
template <bool SYM>
spmv_status sg_phase(const spgemm *h, int *ci_c, float *v_c, hipStream_t st) {
    const int *mp = h->map;
    const int *b = h->base;
    const int *c = h->counts;
    // without rows in bins 2-6 everything runs on the caller's stream
    const bool fork = c[2] + c[3] + c[4] + c[5] + c[6] > 0;
    if (fork) {
        SPMV_HIP(hipEventRecord(h->fork, st));
        for (hipStream_t q : h->side) SPMV_HIP(hipStreamWaitEvent(q, h->fork, 0));
    }
    if (c[6] > 0) {
        if (SYM)
            k_sg_g3_count<<<c[6], G3_WG, 0, h->side[0]>>>(mp + b[6], h->g3off, h->tkeys, h->rpa, h->cia,
                                                          h->rpb, h->cib, h->cnt, h->err);
        else
            k_sg_g3_fill<<<c[6], G3_WG, 0, h->side[0]>>>(mp + b[6], h->g3off, h->tkeys, h->tvals, h->rpa,
                                                         h->cia, h->va, h->rpb, h->cib, h->vb, h->rp, ci_c, v_c,
                                                         h->err);
    }
#define SG_TB(BIN, WG, TMAX, Q)                                                                                     \
    if (c[BIN] > 0) {                                                                                              \
        if (SYM)                                                                                                   \
            k_sg_tb_count<WG, TMAX><<<c[BIN], WG, 0, Q>>>(mp + b[BIN], h->ip, h->rpa, h->cia, h->rpb, h->cib,        \
                                                          h->cnt, h->err);                                        \
        else                                                                                                       \
            k_sg_tb_fill<WG, TMAX><<<c[BIN], WG, 0, Q>>>(mp + b[BIN], h->ip, h->rpa, h->cia, h->va, h->rpb, h->cib,  \
                                                         h->vb, h->rp, ci_c, v_c, h->err);                        \
    }
    SG_TB(5, 1024, 16384, h->side[1])
    SG_TB(4, 1024, 8192, h->side[1])
    SG_TB(3, 512, 4096, h->side[2])
    SG_TB(2, 256, 2048, h->side[2])
    SG_TB(1, 256, 1024, st)
#undef SG_TB
    if (c[0] > 0) {
        const int g = (int)ceil_div(c[0], G0_ROWS);
        if (SYM)
            k_sg_g0_count<<<g, G0_WG, 0, st>>>(c[0], mp + b[0], h->rpa, h->cia, h->rpb, h->cib, h->cnt, h->err);
        else
            k_sg_g0_fill<<<g, G0_WG, 0, st>>>(c[0], mp + b[0], h->rpa, h->cia, h->va, h->rpb, h->cib, h->vb, h->rp,
                                              ci_c, v_c, h->err);
    }
    SPMV_LAUNCHED(SYM ? "the allocation phase" : "the accumulation phase");
    for (int i = 0; fork && i < 3; ++i) {
        SPMV_HIP(hipEventRecord(h->join[i], h->side[i]));
        SPMV_HIP(hipStreamWaitEvent(st, h->join[i], 0));
    }
    return SPMV_OK;
}

}  // namespace
}  // namespace spmv

using namespace spmv;

extern "C" spmv_status spgemm_workspace_size(int32_t m, int32_t k, int32_t n, int32_t nnz_a, const int32_t *rp_a,
                                             const int32_t *ci_a, int32_t nnz_b, const int32_t *rp_b,
                                             const int32_t *ci_b, size_t *bytes, void *scratch,
                                             size_t scratch_bytes, void *stream) {
    static_assert(sizeof(IpTotals) <= SCRATCH_HEAD - SCRATCH_SG_TOTALS, "IpTotals must fit the scratch head");
    if (!bytes) return fail(SPMV_ERR_INVALID_VALUE, "bytes is NULL");
    spmv_status s = sg_check_args(m, k, n, nnz_a, rp_a, ci_a, nnz_b, rp_b, ci_b);
    if (s != SPMV_OK) return s;
    s = check_scratch(scratch, scratch_bytes, m);
    if (s != SPMV_OK) return s;
    hipStream_t st = as_stream(stream);
    int *err = reinterpret_cast<int *>(static_cast<char *>(scratch) + SCRATCH_SG_ERR);
    IpTotals *tot = reinterpret_cast<IpTotals *>(static_cast<char *>(scratch) + SCRATCH_SG_TOTALS);
    IpTotals h{};
    s = sg_validate(m, k, n, nnz_a, rp_a, ci_a, nnz_b, rp_b, ci_b, err, st);
    if (s == SPMV_OK) s = sg_ip(m, rp_a, ci_a, rp_b, nullptr, nullptr, tot, &h, st);
    if (s != SPMV_OK) return s;
    *bytes = sg_layout(m, h.counts[SG_NBIN - 1], (int64_t)h.g3_slots).total;
    return SPMV_OK;
}

extern "C" spmv_status spgemm_create(spgemm_t *handle, int32_t m, int32_t k, int32_t n, int32_t nnz_a,
                                     const int32_t *rp_a, const int32_t *ci_a, const float *v_a, int32_t nnz_b,
                                     const int32_t *rp_b, const int32_t *ci_b, const float *v_b, void *workspace,
                                     size_t workspace_bytes, void *stream) {
    if (!handle) return fail(SPMV_ERR_INVALID_VALUE, "handle is NULL");
    *handle = nullptr;
    spmv_status s = sg_check_args(m, k, n, nnz_a, rp_a, ci_a, nnz_b, rp_b, ci_b);
    if (s != SPMV_OK) return s;
    if ((nnz_a > 0 && !v_a) || (nnz_b > 0 && !v_b)) return fail(SPMV_ERR_INVALID_VALUE, "values are NULL");
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return fail(SPMV_ERR_INVALID_VALUE, "workspace must be non-NULL and 256-byte aligned");
    hipStream_t st = as_stream(stream);
    // the fixed part first (validation, IP and the bin counts need it), then the tables
    const SgLayout L0 = sg_layout(m, 0, 0);
    if (workspace_bytes < L0.total)
        return fail(SPMV_ERR_INVALID_VALUE, "workspace of %zu bytes is smaller than %zu", workspace_bytes, L0.total);
    char *w = static_cast<char *>(workspace);
    s = sg_validate(m, k, n, nnz_a, rp_a, ci_a, nnz_b, rp_b, ci_b, reinterpret_cast<int *>(w + L0.err), st);
    if (s != SPMV_OK) return s;
    IpTotals h{};
    s = sg_ip(m, rp_a, ci_a, rp_b, reinterpret_cast<long long *>(w + L0.ip), reinterpret_cast<int *>(w + L0.bcnt),
              reinterpret_cast<IpTotals *>(w + L0.tot), &h, st);
    if (s != SPMV_OK) return s;
    const int n3 = h.counts[SG_NBIN - 1];
    const SgLayout L = sg_layout(m, n3, (int64_t)h.g3_slots);
    if (workspace_bytes < L.total)
        return fail(SPMV_ERR_INVALID_VALUE, "workspace of %zu bytes is smaller than %zu", workspace_bytes, L.total);
    spgemm *H = new spgemm{};
    H->m = m, H->k = k, H->n = n, H->nnz_a = nnz_a, H->nnz_b = nnz_b;
    H->rpa = rp_a, H->cia = ci_a, H->va = v_a, H->rpb = rp_b, H->cib = ci_b, H->vb = v_b;
    H->ip = reinterpret_cast<long long *>(w + L.ip);
    H->map = reinterpret_cast<int *>(w + L.map);
    H->cnt = reinterpret_cast<int *>(w + L.cnt);
    H->rp = reinterpret_cast<int *>(w + L.rp);
    H->sums = reinterpret_cast<long long *>(w + L.sums);
    H->bcnt = reinterpret_cast<int *>(w + L.bcnt);
    H->dbase = reinterpret_cast<int *>(w + L.dbase);
    H->g3off = reinterpret_cast<long long *>(w + L.g3off);
    H->tot = reinterpret_cast<IpTotals *>(w + L.tot);
    H->err = reinterpret_cast<int *>(w + L.err);
    H->tkeys = reinterpret_cast<unsigned *>(w + L.tkeys);
    H->tvals = reinterpret_cast<float *>(w + L.tvals);
    H->total_ip = (int64_t)h.ip;
    H->base[0] = 0;
    for (int q = 0; q < SG_NBIN; ++q) {
        H->counts[q] = h.counts[q];
        H->base[q + 1] = H->base[q] + h.counts[q];
    }
    auto cleanup = [&](spmv_status e) {
        delete H;
        return e;
    };
    if (!side_streams(H->side)) return cleanup(fail(SPMV_ERR_HIP, "creating the side streams failed"));
    for (int i = 0; i < 3; ++i)
        if (hipEventCreateWithFlags(&H->join[i], hipEventDisableTiming) != hipSuccess)
            return cleanup(fail(SPMV_ERR_HIP, "creating an event failed"));
    if (hipEventCreateWithFlags(&H->fork, hipEventDisableTiming) != hipSuccess)
        return cleanup(fail(SPMV_ERR_HIP, "creating an event failed"));
    // Map[]: rows binned, in row order inside each bin
    if (hipMemcpyAsync(H->dbase, H->base, sizeof(int) * SG_NBIN, hipMemcpyHostToDevice, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return cleanup(fail(SPMV_ERR_HIP, "hipMemcpyAsync failed"));
    if (m > 0) {
        const int nwg = sg_nwg(m);
        k_sg_bin_offsets<<<1, SG_SCAN_WG, 0, st>>>(nwg, H->bcnt);
        k_sg_map<<<nwg, 256, 0, st>>>(m, H->ip, H->dbase, H->bcnt, H->map);
        if (hipGetLastError() != hipSuccess) return cleanup(fail(SPMV_ERR_HIP, "launch of the binning failed"));
    }
    if (n3 > 0) {
        k_sg_g3_offsets<<<1, SG_SCAN_WG, 0, st>>>(n3, H->map + H->base[SG_NBIN - 1], H->ip, H->g3off);
        if (hipGetLastError() != hipSuccess) return cleanup(fail(SPMV_ERR_HIP, "launch of k_sg_g3_offsets failed"));
    }
    // allocation phase: distinct columns per row
    if (hipMemsetAsync(H->err, 0, sizeof(int), st) != hipSuccess) return cleanup(fail(SPMV_ERR_HIP, "memset failed"));
    s = sg_phase<true>(H, nullptr, nullptr, st);
    if (s != SPMV_OK) return cleanup(s);
    // row pointers of C
    int64_t total = 0;
    if (m > 0) {
        const int nb = (int)ceil_div(m, SG_SCAN_WG);
        k_sg_scan_sums<<<nb, SG_SCAN_WG, 0, st>>>(m, H->cnt, H->sums);
        k_sg_scan_top<<<1, SG_SCAN_WG, 0, st>>>(nb, H->sums);
        if (hipGetLastError() != hipSuccess) return cleanup(fail(SPMV_ERR_HIP, "launch of the scan failed"));
        long long t = 0;
        int e = 0;
        if (hipMemcpyAsync(&t, H->sums + nb, sizeof t, hipMemcpyDeviceToHost, st) != hipSuccess ||
            hipMemcpyAsync(&e, H->err, sizeof e, hipMemcpyDeviceToHost, st) != hipSuccess ||
            hipStreamSynchronize(st) != hipSuccess)
            return cleanup(fail(SPMV_ERR_HIP, "reading the allocation phase failed"));
        if (e & SG_ERR_PROBE) return cleanup(fail(SPMV_ERR_HIP, "a hash table probe sequence ran out"));
        if (t > INT32_MAX) return cleanup(fail(SPMV_ERR_OVERFLOW, "nnz(C) = %lld exceeds int32", t));
        total = t;
        k_sg_scan_rows<<<nb, SG_SCAN_WG, 0, st>>>(m, H->cnt, H->sums, H->rp);
        if (hipGetLastError() != hipSuccess) return cleanup(fail(SPMV_ERR_HIP, "launch of k_sg_scan_rows failed"));
    } else {
        if (hipMemsetAsync(H->rp, 0, sizeof(int), st) != hipSuccess) return cleanup(fail(SPMV_ERR_HIP, "memset failed"));
    }
    if (hipStreamSynchronize(st) != hipSuccess) return cleanup(fail(SPMV_ERR_HIP, "synchronise failed"));
    H->nnz_c = total;
    *handle = H;
    return SPMV_OK;
}

extern "C" spmv_status spgemm_info(spgemm_t h, int64_t *nnz_c, int64_t *intermediate_products,
                                   int32_t *group_rows) {
    if (!h) return fail(SPMV_ERR_INVALID_VALUE, "handle is NULL");
    if (nnz_c) *nnz_c = h->nnz_c;
    if (intermediate_products) *intermediate_products = h->total_ip;
    if (group_rows) {
        // the page's four groups: bin 0, bin 1, bins 2-5, bin 6
        group_rows[0] = h->counts[0];
        group_rows[1] = h->counts[1];
        group_rows[2] = h->counts[2] + h->counts[3] + h->counts[4] + h->counts[5];
        group_rows[3] = h->counts[6];
    }
    return SPMV_OK;
}

extern "C" spmv_status spgemm_compute(spgemm_t h, int32_t *rp_c, int32_t *ci_c, float *v_c, void *stream) {
    if (!h) return fail(SPMV_ERR_INVALID_VALUE, "handle is NULL");
    if (!rp_c || (h->nnz_c > 0 && (!ci_c || !v_c))) return fail(SPMV_ERR_INVALID_VALUE, "NULL output");
    hipStream_t st = as_stream(stream);
    SPMV_HIP(hipMemcpyAsync(rp_c, h->rp, sizeof(int32_t) * ((size_t)h->m + 1), hipMemcpyDeviceToDevice, st));
    return sg_phase<false>(h, ci_c, v_c, st);
}

extern "C" spmv_status spgemm_destroy(spgemm_t h) {
    delete h;
    return SPMV_OK;
}
