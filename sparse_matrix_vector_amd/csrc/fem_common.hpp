// Device helper shared by the FE matvec kernels: the atomic scatter of a
// wave's element contributions, merged along x-lines of nodes in LDS.
#pragma once

#include "common.hpp"

namespace spmv {

// Scatter of one element's 24 contributions per lane (lane = element, all
// 64 lanes of the wave present; idle lanes hold index -1 everywhere), by
// node line.  Hex8 local nodes (x, y, z corners; local DOF 3a + component)
// pair along x as (0,1), (3,2), (4,5), (7,6): the second node of lane l's
// pair is the first node of lane l + 1's pair when elements are numbered
// x-fastest on a structured grid.  Each pair forms one line of 65 slots of
// 3 DOFs in LDS (sd/sv: 4 lines x 195 entries for this wave).  Lane l puts
// its first nodes in slot l of the four lines; after one wave sync it reads
// slot l + 1 of each line and adds its second node there where the slot
// holds the same global DOFs (compared per DOF, so any numbering stays
// correct; where they differ the lane adds its value to y itself); after a
// second sync the 780 entries go out with lane i taking entries i, 64 + i,
// ...  Consecutive lanes then add to consecutive DOFs, so one memory-side
// atomic request carries ~16 lanes, against ~5 when each lane adds its own
// element's DOFs, and half the adds disappear.  Which values meet in a slot
// depends only on the lanes' elements, and each is added in a fixed order,
// so the values passed to `add` are deterministic.
//
// `add(dof, on, value)` performs one global accumulation (an atomic add of
// the value, or of a fixed-point image of it) when `on`; it is called the
// same number of times in every lane (on = false where there is nothing to
// add), so a caller can issue it as one memory instruction per call with
// no branch around it.  A final wave sync lets the caller reuse sd/sv.
template <typename T, typename Add>
__device__ __forceinline__ void fe_scatter_lines(const int (&d)[24], const T (&f)[24], int n_dof, Add add, int *sd,
                                                 T *sv) {
    constexpr int P0[4] = {0, 3, 4, 7}, P1[4] = {1, 2, 5, 6};
    constexpr int LS = 3 * 65;                 // entries per line
    constexpr int R = (4 * LS + 63) / 64;      // entries per lane in the final pass
    const int lane = __lane_id();
    auto wave_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            sd[k * LS + 3 * lane + c] = d[3 * P0[k] + c];
            sv[k * LS + 3 * lane + c] = f[3 * P0[k] + c];
        }
    if (lane == 63)
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int c = 0; c < 3; ++c) sd[k * LS + 3 * 64 + c] = -1;
    wave_sync();
    int nd[12];
    T nv[12];
#pragma unroll
    for (int q = 0; q < 12; ++q) {
        nd[q] = sd[(q / 3) * LS + 3 * (lane + 1) + q % 3];
        nv[q] = sv[(q / 3) * LS + 3 * (lane + 1) + q % 3];
    }
#pragma unroll
    for (int q = 0; q < 12; ++q) {
        const int k = q / 3, c = q % 3;
        const int j = k * LS + 3 * (lane + 1) + c;
        const int da = d[3 * P1[k] + c];
        const T fv = f[3 * P1[k] + c];
        const bool valid = (unsigned)da < (unsigned)n_dof;
        const bool same = valid && nd[q] == da;
        const bool open = valid && !same && lane == 63;   // slot 64: past the wave's last element
        if (same || open) sv[j] = same ? nv[q] + fv : fv;
        if (open) sd[j] = da;
        add(da, valid && !same && lane != 63, fv);
    }
    wave_sync();
    int od[R];
    T ov[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = 64 * r + lane;
        od[r] = i < 4 * LS ? sd[i] : -1;
        ov[r] = i < 4 * LS ? sv[i] : T(0);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) add(od[r], (unsigned)od[r] < (unsigned)n_dof, ov[r]);
    wave_sync();
}

}  // namespace spmv
