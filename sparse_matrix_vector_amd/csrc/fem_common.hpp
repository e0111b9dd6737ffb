// Device helper shared by the FE matvec kernels: combining, inside a wave,
// the contributions of x-neighbouring elements to their shared face before
// the atomic scatter.
#pragma once

#include "common.hpp"

namespace spmv {

// Wave-wide lane shifts of the GFX9 DPP encoding: lane i reads lane i + 1
// (WAVE_SHL1) or lane i - 1 (WAVE_SHR1); the end lanes read `old`.
constexpr int DPP_WAVE_SHL1 = 0x130;
constexpr int DPP_WAVE_SHR1 = 0x138;

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v, int old) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xffffffffll), CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xf, 0xf, false);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
__device__ __forceinline__ float dpp_right(float v) { return dpp_f32<DPP_WAVE_SHL1>(v); }
__device__ __forceinline__ double dpp_right(double v) { return dpp_f64<DPP_WAVE_SHL1>(v); }

// Hex8 local nodes (x, y, z corners, the order of the element DOF lists:
// local DOF 3a + component): an element's x = 1 face holds local nodes
// 1, 2, 5, 6; they coincide with local nodes 0, 3, 4, 7 of the element on
// its +x side.  Lane l (element e) and lane l + 1 (element e') compare the
// global DOF numbers of each such pair; where they are equal (and a real
// DOF), lane l adds lane l + 1's contribution to its own and lane l + 1
// drops that DOF from its scatter (its index becomes -1).  Elements numbered
// x-fastest on a structured grid share a face with their successor, so
// about half of the 24 atomic adds per element disappear; for any other
// numbering the comparison fails and nothing changes.  All 64 lanes must
// execute this (idle lanes hold index -1 everywhere).
template <typename T>
__device__ __forceinline__ void fe_combine_x_neighbours(int (&d)[24], T (&f)[24], int n_dof) {
    constexpr int A[4] = {1, 2, 5, 6};   // x = 1 face, taken by this lane
    constexpr int B[4] = {0, 3, 4, 7};   // x = 0 face, handed to the left lane
    int dr[12], dl[12];
    T fr[12];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            const int a = 3 * A[k] + c, b = 3 * B[k] + c, j = 3 * k + c;
            dr[j] = dpp_i32<DPP_WAVE_SHL1>(d[b], -2);   // right lane's index for my a
            fr[j] = dpp_right(f[b]);                      // and its contribution
            dl[j] = dpp_i32<DPP_WAVE_SHR1>(d[a], -2);   // left lane's index for my b
        }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            const int a = 3 * A[k] + c, b = 3 * B[k] + c, j = 3 * k + c;
            if ((unsigned)d[a] < (unsigned)n_dof && d[a] == dr[j]) f[a] += fr[j];
            if ((unsigned)d[b] < (unsigned)n_dof && d[b] == dl[j]) d[b] = -1;
        }
    }
}

}  // namespace spmv
