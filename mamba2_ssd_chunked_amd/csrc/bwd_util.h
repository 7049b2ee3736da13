// Small wave-level helpers of the backward kernels.
#pragma once

#include "ssd_internal.h"

namespace ssd {

template <typename T>
__device__ __forceinline__ void load4(const T* p, float* o) {
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = (float)p[r];
}

// Sum over the four lane groups (lanes l, l^16, l^32, l^48 share a column).
__device__ __forceinline__ float sum_groups(float v) {
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

// DPP lane moves inside rows of 16 lanes (VALU only, no LDS traffic).
#define SSD_DPP(v, ctrl) \
    __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), (ctrl), 0xF, 0xF, false))
#define DPP_ROW_MIRROR 0x140
#define DPP_ROW_HALF_MIRROR 0x141
#define DPP_QUAD_XOR1 0xB1
#define DPP_QUAD_XOR2 0x4E

// Row sums of a 16x16 tile held as 4 rows per lane (rows 4g+r, column l%16):
// reduces v[0..3] over the 16 lanes of each row group and returns, in lane l,
// the sum for row r = 2*(l%16 >= 8) + ((l%8) >= 4) (all four lanes of a quad
// hold the same value).
__device__ __forceinline__ float row_sums16(const float v[4], int lr) {
    const bool hi = lr >= 8;
    const float k0 = hi ? v[2] : v[0], k1 = hi ? v[3] : v[1];
    const float s0 = hi ? v[0] : v[2], s1 = hi ? v[1] : v[3];
    const float a0 = k0 + SSD_DPP(s0, DPP_ROW_MIRROR);
    const float a1 = k1 + SSD_DPP(s1, DPP_ROW_MIRROR);
    const bool h2 = (lr & 4) != 0;
    const float k = h2 ? a1 : a0, s = h2 ? a0 : a1;
    float t = k + SSD_DPP(s, DPP_ROW_HALF_MIRROR);
    t += SSD_DPP(t, DPP_QUAD_XOR2);
    t += SSD_DPP(t, DPP_QUAD_XOR1);
    return t;
}

}  // namespace ssd
