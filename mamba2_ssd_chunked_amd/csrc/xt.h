// Transposed-operand reads from LDS (gfx950), shared by the output pass and
// the chunk backward.
#pragma once

#include "ssd_internal.h"

namespace ssd {

// ---------------------------------------------------------------------------
// Transposed-operand reads of a [token][p] tile kept in LDS in its natural row
// layout.  The result is the k operand of the MFMA that multiplies a weight
// tile (k = source token j) with X: lane l holds column p0 + l % 16 and the k
// slots of KPerm's order (slot s of lane group g is token 16 (s / 4) + 4 g +
// s % 4 of the 32-token block).
//
// bf16: two ds_read_b64_tr_b16.  Within each 16-lane group that instruction
// hands output lane i, element e, the element i % 4 of the 8 bytes addressed by
// lane i / 4 + 4 e of the group; letting lane q of group g address token
// jb + 4 g + q / 4, columns p0 + 4 (q % 4) .. +3, output lane i receives tokens
// jb + 4 g + e of column p0 + i.
// float32: four 4-byte reads (16 tokens per MFMA k step, natural order).
template <typename T> struct XT;
template <> struct XT<bf16> {
    typedef short s4 __attribute__((ext_vector_type(4)));
    __device__ static __forceinline__ bf16x8 load(const bf16* xs, int xr, int jb, int p0, int lane) {
        const int q = lane % 16, g = lane / 16;
        const bf16* a = xs + (jb + 4 * g + q / 4) * xr + p0 + 4 * (q % 4);
        typedef __attribute__((address_space(3))) s4 lds_s4;
        const bf16x4 lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)a));
        const bf16x4 hi =
            __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(a + 16 * xr)));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
};
template <> struct XT<float> {
    __device__ static __forceinline__ f32x4 load(const float* xs, int xr, int jb, int p0, int lane) {
        const int i = lane % 16, g = lane / 16;
        const float* a = xs + (jb + 4 * g) * xr + p0 + i;
        return f32x4{a[0], a[xr], a[2 * xr], a[3 * xr]};
    }
};

}  // namespace ssd
