// Affine scan over segment summaries (gfx950).
//
// Megatron-LM #6808 (first commit): a segment's SSD map is affine in its
// initial state, S_out = a_block * S_in + S_ext, so an exclusive causal scan
// over the per-segment summaries (S_ext, a_block) yields every segment's true
// initial state.  The composition (a2, M2) o (a1, M1) = (a1 a2, a2 M1 + M2) is
// applied element-wise in FP32; with at most SSD_MAX_SEGMENTS segments each
// thread simply walks them in causal order (forward) or reverse causal order
// (backward: the final-state gradients).  The pass is HBM-bound: it reads the
// summaries once and writes one state per segment, 16 bytes per lane access.
#include "ssd_internal.h"

namespace ssd {

__global__ void __launch_bounds__(256) k_boundary_scan(int64_t BH, int PN, int nseg, int reverse,
                                                      const float* __restrict__ summary,
                                                      const float* __restrict__ init,
                                                      float* __restrict__ out,
                                                      float* __restrict__ fin) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // float4 index
    const int64_t nq = BH * (PN / 4);
    if (q >= nq) return;
    const int64_t bh = q / (PN / 4);
    const int64_t perq = nq;  // float4s per segment
    const float* a = summary + (int64_t)nseg * BH * PN;
    const f32x4* M = (const f32x4*)summary;
    f32x4* O = (f32x4*)out;
    f32x4 cur = init ? ((const f32x4*)init)[q] : f32x4{0.f, 0.f, 0.f, 0.f};
    if (!reverse) {
        for (int k = 0; k < nseg; ++k) {
            O[k * perq + q] = cur;
            cur = a[k * BH + bh] * cur + M[k * perq + q];
        }
    } else {
        for (int k = nseg - 1; k >= 0; --k) {
            O[k * perq + q] = cur;
            cur = a[k * BH + bh] * cur + M[k * perq + q];
        }
    }
    if (fin) ((f32x4*)fin)[q] = cur;
}

hipError_t launch_boundary_scan(const Dims& d, int nseg, const float* summary, const float* init,
                                int reverse, float* out, float* final_state, hipStream_t s) {
    const int64_t BH = d.batch * d.H;
    const int PN = d.P * d.N;
    const int64_t nq = BH * (PN / 4);
    return launch(k_boundary_scan, dim3((unsigned)((nq + 255) / 256)), dim3(256), s, BH, PN, nseg,
                  reverse, summary, init, out, final_state);
}

}  // namespace ssd
