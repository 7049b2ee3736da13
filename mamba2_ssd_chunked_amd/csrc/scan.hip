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

// Span summaries -> segment summaries.  The forward walk may split a segment
// into spans (SpanPlan), each walked from a zero state; composing the spans'
// summaries in causal order, (a2, M2) o (a1, M1) = (a1 a2, a2 M1 + M2), gives
// the segment's own S_ext and a_block.  One lane per float4 of a (row, head)
// state; spans and segments use the summary layout ([.][b][H][P*N] then
// [.][b][H]).
__global__ void __launch_bounds__(256) k_span_combine(int64_t BH, int PN, int nseg, SpanPlan sp,
                                                     const float* __restrict__ spsum,
                                                     float* __restrict__ summary) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // float4 index
    const int64_t nq = BH * (PN / 4);
    if (q >= nq) return;
    const int64_t bh = q / (PN / 4);
    const f32x4* M = (const f32x4*)spsum;
    const float* a = spsum + (int64_t)sp.n * BH * PN;
    f32x4* O = (f32x4*)summary;
    float* ao = summary + (int64_t)nseg * BH * PN;
    for (int k = 0; k < nseg; ++k) {
        f32x4 cur = f32x4{0.f, 0.f, 0.f, 0.f};
        float ab = 1.f;
        for (int s = sp.first[k]; s < sp.first[k + 1]; ++s) {
            const float as = a[s * BH + bh];
            cur = as * cur + M[s * nq + q];
            ab *= as;
        }
        O[k * nq + q] = cur;
        if (q % (PN / 4) == 0) ao[k * BH + bh] = ab;
    }
}

// The state entering every span: within each segment an exclusive scan over
// its spans' summaries in causal order, starting from the segment's S_in (or
// from zero when S_in is null: the zero-initial-state entering states).
__global__ void __launch_bounds__(256) k_span_scan(int64_t BH, int PN, int nseg, SpanPlan sp,
                                                  const float* __restrict__ spsum,
                                                  const float* __restrict__ S_in,
                                                  float* __restrict__ spst) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // float4 index
    const int64_t nq = BH * (PN / 4);
    if (q >= nq) return;
    const int64_t bh = q / (PN / 4);
    const f32x4* M = (const f32x4*)spsum;
    const float* a = spsum + (int64_t)sp.n * BH * PN;
    f32x4* O = (f32x4*)spst;
    for (int k = 0; k < nseg; ++k) {
        f32x4 cur = S_in ? ((const f32x4*)S_in)[k * nq + q] : f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s = sp.first[k]; s < sp.first[k + 1]; ++s) {
            O[s * nq + q] = cur;
            cur = a[s * BH + bh] * cur + M[s * nq + q];
        }
    }
}

hipError_t launch_span_combine(const Dims& d, const SpanPlan& sp, const float* spsum,
                               float* summary, hipStream_t s) {
    const int64_t BH = d.batch * d.H;
    const int PN = d.P * d.N;
    const int64_t nq = BH * (PN / 4);
    return launch(k_span_combine, dim3((unsigned)((nq + 255) / 256)), dim3(256), s, BH, PN, d.nseg,
                  sp, spsum, summary);
}

hipError_t launch_span_scan(const Dims& d, const SpanPlan& sp, const float* spsum,
                            const float* S_in, float* spst, hipStream_t s) {
    const int64_t BH = d.batch * d.H;
    const int PN = d.P * d.N;
    const int64_t nq = BH * (PN / 4);
    return launch(k_span_scan, dim3((unsigned)((nq + 255) / 256)), dim3(256), s, BH, PN, d.nseg,
                  sp, spsum, S_in, spst);
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
