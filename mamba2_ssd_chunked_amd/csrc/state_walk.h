// Per-segment walk of chunk states (forward) or state gradients (backward).
//
// One workgroup per (row, segment, head) visits the segment's chunks in causal
// order (forward) or reverse causal order (backward).  The running P x N matrix
// lives in MFMA accumulators (FP32).  For every chunk it first stores the
// running value, then applies the chunk's decay alpha_c = exp(cs_end) (exactly
// 0 when a packed sequence starts inside the chunk) and accumulates the chunk's
// own contribution A^T diag(w) B with MFMA:
//
//   forward : A = x, B = B channels, w_j = exp(cs_end - cs_j) dt_j [seq_j = seq_end]
//             stored value = state entering the chunk (zero initial state),
//             final value = the segment's S_ext.
//   backward: A = dy, B = C channels, w_i = exp(cs_i) [seq_i = seq of the state
//             entering the chunk]; walked from the last chunk, the stored value is
//             the gradient of the state leaving the chunk (zero final-state
//             gradient) and the final value is dL/dS_in of the segment's own
//             outputs.
//
// The product of the alphas is the segment's block decay a_block in both
// directions.  This is the decay-weighted sum over earlier chunk states that
// state-spaces/mamba #482 (second comment) identifies as the part of the scan
// that must cross devices; Megatron-LM #6808 ships its segment-level result as
// the FP32 summary.
#pragma once

#include "ssd_internal.h"

namespace ssd {

enum WalkMode { WALK_FWD_PN = 0, WALK_FWD_NP = 1, WALK_BWD_PN = 2 };

template <typename T, int P, int N, int MODE>
__global__ void __launch_bounds__(256) k_state_walk(Dims d, SegTab tab, const T* __restrict__ a_src,
                                                   int64_t a_stride, const T* __restrict__ xc,
                                                   int64_t b_chan0,
                                                   const float* __restrict__ dt_ws,
                                                   const float* __restrict__ cs_ws,
                                                   const int32_t* __restrict__ seq,
                                                   T* __restrict__ store,
                                                   float* __restrict__ summary) {
    typedef Mma<T> M;
    typedef typename M::Frag Frag;
    constexpr int SL = M::SL, KS = M::KS;
    constexpr int KT = 64;               // tokens per LDS slice
    constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte load
    constexpr int PITCH = KT + VEC;      // padded LDS row (keeps 16-byte alignment)
    constexpr int PT = P / 16, NTT = N / 16, NTW = (NTT + 3) / 4;
    constexpr bool BWD = MODE == WALK_BWD_PN;
    __shared__ __attribute__((aligned(16))) T At[P * PITCH];
    __shared__ __attribute__((aligned(16))) T Bt[N * PITCH];
    __shared__ float wv[KT];
    typedef T vt __attribute__((ext_vector_type(VEC)));

    const int h = blockIdx.x, k = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int wave = wave_id(), lane = threadIdx.x % 64, lr = lane % 16, lg = lane / 16;
    const int g = h / d.hpg;
    const int Q = d.Q;
    const int64_t rb = b * d.L;
    const int64_t s0 = tab.start[k];
    const int nc = (int)(tab.len[k] / Q);
    const int64_t pred = seg_pred_token(tab, k);
    const float* dtp = dt_ws + ((int64_t)b * d.H + h) * d.L;
    const float* csp = cs_ws + ((int64_t)b * d.H + h) * d.L;
    const T* arow = a_src + rb * a_stride + (int64_t)h * P;
    const T* brow = xc + rb * d.C + b_chan0 + (int64_t)g * N;

    f32x4 acc[PT][NTW];
#pragma unroll
    for (int i = 0; i < PT; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float ablk = 1.f;

    for (int step = 0; step < nc; ++step) {
        const int c = BWD ? nc - 1 - step : step;
        const int64_t t0 = s0 + (int64_t)c * Q;
        const int cm = (int)(t0 / Q);
        const float cs_e = csp[t0 + Q - 1];
        const int seq_e = seq ? seq[rb + t0 + Q - 1] : 0;
        // The state entering chunk c belongs to the sequence of the token just
        // before it; for a row's first segment that is the sequence of the
        // row's first token (an initial state feeds the first sequence).
        const int64_t ptok = c > 0 ? t0 - 1 : (pred >= 0 ? pred : s0);
        const int seq_ref = seq ? seq[rb + ptok] : 0;
        const float alpha = (seq_ref == seq_e) ? expf(cs_e) : 0.f;
        ablk *= alpha;
        if (step > 0) {
            T* hp = store + (((int64_t)b * d.nchunk + cm) * d.H + h) * (P * N);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    const int nt = wave + 4 * j;
                    if (nt < NTT) {
                        const int n = nt * 16 + lr;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int p = pt * 16 + 4 * lg + r;
                            if (MODE == WALK_FWD_NP) hp[n * P + p] = (T)acc[pt][j][r];
                            else hp[p * N + n] = (T)acc[pt][j][r];
                        }
                    }
                }
        }
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
            for (int j = 0; j < NTW; ++j) acc[pt][j] *= alpha;

        for (int sl = 0; sl < Q / KT; ++sl) {
            const int64_t tb = t0 + (int64_t)sl * KT;
            __syncthreads();
            for (int idx = threadIdx.x; idx < KT * (P / VEC); idx += blockDim.x) {
                const int jj = idx / (P / VEC), pv = idx % (P / VEC);
                const vt v = *(const vt*)(arow + (tb + jj) * a_stride + pv * VEC);
#pragma unroll
                for (int e = 0; e < VEC; ++e) At[(pv * VEC + e) * PITCH + jj] = v[e];
            }
            for (int idx = threadIdx.x; idx < KT * (N / VEC); idx += blockDim.x) {
                const int jj = idx / (N / VEC), nv = idx % (N / VEC);
                const vt v = *(const vt*)(brow + (tb + jj) * d.C + nv * VEC);
#pragma unroll
                for (int e = 0; e < VEC; ++e) Bt[(nv * VEC + e) * PITCH + jj] = v[e];
            }
            if (threadIdx.x < KT) {
                const int64_t tok = tb + threadIdx.x;
                float w;
                if (BWD) {
                    const bool same = !seq || seq[rb + tok] == seq_ref;
                    w = same ? expf(csp[tok]) : 0.f;
                } else {
                    const bool same = !seq || seq[rb + tok] == seq_e;
                    w = same ? expf(cs_e - csp[tok]) * dtp[tok] : 0.f;
                }
                wv[threadIdx.x] = w;
            }
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < KT / KS; ++kk) {
                const int jl = kk * KS + SL * lg;
                float wl[SL];
#pragma unroll
                for (int s = 0; s < SL; ++s) wl[s] = wv[jl + s];
                Frag a[PT];
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
                    a[pt] = M::load_scaled(&At[(pt * 16 + lr) * PITCH + jl], wl);
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    const int nt = wave + 4 * j;
                    if (nt < NTT) {
                        const Frag bb = M::load(&Bt[(nt * 16 + lr) * PITCH + jl]);
#pragma unroll
                        for (int pt = 0; pt < PT; ++pt) acc[pt][j] = M::mma(a[pt], bb, acc[pt][j]);
                    }
                }
            }
        }
    }

    if (!summary) return;
    const int64_t per = (int64_t)d.batch * d.H * P * N;
    float* sx = summary + (int64_t)k * per + ((int64_t)b * d.H + h) * (P * N);
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int nt = wave + 4 * j;
            if (nt < NTT) {
                const int n = nt * 16 + lr;
#pragma unroll
                for (int r = 0; r < 4; ++r) sx[(pt * 16 + 4 * lg + r) * N + n] = acc[pt][j][r];
            }
        }
    if (threadIdx.x == 0)
        summary[(int64_t)d.nseg * per + ((int64_t)k * d.batch + b) * d.H + h] = ablk;
}

}  // namespace ssd
