// dt prep: dt = clamp(softplus(dt_raw + dt_bias), dt_min, dt_max), the
// chunk-local cumulative sum of dt A with A = -exp(A_log), and the chunk total.
// One wave per (row, chunk, head); lane l owns the Q/64 consecutive tokens
// l*Q/64 ...  The cumsum restarts at every packed-sequence start inside the
// chunk (a segmented scan), so a sequence's decays are computed from its own
// tokens only and perturbing one sequence cannot change another's bits.
#pragma once

#include "ssd_internal.h"

namespace ssd {

__device__ __forceinline__ float softplus_f(float z) {
    return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
}

template <typename T>
__device__ __forceinline__ void dt_prep_wave(const Dims& d, const T* __restrict__ dt_raw,
                                             const float* __restrict__ dt_bias,
                                             const float* __restrict__ A_log,
                                             const int32_t* __restrict__ seq,
                                             float* __restrict__ dt_ws,
                                             float* __restrict__ cs_ws,
                                             float* __restrict__ ctot, int cm, int h, int64_t b,
                                             int lane) {
    const int Q = d.Q;
    const int E = Q / 64;  // tokens per lane (1, 2 or 4)
    const int64_t tok0 = b * d.L + (int64_t)cm * Q + lane * E;
    const float A = -expf(A_log[h]);
    const float bias = dt_bias[h];
    float dtv[4], csl[4];
    bool rs[4];  // a sequence starts at or before this token, inside this lane
    bool lflag = false;
    float run = 0.f;
    int sprev = (seq && lane * E > 0) ? seq[tok0 - 1] : 0;
    // every input of the lane's tokens first, in one memory round trip (slots
    // e >= E repeat the last token and are not used): a load under the e < E
    // branch would be waited for before the next slot's load is issued
    float raw[4];
    int sqs[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) raw[e] = to_f(dt_raw[(tok0 + min(e, E - 1)) * d.H + h]);
    if (seq) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sqs[e] = seq[tok0 + min(e, E - 1)];
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) sqs[e] = 0;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (e < E) {
            const int j = lane * E + e;
            const int sj = sqs[e];
            const bool start = j > 0 && sj != sprev;
            sprev = sj;
            lflag = lflag || start;
            rs[e] = lflag;
            if (start) run = 0.f;
            const float z = raw[e] + bias;
            const float dt = fminf(fmaxf(softplus_f(z), d.dt_min), d.dt_max);
            dtv[e] = dt;
            run += dt * A;
            csl[e] = run;
        }
    }
    // Segmented inclusive scan of (flag, sum) across the wave:
    // (f1, v1) then (f2, v2) -> (f1 | f2, f2 ? v2 : v1 + v2).
    float iv = run;
    bool ifl = lflag;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float v = __shfl_up(iv, off, 64);
        const int f = __shfl_up((int)ifl, off, 64);
        if (lane >= off) {
            if (!ifl) iv += v;
            ifl = ifl || f;
        }
    }
    float ev = __shfl_up(iv, 1, 64);
    if (lane == 0) ev = 0.f;
    const int64_t o = ((int64_t)b * d.H + h) * d.L + (int64_t)cm * Q + lane * E;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (e < E) {
            dt_ws[o + e] = dtv[e];
            cs_ws[o + e] = rs[e] ? csl[e] : ev + csl[e];
        }
    }
    // the chunk total is the last token's cumulative sum, bit for bit
    if (lane == 63)
        ctot[((int64_t)b * d.H + h) * d.nchunk + cm] = rs[E - 1] ? csl[E - 1] : ev + csl[E - 1];
}

}  // namespace ssd
