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

// dt, the segmented cumulative sum and the chunk total of head h of chunk cm,
// one wave: lane `lane` holds the raw dt (before bias) of its E = Q/64
// consecutive tokens in raw[0..E-1], their sequence ids in sqs and the id of
// the token before its first in sprev (all 0 without sequence ids).
__device__ __forceinline__ void dt_prep_scan(const Dims& d, const float (&raw)[4],
                                             const int (&sqs)[4], int sprev,
                                             const float* __restrict__ dt_bias,
                                             const float* __restrict__ A_log,
                                             float* __restrict__ dt_ws, float* __restrict__ cs_ws,
                                             float* __restrict__ ctot, int cm, int h, int64_t b,
                                             int lane) {
    const int Q = d.Q;
    const int E = Q / 64;  // tokens per lane (1, 2 or 4)
    const float A = -expf(A_log[h]);
    const float bias = dt_bias[h];
    float dtv[4], csl[4];
    bool rs[4];  // a sequence starts at or before this token, inside this lane
    bool lflag = false;
    float run = 0.f;
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
    float cso[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) cso[e] = rs[e] ? csl[e] : ev + csl[e];
    if (E == 4) {  // one 16-byte store each (o is a multiple of 4 floats)
        *(f32x4*)(dt_ws + o) = f32x4{dtv[0], dtv[1], dtv[2], dtv[3]};
        *(f32x4*)(cs_ws + o) = f32x4{cso[0], cso[1], cso[2], cso[3]};
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (e < E) {
                dt_ws[o + e] = dtv[e];
                cs_ws[o + e] = cso[e];
            }
        }
    }
    // the chunk total is the last token's cumulative sum, bit for bit
    if (lane == 63) ctot[((int64_t)b * d.H + h) * d.nchunk + cm] = cso[E - 1];
}

// dt prep of head h of chunk cm by one wave, reading its inputs itself.
template <typename T>
__device__ __forceinline__ void dt_prep_wave(const Dims& d, const T* __restrict__ dt_raw,
                                             const float* __restrict__ dt_bias,
                                             const float* __restrict__ A_log,
                                             const int32_t* __restrict__ seq,
                                             float* __restrict__ dt_ws,
                                             float* __restrict__ cs_ws,
                                             float* __restrict__ ctot, int cm, int h, int64_t b,
                                             int lane) {
    const int E = d.Q / 64;
    const int64_t tok0 = b * d.L + (int64_t)cm * d.Q + lane * E;
    const int sprev = (seq && lane * E > 0) ? seq[tok0 - 1] : 0;
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
    dt_prep_scan(d, raw, sqs, sprev, dt_bias, A_log, dt_ws, cs_ws, ctot, cm, h, b, lane);
}

// dt prep of DTB = 4 consecutive heads h0 .. of chunk cm by a workgroup of 256
// threads.  dt_raw is [token][H]: a wave reading one head at a time touches a
// cache line per token for 2 or 4 bytes, so the workgroup reads each token's
// DTB heads at once (one 8- or 16-byte load where H allows), stages them and
// the sequence ids in LDS, and each wave scans one head from there.
constexpr int DTB = 4;
struct DtLds {
    float raw[256][DTB + 1];
    int sq[256];
};
template <typename T>
__device__ __forceinline__ void dt_prep_block(const Dims& d, const T* __restrict__ dt_raw,
                                              const float* __restrict__ dt_bias,
                                              const float* __restrict__ A_log,
                                              const int32_t* __restrict__ seq,
                                              float* __restrict__ dt_ws, float* __restrict__ cs_ws,
                                              float* __restrict__ ctot, int cm, int h0, int64_t b,
                                              DtLds& sm) {
    const int Q = d.Q, E = Q / 64;
    const int j = threadIdx.x;  // token of the chunk
    const int64_t row = b * d.L + (int64_t)cm * Q;
    if (j < Q) {
        const T* src = dt_raw + (row + j) * d.H + h0;
        float v[DTB];
        constexpr int VW = DTB;  // one load of the DTB heads
        if (h0 + DTB <= d.H && d.H % VW == 0) {
            // aligned: dt_raw is (16 bytes), and (token H + h0) is a multiple of VW
            typedef T vt __attribute__((ext_vector_type(VW)));
#pragma unroll
            for (int q = 0; q < DTB / VW; ++q) {
                const vt x = *(const vt*)(src + q * VW);
#pragma unroll
                for (int e = 0; e < VW; ++e) v[q * VW + e] = to_f(x[e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < DTB; ++e) v[e] = (h0 + e < d.H) ? to_f(src[e]) : 0.f;
        }
        const int sv = seq ? seq[row + j] : 0;
#pragma unroll
        for (int e = 0; e < DTB; ++e) sm.raw[j][e] = v[e];
        sm.sq[j] = sv;
    }
    __syncthreads();
    const int lane = threadIdx.x % 64, w = threadIdx.x / 64;
    float raw[4];
    int sqs[4];
    const int t0 = lane * E;
#pragma unroll
    for (int e = 0; e < 4; ++e) sqs[e] = sm.sq[t0 + min(e, E - 1)];
    const int sprev = t0 > 0 ? sm.sq[t0 - 1] : 0;
#pragma unroll
    for (int k = 0; k < DTB / 4; ++k) {
        const int hh = w + 4 * k;
        if (h0 + hh >= d.H) break;  // wave-uniform
#pragma unroll
        for (int e = 0; e < 4; ++e) raw[e] = sm.raw[t0 + min(e, E - 1)][hh];
        dt_prep_scan(d, raw, sqs, sprev, dt_bias, A_log, dt_ws, cs_ws, ctot, cm, h0 + hh, b, lane);
    }
}

}  // namespace ssd
