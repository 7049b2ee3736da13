// Per-segment walk of chunk states (forward) or state gradients (backward).
//
// One workgroup per (row, segment, head) visits the segment's chunks in causal
// order (forward) or reverse causal order (backward).  The running P x N
// matrix lives in MFMA accumulators (FP32).  For every chunk it first stores
// the running value, then applies the chunk's decay alpha_c = exp(cs_end)
// (exactly 0 when a packed sequence starts inside the chunk) and accumulates
// the chunk's own contribution A^T diag(w) B with MFMA:
//
//   forward : A = x, B = B channels, w_j = exp(cs_end - cs_j) dt_j [seq_j = seq_end];
//             the stored value is the state entering the chunk.
//   backward: A = dy, B = C channels, w_i = exp(cs_i) [seq_i = seq of the state
//             entering the chunk]; the stored value is the gradient of the
//             state leaving the chunk.
//
// The walk starts from `init` ([S][b][H][P][N] FP32: S_in forward, dS_out
// backward) or from zero; from zero, the forward walk stores nothing for a
// segment's first chunk (its entering state is zero).  The final value is
// S_ext (forward) or dL/dS_in of the segment's own outputs (backward), and the
// product of the alphas the block decay a_block, both written to `summary` if
// given.  With `gdot`, the forward walk also writes <G_c, H_c> per chunk, G_c
// read from gdot in the stored layout.
//
// This is the decay-weighted sum over earlier chunk states that
// state-spaces/mamba #482 (second comment) identifies as the part of the scan
// that must cross devices; Megatron-LM #6808 ships its segment-level result as
// the FP32 summary.
//
// A chunk is read in 64-token slices: A rows (scaled by w) and B rows go to LDS
// in their natural [token][.] layout and both MFMA operands come from
// transposed LDS reads (XT); the next slice is loaded into registers while the
// current one is multiplied.
#pragma once

#include "ssd_internal.h"
#include "xt.h"

namespace ssd {

template <typename T, int P, int N, bool BWD>
__global__ void __launch_bounds__(256) k_state_walk(Dims d, SegTab tab, const T* __restrict__ xc,
                                                   const T* __restrict__ dy,
                                                   const float* __restrict__ dt_ws,
                                                   const float* __restrict__ cs_ws,
                                                   const int32_t* __restrict__ seq,
                                                   const float* __restrict__ init,
                                                   T* __restrict__ store,
                                                   const T* __restrict__ gdot,
                                                   float* __restrict__ dotgh,
                                                   float* __restrict__ summary) {
    typedef Mma<T> M;
    typedef typename M::Frag Frag;
    constexpr int KS = M::KS;
    constexpr int KT = 64;               // tokens per LDS slice
    constexpr int NTH = 256;
    constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte load
    constexpr int XR = P + VEC, BR = N + VEC;
    constexpr int PT = P / 16, NTT = N / 16, NTW = (NTT + 3) / 4;
    constexpr int VX = (KT * (P / VEC) + NTH - 1) / NTH;  // A vectors per thread and slice
    constexpr int VB = (KT * (N / VEC) + NTH - 1) / NTH;  // B vectors per thread and slice
    __shared__ __attribute__((aligned(16))) T sX[KT * XR];
    __shared__ __attribute__((aligned(16))) T sB[KT * BR];
    __shared__ float sdot[4];
    typedef T vt __attribute__((ext_vector_type(VEC)));

    const int h = blockIdx.x, k = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int wave = wave_id(), lane = threadIdx.x % 64, lr = lane % 16, lg = lane / 16;
    const int g = h / d.hpg;
    const int Q = d.Q;
    const int64_t rb = b * d.L;
    const int64_t s0 = tab.start[k];
    const int nc = (int)(tab.len[k] / Q);
    const int spc = Q / KT;  // slices per chunk
    const int ns = nc * spc;
    const int64_t pred = seg_pred_token(tab, k);
    const float* dtp = dt_ws + ((int64_t)b * d.H + h) * d.L;
    const float* csp = cs_ws + ((int64_t)b * d.H + h) * d.L;
    const int64_t astr = BWD ? (int64_t)d.H * P : (int64_t)d.C;
    const T* arow = (BWD ? dy + rb * astr : xc + rb * astr) + (int64_t)h * P;
    const T* brow = xc + rb * d.C + (int64_t)d.H * P + (BWD ? (int64_t)d.G * N : 0) + (int64_t)g * N;
    auto chunk_of = [&](int si) { return BWD ? nc - 1 - si / spc : si / spc; };

    // ---- one slice: registers, then LDS (A scaled by its token's weight)
    vt rx[VX], rbv[VB];
    float rcs[VX], rdt[VX];
    int rsq[VX];
    auto fetch = [&](int si) {
        const int64_t tb = s0 + (int64_t)chunk_of(si) * Q + (int64_t)(si % spc) * KT;
#pragma unroll
        for (int q = 0; q < VX; ++q) {
            const int idx = threadIdx.x + q * NTH;
            if (idx < KT * (P / VEC)) {
                const int jj = idx / (P / VEC), pv = idx % (P / VEC);
                rx[q] = *(const vt*)(arow + (tb + jj) * astr + pv * VEC);
                rcs[q] = csp[tb + jj];
                rdt[q] = BWD ? 0.f : dtp[tb + jj];
                rsq[q] = seq ? seq[rb + tb + jj] : 0;
            }
        }
#pragma unroll
        for (int q = 0; q < VB; ++q) {
            const int idx = threadIdx.x + q * NTH;
            if (idx < KT * (N / VEC)) {
                const int jj = idx / (N / VEC), nv = idx % (N / VEC);
                rbv[q] = *(const vt*)(brow + (tb + jj) * d.C + nv * VEC);
            }
        }
    };
    // sref: seq_end (forward) or the entering state's sequence (backward)
    auto stash = [&](float cs_e, int sref) {
#pragma unroll
        for (int q = 0; q < VX; ++q) {
            const int idx = threadIdx.x + q * NTH;
            if (idx < KT * (P / VEC)) {
                const int jj = idx / (P / VEC), pv = idx % (P / VEC);
                const float w = rsq[q] != sref ? 0.f
                                : BWD      ? __expf(rcs[q])
                                           : __expf(cs_e - rcs[q]) * rdt[q];
                vt v;
#pragma unroll
                for (int e = 0; e < VEC; ++e) v[e] = (T)((float)rx[q][e] * w);
                *(vt*)&sX[jj * XR + pv * VEC] = v;
            }
        }
#pragma unroll
        for (int q = 0; q < VB; ++q) {
            const int idx = threadIdx.x + q * NTH;
            if (idx < KT * (N / VEC)) {
                const int jj = idx / (N / VEC), nv = idx % (N / VEC);
                *(vt*)&sB[jj * BR + nv * VEC] = rbv[q];
            }
        }
    };

    const int64_t per = (int64_t)d.batch * d.H * P * N;
    const int64_t sg = ((int64_t)k * d.batch + b) * d.H + h;
    f32x4 acc[PT][NTW];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int nt = wave + 4 * j;
            if (init && nt < NTT) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[pt][j][r] = init[sg * (P * N) + (pt * 16 + 4 * lg + r) * N + nt * 16 + lr];
            } else {
                acc[pt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    float ablk = 1.f;
    float cs_e = 0.f;
    int sref = 0;
    int64_t dot_at = -1;  // dotgh index of the chunk whose <G, H> sits in sdot

    fetch(0);
    for (int si = 0; si < ns; ++si) {
        const int c = chunk_of(si);
        if (si % spc == 0) {
            const int64_t t0 = s0 + (int64_t)c * Q;
            const int cm = (int)(t0 / Q);
            cs_e = csp[t0 + Q - 1];
            const int seq_e = seq ? seq[rb + t0 + Q - 1] : 0;
            // The state entering chunk c belongs to the sequence of the token just
            // before it; for a row's first segment that is the sequence of the
            // row's first token (an initial state feeds the first sequence).
            const int64_t ptok = c > 0 ? t0 - 1 : (pred >= 0 ? pred : s0);
            const int seq_ref = seq ? seq[rb + ptok] : 0;
            sref = BWD ? seq_ref : seq_e;
            const float alpha = (seq_ref == seq_e) ? expf(cs_e) : 0.f;
            ablk *= alpha;
            const int64_t so = (((int64_t)b * d.nchunk + cm) * d.H + h) * (P * N);
            if (store && (init || BWD || c > 0)) {
                T* hp = store + so;
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                    for (int j = 0; j < NTW; ++j) {
                        const int nt = wave + 4 * j;
                        if (nt < NTT) {
                            const int n = nt * 16 + lr;
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                hp[(pt * 16 + 4 * lg + r) * N + n] = (T)acc[pt][j][r];
                        }
                    }
            }
            if (gdot) {
                float dot = 0.f;
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                    for (int j = 0; j < NTW; ++j) {
                        const int nt = wave + 4 * j;
                        if (nt < NTT) {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                dot += (float)gdot[so + (pt * 16 + 4 * lg + r) * N + nt * 16 + lr] *
                                       acc[pt][j][r];
                        }
                    }
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
                if (lane == 0) sdot[wave] = dot;
                dot_at = ((int64_t)b * d.nchunk + cm) * d.H + h;
            }
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                for (int j = 0; j < NTW; ++j) acc[pt][j] *= alpha;
        }
        __syncthreads();  // the previous slice's products are done with the LDS
        if (dot_at >= 0 && threadIdx.x == 0) {
            dotgh[dot_at] = sdot[0] + sdot[1] + sdot[2] + sdot[3];
        }
        dot_at = -1;
        stash(cs_e, sref);
        __syncthreads();
        if (si + 1 < ns) fetch(si + 1);
#pragma unroll
        for (int kk = 0; kk < KT / KS; ++kk) {
            const int jb = kk * KS;
            Frag a[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) a[pt] = XT<T>::load(sX, XR, jb, pt * 16, lane);
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int nt = wave + 4 * j;
                if (nt < NTT) {
                    const Frag bb = XT<T>::load(sB, BR, jb, nt * 16, lane);
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) acc[pt][j] = M::mma(a[pt], bb, acc[pt][j]);
                }
            }
        }
    }

    if (!summary) return;
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
