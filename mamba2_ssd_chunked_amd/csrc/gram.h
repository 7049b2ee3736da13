// Causal Gram tiles of a chunk: G_ab[j][i] = B_j . C_i for 16-token tiles
// a >= b (output tile a holds i, source tile b holds j), one per (row, chunk,
// group).  Every head of the group weights the same C B^T by its own decays, so
// the product is formed once here instead of once per head.  This is the
// "local CB computation" of Megatron-LM #6808 (first commit), which it overlaps
// with the summary exchange.
//
// Tile layout: the MFMA output layout, stored lane by lane, so that one wave
// reads a tile back with one 8-byte (bf16) or 16-byte (float32) load per lane:
// lane l holds column i = l % 16 and rows j = 4 (l / 16) + r, r = 0..3.
// Tiles of a (row, chunk, group) are numbered t = a (a + 1) / 2 + b.
// TRANS = true stores the transposed tiles S_ab[i][j] = C_i . B_j instead (lane
// l holds column j = l % 16 and rows i = 4 (l / 16) + r), the orientation the
// chunk backward consumes.
#pragma once

#include "dt_prep.h"
#include "ssd_internal.h"

namespace ssd {

__host__ __device__ constexpr int gram_tiles(int qt) { return qt * (qt + 1) / 2; }
__host__ __device__ constexpr int gram_index(int a, int b) { return a * (a + 1) / 2 + b; }

// One workgroup of QT / 2 waves per (row, chunk, group), split S ways over the
// source tiles when there are fewer than 256 (row, chunk, group) items: split z
// forms the tiles whose source tile b has b % S == z.  It stages those B rows
// in LDS once; wave w holds the C rows of output tiles w and QT-1-w as MFMA
// operands and forms their tiles of the split from the staged rows.  Every B
// row is read from memory once per (chunk, group), every C row once per split.
// The same workgroups run dt prep for the group's heads of their chunk (head j
// of the group in split j % S, one head per wave and round): the two read
// different inputs.
inline int gram_split(const Dims& d) {
    const int64_t items = (int64_t)d.nchunk * d.G * d.batch;
    const int pairs = d.Q / 32;
    int S = 1;
    while (S < pairs && items * S < 256) S *= 2;
    return S;
}

// LDS of a Gram workgroup (elements of T): the staged B rows.
template <typename T, int N, int Q>
constexpr int gram_lds() {
    return Q * (N + 16 / (int)sizeof(T));
}

// One Gram workgroup: workgroup j of n (the XCD-aware item mapping is over this
// range), its B rows staged at sB; with_dt: also the dt prep of its heads.
template <typename T, int N, int Q, bool TRANS>
__device__ __forceinline__ void gram_block(const Dims& d, int S, const T* __restrict__ bc,
                                           int64_t bstr, T* __restrict__ gram, T* sB, int64_t j,
                                           int64_t n, bool with_dt, const T* __restrict__ dt_raw,
                                           const float* __restrict__ dt_bias,
                                           const float* __restrict__ A_log,
                                           const int32_t* __restrict__ seq,
                                           float* __restrict__ dt_ws, float* __restrict__ cs_ws,
                                           float* __restrict__ ctot) {
    typedef Mma<T> M;
    typedef typename M::Frag Frag;
    constexpr int SL = M::SL, KS = M::KS, NKF = N / KS, QT = Q / 16;
    constexpr int VEC = 16 / (int)sizeof(T), BR = N + VEC;
    typedef T vt __attribute__((ext_vector_type(VEC)));
    typedef T t4 __attribute__((ext_vector_type(4)));

    // block -> (split, group, chunk, row); the S splits of a (chunk, group) are
    // consecutive items, and each XCD takes one contiguous range of items
    constexpr int NXCD = 8;
    int64_t item = (n % NXCD == 0) ? (j % NXCD) * (n / NXCD) + j / NXCD : j;
    const int z = (int)(item % S);
    item /= S;
    const int g = (int)(item % d.G);
    item /= d.G;
    const int cm = (int)(item % d.nchunk);
    const int64_t b = item / d.nchunk;
    constexpr int GW = QT / 2;  // waves of the workgroup
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, lr = lane % 16, lg = lane / 16;
    const int a0 = wave, a1 = QT - 1 - wave;
    const int64_t t0 = b * d.L + (int64_t)cm * Q;
    const int64_t boff = (int64_t)g * N;
    const int64_t coff = boff + (int64_t)d.G * N;

    Frag cf[2][NKF];
#pragma unroll
    for (int kn = 0; kn < NKF; ++kn) {
        cf[0][kn] = M::load(bc + (t0 + a0 * 16 + lr) * bstr + coff + kn * KS + SL * lg);
        cf[1][kn] = M::load(bc + (t0 + a1 * 16 + lr) * bstr + coff + kn * KS + SL * lg);
    }
    // B rows of the split's source tiles z, z + S, ...: LDS row (bt / S) * 16 + r
    const int rows = (QT - z + S - 1) / S * 16;
    for (int idx = threadIdx.x; idx < rows * (N / VEC); idx += GW * 64) {
        const int r = idx / (N / VEC), v = idx % (N / VEC);
        const int tok = ((r / 16) * S + z) * 16 + r % 16;
        *(vt*)&sB[r * BR + v * VEC] = *(const vt*)(bc + (t0 + tok) * bstr + boff + v * VEC);
    }
    __syncthreads();
    T* out = gram + (((int64_t)b * d.nchunk + cm) * d.G + g) * (int64_t)gram_tiles(QT) * 256 + lane * 4;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int a = it == 0 ? a0 : a1;
        for (int bt = z; bt <= a; bt += S) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kn = 0; kn < NKF; ++kn) {
                const Frag bf = M::load(&sB[((bt / S) * 16 + lr) * BR + kn * KS + SL * lg]);
                acc = TRANS ? M::mma(cf[it][kn], bf, acc) : M::mma(bf, cf[it][kn], acc);
            }
            *(t4*)(out + (int64_t)gram_index(a, bt) * 256) = t4{(T)acc[0], (T)acc[1], (T)acc[2], (T)acc[3]};
        }
    }
    if (!with_dt) return;
    for (int hj = z + S * wave; hj < d.hpg; hj += S * GW)
        dt_prep_wave<T>(d, dt_raw, dt_bias, A_log, seq, dt_ws, cs_ws, ctot, cm, g * d.hpg + hj, b, lane);
}

template <typename T, int N, int Q, bool TRANS>
__global__ void __launch_bounds__(Q / 32 * 64) k_gram_dt(Dims d, int S, const T* __restrict__ bc,
                                                        int64_t bstr, T* __restrict__ gram,
                                                        const T* __restrict__ dt_raw,
                                                        const float* __restrict__ dt_bias,
                                                        const float* __restrict__ A_log,
                                                        const int32_t* __restrict__ seq,
                                                        float* __restrict__ dt_ws,
                                                        float* __restrict__ cs_ws,
                                                        float* __restrict__ ctot) {
    __shared__ __attribute__((aligned(16))) T sB[gram_lds<T, N, Q>()];
    gram_block<T, N, Q, TRANS>(d, S, bc, bstr, gram, sB, blockIdx.x, gridDim.x, true, dt_raw,
                               dt_bias, A_log, seq, dt_ws, cs_ws, ctot);
}

template <typename T, int N, int Q, bool TRANS>
inline hipError_t launch_gram_dt_q(const Dims& d, const T* bc, int64_t bstr, T* gram,
                                   const void* dt_raw, const float* dt_bias, const float* A_log,
                                   const int32_t* seq, float* dt_ws, float* cs_ws, float* ctot,
                                   hipStream_t s) {
    const int S = gram_split(d);
    const int64_t nblk = (int64_t)d.nchunk * d.G * d.batch * S;
    return launch(k_gram_dt<T, N, Q, TRANS>, dim3((unsigned)nblk), dim3(Q / 32 * 64), s, d, S,
                  bc, bstr, gram, (const T*)dt_raw, dt_bias, A_log, seq, dt_ws, cs_ws, ctot);
}

// The Gram tiles and dt prep in one launch.  B and C channels of token row m at
// bc + m * bstr (B of group g at g N, C at (G + g) N).
template <typename T, int N, bool TRANS = false>
inline hipError_t launch_gram_dt(const Dims& d, const T* bc, int64_t bstr, T* gram,
                                 const void* dt_raw, const float* dt_bias, const float* A_log,
                                 const int32_t* seq, float* dt_ws, float* cs_ws, float* ctot,
                                 hipStream_t s) {
    switch (d.Q) {
        case 64:
            return launch_gram_dt_q<T, N, 64, TRANS>(d, bc, bstr, gram, dt_raw, dt_bias, A_log, seq,
                                                     dt_ws, cs_ws, ctot, s);
        case 128:
            return launch_gram_dt_q<T, N, 128, TRANS>(d, bc, bstr, gram, dt_raw, dt_bias, A_log,
                                                      seq, dt_ws, cs_ws, ctot, s);
        case 256:
            return launch_gram_dt_q<T, N, 256, TRANS>(d, bc, bstr, gram, dt_raw, dt_bias, A_log,
                                                      seq, dt_ws, cs_ws, ctot, s);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace ssd
