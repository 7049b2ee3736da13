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

// One wave per (output tiles w and QT-1-w, every GSPLIT-th source tile, chunk,
// group, row): 2048 waves at the mixer shard's shape, each with a few
// independent tile products to keep loads in flight.
constexpr int GSPLIT = 4;
// One block of the Gram pass: bx = (tile pair, source-tile part), by =
// (chunk, group), b = row.  The B and C channels of token row m are at bc +
// m * bstr (B of group g at g N, C at (G + g) N).
template <typename T, int N, bool TRANS>
__device__ __forceinline__ void gram_block(const Dims& d, const T* __restrict__ bc, int64_t bstr,
                                           T* __restrict__ gram, int bx, int by, int64_t b) {
    typedef Mma<T> M;
    typedef typename M::Frag Frag;
    constexpr int SL = M::SL, KS = M::KS, NKF = N / KS;
    typedef T t4 __attribute__((ext_vector_type(4)));
    const int QT = d.Q / 16;
    const int w = bx / GSPLIT, part = bx % GSPLIT;
    const int g = by % d.G, cm = by / d.G;
    const int lane = threadIdx.x, lr = lane % 16, lg = lane / 16;
    const int64_t t0 = b * d.L + (int64_t)cm * d.Q;
    const int64_t boff = (int64_t)g * N;
    const int64_t coff = boff + (int64_t)d.G * N;
    T* out = gram + (((int64_t)b * d.nchunk + cm) * d.G + g) * (int64_t)gram_tiles(QT) * 256;
    for (int side = 0; side < 2; ++side) {
        const int a = side == 0 ? w : QT - 1 - w;
        if (side == 1 && a == w) break;
        Frag cf[NKF];
#pragma unroll
        for (int kn = 0; kn < NKF; ++kn)
            cf[kn] = M::load(bc + (t0 + a * 16 + lr) * bstr + coff + kn * KS + SL * lg);
#pragma unroll 2
        for (int bt = part; bt <= a; bt += GSPLIT) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kn = 0; kn < NKF; ++kn) {
                const Frag bf = M::load(bc + (t0 + bt * 16 + lr) * bstr + boff + kn * KS + SL * lg);
                acc = TRANS ? M::mma(cf[kn], bf, acc) : M::mma(bf, cf[kn], acc);
            }
            *(t4*)(out + (int64_t)gram_index(a, bt) * 256 + lane * 4) =
                t4{(T)acc[0], (T)acc[1], (T)acc[2], (T)acc[3]};
        }
    }
}

// The Gram pass and dt prep in one launch: the first blocks are Gram blocks,
// the rest one wave per (row, chunk, head) of dt prep.  The two read different
// inputs (B, C and dt_raw) and have no order between them, so their blocks
// share the chip instead of running one kernel after the other.
template <typename T, int N, bool TRANS>
__global__ void __launch_bounds__(64) k_gram_dt(Dims d, const T* __restrict__ bc, int64_t bstr,
                                               T* __restrict__ gram, int64_t ngram,
                                               const T* __restrict__ dt_raw,
                                               const float* __restrict__ dt_bias,
                                               const float* __restrict__ A_log,
                                               const int32_t* __restrict__ seq,
                                               float* __restrict__ dt_ws,
                                               float* __restrict__ cs_ws,
                                               float* __restrict__ ctot) {
    const int64_t i = blockIdx.x;
    if (i < ngram) {
        const int gx = d.Q / 16 / 2 * GSPLIT, gy = d.nchunk * d.G;
        gram_block<T, N, TRANS>(d, bc, bstr, gram, (int)(i % gx), (int)((i / gx) % gy),
                                i / gx / gy);
    } else {
        const int64_t j = i - ngram;
        dt_prep_wave<T>(d, dt_raw, dt_bias, A_log, seq, dt_ws, cs_ws, ctot,
                        (int)((j / d.H) % d.nchunk), (int)(j % d.H), j / d.H / d.nchunk,
                        threadIdx.x);
    }
}

template <typename T, int N, bool TRANS = false>
inline hipError_t launch_gram_dt(const Dims& d, const T* bc, int64_t bstr, T* gram,
                                 const void* dt_raw,
                                 const float* dt_bias, const float* A_log, const int32_t* seq,
                                 float* dt_ws, float* cs_ws, float* ctot, hipStream_t s) {
    const int64_t ngram = (int64_t)(d.Q / 16 / 2 * GSPLIT) * d.nchunk * d.G * d.batch;
    const int64_t ndt = (int64_t)d.nchunk * d.H * d.batch;
    return launch(k_gram_dt<T, N, TRANS>, dim3((unsigned)(ngram + ndt)), dim3(64), s, d, bc, bstr,
                  gram, ngram, (const T*)dt_raw, dt_bias, A_log, seq, dt_ws, cs_ws, ctot);
}

}  // namespace ssd
