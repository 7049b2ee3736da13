// Causal depthwise conv1d + SiLU recomputed inside the kernels that consume
// its output (the conv-fused forward: the x channels never go to memory).
//
// A thread owns one VEC-channel column of one head and NO consecutive output
// rows of a tile, and holds the NO + W - 1 raw input rows their taps reach in
// registers: the first W - 1 of them are the halo before its first row, earlier
// rows of the same tile or, across a segment start, the last rows of the causal
// predecessor segment (the conv halo that Megatron-LM #6808's first commit
// exchanges between causal shards; state-spaces/mamba #482, second comment,
// places the conv before the scan).  Rows that do not exist are zero and their
// taps are skipped, as are taps that reach across a packed sequence start
// (seq_idx).  The arithmetic is the conv pass's own, tap by tap in the same
// order and with the same SiLU, so a fused consumer multiplies exactly the
// values the conv pass would have stored.
#pragma once

#include "ssd_internal.h"

namespace ssd {

// Memory row of window row r, for a window whose first output row is token t
// (memory order) of segment k: token t + r - (W - 1); rows before the segment
// start come from its causal predecessor, -1 where there is none.
template <int W>
__device__ __forceinline__ int64_t window_row(const SegTab& tab, int k, int64_t t, int r) {
    return r >= W - 1 ? t + (r - (W - 1)) : conv_row(tab, k, t, r - (W - 1));
}

// One thread's window: NR raw rows of one VEC-channel column, the sequence id
// of each row and a bit per row that exists.
template <typename T, int VEC, int NR>
struct ConvWindow {
    typedef T vt __attribute__((ext_vector_type(VEC)));
    vt x[NR];
    int sq[NR];
    unsigned ok;
};

// Loads the window of the column at element offset `col` of token rows
// t .. t + NR - W (memory order) of segment k in batch row rb (token row
// stride C elements).
template <typename T, int VEC, int W, int NR>
__device__ __forceinline__ void load_window(ConvWindow<T, VEC, NR>& cw, const T* __restrict__ src,
                                            const int32_t* __restrict__ seq, const SegTab& tab,
                                            int k, int64_t rb, int64_t t, int64_t C, int64_t col) {
    typedef typename ConvWindow<T, VEC, NR>::vt vt;
    cw.ok = 0;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int64_t m = window_row<W>(tab, k, t, r);
        if (m >= 0) {
            cw.x[r] = *(const vt*)(src + (rb + m) * C + col);
            cw.sq[r] = seq ? seq[rb + m] : 0;
            cw.ok |= 1u << r;
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) cw.x[r][e] = (T)0.f;
            cw.sq[r] = 0;
        }
    }
}

// The tap weights of the column's VEC channels, channel c0 first ([C][W] layout).
template <int VEC, int W>
__device__ __forceinline__ void load_taps(float (&w)[VEC][W], const float* __restrict__ conv_w,
                                          int64_t c0) {
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int kk = 0; kk < W; ++kk) w[e][kk] = conv_w[(c0 + e) * W + kk];
}

// True if no tap of the window is skipped: every row exists and all rows
// belong to one sequence.
template <typename T, int VEC, int NR>
__device__ __forceinline__ bool window_clean(const ConvWindow<T, VEC, NR>& cw) {
    bool c = cw.ok == (1u << NR) - 1;
#pragma unroll
    for (int r = 1; r < NR; ++r) c = c && cw.sq[r] == cw.sq[0];
    return c;
}

// conv + SiLU of output row o of the window (taps on rows o .. o + W - 1, the
// last one the output row's own), rounded to T as the conv pass stores it.
template <typename T, int VEC, int W, int NR, bool MASKED>
__device__ __forceinline__ typename ConvWindow<T, VEC, NR>::vt conv_silu(
    const ConvWindow<T, VEC, NR>& cw, int o, const float (&w)[VEC][W]) {
    typename ConvWindow<T, VEC, NR>::vt out;
    float acc[VEC] = {};
    const int ro = o + W - 1;
#pragma unroll
    for (int kk = 0; kk < W; ++kk) {
        const int r = o + kk;
        if (!MASKED || (((cw.ok >> r) & 1u) && cw.sq[r] == cw.sq[ro])) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] += w[e][kk] * (float)cw.x[r][e];
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) out[e] = (T)(acc[e] * __builtin_amdgcn_rcpf(1.f + __expf(-acc[e])));
    return out;
}

}  // namespace ssd
