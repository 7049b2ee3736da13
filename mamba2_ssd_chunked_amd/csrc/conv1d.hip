// Causal depthwise conv1d + SiLU with a causal-predecessor halo (gfx950).
//
// Each workgroup owns 64 consecutive tokens (memory order, inside one segment)
// and 128 channels.  It stages the 64 + W - 1 input rows in LDS with coalesced
// 16-byte loads; the first W - 1 rows are the halo, read from the last tokens
// of the causal predecessor segment when the tile starts a segment (the conv
// halo that Megatron-LM #6808's first commit exchanges between causal shards).  Taps that reach before the row start or across a packed
// sequence start are zero.  HBM-bound: 2*C*sizeof(act) bytes per token.
#include "ssd_internal.h"

namespace ssd {

constexpr int CONV_TT = 64;   // tokens per workgroup
constexpr int CONV_CT = 128;  // channels per workgroup
constexpr int CONV_MAXW = 8;  // widest supported conv
constexpr int CONV_ROWS = CONV_TT + CONV_MAXW - 1;

template <typename T, int W>
__global__ void __launch_bounds__(256) k_conv1d_silu(Dims d, SegTab tab, const T* __restrict__ xBC,
                                                    const float* __restrict__ w,
                                                    const int32_t* __restrict__ seq,
                                                    T* __restrict__ out) {
    constexpr int VEC = 8;                // channels per thread vector
    constexpr int CV = CONV_CT / VEC;     // vectors per row
    typedef T vec_t __attribute__((ext_vector_type(8)));
    __shared__ __attribute__((aligned(16))) T tile[CONV_ROWS * CONV_CT];
    __shared__ int64_t rowmem[CONV_ROWS];
    __shared__ int rowseq[CONV_ROWS];

    const int64_t b = blockIdx.z;
    const int64_t t0 = (int64_t)blockIdx.y * CONV_TT;
    const int c0 = blockIdx.x * CONV_CT;
    const int rows = CONV_TT + W - 1;
    const int64_t rb = b * d.L;

    int k = 0;
    for (int i = 0; i < tab.n; ++i)
        if (t0 >= tab.start[i] && t0 < tab.start[i] + tab.len[i]) k = i;
    const int64_t s0 = tab.start[k];

    // LDS row r holds causal token (t0 - (W-1) + r); find its memory position.
    for (int r = threadIdx.x; r < rows; r += blockDim.x) {
        const int64_t m = t0 - (W - 1) + r;
        int64_t mem;
        if (m >= s0) mem = m;
        else if (k > 0) mem = tab.start[k - 1] + tab.len[k - 1] - (s0 - m);
        else mem = -1;
        rowmem[r] = mem;
        rowseq[r] = (mem >= 0 && seq) ? seq[rb + mem] : 0;
    }
    __syncthreads();

    for (int idx = threadIdx.x; idx < rows * CV; idx += blockDim.x) {
        const int r = idx / CV, v = idx % CV;
        const int c = c0 + v * VEC;
        vec_t val;
        if (c < d.C && rowmem[r] >= 0) {
            val = *(const vec_t*)(xBC + (rb + rowmem[r]) * d.C + c);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) val[e] = (T)0.f;
        }
        *(vec_t*)(tile + r * CONV_CT + v * VEC) = val;
    }
    __syncthreads();

    // Every thread keeps one channel vector (idx % CV is fixed since blockDim % CV == 0).
    const int v = threadIdx.x % CV;
    const int c = c0 + v * VEC;
    if (c >= d.C) return;
    float wr[VEC][W];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int kk = 0; kk < W; ++kk) wr[e][kk] = w[(c + e) * W + kk];

    for (int idx = threadIdx.x; idx < CONV_TT * CV; idx += blockDim.x) {
        const int t = idx / CV;
        const int ro = t + W - 1;  // LDS row of the output token
        const int sq = rowseq[ro];
        float acc[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < W; ++kk) {
            const int r = t + kk;
            if (rowmem[r] < 0 || rowseq[r] != sq) continue;
            const vec_t xv = *(const vec_t*)(tile + r * CONV_CT + v * VEC);
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] += wr[e][kk] * (float)xv[e];
        }
        vec_t o;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float u = acc[e];
            o[e] = (T)(u / (1.f + expf(-u)));
        }
        *(vec_t*)(out + (rb + t0 + t) * d.C + c) = o;
    }
}

template <typename T, int W>
static void launch_w(const Dims& d, const SegTab& t, const void* xBC, const float* w,
                     const int32_t* seq, void* out, hipStream_t s) {
    dim3 grid((d.C + CONV_CT - 1) / CONV_CT, (unsigned)(d.L / CONV_TT), (unsigned)d.batch);
    hipLaunchKernelGGL((k_conv1d_silu<T, W>), grid, dim3(256), 0, s, d, t, (const T*)xBC, w, seq,
                       (T*)out);
}

template <typename T>
static void launch_t(const Dims& d, const SegTab& t, const void* xBC, const float* w,
                     const int32_t* seq, void* out, hipStream_t s) {
    switch (d.W) {
        case 1: launch_w<T, 1>(d, t, xBC, w, seq, out, s); break;
        case 2: launch_w<T, 2>(d, t, xBC, w, seq, out, s); break;
        case 3: launch_w<T, 3>(d, t, xBC, w, seq, out, s); break;
        case 4: launch_w<T, 4>(d, t, xBC, w, seq, out, s); break;
        case 5: launch_w<T, 5>(d, t, xBC, w, seq, out, s); break;
        case 6: launch_w<T, 6>(d, t, xBC, w, seq, out, s); break;
        case 7: launch_w<T, 7>(d, t, xBC, w, seq, out, s); break;
        default: launch_w<T, 8>(d, t, xBC, w, seq, out, s); break;
    }
}

hipError_t launch_conv1d_fwd(const Dims& d, const SegTab& t, int act, const void* xBC,
                             const float* w, const int32_t* seq, void* out, hipStream_t s) {
    if (act == SSD_BF16) launch_t<bf16>(d, t, xBC, w, seq, out, s);
    else launch_t<float>(d, t, xBC, w, seq, out, s);
    return hipGetLastError();
}

}  // namespace ssd
