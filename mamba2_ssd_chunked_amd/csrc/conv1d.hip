// Causal depthwise conv1d + SiLU with a causal-predecessor halo (gfx950).
//
// No LDS: every thread owns 4 consecutive channels and TPT consecutive tokens
// (memory order, inside one segment), loads the TPT + W - 1 input rows it needs
// straight into registers (the first W - 1 are the halo, read from the last
// tokens of the causal predecessor segment when the group starts a segment:
// the conv halo that Megatron-LM #6808's first commit exchanges between causal
// shards) and slides the taps over them.  The 64 lanes of a wave own 256
// consecutive channels of the same tokens, so every load and store of a wave is
// one contiguous run.  Taps that reach before the row start or across a packed
// sequence start are zero.  HBM-bound: 2*C*sizeof(act) bytes per token.
#include <type_traits>

#include "dt_prep.h"
#include "ssd_internal.h"

namespace ssd {

// Channels c0 .. c0 + nc - 1 of xBC go to columns 0 .. nc - 1 of `out`, whose
// token rows are ostr elements apart (the whole conv output: c0 = 0, nc =
// ostr = C).
// Workgroup (bx, by, bz) of the (channel block, token block, row) grid.
template <typename T, int W>
__device__ __forceinline__ void conv_block(const Dims& d, const SegTab& tab,
                                           const T* __restrict__ xBC, const float* __restrict__ w,
                                           const int32_t* __restrict__ seq, int c0, int nc,
                                           int64_t ostr, T* __restrict__ out, int bx, int by,
                                           int bz) {
    constexpr int R = CONV_TPT + W - 1;
    typedef typename Vec4<T>::type vt;
    const int lane = threadIdx.x % 64;
    const int c = c0 + (bx * 64 + lane) * CONV_VEC;
    const int64_t b = bz;
    const int64_t t0 = (int64_t)by * CONV_TT + wave_id() * CONV_TPT;
    const int64_t rb = b * d.L;
    if (c >= c0 + nc) return;  // no barriers below
    const int k = conv_seg(tab, t0);

    float wr[CONV_VEC][W];
#pragma unroll
    for (int e = 0; e < CONV_VEC; ++e)
#pragma unroll
        for (int kk = 0; kk < W; ++kk) wr[e][kk] = w[(c + e) * W + kk];

    // row r is the token r - (W-1) places after t0; rows, their positions and
    // sequence ids are the same for the whole wave (t0 is), so the tap masks are
    // scalar
    float xs[R][CONV_VEC];
    int sq[R];
    bool ok[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int mem = __builtin_amdgcn_readfirstlane(
            (int)(r >= W - 1 ? t0 + (r - (W - 1)) : conv_row(tab, k, t0, r - (W - 1))));
        ok[r] = mem >= 0;
        sq[r] = __builtin_amdgcn_readfirstlane((ok[r] && seq) ? seq[rb + mem] : 0);
        vt v;
        if (ok[r]) {
            v = *(const vt*)(xBC + (rb + mem) * d.C + c);
        } else {
#pragma unroll
            for (int e = 0; e < CONV_VEC; ++e) v[e] = (T)0.f;
        }
#pragma unroll
        for (int e = 0; e < CONV_VEC; ++e) xs[r][e] = (float)v[e];
    }
    // almost every wave sees neither a row start nor a sequence start in its rows:
    // then no tap is masked and the loop runs without selects
    bool clean = true;
#pragma unroll
    for (int r = 0; r < R; ++r) clean = clean && ok[r] && sq[r] == sq[0];
    auto run = [&](auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
        for (int t = 0; t < CONV_TPT; ++t) {
            const int ro = t + W - 1;
            float acc[CONV_VEC] = {};
#pragma unroll
            for (int kk = 0; kk < W; ++kk) {
                const int r = t + kk;
                if (!MASKED || (ok[r] && sq[r] == sq[ro])) {
#pragma unroll
                    for (int e = 0; e < CONV_VEC; ++e) acc[e] += wr[e][kk] * xs[r][e];
                }
            }
            // SiLU with the hardware reciprocal (1 ulp)
            vt o;
#pragma unroll
            for (int e = 0; e < CONV_VEC; ++e)
                o[e] = (T)(acc[e] * __builtin_amdgcn_rcpf(1.f + __expf(-acc[e])));
            *(vt*)(out + (rb + t0 + t) * ostr + (c - c0)) = o;
        }
    };
    if (clean) run(std::false_type{});
    else run(std::true_type{});
}

template <typename T, int W>
__global__ void __launch_bounds__(256) k_conv1d_silu(Dims d, SegTab tab, const T* __restrict__ xBC,
                                                    const float* __restrict__ w,
                                                    const int32_t* __restrict__ seq,
                                                    int c0, int nc, int64_t ostr,
                                                    T* __restrict__ out) {
    conv_block<T, W>(d, tab, xBC, w, seq, c0, nc, ostr, out, blockIdx.x, blockIdx.y, blockIdx.z);
}

// The whole conv pass and dt prep in one launch: the grid's first gx channel
// blocks convolve; the extra ones (their (x - gx, y) numbered within the row)
// run dt prep for DTB heads of one chunk each (dt_prep_block).  The conv is
// bound by memory bandwidth and dt prep by latency, so the two overlap.
template <typename T, int W>
__global__ void __launch_bounds__(256) k_conv1d_silu_dt(Dims d, SegTab tab,
                                                       const T* __restrict__ xBC,
                                                       const float* __restrict__ w,
                                                       const int32_t* __restrict__ seq, int gx,
                                                       T* __restrict__ out,
                                                       const T* __restrict__ dt_raw,
                                                       const float* __restrict__ dt_bias,
                                                       const float* __restrict__ A_log,
                                                       float* __restrict__ dt_ws,
                                                       float* __restrict__ cs_ws,
                                                       float* __restrict__ ctot) {
    if ((int)blockIdx.x < gx) {
        conv_block<T, W>(d, tab, xBC, w, seq, 0, d.C, d.C, out, blockIdx.x, blockIdx.y,
                         blockIdx.z);
        return;
    }
    __shared__ DtLds sm;
    const int64_t item = (int64_t)(blockIdx.x - gx) * gridDim.y + blockIdx.y;
    if (item >= (int64_t)d.nchunk * ((d.H + DTB - 1) / DTB)) return;  // whole workgroup
    const int cm = (int)(item % d.nchunk), h0 = (int)(item / d.nchunk) * DTB;
    dt_prep_block<T>(d, dt_raw, dt_bias, A_log, seq, dt_ws, cs_ws, ctot, cm, h0, blockIdx.z, sm);
}

template <typename T, int W>
static hipError_t launch_w(const Dims& d, const SegTab& t, const void* xBC, const float* w,
                           const int32_t* seq, int c0, int nc, int64_t ostr, void* out,
                           hipStream_t s) {
    dim3 grid((nc + 64 * CONV_VEC - 1) / (64 * CONV_VEC), (unsigned)(d.L / CONV_TT),
              (unsigned)d.batch);
    return launch(k_conv1d_silu<T, W>, grid, dim3(256), s, d, t, (const T*)xBC, w, seq, c0, nc,
                  ostr, (T*)out);
}

template <typename T>
static hipError_t launch_t(const Dims& d, const SegTab& t, const void* xBC, const float* w,
                           const int32_t* seq, int c0, int nc, int64_t ostr, void* out,
                           hipStream_t s) {
    switch (d.W) {
        case 1: return launch_w<T, 1>(d, t, xBC, w, seq, c0, nc, ostr, out, s);
        case 2: return launch_w<T, 2>(d, t, xBC, w, seq, c0, nc, ostr, out, s);
        case 3: return launch_w<T, 3>(d, t, xBC, w, seq, c0, nc, ostr, out, s);
        case 4: return launch_w<T, 4>(d, t, xBC, w, seq, c0, nc, ostr, out, s);
        case 5: return launch_w<T, 5>(d, t, xBC, w, seq, c0, nc, ostr, out, s);
        case 6: return launch_w<T, 6>(d, t, xBC, w, seq, c0, nc, ostr, out, s);
        case 7: return launch_w<T, 7>(d, t, xBC, w, seq, c0, nc, ostr, out, s);
        case 8: return launch_w<T, 8>(d, t, xBC, w, seq, c0, nc, ostr, out, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_conv1d_channels(const Dims& d, const SegTab& t, int act, const void* xBC,
                                  const float* w, const int32_t* seq, int c0, int nc,
                                  int64_t ostr, void* out, hipStream_t s) {
    // whole 16-byte vectors of channels, inside the row
    if (c0 < 0 || nc < 1 || c0 % CONV_VEC || nc % CONV_VEC || c0 + nc > d.C || ostr < nc)
        return hipErrorInvalidValue;
    if (act == SSD_BF16) return launch_t<bf16>(d, t, xBC, w, seq, c0, nc, ostr, out, s);
    return launch_t<float>(d, t, xBC, w, seq, c0, nc, ostr, out, s);
}

hipError_t launch_conv1d_fwd(const Dims& d, const SegTab& t, int act, const void* xBC,
                             const float* w, const int32_t* seq, void* out, hipStream_t s) {
    return launch_conv1d_channels(d, t, act, xBC, w, seq, 0, d.C, d.C, out, s);
}

template <typename T, int W>
static hipError_t launch_dt_w(const Dims& d, const SegTab& t, const void* xBC, const float* w,
                              const int32_t* seq, void* out, const void* dt_raw,
                              const float* dt_bias, const float* A_log, float* dt_ws,
                              float* cs_ws, float* ctot, hipStream_t s) {
    const int gx = (d.C + 64 * CONV_VEC - 1) / (64 * CONV_VEC);
    const int gy = (int)(d.L / CONV_TT);
    const int items = d.nchunk * ((d.H + DTB - 1) / DTB);  // dt prep workgroups per row
    const dim3 grid((unsigned)(gx + (items + gy - 1) / gy), (unsigned)gy, (unsigned)d.batch);
    return launch(k_conv1d_silu_dt<T, W>, grid, dim3(256), s, d, t, (const T*)xBC, w, seq, gx,
                  (T*)out, (const T*)dt_raw, dt_bias, A_log, dt_ws, cs_ws, ctot);
}

template <typename T>
static hipError_t launch_dt_t(const Dims& d, const SegTab& t, const void* xBC, const float* w,
                              const int32_t* seq, void* out, const void* dt_raw,
                              const float* dt_bias, const float* A_log, float* dt_ws,
                              float* cs_ws, float* ctot, hipStream_t s) {
#define SSD_CONV_DT(WW)                                                                     \
    case WW:                                                                                \
        return launch_dt_w<T, WW>(d, t, xBC, w, seq, out, dt_raw, dt_bias, A_log, dt_ws, cs_ws, \
                                  ctot, s);
    switch (d.W) {
        SSD_CONV_DT(1) SSD_CONV_DT(2) SSD_CONV_DT(3) SSD_CONV_DT(4)
        SSD_CONV_DT(5) SSD_CONV_DT(6) SSD_CONV_DT(7) SSD_CONV_DT(8)
        default: return hipErrorInvalidValue;
    }
#undef SSD_CONV_DT
}

hipError_t launch_conv1d_dt(const Dims& d, const SegTab& t, int act, const void* xBC,
                            const float* w, const int32_t* seq, void* out, const void* dt_raw,
                            const float* dt_bias, const float* A_log, float* dt_ws, float* cs_ws,
                            float* ctot, hipStream_t s) {
    if (act == SSD_BF16)
        return launch_dt_t<bf16>(d, t, xBC, w, seq, out, dt_raw, dt_bias, A_log, dt_ws, cs_ws,
                                 ctot, s);
    return launch_dt_t<float>(d, t, xBC, w, seq, out, dt_raw, dt_bias, A_log, dt_ws, cs_ws, ctot,
                              s);
}

}  // namespace ssd
