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

#include "ssd_internal.h"

namespace ssd {

// Channels c0 .. c0 + nc - 1 of xBC go to columns 0 .. nc - 1 of `out`, whose
// token rows are ostr elements apart (the whole conv output: c0 = 0, nc =
// ostr = C).
template <typename T, int W>
__global__ void __launch_bounds__(256) k_conv1d_silu(Dims d, SegTab tab, const T* __restrict__ xBC,
                                                    const float* __restrict__ w,
                                                    const int32_t* __restrict__ seq,
                                                    int c0, int nc, int64_t ostr,
                                                    T* __restrict__ out) {
    constexpr int R = CONV_TPT + W - 1;
    typedef typename Vec4<T>::type vt;
    const int lane = threadIdx.x % 64;
    const int c = c0 + (blockIdx.x * 64 + lane) * CONV_VEC;
    const int64_t b = blockIdx.z;
    const int64_t t0 = (int64_t)blockIdx.y * CONV_TT + wave_id() * CONV_TPT;
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

}  // namespace ssd
