// Segment-local SSD forward and the correction pass (gfx950, wave64, MFMA).
//
// Kernels, in launch order:
//   k_dt_prep      dt = clamp(softplus(dt_raw + dt_bias)), l = dt*A, and the
//                  chunk-local inclusive cumsum cs of l, per (row, head, chunk).
//   k_state_walk   (state_walk.h) one workgroup per (row, segment, head) walks
//                  the segment's chunks in causal order.  The running state H (P x N, FP32)
//                  lives in MFMA accumulators: for chunk c it first writes H
//                  (the state entering c), scales it by the chunk decay
//                  alpha_c = exp(cs_end) (exactly 0 across a sequence start)
//                  and then accumulates the chunk state
//                  Z_c = X^T diag(exp(cs_end - cs_j) dt_j) B with MFMA, so the
//                  inter-chunk recurrence H <- alpha_c H + Z_c costs one scale.
//                  After the last chunk H is the segment's S_ext; the product of
//                  the alphas is a_block.  (state-spaces/mamba #482 names this
//                  decay-weighted sum over earlier chunk states as the step that
//                  must cross devices; Megatron-LM #6808 ships it as the FP32
//                  segment summary.)
//   k_chunk_out    one workgroup per (row, chunk, head): the intra-chunk term
//                  (C B^T masked by exp(cs_i - cs_j) dt_j, j <= i, same sequence)
//                  times X, plus the inter-chunk term exp(cs_i) C_i H_c, into the
//                  zero-initial-state output y_zero.  CB^T is produced tile by
//                  tile in registers and fed straight back as an MFMA operand.
//   k_apply_init   y = y_zero + exp(cs_seg_i) C_i S_in^T + D x_i (the correction
//                  of #6808 once the boundary scan has produced S_in).
#include <type_traits>

#include "ssd_internal.h"
#include "state_walk.h"

namespace ssd {

__device__ __forceinline__ float softplus_f(float z) {
    return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
}

// Operand whose k slots follow the layout of an MFMA output tile reused as the
// B operand: with 16x16 output tiles stacked along k, slot s of lane group g
// stands for k = 16*(s/4) + 4*g + (s%4).  `p` points at k = 4*g of the block.
template <typename T> struct KPerm;
template <> struct KPerm<bf16> {
    __device__ static __forceinline__ bf16x8 load(const bf16* p) {
        const bf16x4 lo = *(const bf16x4*)p;
        const bf16x4 hi = *(const bf16x4*)(p + 16);
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
};
template <> struct KPerm<float> {
    __device__ static __forceinline__ f32x4 load(const float* p) { return *(const f32x4*)p; }
};

// ---------------------------------------------------------------------------
// The cumsum restarts at every packed-sequence start inside the chunk (a
// segmented scan), so a sequence's decays are computed from its own tokens
// only and perturbing one sequence cannot change another's bits.
template <typename T>
__global__ void __launch_bounds__(256) k_dt_prep(Dims d, const T* __restrict__ dt_raw,
                                                const float* __restrict__ dt_bias,
                                                const float* __restrict__ A_log,
                                                const int32_t* __restrict__ seq,
                                                float* __restrict__ dt_ws, float* __restrict__ cs_ws,
                                                float* __restrict__ ctot) {
    __shared__ float raw[256][17];
    __shared__ int sseq[256];
    const int cm = blockIdx.x, h0 = blockIdx.y * 16;
    const int64_t b = blockIdx.z;
    const int Q = d.Q;
    const int64_t tok0 = (int64_t)cm * Q;
    const int nh = min(16, d.H - h0);
    for (int idx = threadIdx.x; idx < Q * 16; idx += blockDim.x) {
        const int j = idx / 16, hh = idx % 16;
        raw[j][hh] = hh < nh ? to_f(dt_raw[(b * d.L + tok0 + j) * d.H + h0 + hh]) : 0.f;
    }
    for (int j = threadIdx.x; j < Q; j += blockDim.x) sseq[j] = seq ? seq[b * d.L + tok0 + j] : 0;
    __syncthreads();
    const int wave = wave_id(), lane = threadIdx.x % 64;
    const int E = Q / 64;  // tokens per lane (1, 2 or 4)
    bool rs[4];            // a sequence starts at or before this token, inside this lane
    bool lflag = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (e < E) {
            const int j = lane * E + e;
            lflag = lflag || (j > 0 && sseq[j] != sseq[j - 1]);
            rs[e] = lflag;
        }
    }
    for (int hh = wave; hh < nh; hh += 4) {
        const int h = h0 + hh;
        const float A = -expf(A_log[h]);
        const float bias = dt_bias[h];
        float dtv[4], csl[4];
        float run = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (e < E) {
                const int j = lane * E + e;
                if (j > 0 && sseq[j] != sseq[j - 1]) run = 0.f;
                const float z = raw[j][hh] + bias;
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
        float* dtp = dt_ws + ((int64_t)b * d.H + h) * d.L + tok0;
        float* csp = cs_ws + ((int64_t)b * d.H + h) * d.L + tok0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (e < E) {
                dtp[lane * E + e] = dtv[e];
                csp[lane * E + e] = rs[e] ? csl[e] : ev + csl[e];
            }
        }
        // the chunk total is the last token's cumulative sum, bit for bit
        if (lane == 63)
            ctot[((int64_t)b * d.H + h) * d.nchunk + cm] =
                rs[E - 1] ? csl[E - 1] : ev + csl[E - 1];
    }
}

// ---------------------------------------------------------------------------
// Waves take 16-column output tiles in the order w, 2NW-1-w, 2NW+w, ... so that
// the causal (triangular) work is balanced across waves.
__device__ __forceinline__ int wave_tile(int wave, int nw, int m) {
    const int pair = m / 2;
    return (m % 2 == 0) ? 2 * nw * pair + wave : 2 * nw * pair + 2 * nw - 1 - wave;
}

template <typename T, int P, int N, int Q, int NW>
__global__ void __launch_bounds__(NW * 64) k_chunk_out(Dims d, SegTab tab, const T* __restrict__ xc,
                                                      const float* __restrict__ dt_ws,
                                                      const float* __restrict__ cs_ws,
                                                      const int32_t* __restrict__ seq,
                                                      const T* __restrict__ hst,
                                                      float* __restrict__ y_zero) {
    typedef Mma<T> M;
    typedef typename M::Frag Frag;
    constexpr int SL = M::SL, KS = M::KS;
    constexpr int VEC = 16 / sizeof(T);
    constexpr int XPITCH = Q + VEC;
    constexpr int BPITCH = N + VEC;
    constexpr int PT = P / 16, QT = Q / 16, NKF = N / KS;
    __shared__ __attribute__((aligned(16))) T Xt[P * XPITCH];
    __shared__ __attribute__((aligned(16))) T Bs[Q * BPITCH];
    __shared__ float scs[Q], sdt[Q];
    __shared__ int ssq[Q];

    const ChunkHead ch = chunk_head_of_block(d);
    const int cm = ch.cm, h = ch.h;
    const int64_t b = ch.b;
    const int wave = wave_id(), lane = threadIdx.x % 64, lr = lane % 16, lg = lane / 16;
    const int g = h / d.hpg;
    const int64_t rb = b * d.L;
    const int64_t t0 = (int64_t)cm * Q;
    const int k = seg_of_chunk(tab, cm, Q);
    const bool first = (t0 == tab.start[k]);
    const int64_t xoff = (int64_t)h * P, boff = (int64_t)d.H * P + (int64_t)g * N;
    const int64_t coff = (int64_t)d.H * P + (int64_t)d.G * N + (int64_t)g * N;

    typedef T vt __attribute__((ext_vector_type(VEC)));
    for (int idx = threadIdx.x; idx < Q * (P / VEC); idx += blockDim.x) {
        const int jj = idx / (P / VEC), pv = idx % (P / VEC);
        const vt v = *(const vt*)(xc + (rb + t0 + jj) * d.C + xoff + pv * VEC);
#pragma unroll
        for (int e = 0; e < VEC; ++e) Xt[(pv * VEC + e) * XPITCH + jj] = v[e];
    }
    for (int idx = threadIdx.x; idx < Q * (N / VEC); idx += blockDim.x) {
        const int jj = idx / (N / VEC), nv = idx % (N / VEC);
        *(vt*)&Bs[jj * BPITCH + nv * VEC] = *(const vt*)(xc + (rb + t0 + jj) * d.C + boff + nv * VEC);
    }
    const float* csp = cs_ws + ((int64_t)b * d.H + h) * d.L + t0;
    const float* dtp = dt_ws + ((int64_t)b * d.H + h) * d.L + t0;
    for (int j = threadIdx.x; j < Q; j += blockDim.x) {
        scs[j] = csp[j];
        sdt[j] = dtp[j];
        ssq[j] = seq ? seq[rb + t0 + j] : 0;
    }
    const int seq_prev = (!first && seq) ? seq[rb + t0 - 1] : 0;
    __syncthreads();

    const T* hp = hst + (((int64_t)b * d.nchunk + cm) * d.H + h) * (P * N);
#pragma unroll 1
    for (int m = 0;; ++m) {
        const int it = wave_tile(wave, NW, m);
        if (it >= QT) break;
        const int i0 = it * 16;
        const int i = i0 + lr;
        const float cs_i = scs[i];
        const int sq_i = ssq[i];

        Frag cf[NKF];
#pragma unroll
        for (int kn = 0; kn < NKF; ++kn)
            cf[kn] = M::load(xc + (rb + t0 + i) * d.C + coff + kn * KS + SL * lg);

        f32x4 acc[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};

        if (!first) {
            // inter-chunk term: exp(cs_i) C_i H_c^T, for tokens still in the
            // sequence that was running when the chunk started.
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                for (int kn = 0; kn < NKF; ++kn)
                    acc[pt] = M::mma(M::load(hp + (pt * 16 + lr) * N + kn * KS + SL * lg), cf[kn],
                                     acc[pt]);
            const float f = (sq_i == seq_prev) ? expf(cs_i) : 0.f;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[pt] *= f;
        }

        // intra-chunk term, j-blocks of KS tokens up to the diagonal
#pragma unroll 1
        for (int j0 = 0; j0 <= i0 + 15; j0 += KS) {
            float tv[SL];
#pragma unroll
            for (int st = 0; st < KS / 16; ++st) {
                const int js = j0 + st * 16;
                f32x4 tacc = f32x4{0.f, 0.f, 0.f, 0.f};
                if (js <= i0 + 15) {
#pragma unroll
                    for (int kn = 0; kn < NKF; ++kn)
                        tacc = M::mma(M::load(&Bs[(js + lr) * BPITCH + kn * KS + SL * lg]), cf[kn],
                                      tacc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = js + 4 * lg + r;
                    float val = 0.f;
                    if (j <= i && ssq[j] == sq_i) val = tacc[r] * expf(cs_i - scs[j]) * sdt[j];
                    tv[st * 4 + r] = val;
                }
            }
            const Frag tb = M::from_f(tv);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
                acc[pt] = M::mma(KPerm<T>::load(&Xt[(pt * 16 + lr) * XPITCH + j0 + 4 * lg]), tb,
                                 acc[pt]);
        }

        float* yo = y_zero + ((rb + t0 + i) * d.H + h) * P;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) *(f32x4*)(yo + pt * 16 + 4 * lg) = acc[pt];
    }
}

// ---------------------------------------------------------------------------
template <typename T, int P, int N>
__global__ void __launch_bounds__(256) k_apply_init(Dims d, SegTab tab, const float* __restrict__ y_zero,
                                                   const T* __restrict__ xc,
                                                   const float* __restrict__ Dp,
                                                   const int32_t* __restrict__ seq,
                                                   const float* __restrict__ S_in,
                                                   const float* __restrict__ cs_ws,
                                                   const float* __restrict__ ctot,
                                                   T* __restrict__ y) {
    typedef Mma<T> M;
    typedef typename M::Frag Frag;
    constexpr int SL = M::SL, KS = M::KS;
    constexpr int PT = P / 16, NKF = N / KS;
    __shared__ float s_pre;

    const ChunkHead ch = chunk_head_of_block(d);
    const int cm = ch.cm, h = ch.h;
    const int64_t b = ch.b;
    const int wave = wave_id(), lane = threadIdx.x % 64, lr = lane % 16, lg = lane / 16;
    const int g = h / d.hpg;
    const int Q = d.Q;
    const int64_t rb = b * d.L;
    const int64_t t0 = (int64_t)cm * Q;
    const int k = seg_of_chunk(tab, cm, Q);
    const int cseg0 = (int)(tab.start[k] / Q);
    const float* ct = ctot + ((int64_t)b * d.H + h) * d.nchunk;
    if (threadIdx.x == 0) {
        float pre = 0.f;  // sum of dt*A over the segment's earlier chunks
        for (int c = cseg0; c < cm; ++c) pre += ct[c];
        s_pre = pre;
    }
    __syncthreads();
    const float pre = s_pre;
    const int64_t pred = seg_pred_token(tab, k);
    const int seq_ref = seq ? seq[rb + (pred >= 0 ? pred : tab.start[k])] : 0;
    const float* sin = S_in + (((int64_t)k * d.batch + b) * d.H + h) * (P * N);
    const int64_t xoff = (int64_t)h * P;
    const int64_t coff = (int64_t)d.H * P + (int64_t)d.G * N + (int64_t)g * N;
    const float Dh = Dp[h];
    const float* csp = cs_ws + ((int64_t)b * d.H + h) * d.L;

    Frag sa[PT][NKF];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int kn = 0; kn < NKF; ++kn) {
            float f[SL];
            const float* src = sin + (pt * 16 + lr) * N + kn * KS + SL * lg;
#pragma unroll
            for (int s = 0; s < SL; ++s) f[s] = src[s];
            sa[pt][kn] = M::from_f(f);
        }

    for (int it = wave; it < Q / 16; it += 4) {
        const int i = it * 16 + lr;
        const int64_t tok = t0 + i;
        f32x4 acc[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kn = 0; kn < NKF; ++kn) {
            const Frag cf = M::load(xc + (rb + tok) * d.C + coff + kn * KS + SL * lg);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[pt] = M::mma(sa[pt][kn], cf, acc[pt]);
        }
        const bool same = !seq || seq[rb + tok] == seq_ref;
        const float f = same ? expf(pre + csp[tok]) : 0.f;
        const float* yz = y_zero + ((rb + tok) * d.H + h) * P;
        T* yo = y + ((rb + tok) * d.H + h) * P;
        const T* xr = xc + (rb + tok) * d.C + xoff;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const int p = pt * 16 + 4 * lg;
            const f32x4 z = *(const f32x4*)(yz + p);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                yo[p + r] = (T)(z[r] + f * acc[pt][r] + Dh * to_f(xr[p + r]));
        }
    }
}

// ---------------------------------------------------------------------------
// Dispatch over the compiled (activation type, P, N, Q) combinations.

template <typename T, int P, int N, int Q>
constexpr size_t chunk_out_lds() {
    return sizeof(T) * ((size_t)P * (Q + 16 / sizeof(T)) + (size_t)Q * (N + 16 / sizeof(T))) +
           (size_t)Q * 12;
}
constexpr size_t LDS_LIMIT = 160 * 1024;

template <typename T, int P, int N>
static bool shape_ok(int Q) {
    if (Q == 64) return chunk_out_lds<T, P, N, 64>() <= LDS_LIMIT;
    if (Q == 128) return chunk_out_lds<T, P, N, 128>() <= LDS_LIMIT;
    if (Q == 256) return chunk_out_lds<T, P, N, 256>() <= LDS_LIMIT;
    return false;
}

template <typename T, int P, int N, int Q>
static void launch_chunk_out(const Dims& d, const SegTab& t, const T* xc, const float* dtw,
                             const float* csw, const int32_t* seq, const T* hst, float* y_zero,
                             hipStream_t s) {
    if constexpr (chunk_out_lds<T, P, N, Q>() <= LDS_LIMIT) {
        constexpr int NW = Q >= 128 ? 8 : 4;
        hipLaunchKernelGGL((k_chunk_out<T, P, N, Q, NW>), chunk_head_grid(d), dim3(NW * 64), 0, s, d, t, xc, dtw,
                           csw, seq, hst, y_zero);
    }
}

template <typename T, int P, int N>
static void segment_states_t(const Dims& d, const SegTab& t, const void* xc_, const void* dt_raw,
                             const float* dt_bias, const float* A_log, const int32_t* seq,
                             float* summary, void* ws, hipStream_t s) {
    const T* xc = (const T*)xc_;
    const FwdWs L = fwd_ws_layout(d, std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32);
    char* w = (char*)ws;
    float* dtw = (float*)(w + L.dt);
    float* csw = (float*)(w + L.cs);
    float* ctot = (float*)(w + L.ctot);
    T* hst = (T*)(w + L.hst);
    launch_dt_prep(d, std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32, dt_raw, dt_bias, A_log,
                   seq, dtw, csw, ctot, s);
    hipLaunchKernelGGL((k_state_walk<T, P, N, WALK_FWD_PN>),
                       dim3((unsigned)d.H, (unsigned)d.nseg, (unsigned)d.batch), dim3(256), 0, s,
                       d, t, xc, (int64_t)d.C, xc, (int64_t)d.H * P, dtw, csw, seq, hst, summary);
}

template <typename T, int P, int N>
static void segment_output_t(const Dims& d, const SegTab& t, const void* xc_, const int32_t* seq,
                             const void* ws, float* y_zero, hipStream_t s) {
    const T* xc = (const T*)xc_;
    const FwdWs L = fwd_ws_layout(d, std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32);
    const char* w = (const char*)ws;
    const float* dtw = (const float*)(w + L.dt);
    const float* csw = (const float*)(w + L.cs);
    const T* hst = (const T*)(w + L.hst);
    switch (d.Q) {
        case 64: launch_chunk_out<T, P, N, 64>(d, t, xc, dtw, csw, seq, hst, y_zero, s); break;
        case 128: launch_chunk_out<T, P, N, 128>(d, t, xc, dtw, csw, seq, hst, y_zero, s); break;
        default: launch_chunk_out<T, P, N, 256>(d, t, xc, dtw, csw, seq, hst, y_zero, s); break;
    }
}

template <typename T, int P, int N>
static void apply_init_t(const Dims& d, const SegTab& t, const float* y_zero, const void* xc,
                         const float* D, const int32_t* seq, const float* S_in, const void* ws,
                         void* y, hipStream_t s) {
    const FwdWs L = fwd_ws_layout(d, std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32);
    const char* w = (const char*)ws;
    hipLaunchKernelGGL((k_apply_init<T, P, N>), chunk_head_grid(d),
                       dim3(256), 0, s, d, t, y_zero, (const T*)xc, D, seq, S_in,
                       (const float*)(w + L.cs), (const float*)(w + L.ctot), (T*)y);
}

hipError_t launch_dt_prep(const Dims& d, int act, const void* dt_raw, const float* dt_bias,
                          const float* A_log, const int32_t* seq, float* dt_ws, float* cs_ws,
                          float* ctot, hipStream_t s) {
    const dim3 grid((unsigned)d.nchunk, (unsigned)((d.H + 15) / 16), (unsigned)d.batch);
    if (act == SSD_BF16)
        hipLaunchKernelGGL(k_dt_prep<bf16>, grid, dim3(256), 0, s, d, (const bf16*)dt_raw, dt_bias,
                           A_log, seq, dt_ws, cs_ws, ctot);
    else
        hipLaunchKernelGGL(k_dt_prep<float>, grid, dim3(256), 0, s, d, (const float*)dt_raw,
                           dt_bias, A_log, seq, dt_ws, cs_ws, ctot);
    return hipGetLastError();
}

// (P, N) pairs with kernels.  bf16 needs N % 32 == 0 (one MFMA consumes 32 of k).
#define SSD_F32_SHAPES(X) X(16, 16) X(32, 32) X(64, 64) X(64, 128)
#define SSD_BF16_SHAPES(X) X(32, 64) X(64, 64) X(64, 128) X(128, 128)

bool kernels_supported(int P, int N, int act) {
#define X(p, n) if (P == p && N == n) return true;
    if (act == SSD_F32) { SSD_F32_SHAPES(X) }
    else { SSD_BF16_SHAPES(X) }
#undef X
    return false;
}

bool chunk_supported(int P, int N, int Q, int act) {
#define X(p, n) if (P == p && N == n) return shape_ok<T, p, n>(Q);
    if (act == SSD_F32) {
        typedef float T;
        SSD_F32_SHAPES(X)
    } else {
        typedef bf16 T;
        SSD_BF16_SHAPES(X)
    }
#undef X
    return false;
}

hipError_t launch_segment_states(const Dims& d, const SegTab& t, int act, const void* xBC_conv,
                                 const void* dt_raw, const float* dt_bias, const float* A_log,
                                 const int32_t* seq, float* summary, void* ws, hipStream_t s) {
#define X(p, n)                                                                               \
    if (d.P == p && d.N == n) {                                                               \
        segment_states_t<T, p, n>(d, t, xBC_conv, dt_raw, dt_bias, A_log, seq, summary, ws, s); \
        return hipGetLastError();                                                             \
    }
    if (act == SSD_F32) {
        typedef float T;
        SSD_F32_SHAPES(X)
    } else {
        typedef bf16 T;
        SSD_BF16_SHAPES(X)
    }
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_segment_output(const Dims& d, const SegTab& t, int act, const void* xBC_conv,
                                 const int32_t* seq, const void* ws, float* y_zero,
                                 hipStream_t s) {
#define X(p, n)                                                            \
    if (d.P == p && d.N == n) {                                            \
        segment_output_t<T, p, n>(d, t, xBC_conv, seq, ws, y_zero, s);     \
        return hipGetLastError();                                          \
    }
    if (act == SSD_F32) {
        typedef float T;
        SSD_F32_SHAPES(X)
    } else {
        typedef bf16 T;
        SSD_BF16_SHAPES(X)
    }
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_apply_init_state(const Dims& d, const SegTab& t, int act, const float* y_zero,
                                   const void* xBC_conv, const float* D, const int32_t* seq,
                                   const float* S_in, const void* ws, void* y, hipStream_t s) {
#define X(p, n)                                                                     \
    if (d.P == p && d.N == n) {                                                     \
        apply_init_t<T, p, n>(d, t, y_zero, xBC_conv, D, seq, S_in, ws, y, s);     \
        return hipGetLastError();                                                   \
    }
    if (act == SSD_F32) {
        typedef float T;
        SSD_F32_SHAPES(X)
    } else {
        typedef bf16 T;
        SSD_BF16_SHAPES(X)
    }
#undef X
    return hipErrorInvalidValue;
}

}  // namespace ssd
