// Backward of the conv1d + SSD state-passing path (gfx950, wave64, MFMA).
//
// Megatron-LM #6808 (first commit): the backward mirrors the forward with a
// reverse boundary scan and recomputes every sequence-length-sized
// intermediate instead of saving it.  Here:
//
//   summary phase (ssd_segment_bwd_summary)
//     conv recompute -> xBC_conv (+ a chunk-transposed copy of the B and C
//     channels, k_bc_transpose), dt/cumsum recompute (k_dt_prep), every
//     chunk's own contribution to the state and to the state gradient, in
//     parallel over chunks (k_bwd_chunk_states), and the reverse passing of
//     those contributions inside each segment (k_state_pass) that leaves, per
//     segment, dL/dS_in of the segment's own outputs and its block decay, in
//     the same packed layout as the forward summary.
//   reverse boundary scan (ssd_boundary_scan, reverse = 1) -> the gradient of
//     every segment's final state.
//   pass phase (ssd_segment_bwd_pass): the true exit gradient and entering
//     state of every chunk (the reverse walk from dS_out and the forward walk
//     from S_in; k_state_pass on the headdim-128 path).
//   chunk phase (ssd_segment_bwd_chunks): k_chunk_bwd per chunk and head: dx,
//     dB, dC and the ddt partial sums, written into the buffers the conv
//     backward consumes.
//   conv phase (ssd_conv1d_bwd): k_bc_blocksum (dB, dC summed over head
//     blocks), k_conv_bwd_ddt (SiLU' and the transposed conv, with a right halo
//     from the causal successor segment, and in the same launch the ddt
//     assembly per token) and k_bwd_reduce (deterministic parameter gradients).
//
// ddt without recomputing y.  dL/d(dt_t A) sums, over every (source j, output
// i) pair with j < t <= i, the derivative of their decay.  Per chunk that is
//   sum_{i >= t} (R_i - K_i)      sources and outputs inside the chunk, with
//                                 R, K the row / column sums of
//                                 F[i][j] = (C_i.B_j)(dy_i.x_j) decay dt_j,
//   + sum_{i >= t} u_i            the entering state seen by outputs i,
//   + sum_{j < t} v_j             sources j feeding the exit state,
//   + <G_exit, decay H_enter>     entering state straight to the exit,
// and exactly 0 at a token that starts a packed sequence.  R and K come from
// the same fp32 F tiles, so their telescoping cancels without bf16 noise.
#include <type_traits>

#include "bwd_util.h"
#include "chunk_bwd.h"
#include "gram.h"
#include "ssd_internal.h"
#include "state_walk.h"
#include "xt.h"

namespace ssd {

__device__ __forceinline__ float softplus_b(float z) {
    return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
}

// Token order inside the transposed [row][token] tiles of the backward.  A bf16
// MFMA takes 32 tokens as its k dimension, 8 per lane group g, and an output
// tile gives lane group g its rows 4g..4g+3.  Each 32-token block is stored as
// tokens 4g..4g+3 and 16+4g..16+4g+3 at positions 8g..8g+7, so that one
// 16-byte load fetches exactly the tokens that two stacked output tiles hold
// in one lane: MFMA results then feed the next MFMA as its k operand.
// float32 MFMAs take 16 tokens, 4 per lane group, in natural order.
template <typename T> struct TokPerm;
template <> struct TokPerm<bf16> {
    static constexpr int BLK = 32;
    __host__ __device__ static constexpr int pos(int i) {
        return ((i & 15) >> 2) * 8 + (i >> 4) * 4 + (i & 3);
    }
};
template <> struct TokPerm<float> {
    static constexpr int BLK = 16;
    __host__ __device__ static constexpr int pos(int i) { return i; }
};
// Position of chunk-local token t in a permuted row.
template <typename T>
__device__ __forceinline__ int tpos(int t) {
    constexpr int B = TokPerm<T>::BLK;
    return (t & ~(B - 1)) + TokPerm<T>::pos(t & (B - 1));
}

// ---------------------------------------------------------------------------
// B and C channels of one chunk, transposed to [part][n][token] (part 0 = B,
// 1 = C) in the permuted token order, so that operands needing the token
// dimension as the MFMA k index read them with 16-byte loads.
template <typename T>
__global__ void __launch_bounds__(256) k_bc_transpose(Dims d, const T* __restrict__ xc,
                                                     T* __restrict__ bct) {
    constexpr int VEC = 16 / sizeof(T);
    constexpr int SLAB = 32;                 // channels per pass
    constexpr int QMAXP = 256 + VEC;
    __shared__ __attribute__((aligned(16))) T tile[SLAB * QMAXP];
    typedef T vt __attribute__((ext_vector_type(VEC)));
    const int cm = blockIdx.x, g = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int Q = d.Q, N = d.N;
    const int QP = Q + VEC;
    const int64_t rb = b * d.L, t0 = (int64_t)cm * Q;
    for (int part = 0; part < 2; ++part) {
        const int64_t chan0 = (int64_t)d.H * d.P + (int64_t)part * d.G * N + (int64_t)g * N;
        T* dst = bct + ((((int64_t)b * d.nchunk + cm) * d.G + g) * 2 + part) * (int64_t)N * Q;
        for (int n0 = 0; n0 < N; n0 += SLAB) {
            const int ns = min(SLAB, N - n0);
            __syncthreads();
            for (int idx = threadIdx.x; idx < Q * (ns / VEC); idx += blockDim.x) {
                const int jj = idx / (ns / VEC), nv = idx % (ns / VEC);
                const vt v = *(const vt*)(xc + (rb + t0 + jj) * d.C + chan0 + n0 + nv * VEC);
#pragma unroll
                for (int e = 0; e < VEC; ++e) tile[(nv * VEC + e) * QP + tpos<T>(jj)] = v[e];
            }
            __syncthreads();
            for (int idx = threadIdx.x; idx < ns * (Q / VEC); idx += blockDim.x) {
                const int n = idx / (Q / VEC), qv = idx % (Q / VEC);
                *(vt*)(dst + (int64_t)(n0 + n) * Q + qv * VEC) = *(const vt*)(tile + n * QP + qv * VEC);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Chunk states of the backward, every chunk in parallel (one workgroup per
// chunk and head):
//   Zh_c = sum_j exp(cs_e - cs_j) dt_j [seq_j = seq_e] x_j B_j^T   (what the
//          chunk adds to the state leaving it),
//   Zg_c = sum_i exp(cs_i) [seq_i = seq of the entering state] dy_i C_i^T
//          (the gradient its outputs send to the state entering it),
// both P x N in FP32, and (for the per-head chunk kernel only) the chunk's dy
// transposed to [p][token] in the permuted token order.
template <typename T, int P, int N>
__global__ void __launch_bounds__(256) k_bwd_chunk_states(
    Dims d, SegTab tab, const T* __restrict__ xc, const T* __restrict__ bct,
    const T* __restrict__ dy, const float* __restrict__ dt_ws, const float* __restrict__ cs_ws,
    const int32_t* __restrict__ seq, float* __restrict__ zh, float* __restrict__ zg,
    T* __restrict__ dyT) {
    typedef Mma<T> M;
    typedef typename M::Frag Frag;
    constexpr int SL = M::SL, KS = M::KS, TPK = KS / 16;
    constexpr int KT = 64;               // tokens per LDS slice
    constexpr int VEC = 16 / sizeof(T);
    constexpr int XR = P + VEC;          // [token][p] row pitch
    constexpr int PT = P / 16, NT = N / 16, NTW = (NT + 3) / 4;
    // x rows scaled by their state weight, and dy rows, natural layout; the MFMA
    // A operands (k = token) come from transposed reads (XT)
    __shared__ __attribute__((aligned(16))) T sX[KT * XR];
    __shared__ __attribute__((aligned(16))) T sY[KT * XR];
    __shared__ __attribute__((aligned(16))) float wz[KT];
    typedef T vt __attribute__((ext_vector_type(VEC)));

    const ChunkHead ch = chunk_head_of_block(d);
    const int cm = ch.cm, h = ch.h;
    const int64_t b = ch.b;
    const int wave = wave_id(), lane = threadIdx.x % 64, lr = lane % 16, lg = lane / 16;
    const int g = h / d.hpg;
    const int Q = d.Q;
    const int64_t rb = b * d.L, t0 = (int64_t)cm * Q, HPd = (int64_t)d.H * P;
    const int k = seg_of_chunk(tab, cm, Q);
    const int64_t s0 = tab.start[k];
    const int64_t pred = seg_pred_token(tab, k);
    const int64_t ptok = t0 > s0 ? t0 - 1 : (pred >= 0 ? pred : s0);
    const int seq_ref = seq ? seq[rb + ptok] : 0;
    const int seq_e = seq ? seq[rb + t0 + Q - 1] : 0;
    const int64_t hl = ((int64_t)b * d.H + h) * d.L + t0;
    const float cs_e = cs_ws[hl + Q - 1];
    const T* bctB = bct + ((((int64_t)b * d.nchunk + cm) * d.G + g) * 2) * (int64_t)N * Q;
    const T* bctC = bctB + (int64_t)N * Q;

    f32x4 ah[PT][NTW], ag[PT][NTW];
#pragma unroll
    for (int i = 0; i < PT; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) ah[i][j] = ag[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int sl = 0; sl < Q / KT; ++sl) {
        const int tb = sl * KT;
        __syncthreads();
        for (int idx = threadIdx.x; idx < KT * (P / VEC); idx += blockDim.x) {
            const int jj = idx / (P / VEC), pv = idx % (P / VEC);
            const int64_t tok = rb + t0 + tb + jj;
            const bool same = !seq || seq[tok] == seq_e;
            const float w = same ? __expf(cs_e - cs_ws[hl + tb + jj]) * dt_ws[hl + tb + jj] : 0.f;
            const vt xv = *(const vt*)(xc + tok * d.C + (int64_t)h * P + pv * VEC);
            vt xs;
#pragma unroll
            for (int e = 0; e < VEC; ++e) xs[e] = (T)((float)xv[e] * w);
            *(vt*)&sX[jj * XR + pv * VEC] = xs;
            *(vt*)&sY[jj * XR + pv * VEC] = *(const vt*)(dy + tok * HPd + (int64_t)h * P + pv * VEC);
        }
        if (threadIdx.x < KT) {
            const int jj = threadIdx.x;
            const bool same = !seq || seq[rb + t0 + tb + jj] == seq_ref;
            wz[jj] = same ? __expf(cs_ws[hl + tb + jj]) : 0.f;
        }
        __syncthreads();
        if (dyT) {  // dy as [p][token] in the permuted token order (per-head chunk kernel)
            T* yT = dyT + (((int64_t)b * d.nchunk + cm) * d.H + h) * (int64_t)P * Q;
            for (int idx = threadIdx.x; idx < P * KT; idx += blockDim.x) {
                const int p = idx / KT, jj = idx % KT;
                yT[(int64_t)p * Q + tb + tpos<T>(jj)] = sY[jj * XR + p];
            }
        }
#pragma unroll
        for (int kk = 0; kk < KT / KS; ++kk) {
            const int jb = kk * KS;
            Frag ax[PT], ay[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                ax[pt] = XT<T>::load(sX, XR, jb, pt * 16, lane);
                ay[pt] = XT<T>::load(sY, XR, jb, pt * 16, lane);
            }
            // weight of k slot s: the token XT puts there
            float wl[SL];
#pragma unroll
            for (int s2 = 0; s2 < SL; ++s2)
                wl[s2] = wz[jb + (TPK == 2 ? 16 * (s2 / 4) + 4 * lg + s2 % 4 : 4 * lg + s2)];
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int nt = wave + 4 * j;
                if (nt < NT) {
                    const int64_t o = (int64_t)(nt * 16 + lr) * Q + tb + jb + SL * lg;
                    const Frag bB = M::load(bctB + o);
                    const Frag bC = M::load_scaled(bctC + o, wl);
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        ah[pt][j] = M::mma(ax[pt], bB, ah[pt][j]);
                        ag[pt][j] = M::mma(ay[pt], bC, ag[pt][j]);
                    }
                }
            }
        }
    }
    const int64_t so = (((int64_t)b * d.nchunk + cm) * d.H + h) * (P * N);
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int nt = wave + 4 * j;
            if (nt < NT) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t o = so + (int64_t)(pt * 16 + 4 * lg + r) * N + nt * 16 + lr;
                    zh[o] = ah[pt][j][r];
                    zg[o] = ag[pt][j][r];
                }
            }
        }
}

// ---------------------------------------------------------------------------
// Chunk-to-chunk passing inside a segment, elementwise over P x N in FP32
// (one workgroup per head, segment and row).  alpha_c = exp(cs at the chunk's
// last token) when the state entering chunk c and that token belong to one
// sequence, else exactly 0.  With G_c the gradient of the state leaving chunk
// c and H_c the state entering it:
//   PASS_SUMMARY: G <- alpha_c G + Zg_c from the last chunk with zero final
//                 gradient; leaves L_k (dL/dS_in of the segment's own outputs)
//                 and a_k = prod alpha_c in the summary layout.
//   PASS_TRUE:    G from dS_out backwards, storing every G_c as [p][n] (and
//                 [n][p] if gnp is given); then H from S_in forwards, storing
//                 every H_c as [p][n] and / or [n][p] (whichever of hpn, hnp
//                 is given) and <G_c, H_c> per chunk.
enum PassMode { PASS_SUMMARY = 0, PASS_TRUE = 1 };

template <typename T, int P, int N, int MODE>
__global__ void __launch_bounds__(256) k_state_pass(
    Dims d, SegTab tab, const float* __restrict__ ctot, const int32_t* __restrict__ seq,
    const float* __restrict__ zg, const float* __restrict__ zh, const float* __restrict__ S_in,
    const float* __restrict__ dS_out, float* __restrict__ summary, T* __restrict__ gpn,
    T* __restrict__ gnp, T* __restrict__ hnp, T* __restrict__ hpn, float* __restrict__ dotgh) {
    constexpr int PN4 = P * N / 4;
    constexpr int E4 = (PN4 + 255) / 256;  // float4 groups per thread
    constexpr int TP = N + 1;              // fp32 transpose tile pitch
    constexpr int VEC = 16 / sizeof(T);
    typedef T vt __attribute__((ext_vector_type(VEC)));
    typedef T vt4 __attribute__((ext_vector_type(4)));
    __shared__ float tile[MODE == PASS_TRUE ? P * TP : 1];
    __shared__ float sred[4];
    const int h = blockIdx.x, k = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int Q = d.Q;
    const int64_t rb = b * d.L;
    const int64_t s0 = tab.start[k];
    const int nc = (int)(tab.len[k] / Q);
    const int cm0 = (int)(s0 / Q);
    const int64_t pred = seg_pred_token(tab, k);
    const float* ct = ctot + ((int64_t)b * d.H + h) * d.nchunk;
    const int64_t per = (int64_t)d.batch * d.H * P * N;
    const int64_t sg = ((int64_t)k * d.batch + b) * d.H + h;
    auto alpha_of = [&](int c) {
        const int64_t t0 = (int64_t)(cm0 + c) * Q;
        const int64_t ptok = c > 0 ? t0 - 1 : (pred >= 0 ? pred : s0);
        const bool same = !seq || seq[rb + ptok] == seq[rb + t0 + Q - 1];
        return same ? expf(ct[cm0 + c]) : 0.f;
    };
    auto st_off = [&](int c) { return (((int64_t)b * d.nchunk + cm0 + c) * d.H + h) * (P * N); };

    f32x4 acc[E4];
    // reverse pass over the gradient
#pragma unroll
    for (int q = 0; q < E4; ++q) {
        const int i4 = threadIdx.x + q * 256;
        acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (MODE == PASS_TRUE && i4 < PN4) acc[q] = *(const f32x4*)(dS_out + sg * P * N + 4 * i4);
    }
    float ablk = 1.f;
    for (int c = nc - 1; c >= 0; --c) {
        const int64_t so = st_off(c);
        if (MODE == PASS_TRUE) {
#pragma unroll
            for (int q = 0; q < E4; ++q) {
                const int i4 = threadIdx.x + q * 256;
                if (i4 < PN4) {
                    vt4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = (T)acc[q][e];
                    *(vt4*)(gpn + so + 4 * i4) = v;
                    if (gnp) {
                        const int p = (4 * i4) / N, n = (4 * i4) % N;
#pragma unroll
                        for (int e = 0; e < 4; ++e) tile[p * TP + n + e] = acc[q][e];
                    }
                }
            }
            if (gnp) {
                __syncthreads();
                for (int idx = threadIdx.x; idx < N * (P / VEC); idx += 256) {
                    const int n = idx / (P / VEC), p0 = (idx % (P / VEC)) * VEC;
                    vt v;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) v[e] = (T)tile[(p0 + e) * TP + n];
                    *(vt*)(gnp + so + (int64_t)n * P + p0) = v;
                }
                __syncthreads();
            }
        }
        const float a = alpha_of(c);
        ablk *= a;
#pragma unroll
        for (int q = 0; q < E4; ++q) {
            const int i4 = threadIdx.x + q * 256;
            if (i4 < PN4) {
                const f32x4 z = *(const f32x4*)(zg + so + 4 * i4);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[q][e] = a * acc[q][e] + z[e];
            }
        }
    }
    if (MODE == PASS_SUMMARY) {
#pragma unroll
        for (int q = 0; q < E4; ++q) {
            const int i4 = threadIdx.x + q * 256;
            if (i4 < PN4) *(f32x4*)(summary + (int64_t)k * per + sg % (d.batch * d.H) * (P * N) +
                                    4 * i4) = acc[q];
        }
        if (threadIdx.x == 0) summary[(int64_t)d.nseg * per + sg] = ablk;
        return;
    }
    // forward pass over the state
#pragma unroll
    for (int q = 0; q < E4; ++q) {
        const int i4 = threadIdx.x + q * 256;
        acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (i4 < PN4) acc[q] = *(const f32x4*)(S_in + sg * P * N + 4 * i4);
    }
    const int wave = wave_id(), lane = threadIdx.x % 64;
    for (int c = 0; c < nc; ++c) {
        const int64_t so = st_off(c);
        float dot = 0.f;
#pragma unroll
        for (int q = 0; q < E4; ++q) {
            const int i4 = threadIdx.x + q * 256;
            if (i4 < PN4) {
                const vt4 gv = *(const vt4*)(gpn + so + 4 * i4);  // written by this thread
                const int p = (4 * i4) / N, n = (4 * i4) % N;
                vt4 hv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dot += (float)gv[e] * acc[q][e];
                    if (hnp) tile[p * TP + n + e] = acc[q][e];
                    hv[e] = (T)acc[q][e];
                }
                if (hpn) *(vt4*)(hpn + so + 4 * i4) = hv;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
        if (lane == 0) sred[wave] = dot;
        __syncthreads();
        if (hnp) {
            for (int idx = threadIdx.x; idx < N * (P / VEC); idx += 256) {
                const int n = idx / (P / VEC), p0 = (idx % (P / VEC)) * VEC;
                vt v;
#pragma unroll
                for (int e = 0; e < VEC; ++e) v[e] = (T)tile[(p0 + e) * TP + n];
                *(vt*)(hnp + so + (int64_t)n * P + p0) = v;
            }
        }
        if (threadIdx.x == 0)
            dotgh[((int64_t)b * d.nchunk + cm0 + c) * d.H + h] = sred[0] + sred[1] + sred[2] + sred[3];
        const float a = alpha_of(c);
#pragma unroll
        for (int q = 0; q < E4; ++q) {
            const int i4 = threadIdx.x + q * 256;
            if (i4 < PN4) {
                const f32x4 z = *(const f32x4*)(zh + so + 4 * i4);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[q][e] = a * acc[q][e] + z[e];
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// The chunk backward, one workgroup per (chunk, head) with NW = Q/(16 TPW)
// waves of TPW 16-token tiles each.  Tiles come in pairs (t, Q/16-1-t), one
// from each end of the chunk, so that every wave meets the same number of
// causal (i >= j) tile pairs; every operand fragment read from LDS feeds the
// MFMAs of all TPW tiles of the wave.
//
//   phase A (its tiles as outputs i):  dC_i = f_i H^T dy_i
//                                        + sum_{j<=i} M_ij dt_j (dy_i.x_j) B_j
//   phase B1 (its tiles as sources j): dx_j = dt_j (g_j G B_j + sum_{i>=j} M_ij (C_i.B_j) dy_i)
//                                      and the per-token ddt terms
//   phase B2 (its tiles as sources j): dB_j = dt_j (g_j G^T x_j + sum_{i>=j} M_ij (dy_i.x_j) C_i)
// with M_ij = exp(cs_i - cs_j) [same sequence], f_i = exp(cs_i) [i in the
// entering state's sequence], g_j = exp(cs_e - cs_j) [j in the last token's
// sequence], H the state entering the chunk and G the gradient of the state
// leaving it.  B1 and B2 are separate passes (B2 recomputes dy_i.x_j) so that
// the dx and dB accumulators are never live together.  The i-blocks (phase B)
// and j-blocks (phase A) of KS tokens are
// staged once per workgroup in LDS, double buffered; transposed operands come
// pre-transposed in the permuted token order.  Per-token partial sums for ddt
// go to the workspace; the ddt assembly (ddt_wave) combines them per chunk.
template <typename T, int P, int N, int Q, int TPW>
struct ChunkBwd {
    typedef Mma<T> M;
    static constexpr int SL = M::SL, KS = M::KS;
    static constexpr int VEC = 16 / sizeof(T);
    static constexpr int QT = Q / 16, NW = QT / TPW, NTH = NW * 64;
    static constexpr int PT = P / 16, NT = N / 16, KP = P / KS, KN = N / KS;
    static constexpr int RPN = N + VEC, RPP = P + VEC, TPK = KS + VEC;
    // staging buffers, elements per buffer
    static constexpr int S_CROW = KS * RPN, S_DROW = KS * RPP, S_CT = N * TPK, S_DT = P * TPK;
    static constexpr int STAGE_A = S_DROW + S_CT;            // phase A: x rows, B^T
    static constexpr int STAGE_B1 = S_CROW + S_DROW + S_DT;  // phase B1: C rows, dy rows, dy^T
    static constexpr int STAGE_B2 = S_DROW + S_CT;           // phase B2: dy rows, C^T
    static constexpr int ST_G = P * RPN;                     // G [p][n]
    static constexpr int ST_GT = N * RPP;                    // G^T or H^T [n][p]
    static constexpr int cmax(int a, int b) { return a > b ? a : b; }
    static constexpr int U_ELEMS =
        cmax(cmax(2 * STAGE_A, 2 * STAGE_B1), cmax(2 * STAGE_B2, cmax(ST_G, ST_GT)));
    static constexpr size_t U_BYTES = (size_t)U_ELEMS * sizeof(T);
    static constexpr size_t TOK_BYTES = (size_t)Q * 20 + (size_t)NW * Q * 4 + QT * QT * 4;
    static constexpr size_t LDS = U_BYTES + TOK_BYTES + 64;
    static_assert(NW * TPW == QT && TPW % 2 == 0, "tiles in pairs");
    // tile index of slot s of wave w: pairs (t, QT-1-t)
    __device__ static __forceinline__ int tile(int w, int s) {
        const int t = (s / 2) * (QT / 2) + ((s / 2) % 2 ? NW - 1 - w : w);
        return s % 2 ? QT - 1 - t : t;
    }
};

template <typename T, int P, int N, int Q, int TPW>
__global__ void __launch_bounds__(Q / (16 * TPW) * 64) k_chunk_bwd(
    Dims d, SegTab tab, const T* __restrict__ xc, const T* __restrict__ bct,
    const T* __restrict__ dy, const T* __restrict__ dyT, const float* __restrict__ Dp,
    const float* __restrict__ dt_ws, const float* __restrict__ cs_ws,
    const int32_t* __restrict__ seq, const T* __restrict__ gpn, const T* __restrict__ gnp,
    const T* __restrict__ hnp, T* __restrict__ dv, T* __restrict__ dbc,
    float* __restrict__ rpart, float* __restrict__ tokp, float* __restrict__ red4) {
    typedef ChunkBwd<T, P, N, Q, TPW> K;
    typedef Mma<T> M;
    typedef typename M::Frag Frag;
    typedef typename M::Elem E;
    constexpr int SL = K::SL, KS = K::KS, VEC = K::VEC, NW = K::NW, NTH = K::NTH;
    constexpr int PT = K::PT, NT = K::NT, KP = K::KP, KN = K::KN;
    constexpr int RPN = K::RPN, RPP = K::RPP, TPK = K::TPK;
    typedef T vt __attribute__((ext_vector_type(VEC)));
    __shared__ __attribute__((aligned(16))) T U[K::U_ELEMS];
    __shared__ __attribute__((aligned(16))) float scs[Q];
    __shared__ __attribute__((aligned(16))) float sdt[Q];
    __shared__ __attribute__((aligned(16))) int ssq[Q];
    __shared__ float s_rw[NW][Q];  // per-wave row sums of F
    __shared__ float s_red[NW];
    // Decay factors for chunks without a sequence start inside (one continuous
    // cumulative sum): with F_a, L_a the cumulative sums at the first and last
    // token of 16-token tile a,
    //   exp(cs_i - cs_j) = exp(cs_i - F_a(i)) exp(F_a(i) - L_b(j)) exp(L_b(j) - cs_j),
    // every factor bounded by exp(24) (a tile spans 16 tokens, |dt A| <= 1.6), so
    // the intra-chunk decays need no transcendental in the inner loops.
    __shared__ __attribute__((aligned(16))) float sea[Q];  // exp(cs_t - F(t))
    __shared__ __attribute__((aligned(16))) float seb[Q];  // exp(L(t) - cs_t) dt_t
    __shared__ float stab[K::QT * K::QT];                   // exp(F_a - L_b), a >= b; else 0

    const ChunkHead ch = chunk_head_of_block(d);
    const int cm = ch.cm, h = ch.h;
    const int64_t b = ch.b;
    const int wave = wave_id(), lane = threadIdx.x % 64, lr = lane % 16, lg = lane / 16;
    const int g = h / d.hpg;
    const int64_t rb = b * d.L, t0 = (int64_t)cm * Q;
    const int64_t HPd = (int64_t)d.H * P;
    const int k = seg_of_chunk(tab, cm, Q);
    const int64_t s0 = tab.start[k];
    const int64_t pred = seg_pred_token(tab, k);
    const int64_t refc = t0 > s0 ? t0 - 1 : (pred >= 0 ? pred : s0);
    const int seq_refc = seq ? seq[rb + refc] : 0;
    const int seq_e = seq ? seq[rb + t0 + Q - 1] : 0;
    // a packed sequence starts inside the chunk: pairs need the sequence mask
    const bool split = seq && seq[rb + t0] != seq_e;
    const int64_t xoff = (int64_t)h * P, boff = HPd + (int64_t)g * N;
    const int64_t coff = HPd + (int64_t)d.G * N + (int64_t)g * N;
    const T* bctB = bct + ((((int64_t)b * d.nchunk + cm) * d.G + g) * 2 + 0) * (int64_t)N * Q;
    const T* bctC = bctB + (int64_t)N * Q;
    const T* yT = dyT + (((int64_t)b * d.nchunk + cm) * d.H + h) * (int64_t)P * Q;
    const int64_t st_off = (((int64_t)b * d.nchunk + cm) * d.H + h) * (P * N);
    const int64_t hl = ((int64_t)b * d.H + h) * d.L + t0;  // (row, head) token base

    int tt[TPW];  // first token of each of this wave's tiles
#pragma unroll
    for (int s = 0; s < TPW; ++s) tt[s] = K::tile(wave, s) * 16;

    for (int j = threadIdx.x; j < Q; j += NTH) {
        scs[j] = cs_ws[hl + j];
        sdt[j] = dt_ws[hl + j];
        ssq[j] = seq ? seq[rb + t0 + j] : 0;
    }
    for (int j = threadIdx.x; j < NW * Q; j += NTH) (&s_rw[0][0])[j] = 0.f;
    // H^T [n][p]
    for (int idx = threadIdx.x; idx < N * (P / VEC); idx += NTH) {
        const int n = idx / (P / VEC), pv = idx % (P / VEC);
        *(vt*)&U[n * RPP + pv * VEC] = *(const vt*)(hnp + st_off + (int64_t)n * P + pv * VEC);
    }
    __syncthreads();
    constexpr int QT = K::QT;
    if (!split) {
        for (int t = threadIdx.x; t < Q; t += NTH) {
            const int t16 = t & ~15;
            sea[t] = __expf(scs[t] - scs[t16]);
            seb[t] = __expf(scs[t16 + 15] - scs[t]) * sdt[t];
        }
        for (int q = threadIdx.x; q < QT * QT; q += NTH) {
            const int a = q / QT, c = q % QT;
            stab[q] = a >= c ? __expf(scs[16 * a] - scs[16 * c + 15]) : 0.f;
        }
        __syncthreads();
    }

    const float cs_e = scs[Q - 1];
    const float Dh = Dp[h];

    // =================== phase A: dC of the wave's tiles (outputs i) ===================
    float u_t[TPW];
    {
        f32x4 adc[TPW][NT];
        Frag Dn[TPW][KP];
        float cs_i[TPW], e3[TPW];
        int sq_i[TPW];
#pragma unroll
        for (int it = 0; it < TPW; ++it) {
            const int ti = tt[it] + lr;
            const int64_t trow = rb + t0 + ti;
            cs_i[it] = scs[ti];
            sq_i[it] = ssq[ti];
            e3[it] = split ? 0.f : sea[ti];
            const float f_i = (sq_i[it] == seq_refc) ? __expf(cs_i[it]) : 0.f;
#pragma unroll
            for (int kp = 0; kp < KP; ++kp)
                Dn[it][kp] = M::load(dy + trow * HPd + xoff + kp * KS + SL * lg);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kp = 0; kp < KP; ++kp)
                    a = M::mma(M::load(&U[(nt * 16 + lr) * RPP + kp * KS + SL * lg]), Dn[it][kp], a);
                adc[it][nt] = a * f_i;
            }
            // u_i = C_i . (entering-state part of dC_i)
            float up = 0.f;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                float cv[4];
                load4(xc + trow * d.C + coff + nt * 16 + 4 * lg, cv);
#pragma unroll
                for (int r = 0; r < 4; ++r) up += cv[r] * adc[it][nt][r];
            }
            u_t[it] = sum_groups(up);
        }
        __syncthreads();  // H^T consumed; the union now holds staging

        constexpr int V_X = (KS * (P / VEC) + NTH - 1) / NTH;
        constexpr int V_B = (N * (KS / VEC) + NTH - 1) / NTH;
        auto fetchA = [&](int j0, vt (&rx)[V_X], vt (&rbt)[V_B]) {
#pragma unroll
            for (int q = 0; q < V_X; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < KS * (P / VEC)) {
                    const int jj = idx / (P / VEC), pv = idx % (P / VEC);
                    rx[q] = *(const vt*)(xc + (rb + t0 + j0 + jj) * d.C + xoff + pv * VEC);
                }
            }
#pragma unroll
            for (int q = 0; q < V_B; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < N * (KS / VEC)) {
                    const int n = idx / (KS / VEC), kv = idx % (KS / VEC);
                    rbt[q] = *(const vt*)(bctB + (int64_t)n * Q + j0 + kv * VEC);
                }
            }
        };
        auto storeA = [&](T* s, const vt (&rx)[V_X], const vt (&rbt)[V_B]) {
#pragma unroll
            for (int q = 0; q < V_X; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < KS * (P / VEC))
                    *(vt*)&s[(idx / (P / VEC)) * RPP + (idx % (P / VEC)) * VEC] = rx[q];
            }
#pragma unroll
            for (int q = 0; q < V_B; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < N * (KS / VEC))
                    *(vt*)&s[K::S_DROW + (idx / (KS / VEC)) * TPK + (idx % (KS / VEC)) * VEC] = rbt[q];
            }
        };
        {
            vt rx[V_X], rbt[V_B];
            fetchA(0, rx, rbt);
            storeA(U, rx, rbt);
        }
        __syncthreads();
        int buf = 0;
#pragma unroll 1
        for (int j0 = 0; j0 < Q; j0 += KS, buf ^= 1) {
            const bool more = j0 + KS < Q;
            vt rx[V_X], rbt[V_B];
            if (more) fetchA(j0 + KS, rx, rbt);
            const T* sX = U + buf * K::STAGE_A;
            const T* sBT = sX + K::S_DROW;
            // a tile is active for the block when some j of the block is <= some i of the tile
            bool act[TPW], any_act = false;
#pragma unroll
            for (int it = 0; it < TPW; ++it) {
                act[it] = j0 <= tt[it] + 15;
                any_act = any_act || act[it];
            }
            if (any_act) {
                Frag vf[TPW];
#pragma unroll
                for (int st = 0; st < KS / 16; ++st) {
                    const int js = j0 + st * 16;
                    Frag xf[KP];
#pragma unroll
                    for (int kp = 0; kp < KP; ++kp)
                        xf[kp] = M::load(&sX[(st * 16 + lr) * RPP + kp * KS + SL * lg]);
                    const f32x4 ej = *(const f32x4*)&seb[js + 4 * lg];
#pragma unroll
                    for (int it = 0; it < TPW; ++it) {
                        const int i0 = tt[it];
                        float vv[4] = {0.f, 0.f, 0.f, 0.f};
                        if (js <= i0 + 15) {
                            f32x4 w = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int kp = 0; kp < KP; ++kp) w = M::mma(xf[kp], Dn[it][kp], w);
                            const int ti = i0 + lr;
                            if (!split) {
                                const float bi = e3[it] * stab[(i0 / 16) * QT + js / 16];
#pragma unroll
                                for (int r = 0; r < 4; ++r) vv[r] = w[r] * (ej[r] * bi);
                                if (js == i0) {
#pragma unroll
                                    for (int r = 0; r < 4; ++r)
                                        if (js + 4 * lg + r > ti) vv[r] = 0.f;
                                }
                            } else {
                                const f32x4 cj = *(const f32x4*)&scs[js + 4 * lg];
                                const f32x4 dj = *(const f32x4*)&sdt[js + 4 * lg];
                                const int4 sj = *(const int4*)&ssq[js + 4 * lg];
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    const int j = js + 4 * lg + r;
                                    const bool ok = j <= ti && sj[r] == sq_i[it];
                                    vv[r] = ok ? w[r] * (__expf(cs_i[it] - cj[r]) * dj[r]) : 0.f;
                                }
                            }
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) vf[it][st * 4 + r] = (E)vv[r];
                    }
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const Frag bt = M::load(&sBT[(nt * 16 + lr) * TPK + SL * lg]);
#pragma unroll
                    for (int it = 0; it < TPW; ++it) adc[it][nt] = M::mma(bt, vf[it], adc[it][nt]);
                }
            }
            if (more) storeA(U + (buf ^ 1) * K::STAGE_A, rx, rbt);
            __syncthreads();
        }
#pragma unroll
        for (int it = 0; it < TPW; ++it) {
            const int64_t trow = rb + t0 + tt[it] + lr;
            T* dcrow = dbc + (trow * d.H + h) * (2 * N) + N;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) dcrow[nt * 16 + 4 * lg + r] = (T)adc[it][nt][r];
        }
    }

    // ============ phase B1: dx and the ddt terms of the wave's tiles (sources j) ============
    // G [p][n] into the union (every wave is past its last staging read)
    for (int idx = threadIdx.x; idx < P * (N / VEC); idx += NTH) {
        const int p = idx / (N / VEC), nv = idx % (N / VEC);
        *(vt*)&U[p * RPN + nv * VEC] = *(const vt*)(gpn + st_off + (int64_t)p * N + nv * VEC);
    }
    __syncthreads();

    float cs_j[TPW], dt_j[TPW], e2[TPW], gj[TPW];
    int sq_j[TPW];
#pragma unroll
    for (int jt = 0; jt < TPW; ++jt) {
        const int tj = tt[jt] + lr;
        cs_j[jt] = scs[tj];
        dt_j[jt] = sdt[tj];
        sq_j[jt] = ssq[tj];
        e2[jt] = split ? 0.f : __expf(scs[tt[jt] + 15] - cs_j[jt]);
        gj[jt] = (sq_j[jt] == seq_e) ? __expf(cs_e - cs_j[jt]) : 0.f;
    }
    // decay of pair (i, j) for the i-sub-tile starting at `is`, rows 4 lg + r
    auto pair_decay = [&](int is, int jt, const f32x4& ea, float (&m)[4]) {
        const int j0 = tt[jt], tj = j0 + lr;
        if (!split) {
            const float bj = stab[(is / 16) * QT + j0 / 16] * e2[jt];
#pragma unroll
            for (int r = 0; r < 4; ++r) m[r] = ea[r] * bj;
            if (is == j0) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (is + 4 * lg + r < tj) m[r] = 0.f;
            }
        } else {
            const f32x4 ci = *(const f32x4*)&scs[is + 4 * lg];
            const int4 si = *(const int4*)&ssq[is + 4 * lg];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool ok = is + 4 * lg + r >= tj && si[r] == sq_j[jt];
                m[r] = ok ? __expf(ci[r] - cs_j[jt]) : 0.f;
            }
        }
    };

    float v_t[TPW], kq[TPW], q_t[TPW];
    float dD_part = 0.f;
    {
        Frag Bn[TPW][KN], Xn[TPW][KP];
        f32x4 adx[TPW][PT];
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
            const int64_t trow = rb + t0 + tt[jt] + lr;
            kq[jt] = 0.f;
#pragma unroll
            for (int kn = 0; kn < KN; ++kn)
                Bn[jt][kn] = M::load(xc + trow * d.C + boff + kn * KS + SL * lg);
#pragma unroll
            for (int kp = 0; kp < KP; ++kp)
                Xn[jt][kp] = M::load(xc + trow * d.C + xoff + kp * KS + SL * lg);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kn = 0; kn < KN; ++kn)
                    a = M::mma(M::load(&U[(pt * 16 + lr) * RPN + kn * KS + SL * lg]), Bn[jt][kn], a);
                adx[jt][pt] = a * gj[jt];
            }
            // v_j: what source j adds, through the exit state, to every decay inside the chunk
            float vp = 0.f;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                float xv[4];
                load4(xc + trow * d.C + xoff + pt * 16 + 4 * lg, xv);
#pragma unroll
                for (int r = 0; r < 4; ++r) vp += xv[r] * adx[jt][pt][r];
            }
            v_t[jt] = dt_j[jt] * sum_groups(vp);
        }
        __syncthreads();  // G consumed

        constexpr int V_RN = (KS * (N / VEC) + NTH - 1) / NTH;
        constexpr int V_RP = (KS * (P / VEC) + NTH - 1) / NTH;
        constexpr int V_DT = (P * (KS / VEC) + NTH - 1) / NTH;
        constexpr int SB1 = K::S_CROW + K::S_DROW + K::S_DT;  // C rows, dy rows, dy^T
        auto fetch = [&](int i0, vt (&rn)[V_RN], vt (&rp)[V_RP], vt (&rd)[V_DT]) {
#pragma unroll
            for (int q = 0; q < V_RN; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < KS * (N / VEC)) {
                    const int ii = idx / (N / VEC), nv = idx % (N / VEC);
                    rn[q] = *(const vt*)(xc + (rb + t0 + i0 + ii) * d.C + coff + nv * VEC);
                }
            }
#pragma unroll
            for (int q = 0; q < V_RP; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < KS * (P / VEC)) {
                    const int ii = idx / (P / VEC), pv = idx % (P / VEC);
                    rp[q] = *(const vt*)(dy + (rb + t0 + i0 + ii) * HPd + xoff + pv * VEC);
                }
            }
#pragma unroll
            for (int q = 0; q < V_DT; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < P * (KS / VEC)) {
                    const int p = idx / (KS / VEC), kv = idx % (KS / VEC);
                    rd[q] = *(const vt*)(yT + (int64_t)p * Q + i0 + kv * VEC);
                }
            }
        };
        auto store = [&](T* s, const vt (&rn)[V_RN], const vt (&rp)[V_RP], const vt (&rd)[V_DT]) {
#pragma unroll
            for (int q = 0; q < V_RN; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < KS * (N / VEC))
                    *(vt*)&s[(idx / (N / VEC)) * RPN + (idx % (N / VEC)) * VEC] = rn[q];
            }
#pragma unroll
            for (int q = 0; q < V_RP; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < KS * (P / VEC))
                    *(vt*)&s[K::S_CROW + (idx / (P / VEC)) * RPP + (idx % (P / VEC)) * VEC] = rp[q];
            }
#pragma unroll
            for (int q = 0; q < V_DT; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < P * (KS / VEC))
                    *(vt*)&s[K::S_CROW + K::S_DROW + (idx / (KS / VEC)) * TPK +
                             (idx % (KS / VEC)) * VEC] = rd[q];
            }
        };
        {
            vt rn[V_RN], rp[V_RP], rd[V_DT];
            fetch(0, rn, rp, rd);
            store(U, rn, rp, rd);
        }
        __syncthreads();
        int buf = 0;
#pragma unroll 1
        for (int i0 = 0; i0 < Q; i0 += KS, buf ^= 1) {
            const bool more = i0 + KS < Q;
            vt rn[V_RN], rp[V_RP], rd[V_DT];
            if (more) fetch(i0 + KS, rn, rp, rd);
            const T* sC = U + buf * SB1;
            const T* sD = sC + K::S_CROW;
            const T* sDT = sD + K::S_DROW;
            // a tile is active for the block when some i of the block is >= some j of the tile
            bool any_act = false;
#pragma unroll
            for (int jt = 0; jt < TPW; ++jt) any_act = any_act || (i0 + KS - 1 >= tt[jt]);
            if (any_act) {
                Frag uf[TPW];
#pragma unroll
                for (int st = 0; st < KS / 16; ++st) {
                    const int is = i0 + st * 16;
                    Frag cf[KN], df[KP];
#pragma unroll
                    for (int kn = 0; kn < KN; ++kn)
                        cf[kn] = M::load(&sC[(st * 16 + lr) * RPN + kn * KS + SL * lg]);
#pragma unroll
                    for (int kp = 0; kp < KP; ++kp)
                        df[kp] = M::load(&sD[(st * 16 + lr) * RPP + kp * KS + SL * lg]);
                    const f32x4 ea = *(const f32x4*)&sea[is + 4 * lg];
                    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int jt = 0; jt < TPW; ++jt) {
                        float uv[4] = {0.f, 0.f, 0.f, 0.f};
                        if (is + 15 >= tt[jt]) {
                            f32x4 ut = f32x4{0.f, 0.f, 0.f, 0.f}, wt = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int kn = 0; kn < KN; ++kn) ut = M::mma(cf[kn], Bn[jt][kn], ut);
#pragma unroll
                            for (int kp = 0; kp < KP; ++kp) wt = M::mma(df[kp], Xn[jt][kp], wt);
                            float m[4];
                            pair_decay(is, jt, ea, m);
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                uv[r] = ut[r] * m[r];
                                const float f = uv[r] * wt[r];  // F_ij / dt_j
                                kq[jt] += f;
                                rs[r] += f * dt_j[jt];
                            }
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) uf[jt][st * 4 + r] = (E)uv[r];
                    }
                    const float t = row_sums16(rs, lr);
                    if ((lr & 3) == 0) {
                        const int r = 2 * (lr >> 3) + ((lr >> 2) & 1);
                        s_rw[wave][is + 4 * lg + r] = t;
                    }
                }
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const Frag a = M::load(&sDT[(pt * 16 + lr) * TPK + SL * lg]);
#pragma unroll
                    for (int jt = 0; jt < TPW; ++jt) adx[jt][pt] = M::mma(a, uf[jt], adx[jt][pt]);
                }
            }
            if (more) store(U + (buf ^ 1) * SB1, rn, rp, rd);
            __syncthreads();
        }
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
            const int64_t trow = rb + t0 + tt[jt] + lr;
            float qp = 0.f;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                float xv[4], dyv[4];
                load4(xc + trow * d.C + xoff + pt * 16 + 4 * lg, xv);
                load4(dy + trow * HPd + xoff + pt * 16 + 4 * lg, dyv);
                typedef T ot4 __attribute__((ext_vector_type(4)));
                ot4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    qp += xv[r] * adx[jt][pt][r];
                    o[r] = (T)(dt_j[jt] * adx[jt][pt][r] + Dh * dyv[r]);
                    dD_part += dyv[r] * xv[r];
                }
                *(ot4*)(dv + trow * HPd + xoff + pt * 16 + 4 * lg) = o;
            }
            q_t[jt] = sum_groups(qp);
        }
    }

    // =================== phase B2: dB of the wave's tiles (sources j) ===================
    // G^T [n][p] into the union
    for (int idx = threadIdx.x; idx < N * (P / VEC); idx += NTH) {
        const int n = idx / (P / VEC), pv = idx % (P / VEC);
        *(vt*)&U[n * RPP + pv * VEC] = *(const vt*)(gnp + st_off + (int64_t)n * P + pv * VEC);
    }
    __syncthreads();
    {
        Frag Xn[TPW][KP];
        f32x4 adb[TPW][NT];
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
            const int64_t trow = rb + t0 + tt[jt] + lr;
#pragma unroll
            for (int kp = 0; kp < KP; ++kp)
                Xn[jt][kp] = M::load(xc + trow * d.C + xoff + kp * KS + SL * lg);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kp = 0; kp < KP; ++kp)
                    a = M::mma(M::load(&U[(nt * 16 + lr) * RPP + kp * KS + SL * lg]), Xn[jt][kp], a);
                adb[jt][nt] = a * gj[jt];
            }
        }
        __syncthreads();  // G^T consumed

        constexpr int V_RP = (KS * (P / VEC) + NTH - 1) / NTH;
        constexpr int V_CT = (N * (KS / VEC) + NTH - 1) / NTH;
        constexpr int SB2 = K::S_DROW + K::S_CT;  // dy rows, C^T
        auto fetch = [&](int i0, vt (&rp)[V_RP], vt (&rc)[V_CT]) {
#pragma unroll
            for (int q = 0; q < V_RP; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < KS * (P / VEC)) {
                    const int ii = idx / (P / VEC), pv = idx % (P / VEC);
                    rp[q] = *(const vt*)(dy + (rb + t0 + i0 + ii) * HPd + xoff + pv * VEC);
                }
            }
#pragma unroll
            for (int q = 0; q < V_CT; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < N * (KS / VEC)) {
                    const int n = idx / (KS / VEC), kv = idx % (KS / VEC);
                    rc[q] = *(const vt*)(bctC + (int64_t)n * Q + i0 + kv * VEC);
                }
            }
        };
        auto store = [&](T* s, const vt (&rp)[V_RP], const vt (&rc)[V_CT]) {
#pragma unroll
            for (int q = 0; q < V_RP; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < KS * (P / VEC))
                    *(vt*)&s[(idx / (P / VEC)) * RPP + (idx % (P / VEC)) * VEC] = rp[q];
            }
#pragma unroll
            for (int q = 0; q < V_CT; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < N * (KS / VEC))
                    *(vt*)&s[K::S_DROW + (idx / (KS / VEC)) * TPK + (idx % (KS / VEC)) * VEC] = rc[q];
            }
        };
        {
            vt rp[V_RP], rc[V_CT];
            fetch(0, rp, rc);
            store(U, rp, rc);
        }
        __syncthreads();
        int buf = 0;
#pragma unroll 1
        for (int i0 = 0; i0 < Q; i0 += KS, buf ^= 1) {
            const bool more = i0 + KS < Q;
            vt rp[V_RP], rc[V_CT];
            if (more) fetch(i0 + KS, rp, rc);
            const T* sD = U + buf * SB2;
            const T* sCT = sD + K::S_DROW;
            bool any_act = false;
#pragma unroll
            for (int jt = 0; jt < TPW; ++jt) any_act = any_act || (i0 + KS - 1 >= tt[jt]);
            if (any_act) {
                Frag wf[TPW];
#pragma unroll
                for (int st = 0; st < KS / 16; ++st) {
                    const int is = i0 + st * 16;
                    Frag df[KP];
#pragma unroll
                    for (int kp = 0; kp < KP; ++kp)
                        df[kp] = M::load(&sD[(st * 16 + lr) * RPP + kp * KS + SL * lg]);
                    const f32x4 ea = *(const f32x4*)&sea[is + 4 * lg];
#pragma unroll
                    for (int jt = 0; jt < TPW; ++jt) {
                        float wv[4] = {0.f, 0.f, 0.f, 0.f};
                        if (is + 15 >= tt[jt]) {
                            f32x4 wt = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int kp = 0; kp < KP; ++kp) wt = M::mma(df[kp], Xn[jt][kp], wt);
                            float m[4];
                            pair_decay(is, jt, ea, m);
#pragma unroll
                            for (int r = 0; r < 4; ++r) wv[r] = wt[r] * m[r];
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) wf[jt][st * 4 + r] = (E)wv[r];
                    }
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const Frag a = M::load(&sCT[(nt * 16 + lr) * TPK + SL * lg]);
#pragma unroll
                    for (int jt = 0; jt < TPW; ++jt) adb[jt][nt] = M::mma(a, wf[jt], adb[jt][nt]);
                }
            }
            if (more) store(U + (buf ^ 1) * SB2, rp, rc);
            __syncthreads();
        }
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
            const int64_t trow = rb + t0 + tt[jt] + lr;
            T* dbrow = dbc + (trow * d.H + h) * (2 * N);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dbrow[nt * 16 + 4 * lg + r] = (T)(adb[jt][nt][r] * dt_j[jt]);
        }
    }

#pragma unroll
    for (int jt = 0; jt < TPW; ++jt) {
        const int tj = tt[jt] + lr;
        const float K_j = dt_j[jt] * sum_groups(kq[jt]);
        if (lg == 0) {
            float* tp = tokp + (hl + tj) * 4;
            tp[0] = u_t[jt] - K_j;  // R_i is added by the ddt assembly from the row sums
            tp[1] = q_t[jt];
            tp[2] = v_t[jt];
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dD_part += __shfl_xor(dD_part, off, 64);
    if (lane == 0) s_red[wave] = dD_part;
    __syncthreads();
    for (int t = threadIdx.x; t < Q; t += NTH) {
        float rsum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) rsum += s_rw[w][t];
        rpart[hl + t] = rsum;
    }
    if (threadIdx.x == 0) {
        float dd = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) dd += s_red[w];
        red4[((int64_t)b * d.nchunk + cm) * d.H + h] = dd;
    }
}

// ---------------------------------------------------------------------------
// ddt per chunk and head (one wave):
//   dL/d(dt_t A) = sum_{i >= t in t's sequence run} (R_i - K_i + u_i)
//                  + sum_{j < t} v_j + exp(cs_end) <G_exit, H_enter>,
// exactly 0 at a token that starts a packed sequence; then
// ddt_t = q_t + A dL/d(dt_t A) and the chain through clamp and softplus.
// The arguments of the ddt assembly, passed whole to the kernels that run it.
template <typename T>
struct DdtArgs {
    const T* dt_raw;
    const float *dt_bias, *A_log, *dt_ws, *cs_ws;
    const int32_t* seq;
    const float *rpart, *tokp, *dotgh, *red4;
    T* ddt_raw;
    float* red;
};

template <typename T>
__device__ __forceinline__ void ddt_wave(const Dims& d, const SegTab& tab, const DdtArgs<T>& g,
                                         int cm, int h, int64_t b, int lane) {
    const T* __restrict__ dt_raw = g.dt_raw;
    const float* __restrict__ dt_bias = g.dt_bias;
    const float* __restrict__ A_log = g.A_log;
    const float* __restrict__ dt_ws = g.dt_ws;
    const float* __restrict__ cs_ws = g.cs_ws;
    const int32_t* __restrict__ seq = g.seq;
    const float* __restrict__ rpart = g.rpart;
    const float* __restrict__ tokp = g.tokp;
    const float* __restrict__ dotgh = g.dotgh;
    const float* __restrict__ red4 = g.red4;
    T* __restrict__ ddt_raw = g.ddt_raw;
    float* __restrict__ red = g.red;
    const int Q = d.Q, E = Q / 64;
    const int64_t rb = b * d.L, t0 = (int64_t)cm * Q;
    const int64_t hl = ((int64_t)b * d.H + h) * d.L + t0;
    const int k = seg_of_chunk(tab, cm, Q);
    const int64_t s0 = tab.start[k];
    const int64_t pred = seg_pred_token(tab, k);
    const int64_t refc = (t0 == s0) ? (pred >= 0 ? pred : s0) : t0 - 1;
    const int seq_refc = seq ? seq[rb + refc] : 0;
    const int seq_e = seq ? seq[rb + t0 + Q - 1] : 0;
    const float A = -expf(A_log[h]);
    const float cs_e = cs_ws[hl + Q - 1];
    const float const4 = (seq_refc == seq_e ? expf(cs_e) : 0.f) *
                         dotgh[((int64_t)b * d.nchunk + cm) * d.H + h];
    // every per-token input of the lane's tokens lane*E .. lane*E+E-1 up front
    // (one memory round trip), with the sequence ids of the tokens on either side
    // (three of tokp's four floats per token: a loaded register that is never
    // read gets reused at once, and the reuse waits for that load)
    typedef float f32x3 __attribute__((ext_vector_type(3)));
    f32x3 tp[4];
    float rp[4], dtr[4], dtw[4];
    int sqv[6];  // sequence ids of tokens lane*E-1 .. lane*E+E
    // (slots e >= E load token lane*E+E-1 again, unused: no branch around the loads)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int t = lane * E + min(e, E - 1);
        tp[e] = *(const f32x3*)&tokp[(hl + t) * 4];
        rp[e] = rpart[hl + t];
        dtr[e] = (float)dt_raw[(rb + t0 + t) * d.H + h];
        dtw[e] = dt_ws[hl + t];
    }
    if (seq) {
#pragma unroll
        for (int e = 0; e < 6; ++e) sqv[e] = seq[rb + t0 + min(max(lane * E + e - 1, 0), Q - 1)];
    } else {
#pragma unroll
        for (int e = 0; e < 6; ++e) sqv[e] = 0;
    }
    auto sq = [&](int e) { return sqv[e + 1]; };  // id of token lane*E + e

    // segmented suffix of s (runs end where the sequence changes), lanes hold
    // tokens lane*E .. lane*E+E-1
    float sl[4], run = 0.f;
    bool rs[4], cut_any = false;
#pragma unroll
    for (int e = 3; e >= 0; --e) {
        if (e < E) {
            const int t = lane * E + e;
            const bool cut = t < Q - 1 && sq(e + 1) != sq(e);
            if (cut) run = 0.f;
            cut_any = cut_any || cut;
            const float s = tp[e][0] + rp[e];
            run += s;
            sl[e] = run;
            rs[e] = cut_any;
        }
    }
    // (f1, v1) left of (f2, v2) -> (f1 | f2, f1 ? v1 : v1 + v2), inclusive from the right
    float iv = run;
    bool ifl = cut_any;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float v = __shfl_down(iv, off, 64);
        const int f = __shfl_down((int)ifl, off, 64);
        if (lane + off < 64) {
            if (!ifl) iv += v;
            ifl = ifl || f;
        }
    }
    float carry = __shfl_down(iv, 1, 64);
    if (lane == 63) carry = 0.f;
    // exclusive prefix of v over the chunk
    float vl[4], vrun = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (e < E) {
            vl[e] = vrun;
            vrun += tp[e][2];
        }
    }
    float vin = vrun;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(vin, off, 64);
        if (lane >= off) vin += y;
    }
    const float vbefore = vin - vrun;
    const float bias = dt_bias[h];
    float s_db = 0.f, s_da = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (e < E) {
            const int t = lane * E + e;
            // the decay of a token that starts a sequence is the constant 0
            const bool starts = t > 0 ? sq(e) != sq(e - 1) : sq(e) != seq_refc;
            const float dl = starts ? 0.f : sl[e] + (rs[e] ? 0.f : carry) + vbefore + vl[e] + const4;
            const float ddt = tp[e][1] + A * dl;
            const float z = dtr[e] + bias;
            const float sp = softplus_b(z);
            const bool pass = sp >= d.dt_min && sp <= d.dt_max;
            const float gr = pass ? ddt / (1.f + expf(-z)) : 0.f;
            ddt_raw[(rb + t0 + t) * d.H + h] = (T)gr;
            s_db += gr;
            s_da += dtw[e] * dl;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        s_db += __shfl_xor(s_db, off, 64);
        s_da += __shfl_xor(s_da, off, 64);
    }
    if (lane == 0) {
        const float dd = red4[((int64_t)b * d.nchunk + cm) * d.H + h];
        float* rp = red + (((int64_t)b * d.nchunk + cm) * d.H + h) * 3;
        rp[0] = s_db;
        rp[1] = s_da;
        rp[2] = dd;
    }
}

// ---------------------------------------------------------------------------
// dB and dC of a group are the sums of its head blocks' contributions
// (dbc[token][nblk][2N], blocks of group g at g*bpg..) -> dbcs[token][G][2N].
template <typename T>
__global__ void __launch_bounds__(256) k_bc_blocksum(Dims d, int nblk, int bpg,
                                                    const T* __restrict__ dbc,
                                                    T* __restrict__ dbcs) {
    constexpr int VEC = 16 / sizeof(T);
    typedef T vt __attribute__((ext_vector_type(VEC)));
    const int n2 = 2 * d.N, nv = d.G * n2 / VEC;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= d.batch * d.L * nv) return;
    const int64_t tok = idx / nv;
    const int o = (int)(idx % nv) * VEC, g = o / n2, r = o % n2;
    const T* src = dbc + (tok * nblk + (int64_t)g * bpg) * n2 + r;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
    for (int q = 0; q < bpg; ++q) {
        const vt v = *(const vt*)(src + (int64_t)q * n2);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += (float)v[e];
    }
    vt out;
#pragma unroll
    for (int e = 0; e < VEC; ++e) out[e] = (T)acc[e];
    *(vt*)(dbcs + tok * (d.G * n2) + o) = out;
}

// ---------------------------------------------------------------------------
// SiLU' and the transposed causal conv, without LDS staging: every thread owns 4
// consecutive channels and 16 consecutive tokens (one token group per wave,
// 64 lanes = 256 consecutive channels).  It needs xBC for W-1 tokens before and
// after its own (to rebuild the pre-activation u of its tokens and of the W-1
// that follow) and d(conv output) for its tokens and the W-1 that follow in
// causal order (the right halo, from the causal successor segment), all loaded
// into registers; du is produced in causal order and the transposed conv
// slides a W-row window over it.  The gradient of a conv output channel is
// read from dvx (x channels, [token][H*P]) or dbc (B and C channels,
// [token][G][2N]).  dconv_w is written per 64-token block and reduced later.
template <typename T, int W>
__device__ __forceinline__ void conv_bwd_block(const Dims& d, const SegTab& tab,
                                               const T* __restrict__ xBC,
                                               const float* __restrict__ w,
                                               const int32_t* __restrict__ seq,
                                               const T* __restrict__ dvx,
                                               const T* __restrict__ dbc, T* __restrict__ dxBC,
                                               float* __restrict__ dwp, int bx, int by,
                                               int64_t bz) {
    constexpr int TPT = CONV_TPT;
    constexpr int RX = TPT + 2 * (W - 1);  // x rows: offsets -(W-1) .. TPT+W-2
    constexpr int RD = TPT + W - 1;        // du rows: offsets 0 .. TPT+W-2
    typedef T vt __attribute__((ext_vector_type(4)));
    __shared__ float wred[4][64][4 * W];
    const int lane = threadIdx.x % 64, wave = wave_id();
    const int c = (bx * 64 + lane) * 4;
    const int64_t b = bz;
    const int64_t t0 = (int64_t)by * CONV_TT + wave * TPT;
    const int64_t rb = b * d.L;
    const bool active = c < d.C;
    const int k = conv_seg(tab, t0);
    // where this thread's four channels take their output gradient from
    const int64_t HP = (int64_t)d.H * d.P;
    const bool xch = c < HP;
    const int64_t GN2 = 2 * (int64_t)d.G * d.N;
    const int64_t bco = xch ? 0 : [&] {
        const int o = (int)(c - HP), part = o / (d.G * d.N), gn = o % (d.G * d.N);
        return (int64_t)(gn / d.N) * 2 * d.N + part * d.N + gn % d.N;
    }();
    // The output gradients of the rows are loaded GD rows ahead of their use
    // (a load right before its use costs a memory round trip per row).  Each
    // load is unconditional: a lane past the channels reads channel 0, a row
    // outside the sequence reads row 0, and the products drop those values.
    // Every other access of the loop is a bounded buffer access without a
    // branch, so the wait for a row's gradient counts the stores issued since
    // (a store under a branch might not have been issued, and the wait would
    // then also take the loads of the rows after it).
    constexpr int GD = 6;
    const T* gsrc = !active ? dvx : xch ? dvx + c : dbc + bco;
    const int64_t gstr = (!active || xch) ? HP : GN2;

    float wr[4][W];
    const __amdgpu_buffer_rsrc_t wrs = buf_rsrc(w, d.C * W * (int)sizeof(float));
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int kk = 0; kk < W; ++kk) wr[e][kk] = buf_load<float>(wrs, ((c + e) * W + kk) * 4);

    // x row r is the token r - (W-1) places after t0 in causal order.  Rows,
    // their positions and sequence ids are the same for the whole wave (t0 is),
    // so the tap masks are scalar.
    float xs[RX][4];
    int mem[RX];  // position in the row (< 2^31), -1 outside
    int sq[RX];
#pragma unroll
    for (int r = 0; r < RX; ++r) {
        const int o = r - (W - 1);
        mem[r] = __builtin_amdgcn_readfirstlane(
            (int)((o >= 0 && o < TPT) ? t0 + o : conv_row(tab, k, t0, o)));
        sq[r] = __builtin_amdgcn_readfirstlane((mem[r] >= 0 && seq) ? seq[rb + mem[r]] : 0);
        // a row outside the sequence gets an empty resource (reads zeros)
        const vt v = buf_load<vt>(buf_rsrc(xBC + (rb + max(mem[r], 0)) * d.C,
                                           mem[r] >= 0 ? d.C * (int)sizeof(T) : 0),
                                  c * (int)sizeof(T));
#pragma unroll
        for (int e = 0; e < 4; ++e) xs[r][e] = (float)v[e];
    }
    auto tap = [&](int src, int dst) { return mem[src] >= 0 && mem[dst] >= 0 && sq[src] == sq[dst]; };

    float dw[4][W];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int kk = 0; kk < W; ++kk) dw[e][kk] = 0.f;
    auto gload = [&](int o) {
        return *(const vt*)(gsrc + (rb + max(mem[o + W - 1], 0)) * gstr);
    };
    vt gbuf[GD];
#pragma unroll
    for (int q = 0; q < GD; ++q)
        if (q < RD) gbuf[q] = gload(q);
    float win[W][4];  // du of offsets o-(W-1) .. o
#pragma unroll
    for (int q = 0; q < W; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) win[q][e] = 0.f;

#pragma unroll
    for (int o = 0; o < RD; ++o) {
        const int r = o + W - 1;  // x row of du offset o
        float u[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < W; ++kk) {
            if (tap(o + kk, r)) {
#pragma unroll
                for (int e = 0; e < 4; ++e) u[e] += wr[e][kk] * xs[o + kk][e];
            }
        }
        const vt dv4 = gbuf[o % GD];
        if (o + GD < RD) gbuf[o % GD] = gload(o + GD);
        // zero outside the sequence (that row's gradient load read row 0); a
        // lane past the channels has zero x and weights, so its g only meets
        // zeros and its stores are dropped.  A factor, not a branch: the load
        // of the gradient stays where it was issued.
        const float gm = mem[r] >= 0 ? 1.f : 0.f;
        float g[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-u[e]));
            g[e] = gm * (float)dv4[e] * sg * (1.f + u[e] * (1.f - sg));
        }
        if (o < TPT) {  // dconv_w from this thread's own outputs
#pragma unroll
            for (int kk = 0; kk < W; ++kk) {
                if (tap(o + kk, r)) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) dw[e][kk] += g[e] * xs[o + kk][e];
                }
            }
        }
#pragma unroll
        for (int q = 0; q + 1 < W; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) win[q][e] = win[q + 1][e];
#pragma unroll
        for (int e = 0; e < 4; ++e) win[W - 1][e] = g[e];
        if (o >= W - 1) {
            // source s = o-(W-1) feeds outputs s .. s+W-1 (du offsets), tap kk = W-1-(t-s)
            const int s = o - (W - 1), rs = s + W - 1;
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < W; ++kk) {
                const int ot = s + W - 1 - kk;  // du offset of the output
                if (tap(rs, ot + W - 1)) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] += wr[e][kk] * win[ot - s][e];
                }
            }
            vt ov;
#pragma unroll
            for (int e = 0; e < 4; ++e) ov[e] = (T)acc[e];
            buf_store(ov, buf_rsrc(dxBC + (rb + t0 + s) * d.C, d.C * (int)sizeof(T)),
                      c * (int)sizeof(T));
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int kk = 0; kk < W; ++kk) wred[wave][lane][e * W + kk] = dw[e][kk];
    __syncthreads();
    for (int q = threadIdx.x; q < 64 * 4 * W; q += blockDim.x) {
        const int ln = q / (4 * W), j = q % (4 * W);
        const int cc = (bx * 64 + ln) * 4 + j / W;
        const float sum = wred[0][ln][j] + wred[1][ln][j] + wred[2][ln][j] + wred[3][ln][j];
        if (cc < d.C) dwp[(((int64_t)b * (d.L / CONV_TT) + by) * d.C + cc) * W + (j % W)] = sum;
    }
}

// The conv backward blocks, then the ddt assembly, one wave per (row, chunk,
// head), in the same launch: the two are independent (only the final
// reduction needs both), and the ddt waves fill the last, partial round of
// conv blocks.
template <typename T, int W>
__global__ void __launch_bounds__(256) k_conv_bwd_ddt(Dims d, SegTab tab, const T* __restrict__ xBC,
                                                     const float* __restrict__ w,
                                                     const int32_t* __restrict__ seq,
                                                     const T* __restrict__ dvx,
                                                     const T* __restrict__ dbc,
                                                     T* __restrict__ dxBC,
                                                     float* __restrict__ dwp, DdtArgs<T> g) {
    const int gx = (d.C + 255) / 256, gy = d.L / CONV_TT;
    const int64_t nconv = (int64_t)gx * gy * d.batch;
    const int64_t i = blockIdx.x;
    if (i < nconv) {
        conv_bwd_block<T, W>(d, tab, xBC, w, seq, dvx, dbc, dxBC, dwp, (int)(i % gx),
                             (int)((i / gx) % gy), i / gx / gy);
        return;
    }
    const int64_t item = (i - nconv) * 4 + wave_id();
    if (item >= (int64_t)d.nchunk * d.H * d.batch) return;
    ddt_wave<T>(d, tab, g, (int)((item / d.H) % d.nchunk), (int)(item % d.H),
                item / d.H / d.nchunk, threadIdx.x % 64);
}

// ---------------------------------------------------------------------------
// Parameter gradients from their per-tile / per-chunk partials.  A block owns
// 32 outputs; eight thread groups sum interleaved partials, then one group adds
// the eight results in a fixed order (deterministic, no atomics).
__global__ void __launch_bounds__(256) k_bwd_reduce(Dims d, const float* __restrict__ dwp,
                                                   const float* __restrict__ red,
                                                   const float* __restrict__ A_log,
                                                   float* __restrict__ dconv_w,
                                                   float* __restrict__ ddt_bias,
                                                   float* __restrict__ dA_log,
                                                   float* __restrict__ dD) {
    __shared__ float part[8][32];
    const int CW = d.C * d.W;
    const int nout = CW + 3 * d.H;
    const int col = threadIdx.x % 32, gq = threadIdx.x / 32;
    const int o = blockIdx.x * 32 + col;
    // each group sums its partials in four interleaved chains, so four loads
    // are in flight at a time; the order of the additions is fixed
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
    if (o < CW) {
        const int64_t ntot = d.batch * (d.L / 64);
        int64_t t = gq;
        for (; t + 24 < ntot; t += 32)
#pragma unroll
            for (int u = 0; u < 4; ++u) s4[u] += dwp[(t + 8 * u) * CW + o];
        for (; t < ntot; t += 8) s4[0] += dwp[t * CW + o];
    } else if (o < nout) {
        const int j = o - CW, h = j / 3, q = j % 3;
        const int64_t ntot = d.batch * d.nchunk;
        int64_t bc = gq;
        for (; bc + 24 < ntot; bc += 32)
#pragma unroll
            for (int u = 0; u < 4; ++u) s4[u] += red[((bc + 8 * u) * d.H + h) * 3 + q];
        for (; bc < ntot; bc += 8) s4[0] += red[(bc * d.H + h) * 3 + q];
    }
    const float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    part[gq][col] = s;
    __syncthreads();
    if (gq == 0 && o < nout) {
        float t = 0.f;
#pragma unroll
        for (int g = 0; g < 8; ++g) t += part[g][col];
        if (o < CW) {
            dconv_w[o] = t;
        } else {
            const int j = o - CW, h = j / 3, q = j % 3;
            if (q == 0) ddt_bias[h] = t;
            else if (q == 1) dA_log[h] = -expf(A_log[h]) * t;
            else dD[h] = t;
        }
    }
}

// ---------------------------------------------------------------------------
// Dispatch.

constexpr size_t BWD_LDS_LIMIT = 160 * 1024;

// Tiles per wave (two: with four the accumulators no longer fit in registers).
template <typename T, int Q>
constexpr int chunk_bwd_tpw() {
    return 2;
}

template <typename T, int P, int N, int Q>
constexpr bool chunk_bwd_fits() {
    return ChunkBwd<T, P, N, Q, chunk_bwd_tpw<T, Q>()>::LDS <= BWD_LDS_LIMIT;
}

// The head-blocked chunk kernel takes P <= 64 (its Z and dx accumulators share
// the registers); larger heads use the per-head kernel.
template <typename T, int P, int N, int Q>
constexpr bool hb_fits() {
    return P <= 64 && ChunkBwdHB<T, P, N, Q>::LDS <= BWD_LDS_LIMIT;
}
template <typename T, int P, int N>
static bool hb_path(int Q) {
    if (Q == 64) return hb_fits<T, P, N, 64>();
    if (Q == 128) return hb_fits<T, P, N, 128>();
    if (Q == 256) return hb_fits<T, P, N, 256>();
    return false;
}
constexpr int HB_MAX = 8;  // heads per workgroup of the head-blocked kernel
// heads per block: the largest divisor of the heads per group up to HB_MAX
static int head_block(const Dims& d) {
    int hb = 1;
    for (int c = 1; c <= HB_MAX; ++c)
        if (d.hpg % c == 0) hb = c;
    return hb;
}

template <typename T, int P, int N>
static bool bwd_shape_ok(int Q) {
    if (hb_path<T, P, N>(Q)) return true;
    if (Q == 64) return chunk_bwd_fits<T, P, N, 64>();
    if (Q == 128) return chunk_bwd_fits<T, P, N, 128>();
    if (Q == 256) return chunk_bwd_fits<T, P, N, 256>();
    return false;
}

template <typename T, int P, int N, int Q>
static void launch_chunk_bwd(const Dims& d, const SegTab& t, const BwdArgs& a, const BwdWs& L,
                             char* ws, hipStream_t s) {
    if constexpr (hb_fits<T, P, N, Q>()) {
        const int hbs = head_block(d);
        const unsigned nblk = (unsigned)((int64_t)d.nchunk * (d.H / hbs) * d.batch);
        hipLaunchKernelGGL((k_chunk_bwd_hb<T, P, N, Q>), dim3(nblk),
                           dim3(ChunkBwdHB<T, P, N, Q>::NTH), 0, s, d, t, hbs,
                           (const T*)(ws + L.xc), (const T*)a.dy, (const T*)(ws + L.gramt), a.D, (const float*)(ws + L.dt),
                           (const float*)(ws + L.cs), a.seq, (const T*)(ws + L.gpn),
                           (const T*)(ws + L.hpn), (T*)(ws + L.dv), (T*)(ws + L.dbc),
                           (float*)(ws + L.rpart),
                           (float*)(ws + L.tokp), (float*)(ws + L.red4), (float*)(ws + L.dotgh));
    } else if constexpr (chunk_bwd_fits<T, P, N, Q>()) {
        constexpr int TPW = chunk_bwd_tpw<T, Q>();
        constexpr int NW = ChunkBwd<T, P, N, Q, TPW>::NW;
        hipLaunchKernelGGL((k_chunk_bwd<T, P, N, Q, TPW>), chunk_head_grid(d),
                           dim3(NW * 64), 0, s, d, t, (const T*)(ws + L.xc),
                           (const T*)(ws + L.bct), (const T*)a.dy, (const T*)(ws + L.dyT), a.D,
                           (const float*)(ws + L.dt), (const float*)(ws + L.cs), a.seq,
                           (const T*)(ws + L.gpn), (const T*)(ws + L.gnp), (const T*)(ws + L.hnp),
                           (T*)(ws + L.dv), (T*)(ws + L.dbc), (float*)(ws + L.rpart),
                           (float*)(ws + L.tokp), (float*)(ws + L.red4));
    }
}

template <typename T, int W>
static void launch_conv_bwd_w(const Dims& d, const SegTab& t, const BwdArgs& a, const BwdWs& L,
                              int hbs, char* ws, hipStream_t s) {
    const int64_t nconv = (int64_t)((d.C + 255) / 256) * (d.L / CONV_TT) * d.batch;
    const int64_t nddt = ((int64_t)d.nchunk * d.H * d.batch + 3) / 4;
    // one head block per group: its partials are already [token][G][2N]
    const T* dbc = (const T*)(ws + (d.hpg / hbs == 1 ? L.dbc : L.dbcs));

    const DdtArgs<T> g = {(const T*)a.dt_raw, a.dt_bias, a.A_log, (const float*)(ws + L.dt),
                          (const float*)(ws + L.cs), a.seq, (const float*)(ws + L.rpart),
                          (const float*)(ws + L.tokp), (const float*)(ws + L.dotgh),
                          (const float*)(ws + L.red4), (T*)a.ddt_raw, (float*)(ws + L.red)};
    hipLaunchKernelGGL((k_conv_bwd_ddt<T, W>), dim3((unsigned)(nconv + nddt)), dim3(256), 0, s, d, t,
                       (const T*)a.xBC, a.conv_w, a.seq, (const T*)(ws + L.dv), dbc, (T*)a.dxBC,
                       (float*)(ws + L.dwp), g);
}

template <typename T>
static void launch_conv_bwd(const Dims& d, const SegTab& t, const BwdArgs& a, const BwdWs& L,
                            int hbs, char* ws, hipStream_t s) {
    switch (d.W) {
        case 1: launch_conv_bwd_w<T, 1>(d, t, a, L, hbs, ws, s); break;
        case 2: launch_conv_bwd_w<T, 2>(d, t, a, L, hbs, ws, s); break;
        case 3: launch_conv_bwd_w<T, 3>(d, t, a, L, hbs, ws, s); break;
        case 4: launch_conv_bwd_w<T, 4>(d, t, a, L, hbs, ws, s); break;
        case 5: launch_conv_bwd_w<T, 5>(d, t, a, L, hbs, ws, s); break;
        case 6: launch_conv_bwd_w<T, 6>(d, t, a, L, hbs, ws, s); break;
        case 7: launch_conv_bwd_w<T, 7>(d, t, a, L, hbs, ws, s); break;
        default: launch_conv_bwd_w<T, 8>(d, t, a, L, hbs, ws, s); break;
    }
}

template <typename T, int P, int N>
static void bwd_summary_t(const Dims& d, const SegTab& t, const BwdArgs& a, float* summary,
                          void* ws_, hipStream_t s) {
    const BwdWs L = bwd_ws_layout(d, std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32);
    char* ws = (char*)ws_;
    T* xc = (T*)(ws + L.xc);
    launch_conv1d_fwd(d, t, std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32, a.xBC, a.conv_w,
                      a.seq, xc, s);
    if (hb_path<T, P, N>(d.Q)) {
        // the transposed Gram tiles and dt prep in one launch
        launch_gram_dt<T, N, true>(d, xc, (T*)(ws + L.gramt), a.dt_raw, a.dt_bias, a.A_log, a.seq,
                                   (float*)(ws + L.dt), (float*)(ws + L.cs),
                                   (float*)(ws + L.ctot), s);
    } else {
        hipLaunchKernelGGL(k_bc_transpose<T>,
                           dim3((unsigned)d.nchunk, (unsigned)d.G, (unsigned)d.batch), dim3(256), 0,
                           s, d, (const T*)xc, (T*)(ws + L.bct));
        launch_dt_prep(d, std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32, a.dt_raw, a.dt_bias,
                       a.A_log, a.seq, (float*)(ws + L.dt), (float*)(ws + L.cs),
                       (float*)(ws + L.ctot), s);
    }
    if (hb_path<T, P, N>(d.Q)) {
        // the reverse walk from a zero final gradient: dL/dS_in of each segment's
        // own outputs and its block decay
        const WalkArgs<T> wa = {(const T*)xc, (const T*)a.dy, (const float*)(ws + L.dt),
                                (const float*)(ws + L.cs), a.seq, nullptr, nullptr, summary};
        launch_state_walk<T, P, N, true>(d, t, wa, s);
        return;
    }
    hipLaunchKernelGGL((k_bwd_chunk_states<T, P, N>), chunk_head_grid(d), dim3(256), 0, s,
                       d, t, (const T*)xc, (const T*)(ws + L.bct), (const T*)a.dy,
                       (const float*)(ws + L.dt), (const float*)(ws + L.cs), a.seq,
                       (float*)(ws + L.zh), (float*)(ws + L.zg),
                       hb_path<T, P, N>(d.Q) ? (T*)nullptr : (T*)(ws + L.dyT));
    hipLaunchKernelGGL((k_state_pass<T, P, N, PASS_SUMMARY>),
                       dim3((unsigned)d.H, (unsigned)d.nseg, (unsigned)d.batch), dim3(256), 0, s,
                       d, t, (const float*)(ws + L.ctot), a.seq, (const float*)(ws + L.zg),
                       (const float*)(ws + L.zh), (const float*)nullptr, (const float*)nullptr,
                       summary, (T*)nullptr, (T*)nullptr, (T*)nullptr, (T*)nullptr, (float*)nullptr);
}

template <typename T, int P, int N>
static void bwd_pass_t(const Dims& d, const SegTab& t, const BwdArgs& a, void* ws_,
                       hipStream_t s) {
    // the head-blocked chunk kernel reads G and H as [p][n] only (written by the
    // two walks); the per-head one reads G as [p][n] and [n][p] and H as [n][p]
    // (written by the pass kernel from the chunk contributions)
    const bool hb = hb_path<T, P, N>(d.Q);
    const BwdWs L = bwd_ws_layout(d, std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32);
    char* ws = (char*)ws_;
    if (hb) {
        // G of every chunk: the reverse walk from dS_out; H of every chunk: the
        // forward walk from S_in; both in one launch (<G_c, H_c> comes from the
        // chunk kernel)
        const WalkArgs<T> bwd = {(const T*)(ws + L.xc), (const T*)a.dy, (const float*)(ws + L.dt),
                                 (const float*)(ws + L.cs), a.seq, a.dS_out, (T*)(ws + L.gpn),
                                 nullptr};
        const WalkArgs<T> fwd = {(const T*)(ws + L.xc), nullptr, (const float*)(ws + L.dt),
                                 (const float*)(ws + L.cs), a.seq, a.S_in, (T*)(ws + L.hpn),
                                 nullptr};
        launch_state_walk_pair<T, P, N>(d, t, bwd, fwd, s);
        return;
    }
    hipLaunchKernelGGL((k_state_pass<T, P, N, PASS_TRUE>),
                       dim3((unsigned)d.H, (unsigned)d.nseg, (unsigned)d.batch), dim3(256), 0, s,
                       d, t, (const float*)(ws + L.ctot), a.seq, (const float*)(ws + L.zg),
                       (const float*)(ws + L.zh), a.S_in, a.dS_out, (float*)nullptr,
                       (T*)(ws + L.gpn), (T*)(ws + L.gnp), (T*)(ws + L.hnp), (T*)nullptr,
                       (float*)(ws + L.dotgh));
}

template <typename T, int P, int N>
static void bwd_chunks_t(const Dims& d, const SegTab& t, const BwdArgs& a, void* ws_,
                         hipStream_t s) {
    const BwdWs L = bwd_ws_layout(d, std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32);
    char* ws = (char*)ws_;
    switch (d.Q) {
        case 64: launch_chunk_bwd<T, P, N, 64>(d, t, a, L, ws, s); break;
        case 128: launch_chunk_bwd<T, P, N, 128>(d, t, a, L, ws, s); break;
        default: launch_chunk_bwd<T, P, N, 256>(d, t, a, L, ws, s); break;
    }
}

template <typename T>
static void conv_bwd_t(const Dims& d, const SegTab& t, const BwdArgs& a, int hbs, void* ws_,
                       hipStream_t s) {
    const BwdWs L = bwd_ws_layout(d, std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32);
    char* ws = (char*)ws_;
    if (d.hpg / hbs > 1) {
        const int64_t nv = d.batch * d.L * d.G * 2 * d.N / (16 / sizeof(T));
        hipLaunchKernelGGL(k_bc_blocksum<T>, dim3((unsigned)((nv + 255) / 256)), dim3(256), 0, s, d,
                           d.H / hbs, d.hpg / hbs, (const T*)(ws + L.dbc), (T*)(ws + L.dbcs));
    }
    launch_conv_bwd<T>(d, t, a, L, hbs, ws, s);
    const int nout = d.C * d.W + 3 * d.H;
    hipLaunchKernelGGL(k_bwd_reduce, dim3((unsigned)((nout + 31) / 32)), dim3(256), 0, s, d,
                       (const float*)(ws + L.dwp), (const float*)(ws + L.red), a.A_log, a.dconv_w,
                       a.ddt_bias, a.dA_log, a.dD);
}

#define SSD_BWD_F32_SHAPES(X) X(16, 16) X(32, 32) X(64, 64) X(64, 128)
#define SSD_BWD_BF16_SHAPES(X) X(32, 64) X(64, 64) X(64, 128) X(128, 128)

bool bwd_supported(int P, int N, int Q, int act) {
#define X(p, n) if (P == p && N == n) return bwd_shape_ok<T, p, n>(Q);
    if (act == SSD_F32) {
        typedef float T;
        SSD_BWD_F32_SHAPES(X)
    } else {
        typedef bf16 T;
        SSD_BWD_BF16_SHAPES(X)
    }
#undef X
    return false;
}

hipError_t launch_bwd_summary(const Dims& d, const SegTab& t, int act, const BwdArgs& a,
                              float* summary, void* ws, hipStream_t s) {
#define X(p, n)                                                   \
    if (d.P == p && d.N == n) {                                   \
        bwd_summary_t<T, p, n>(d, t, a, summary, ws, s);          \
        return hipGetLastError();                                 \
    }
    if (act == SSD_F32) {
        typedef float T;
        SSD_BWD_F32_SHAPES(X)
    } else {
        typedef bf16 T;
        SSD_BWD_BF16_SHAPES(X)
    }
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_pass(const Dims& d, const SegTab& t, int act, const BwdArgs& a, void* ws,
                           hipStream_t s) {
#define X(p, n)                                \
    if (d.P == p && d.N == n) {                \
        bwd_pass_t<T, p, n>(d, t, a, ws, s);   \
        return hipGetLastError();              \
    }
    if (act == SSD_F32) {
        typedef float T;
        SSD_BWD_F32_SHAPES(X)
    } else {
        typedef bf16 T;
        SSD_BWD_BF16_SHAPES(X)
    }
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_chunks(const Dims& d, const SegTab& t, int act, const BwdArgs& a, void* ws,
                             hipStream_t s) {
#define X(p, n)                                  \
    if (d.P == p && d.N == n) {                  \
        bwd_chunks_t<T, p, n>(d, t, a, ws, s);   \
        return hipGetLastError();                \
    }
    if (act == SSD_F32) {
        typedef float T;
        SSD_BWD_F32_SHAPES(X)
    } else {
        typedef bf16 T;
        SSD_BWD_BF16_SHAPES(X)
    }
#undef X
    return hipErrorInvalidValue;
}

// Heads per dB / dC partial the chunk phase leaves: the head block of the
// head-blocked kernel, else 1.
static int dbc_heads(const Dims& d, int act) {
#define X(p, n) \
    if (d.P == p && d.N == n) return hb_path<T, p, n>(d.Q) ? head_block(d) : 1;
    if (act == SSD_F32) {
        typedef float T;
        SSD_BWD_F32_SHAPES(X)
    } else {
        typedef bf16 T;
        SSD_BWD_BF16_SHAPES(X)
    }
#undef X
    return 1;
}

hipError_t launch_conv1d_bwd(const Dims& d, const SegTab& t, int act, const BwdArgs& a, void* ws,
                             hipStream_t s) {
    const int hbs = dbc_heads(d, act);
    if (act == SSD_BF16) conv_bwd_t<bf16>(d, t, a, hbs, ws, s);
    else conv_bwd_t<float>(d, t, a, hbs, ws, s);
    return hipGetLastError();
}

}  // namespace ssd
