// Backward of the conv1d + SSD state-passing path (gfx950, wave64, MFMA).
//
// Megatron-LM #6808 (first commit): the backward mirrors the forward with a
// reverse boundary scan and recomputes every sequence-length-sized
// intermediate instead of saving it.  Here:
//
//   summary phase (ssd_segment_bwd_summary)
//     conv recompute -> xBC_conv and dt/cumsum recompute in one launch
//     (k_conv1d_silu_dt), then the reverse walk of every segment from a zero
//     state gradient and the chunk's causal Gram tiles in transposed
//     orientation, in one launch (k_walk_gram<bwd, TRANS>; other shapes run
//     k_gram_dt<TRANS> and k_state_walk<bwd>), which leaves, per segment,
//     dL/dS_in of the segment's own outputs and its block decay, in the same
//     packed layout as the forward summary.
//   reverse boundary scan (ssd_boundary_scan, reverse = 1) -> the gradient of
//     every segment's final state.
//   pass phase (ssd_segment_bwd_pass): the exit gradient and the entering
//     state of every chunk, the reverse walk from dS_out and the forward walk
//     from S_in as the two halves of one launch (k_state_walk_pair).
//   chunk phase (ssd_segment_bwd_chunks): k_chunk_bwd_hb per chunk and block
//     of heads of one group: dx, dB, dC and the ddt partial sums, written into
//     the buffers the conv backward consumes.
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
#include "walk_gram.h"
#include "xt.h"

namespace ssd {

__device__ __forceinline__ float softplus_b(float z) {
    return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
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
    // (tokp per token: -K, q, v, u)
    f32x4 tp[4];
    float rp[4], dtr[4], dtw[4];
    int sqv[6];  // sequence ids of tokens lane*E-1 .. lane*E+E
    // (slots e >= E load token lane*E+E-1 again, unused: no branch around the loads)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int t = lane * E + min(e, E - 1);
        tp[e] = *(const f32x4*)&tokp[(hl + t) * 4];
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
            const float s = tp[e][0] + tp[e][3] + rp[e];
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

// Shapes the backward runs: the head-blocked chunk kernel takes P <= 64 (its Z
// and dx accumulators share the registers) and must fit the LDS of a CU.
template <typename T, int P, int N, int Q>
constexpr bool hb_fits() {
    return P <= 64 && ChunkBwdHB<T, P, N, Q>::LDS <= BWD_LDS_LIMIT;
}
template <typename T, int P, int N>
static bool bwd_shape_ok(int Q) {
    if (Q == 64) return hb_fits<T, P, N, 64>();
    if (Q == 128) return hb_fits<T, P, N, 128>();
    if (Q == 256) return hb_fits<T, P, N, 256>();
    return false;
}

template <typename T, int P, int N, int Q>
static hipError_t launch_chunk_bwd(const Dims& d, const SegTab& t, const BwdArgs& a,
                                   const BwdWs& L, char* ws, hipStream_t s) {
    if constexpr (hb_fits<T, P, N, Q>()) {
        const int hbs = head_block(d);
        const unsigned nblk = (unsigned)((int64_t)d.nchunk * (d.H / hbs) * d.batch);
        return launch(k_chunk_bwd_hb<T, P, N, Q>, dim3(nblk), dim3(ChunkBwdHB<T, P, N, Q>::NTH), s,
                      d, t, hbs, (const T*)(ws + L.xc), (const T*)a.dy, (const T*)(ws + L.gramt),
                      a.D, (const float*)(ws + L.dt), (const float*)(ws + L.cs), a.seq,
                      (const T*)(ws + L.gpn), (const T*)(ws + L.hpn), (T*)(ws + L.dv),
                      (T*)(ws + L.dbc), (float*)(ws + L.rpart), (float*)(ws + L.tokp),
                      (float*)(ws + L.red4), (float*)(ws + L.dotgh));
    }
    return hipErrorInvalidValue;
}

template <typename T, int W>
static hipError_t launch_conv_bwd_w(const Dims& d, const SegTab& t, const BwdArgs& a,
                                    const BwdWs& L, int hbs, char* ws, hipStream_t s) {
    const int64_t nconv = (int64_t)((d.C + 255) / 256) * (d.L / CONV_TT) * d.batch;
    const int64_t nddt = ((int64_t)d.nchunk * d.H * d.batch + 3) / 4;
    // one head block per group: its partials are already [token][G][2N]
    const T* dbc = (const T*)(ws + (d.hpg / hbs == 1 ? L.dbc : L.dbcs));
    const DdtArgs<T> g = {(const T*)a.dt_raw, a.dt_bias, a.A_log, (const float*)(ws + L.dt),
                          (const float*)(ws + L.cs), a.seq, (const float*)(ws + L.rpart),
                          (const float*)(ws + L.tokp), (const float*)(ws + L.dotgh),
                          (const float*)(ws + L.red4), (T*)a.ddt_raw, (float*)(ws + L.red)};
    return launch(k_conv_bwd_ddt<T, W>, dim3((unsigned)(nconv + nddt)), dim3(256), s, d, t,
                  (const T*)a.xBC, a.conv_w, a.seq, (const T*)(ws + L.dv), dbc, (T*)a.dxBC,
                  (float*)(ws + L.dwp), g);
}

template <typename T>
static hipError_t launch_conv_bwd(const Dims& d, const SegTab& t, const BwdArgs& a,
                                  const BwdWs& L, int hbs, char* ws, hipStream_t s) {
    switch (d.W) {
        case 1: return launch_conv_bwd_w<T, 1>(d, t, a, L, hbs, ws, s);
        case 2: return launch_conv_bwd_w<T, 2>(d, t, a, L, hbs, ws, s);
        case 3: return launch_conv_bwd_w<T, 3>(d, t, a, L, hbs, ws, s);
        case 4: return launch_conv_bwd_w<T, 4>(d, t, a, L, hbs, ws, s);
        case 5: return launch_conv_bwd_w<T, 5>(d, t, a, L, hbs, ws, s);
        case 6: return launch_conv_bwd_w<T, 6>(d, t, a, L, hbs, ws, s);
        case 7: return launch_conv_bwd_w<T, 7>(d, t, a, L, hbs, ws, s);
        case 8: return launch_conv_bwd_w<T, 8>(d, t, a, L, hbs, ws, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, int P, int N>
static hipError_t bwd_summary_t(const Dims& d, const SegTab& t, const BwdArgs& a,
                                float* summary, void* ws_, hipStream_t s) {
    constexpr int act = std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32;
    const BwdWs L = bwd_ws_layout(d, act);
    char* ws = (char*)ws_;
    T* xc = (T*)(ws + L.xc);
    float* dtw = (float*)(ws + L.dt);
    float* csw = (float*)(ws + L.cs);
    float* ctot = (float*)(ws + L.ctot);
    const T* bc = xc + (int64_t)d.H * P;
    T* gramt = (T*)(ws + L.gramt);
    // the reverse walk from a zero final gradient: dL/dS_in of each segment's own
    // outputs and its block decay
    const WalkArgs<T> wa = {(const T*)xc, (const T*)a.dy, dtw, csw, a.seq, nullptr, nullptr,
                            summary, span_plan(d, t, false)};
    if (walk_gram_fits<T>(d)) {
        // the conv recompute with dt prep, then the walk and the transposed Gram
        // tiles in one launch
        SSD_TRY(launch_conv1d_dt(d, t, act, a.xBC, a.conv_w, a.seq, xc, a.dt_raw, a.dt_bias,
                                 a.A_log, dtw, csw, ctot, s));
        return launch_walk_gram<T, P, N, true, true>(d, t, wa, bc, (int64_t)d.C, gramt, s);
    }
    SSD_TRY(launch_conv1d_fwd(d, t, act, a.xBC, a.conv_w, a.seq, xc, s));
    // the transposed Gram tiles and dt prep in one launch, then the walk
    SSD_TRY(launch_gram_dt<T, N, true>(d, bc, (int64_t)d.C, gramt, a.dt_raw, a.dt_bias, a.A_log,
                                       a.seq, dtw, csw, ctot, s));
    return launch_state_walk<T, P, N, true>(d, t, wa, s);
}

template <typename T, int P, int N>
static hipError_t bwd_pass_t(const Dims& d, const SegTab& t, const BwdArgs& a, void* ws_,
                             hipStream_t s) {
    const BwdWs L = bwd_ws_layout(d, std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32);
    char* ws = (char*)ws_;
    // G of every chunk: the reverse walk from dS_out; H of every chunk: the forward
    // walk from S_in; both in one launch (<G_c, H_c> comes from the chunk kernel)
    const SpanPlan one = span_plan(d, t, false);  // one span per segment
    const WalkArgs<T> bwd = {(const T*)(ws + L.xc), (const T*)a.dy, (const float*)(ws + L.dt),
                             (const float*)(ws + L.cs), a.seq, a.dS_out, (T*)(ws + L.gpn),
                             nullptr, one};
    const WalkArgs<T> fwd = {(const T*)(ws + L.xc), nullptr, (const float*)(ws + L.dt),
                             (const float*)(ws + L.cs), a.seq, a.S_in, (T*)(ws + L.hpn),
                             nullptr, one};
    return launch_state_walk_pair<T, P, N>(d, t, bwd, fwd, s);
}

template <typename T, int P, int N>
static hipError_t bwd_chunks_t(const Dims& d, const SegTab& t, const BwdArgs& a, void* ws_,
                               hipStream_t s) {
    const BwdWs L = bwd_ws_layout(d, std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32);
    char* ws = (char*)ws_;
    switch (d.Q) {
        case 64: return launch_chunk_bwd<T, P, N, 64>(d, t, a, L, ws, s);
        case 128: return launch_chunk_bwd<T, P, N, 128>(d, t, a, L, ws, s);
        case 256: return launch_chunk_bwd<T, P, N, 256>(d, t, a, L, ws, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
static hipError_t conv_bwd_t(const Dims& d, const SegTab& t, const BwdArgs& a, int hbs,
                             void* ws_, hipStream_t s) {
    const BwdWs L = bwd_ws_layout(d, std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32);
    char* ws = (char*)ws_;
    if (d.hpg / hbs > 1) {
        const int64_t nv = d.batch * d.L * d.G * 2 * d.N / (16 / sizeof(T));
        SSD_TRY(launch(k_bc_blocksum<T>, dim3((unsigned)((nv + 255) / 256)), dim3(256), s, d,
                       d.H / hbs, d.hpg / hbs, (const T*)(ws + L.dbc), (T*)(ws + L.dbcs)));
    }
    SSD_TRY(launch_conv_bwd<T>(d, t, a, L, hbs, ws, s));
    const int nout = d.C * d.W + 3 * d.H;
    return launch(k_bwd_reduce, dim3((unsigned)((nout + 31) / 32)), dim3(256), s, d,
                  (const float*)(ws + L.dwp), (const float*)(ws + L.red), a.A_log, a.dconv_w,
                  a.ddt_bias, a.dA_log, a.dD);
}

bool bwd_supported(int P, int N, int Q, int act) {
#define X(p, n) if (P == p && N == n) return bwd_shape_ok<T, p, n>(Q);
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

hipError_t launch_bwd_summary(const Dims& d, const SegTab& t, int act, const BwdArgs& a,
                              float* summary, void* ws, hipStream_t s) {
#define X(p, n) \
    if (d.P == p && d.N == n) return bwd_summary_t<T, p, n>(d, t, a, summary, ws, s);
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

hipError_t launch_bwd_pass(const Dims& d, const SegTab& t, int act, const BwdArgs& a, void* ws,
                           hipStream_t s) {
#define X(p, n) \
    if (d.P == p && d.N == n) return bwd_pass_t<T, p, n>(d, t, a, ws, s);
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

hipError_t launch_bwd_chunks(const Dims& d, const SegTab& t, int act, const BwdArgs& a, void* ws,
                             hipStream_t s) {
#define X(p, n) \
    if (d.P == p && d.N == n) return bwd_chunks_t<T, p, n>(d, t, a, ws, s);
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

hipError_t launch_conv1d_bwd(const Dims& d, const SegTab& t, int act, const BwdArgs& a, void* ws,
                             hipStream_t s) {
    const int hbs = head_block(d);
    if (act == SSD_BF16) return conv_bwd_t<bf16>(d, t, a, hbs, ws, s);
    return conv_bwd_t<float>(d, t, a, hbs, ws, s);
}

}  // namespace ssd
