// Chunk backward with the heads of a group blocked: one workgroup per (chunk,
// block of HB heads of one group).
//
// Per chunk, with S_ij = C_i . B_j (the group's causal Gram tiles, transposed
// orientation from the Gram pass with TRANS), W^h_ij = dy^h_i . x^h_j, the decay
// L^h_ij = exp(cs_i - cs_j) [j <= i, same sequence] and
//   Z_ij = sum over the block's heads of W^h_ij L^h_ij dt^h_j,
// the gradients of the intra-chunk term are
//   dx^h_j = dt_j sum_i S_ij L_ij dy_i          (per head)
//   dB_j   = sum_i Z_ij C_i                      (per group: B and C are shared
//   dC_i   = sum_j Z_ij B_j                       by the heads of a group)
// so dB and dC cost two products per chunk and head block instead of two per
// head, and the per-head dB / dC never go to memory.  The entering state H and
// the exit gradient G of every chunk (from the pass phase) add
//   dx_j += dt_j g_j G B_j,  dB_j += sum_h dt_j g_j G^T x_j,
//   dC_i += sum_h f_i H^T dy_i,
// with f_i = exp(cs_i) [i in the entering state's sequence] and
// g_j = exp(cs_e - cs_j) [j in the last token's sequence].  The ddt terms are
// the ones the per-head kernel produced (see ddt_wave): row and column sums of
// F = S W L dt, u_i = f_i dy_i . (H C_i), v_j = dt_j x_j . (g_j G B_j),
// q_j = x_j . (dx_j / dt_j without the D term), the dD partial, and <G, H>
// of every chunk and head.
//
// Work split: NW = Q/32 waves; wave w owns the 16-token tiles w and QT-1-w,
// as columns j (dx, column sums, v, q, dB) and as rows i (u, dC).  For a
// column tile the rows i >= j are visited one MFMA k step (KS tokens, TPK
// row tiles) at a time; the (k step, column) blocks of the wave are mapped to
// NKS + 1 fixed register slots of Z (column QT-1-w: slots 0.., column w:
// slot = k step + 1), so Z stays in registers across the heads.  The chunk's
// Gram tiles are the same for every head: they are staged in LDS once per
// workgroup, so the k steps issue no global loads.  dy and G of a head sit
// in LDS in their natural rows: row reads for the W and state products,
// transposed reads (XT) of dy for dx.  (H is loaded for <G, H> only: u is
// formed in the final phase from the H and dy rows its dC rounds load anyway,
// which spares the head loop the group's C rows and the u products; at shapes
// where that would not fit the registers, H is staged and u formed here.)
// x is read only by the wave that owns
// its rows: each wave loads its two column tiles' x rows from memory straight
// into MFMA operands, in the k-slot order of KPermRow (the W product reads dy
// in the same order), which is also the order of the dx accumulator's values,
// so the same registers give the x . dx, x . (state term) and dy . x dot
// products.  After the heads, Z goes to LDS as rows for dC,
// the chunk's C and B rows are staged in turn for the Z products (read
// transposed), and each
// head's G and H for its state terms (read transposed); dB is finished before
// dC starts.  The per-token partials of the ddt assembly are -K_j, q_j, v_j
// and u_j.
#pragma once

#include "bwd_util.h"
#include "gram.h"
#include "ssd_internal.h"
#include "xt.h"

namespace ssd {

// A k operand of consecutive row elements (bf16: 32, float32: 16, from the
// k-th block) in the k slot order of XT, so that it meets an XT read of the
// other operand: bf16 slot s of lane group g holds element 16 (s / 4) + 4 g +
// s % 4, float32 slot s holds 4 g + s.
template <typename T> struct KPermRow;
template <> struct KPermRow<bf16> {
    __device__ static __forceinline__ bf16x8 load(const bf16* row, int lg) {
        const bf16x4 lo = *(const bf16x4*)(row + 4 * lg);
        const bf16x4 hi = *(const bf16x4*)(row + 16 + 4 * lg);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // the row at base + off (elements, a 32-bit lane offset: see at32)
    __device__ static __forceinline__ bf16x8 load(const bf16* base, uint32_t off, int lg) {
        const bf16x4 lo = *(const bf16x4*)at32(base, off + 4 * lg);
        const bf16x4 hi = *(const bf16x4*)at32(base, off + 16 + 4 * lg);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
};
template <> struct KPermRow<float> {
    __device__ static __forceinline__ f32x4 load(const float* row, int lg) {
        return *(const f32x4*)(row + 4 * lg);
    }
    __device__ static __forceinline__ f32x4 load(const float* base, uint32_t off, int lg) {
        return *(const f32x4*)at32(base, off + 4 * lg);
    }
};

template <typename T, int P, int N, int Q>
struct ChunkBwdHB {
    typedef Mma<T> M;
    static constexpr int SL = M::SL, KS = M::KS, VEC = 16 / (int)sizeof(T);
    static constexpr int QT = Q / 16, NW = QT / 2, NTH = NW * 64;
    static constexpr int TPK = KS / 16;  // row tiles per MFMA k step
    static constexpr int NKS = Q / KS;   // k steps per chunk
    static constexpr int NB = NKS + 1;   // Z slots per wave
    // slots of the later column QT-1-w (at most)
    static constexpr int MAXA = TPK == 2 ? (NW - 1) / 2 + 1 : NW;
    static constexpr int PT = P / 16, NT = N / 16, KP = P / KS, KN = N / KS;
    static constexpr int XR = P + VEC;  // x / dy rows [token][p]
    static constexpr int GR = N + VEC;  // G / H rows [p][n]
    static constexpr int BR = N + VEC;  // B / C rows [token][n]
    // Z rows in LDS for dC: row tile a keeps columns [0, cw(a)) (whole k steps)
    __host__ __device__ static constexpr int cw(int a) { return KS * (a / TPK + 1); }
    __host__ __device__ static constexpr int zpitch(int a) { return cw(a) + VEC; }
    __host__ __device__ static constexpr int zoff(int a) {
        int o = 0;
        for (int t = 0; t < a; ++t) o += 16 * zpitch(t);
        return o;
    }
    static constexpr int cmax(int a, int b) { return a > b ? a : b; }
    // u_t = f_t dy_t . (H C_t) in the final phase's dC rounds, from the H and
    // dy rows loaded there, where a round's loaded rows take at most two
    // vectors per thread (every Q = 256 shape); otherwise in the head loop
    // (the C rows and H beside the u products spill at those shapes)
    static constexpr bool U_FIN = (P * (N / VEC) + NTH - 1) / NTH <= 2;
    // head loop: dy, G (and H, for u) of the head, the per-wave row sums and
    // the chunk's Gram tiles
    static constexpr int O_D = 0, O_G = Q * XR, O_H = O_G + P * GR;
    static constexpr int O_RW = O_H + (U_FIN ? 0 : P * GR);
    static constexpr int O_GM = O_RW + NW * Q * 4 / (int)sizeof(T);
    static constexpr int E_HEAD = O_GM + gram_tiles(QT) * 256;
    // final phase: Z rows and C^T (then G of HG heads), later B^T and H
    // heads per round of state terms: two keep a round's loaded rows beside the
    // dB / dC accumulators within the register file (four spilled), and below
    // Q = 256 keep the LDS of a workgroup within half a CU's
    static constexpr int HG = 2;
    static constexpr int O_BT = zoff(QT), E_FIN = O_BT + Q * BR, E_FS = O_BT + HG * P * GR;
    static constexpr int E_U = cmax(E_HEAD, cmax(E_FIN, E_FS));
    static constexpr size_t LDS =
        (size_t)E_U * sizeof(T) + (size_t)Q * 20 + (size_t)NW * 16 + 64;
    static_assert(QT % 2 == 0 && P % KS == 0 && N % KS == 0, "shape");
};

template <typename T, int P, int N, int Q>
__global__ void __launch_bounds__(Q / 32 * 64, 2) k_chunk_bwd_hb(
    Dims d, SegTab tab, int hbs, const T* __restrict__ xc, const T* __restrict__ dy,
    const T* __restrict__ gramT, const float* __restrict__ Dp,
    const float* __restrict__ dt_ws, const float* __restrict__ cs_ws,
    const int32_t* __restrict__ seq, const T* __restrict__ gpn, const T* __restrict__ hpn,
    T* __restrict__ dv,
    T* __restrict__ dbcp, float* __restrict__ rpart, float* __restrict__ tokp,
    float* __restrict__ red4, float* __restrict__ dotgh) {
    typedef ChunkBwdHB<T, P, N, Q> K;
    typedef Mma<T> M;
    typedef typename M::Frag Frag;
    typedef typename M::Elem E;
    constexpr int SL = K::SL, KS = K::KS, VEC = K::VEC, NW = K::NW, NTH = K::NTH, QT = K::QT;
    constexpr int TPK = K::TPK, NKS = K::NKS, NB = K::NB, MAXA = K::MAXA;
    constexpr int PT = K::PT, NT = K::NT, KP = K::KP, KN = K::KN, XR = K::XR;
    typedef T vt __attribute__((ext_vector_type(VEC)));
    typedef T t4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) T U[K::E_U];
    T* const sD = U + K::O_D;                   // dy of the current head [Q][XR]
    T* const sG = U + K::O_G;                   // exit gradient G [P][GR]
    T* const sH = U + K::O_H;                   // entering state H [P][GR] (u in the head loop)
    float* const s_rw = (float*)(U + K::O_RW);  // per-wave row sums of F [NW][Q]
    T* const sGm = U + K::O_GM;                 // the chunk's Gram tiles (head loop)
    T* const sZ = U;                            // final phase: Z rows, strip per row tile
    T* const sBT = U + K::O_BT;                 // final phase: C rows, then B rows [Q][BR]
    constexpr int GR = K::GR, BR = K::BR;
    __shared__ __attribute__((aligned(16))) float scs[Q];
    __shared__ __attribute__((aligned(16))) float sdt[Q];
    __shared__ __attribute__((aligned(16))) float sea[Q];  // exp(cs_t - F(t))
    __shared__ __attribute__((aligned(16))) float seb[Q];  // exp(L(t) - cs_t)
    __shared__ __attribute__((aligned(16))) int ssq[Q];
    // per-wave parts of dy . x and <G, H> of a head, by head parity (a head's are
    // summed after the next head's first barrier, while the next head writes
    // its own)
    __shared__ float s_dd[2][NW];
    __shared__ float s_gh[2][NW];

    // block -> (head block, chunk, row); the head blocks of a chunk are adjacent
    // items, and consecutive items go to one XCD
    const int nhb = d.H / hbs;
    int hbi, cm;
    int64_t b;
    {
        constexpr int NXCD = 8;
        const int64_t n = gridDim.x, i = blockIdx.x;
        const int64_t item = (n % NXCD == 0) ? (i % NXCD) * (n / NXCD) + i / NXCD : i;
        hbi = (int)(item % nhb);
        const int64_t rest = item / nhb;
        cm = (int)(rest % d.nchunk);
        b = rest / d.nchunk;
    }
    const int wave = wave_id(), lane = threadIdx.x % 64, lr = lane % 16, lg = lane / 16;
    const int h0 = hbi * hbs;
    const int g = h0 / d.hpg;
    const int64_t rb = b * d.L, t0 = (int64_t)cm * Q;
    const int64_t HPd = (int64_t)d.H * P;
    const int kseg = seg_of_chunk(tab, cm, Q);
    const int64_t s0 = tab.start[kseg];
    const int64_t pred = seg_pred_token(tab, kseg);
    const int64_t refc = t0 > s0 ? t0 - 1 : (pred >= 0 ? pred : s0);
    const int seq_refc = seq ? seq[rb + refc] : 0;
    const int seq_e = seq ? seq[rb + t0 + Q - 1] : 0;
    const bool split = seq && seq[rb + t0] != seq_e;
    const int64_t boff = HPd + (int64_t)g * N;
    const int64_t coff = HPd + (int64_t)d.G * N + (int64_t)g * N;
    const int64_t cg = ((int64_t)b * d.nchunk + cm) * d.G + g;
    const int j0 = wave, j1 = QT - 1 - wave;  // the wave's tiles
    const int ks0 = j0 / TPK, ks1 = j1 / TPK;  // first k step of each as a column
    const int n1 = NKS - ks1;                  // k steps of column j1
    auto st_of = [&](int h) { return (((int64_t)b * d.nchunk + cm) * d.H + h) * (int64_t)(P * N); };
    auto hl_of = [&](int h) { return ((int64_t)b * d.H + h) * d.L + t0; };
    const uint32_t Cu = (uint32_t)d.C;  // token row pitch of xBC (32-bit lane offsets)

    // ---- staging of dy, G and H of one head (registers, then LDS; H only for
    // <G, H> unless u is formed in the head loop), and the x
    // rows of the wave's columns j0, j1 (registers, in KPermRow order)
    constexpr int V_X = (Q * (P / VEC) + NTH - 1) / NTH;
    constexpr int V_S = (P * (N / VEC) + NTH - 1) / NTH;
    vt rd[V_X], rg[V_S], rh[V_S];
    Frag xf[2][KP];
    float rcs = 0.f, rdt = 0.f;  // cumulative sum and dt of token threadIdx.x (< Q)
    // tid: threadIdx.x plus the head's opaque zero (below), so that the lane
    // offsets are recomputed per head instead of held across the head loop
    auto fetch = [&](int h, int tid) {
        const int64_t so = st_of(h);
        if (tid < Q) {
            rcs = *at32(cs_ws + hl_of(h), tid);
            rdt = *at32(dt_ws + hl_of(h), tid);
        }
        const T* const dyh = dy + (rb + t0) * HPd + (int64_t)h * P;
#pragma unroll
        for (int q = 0; q < V_X; ++q) {
            const int idx = tid + q * NTH;
            if (V_X * NTH == Q * (P / VEC) || idx < Q * (P / VEC)) {
                const int j = idx / (P / VEC), pv = idx % (P / VEC);
                rd[q] = *(const vt*)at32(dyh, (uint32_t)(j * HPd + pv * VEC));
            }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int kp = 0; kp < KP; ++kp)
                xf[c][kp] = KPermRow<T>::load(
                    xc + (rb + t0 + (c == 0 ? j0 : j1) * 16 + lr) * d.C + (int64_t)h * P + kp * KS, lg);
#pragma unroll
        for (int q = 0; q < V_S; ++q) {
            const int idx = threadIdx.x + q * NTH;
            if (idx < P * (N / VEC)) {
                rg[q] = *(const vt*)(gpn + so + (int64_t)idx * VEC);
                rh[q] = *(const vt*)(hpn + so + (int64_t)idx * VEC);
            }
        }
    };
    auto stash = [&](int tid, int par) {
#pragma unroll
        for (int q = 0; q < V_X; ++q) {
            const int idx = tid + q * NTH;
            if (V_X * NTH == Q * (P / VEC) || idx < Q * (P / VEC)) {
                const int j = idx / (P / VEC), pv = idx % (P / VEC);
                *(vt*)&sD[j * XR + pv * VEC] = rd[q];
            }
        }
        float gh = 0.f;  // this thread's part of <G, H>
#pragma unroll
        for (int q = 0; q < V_S; ++q) {
            const int idx = tid + q * NTH;
            if (V_S * NTH == P * (N / VEC) || idx < P * (N / VEC)) {
                const int p = idx / (N / VEC), nv = idx % (N / VEC);
                *(vt*)&sG[p * GR + nv * VEC] = rg[q];
                if constexpr (!K::U_FIN) *(vt*)&sH[p * GR + nv * VEC] = rh[q];
#pragma unroll
                for (int e = 0; e < VEC; ++e) gh += (float)rg[q][e] * (float)rh[q][e];
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) gh += __shfl_xor(gh, off, 64);
        if (tid % 64 == 0) s_gh[par][wave] = gh;
    };

    f32x4 Z[NB][TPK];
#pragma unroll
    for (int s = 0; s < NB; ++s)
#pragma unroll
        for (int it = 0; it < TPK; ++it) Z[s][it] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int j = threadIdx.x; j < Q; j += NTH) ssq[j] = seq ? seq[rb + t0 + j] : 0;
    {
        // the chunk's Gram tiles, read by every head's k steps (the first head's
        // barriers order these writes before the first read)
        // Every load of the thread before the first LDS write: a load followed
        // by its write in the loop would wait for it before the next is issued.
        const T* gsrc = gramT + cg * (int64_t)gram_tiles(QT) * 256;
        constexpr int NGV = gram_tiles(QT) * 256 / VEC, NGI = (NGV + NTH - 1) / NTH;
        vt gv[NGI];
#pragma unroll
        for (int q = 0; q < NGI; ++q) {
            const int idx = threadIdx.x + q * NTH;
            if (NGV % NTH == 0 || idx < NGV) gv[q] = *(const vt*)(gsrc + (int64_t)idx * VEC);
        }
#pragma unroll
        for (int q = 0; q < NGI; ++q) {
            const int idx = threadIdx.x + q * NTH;
            if (NGV % NTH == 0 || idx < NGV) *(vt*)&sGm[idx * VEC] = gv[q];
        }
    }

    // The end of head h (parity par), once every wave is past its k steps: the
    // token row sums of F (rpart; each thread then clears the s_rw entries it
    // read, for the next head), dy . x and <G, H>.
    auto finish_head = [&](int h, int par, int tid) {
        const int64_t hl = hl_of(h);
        for (int t = tid; t < Q; t += NTH) {
            float rsum = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                rsum += s_rw[w * Q + t];
                s_rw[w * Q + t] = 0.f;
            }
            *at32(rpart + hl, t) = rsum;
        }
        if (tid == 0) {
            float dd = 0.f, gh = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                dd += s_dd[par][w];
                gh += s_gh[par][w];
            }
            red4[((int64_t)b * d.nchunk + cm) * d.H + h] = dd;
            dotgh[((int64_t)b * d.nchunk + cm) * d.H + h] = gh;
        }
    };
    for (int j = threadIdx.x; j < NW * Q; j += NTH) s_rw[j] = 0.f;  // ordered by the first barrier
    for (int hh = 0; hh < hbs; ++hh) {
        const int h = h0 + hh;
        const int64_t hl = hl_of(h);
        // An opaque zero, new every head: lane-derived indices, masks, load
        // offsets and the Gram tile addresses depend on it, so they are
        // recomputed where they are used instead of being hoisted out of the
        // head loop (where they would hold registers for its whole length).
        int opq;
        asm volatile("s_mov_b32 %0, 0" : "=s"(opq));
        const int tid = (int)threadIdx.x + opq;
        fetch(h, tid);
        const int lane = tid % 64, lr = lane % 16, lg = lane / 16;
        // B rows of tile j1 (its column's state part); C rows of the wave's two
        // tiles where u is formed here
        Frag bfr[KN], cfr[2][KN];
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) {
            if constexpr (!K::U_FIN) {
                cfr[0][kn] = M::load(xc + (rb + t0 + j0 * 16 + lr) * d.C + coff + kn * KS + SL * lg);
                cfr[1][kn] = M::load(xc + (rb + t0 + j1 * 16 + lr) * d.C + coff + kn * KS + SL * lg);
            }
            bfr[kn] = M::load(xc + (rb + t0 + j1 * 16 + lr) * d.C + boff + kn * KS + SL * lg);
        }
        __syncthreads();  // the previous head is done with the LDS
        if (hh > 0) finish_head(h - 1, (hh - 1) & 1, tid);
        stash(tid, hh & 1);
        if (tid < Q) {  // loaded with the head's rows
            scs[tid] = rcs;
            sdt[tid] = rdt;
            // the factored decay's token factors (unused on the exact path), from
            // the cumulative sums at the first and last token of the token's
            // 16-token tile, which lanes of this wave hold (Q = NTH / 2: whole
            // waves take this branch)
            const float cf = __shfl(rcs, lane & ~15, 64), cl = __shfl(rcs, lane | 15, 64);
            sea[tid] = __expf(rcs - cf);
            seb[tid] = __expf(cl - rcs);
        }
        __syncthreads();
        // factored decay unless a sequence starts in the chunk or a tile's span
        // would leave the normal float range
        const bool exact = split || tile_span_wide<QT>(scs, lane);
        const float cs_e = scs[Q - 1];
        const float Dh = Dp[h];
        float ddp = 0.f;  // dy . x over the wave's tokens

        // u_i = f_i dy_i . (H C_i) for the wave's two tiles as rows, where it is
        // formed in the head loop (both tiles from each H fragment read)
        float u[2] = {0.f, 0.f};
        if constexpr (!K::U_FIN) {
            f32x4 ys[2][PT];
#pragma unroll
            for (int it = 0; it < 2; ++it)
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) ys[it][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kn = 0; kn < KN; ++kn)
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const Frag hf = M::load(&sH[(pt * 16 + lr) * GR + kn * KS + SL * lg]);
                    ys[0][pt] = M::mma(hf, cfr[0][kn], ys[0][pt]);
                    ys[1][pt] = M::mma(hf, cfr[1][kn], ys[1][pt]);
                }
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int i = (it == 0 ? j0 : j1) * 16 + lr;
                float up = 0.f;
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    float dyv[4];
                    load4(&sD[i * XR + pt * 16 + 4 * lg], dyv);
#pragma unroll
                    for (int r = 0; r < 4; ++r) up += dyv[r] * ys[it][pt][r];
                }
                const float f_i = (ssq[i] == seq_refc) ? __expf(scs[i]) : 0.f;
                u[it] = f_i * sum_groups(up);
            }
        }

        // ---- one column tile: its state part, its k steps, its outputs
        int jc = 0;
        float csj = 0.f, dtj = 0.f, e2j = 0.f, vj = 0.f, kacc = 0.f;
        // the column's tile factors exp(F_a - L_jc), a >= jc: lane a holds row
        // tile a's, read with readlane in the k steps
        float stc = 0.f;
        int sqj = 0;
        f32x4 acc[PT];
        Frag xB[KP];
        // element p = pt * 16 + 4 lg + r of the column's x row (this lane's row
        // j): KPermRow order puts it in slot (pt % TPK) * 4 + r of block pt / TPK
        auto xval = [&](int pt, int r) { return (float)xB[pt / TPK][(pt % TPK) * 4 + r]; };
        auto col_begin = [&](int jc_, const Frag (&bf)[KN], const Frag (&xq)[KP]) {
            jc = jc_;
            const int j = 16 * jc + lr;
            csj = scs[j];
            dtj = sdt[j];
            sqj = ssq[j];
            e2j = exact ? 0.f : seb[j];
            stc = (!exact && lane < QT && lane >= jc) ? __expf(scs[16 * lane] - scs[16 * jc + 15]) : 0.f;
            const float gj = (sqj == seq_e) ? __expf(cs_e - csj) : 0.f;
#pragma unroll
            for (int kp = 0; kp < KP; ++kp) xB[kp] = xq[kp];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kn = 0; kn < KN; ++kn)
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
                    acc[pt] = M::mma(M::load(&sG[(pt * 16 + lr) * GR + kn * KS + SL * lg]), bf[kn], acc[pt]);
            float vp = 0.f;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                acc[pt] *= gj;
#pragma unroll
                for (int r = 0; r < 4; ++r) vp += xval(pt, r) * acc[pt][r];
            }
            vj = dtj * sum_groups(vp);
            kacc = 0.f;
        };
        // k step ks of the current column, accumulating into Z slot z
        auto kstep = [&](f32x4 (&z)[TPK], int ks) {
            Frag sl;
#pragma unroll
            for (int it = 0; it < TPK; ++it) {
                const int a = ks * TPK + it;
                float dd[4] = {0.f, 0.f, 0.f, 0.f}, ss[4] = {0.f, 0.f, 0.f, 0.f};
                f32x4 w = f32x4{0.f, 0.f, 0.f, 0.f};
                const bool live = a >= jc;  // wave-uniform
                if (live) {
                    const t4 gv = *(const t4*)&sGm[gram_index(a, jc) * 256 + lane * 4];
#pragma unroll
                    for (int kp = 0; kp < KP; ++kp)
                        w = M::mma(KPermRow<T>::load(&sD[(16 * a + lr) * XR + kp * KS], lg), xB[kp], w);
                    const int ib = 16 * a + 4 * lg;
                    if (!exact) {
                        const float bj = __builtin_bit_cast(
                            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, stc), a)) * e2j;
                        const f32x4 ea = *(const f32x4*)&sea[ib];
#pragma unroll
                        for (int r = 0; r < 4; ++r) dd[r] = ea[r] * bj;
                        if (a == jc) {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (4 * lg + r < lr) dd[r] = 0.f;
                        }
                    } else {
                        const f32x4 ci = *(const f32x4*)&scs[ib];
                        const int4 si = *(const int4*)&ssq[ib];
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            dd[r] = (ib + r >= 16 * jc + lr && si[r] == sqj) ? __expf(ci[r] - csj) : 0.f;
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) ss[r] = (float)gv[r];
                }
                float fr[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float wd = w[r] * (dd[r] * dtj);
                    z[it][r] += wd;
                    fr[r] = ss[r] * wd;
                    kacc += fr[r];
                    sl[it * 4 + r] = (E)(ss[r] * dd[r]);
                }
                if (live) {
                    const float t = row_sums16(fr, lr);
                    if ((lr & 3) == 0) {
                        const int r = 2 * (lr >> 3) + ((lr >> 2) & 1);
                        s_rw[wave * Q + 16 * a + 4 * lg + r] += t;
                    }
                }
            }
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
                acc[pt] = M::mma(XT<T>::load(sD, XR, ks * KS, pt * 16, lane), sl, acc[pt]);
        };
        auto col_end = [&](float ui) {
            const int j = 16 * jc + lr;
            float qp = 0.f;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                float dyv[4];
                load4(&sD[j * XR + pt * 16 + 4 * lg], dyv);
                t4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float xv = xval(pt, r);
                    qp += xv * acc[pt][r];
                    o[r] = (T)(dtj * acc[pt][r] + Dh * dyv[r]);
                    ddp += dyv[r] * xv;
                }
                *(t4*)(dv + (rb + t0 + j) * HPd + (int64_t)h * P + pt * 16 + 4 * lg) = o;
            }
            const float qj = sum_groups(qp);
            const float Kj = sum_groups(kacc);
            if (lg == 0) {
                float* tp = tokp + (hl + j) * 4;
                // R_j (row sums) and u_j (the fourth float, from here or the
                // final phase) are added by the ddt assembly
                tp[0] = -Kj;
                if constexpr (!K::U_FIN) tp[3] = ui;
                tp[1] = qj;
                tp[2] = vj;
            }
        };

        // (scheduling barriers keep the unrolled k steps from being interleaved,
        // which would need more registers than Z leaves)
        col_begin(j1, bfr, xf[1]);
        Frag bf0[KN];  // B rows of tile j0, for its column start
#pragma unroll
        for (int kn = 0; kn < KN; ++kn)
            bf0[kn] = M::load(xc + (rb + t0 + j0 * 16 + lr) * d.C + boff + kn * KS + SL * lg);
#pragma unroll
        for (int m = 0; m < MAXA; ++m) {
            __builtin_amdgcn_sched_barrier(0);
            if (m < n1) kstep(Z[m], ks1 + m);
        }
        __builtin_amdgcn_sched_barrier(0);
        col_end(u[1]);
        col_begin(j0, bf0, xf[0]);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            __builtin_amdgcn_sched_barrier(0);
            if (ks >= ks0) kstep(Z[ks + 1], ks);
        }
        __builtin_amdgcn_sched_barrier(0);
        col_end(u[0]);

#pragma unroll
        for (int off = 32; off > 0; off >>= 1) ddp += __shfl_xor(ddp, off, 64);
        if (lane % 64 == 0) s_dd[hh & 1][wave] = ddp;
    }
    __syncthreads();  // every wave is past the last head's k steps
    finish_head(h0 + hbs - 1, (hbs - 1) & 1, threadIdx.x);

    // ================= dB and dC of the head block =================
    // dB first (Z from registers, then the exit-gradient terms), then dC (Z
    // rows from LDS, then the entering-state terms): one set of 2 x NT
    // accumulators is live at a time.
    int opq;
    asm volatile("s_mov_b32 %0, 0" : "=s"(opq));
    const int lane2 = threadIdx.x % 64 + opq, lr2 = lane2 % 16, lg2 = lane2 / 16;
    constexpr int V_T = (N * (Q / VEC) + NTH - 1) / NTH;
    // B or C rows of the chunk -> sBT [Q][BR]: every load of the thread before
    // the first LDS write (a load followed by its write would wait for it
    // before the next load is issued)
    auto stage_rows = [&](int64_t choff) {
        vt rv[V_T];
        const T* const src = xc + (rb + t0) * d.C + choff;
#pragma unroll
        for (int q = 0; q < V_T; ++q) {
            const int idx = threadIdx.x + q * NTH;
            if (V_T * NTH == Q * (N / VEC) || idx < Q * (N / VEC))
                rv[q] = *(const vt*)at32(src, (uint32_t)(idx / (N / VEC)) * Cu + (idx % (N / VEC)) * VEC);
        }
#pragma unroll
        for (int q = 0; q < V_T; ++q) {
            const int idx = threadIdx.x + q * NTH;
            if (V_T * NTH == Q * (N / VEC) || idx < Q * (N / VEC))
                *(vt*)&sBT[(idx / (N / VEC)) * BR + (idx % (N / VEC)) * VEC] = rv[q];
        }
    };
    T* const dbp = dbcp + (int64_t)hbi * 2 * N;
    const int64_t dbs = (int64_t)nhb * 2 * N;  // token stride of the partials
    f32x4 ab[2][NT];  // [tile j0 / j1][n tile], transposed ([n][token])
    auto ab_zero = [&]() {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) ab[c][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // lane ids are passed in: each part takes them from its own opaque zero, so
    // that the addresses derived from them are recomputed per part instead of
    // being held (and spilled) across the other part
    auto ab_store = [&](int part, int lr2, int lg2) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            T* o = dbp + (rb + t0 + (c == 0 ? j0 : j1) * 16 + lr2) * dbs + part * N;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                *(t4*)(o + nt * 16 + 4 * lg2) =
                    t4{(T)ab[c][nt][0], (T)ab[c][nt][1], (T)ab[c][nt][2], (T)ab[c][nt][3]};
        }
    };
    // the state terms of one part over the heads: ab[c] += S^T (scaled rows of
    // tile c), S = G (dB, rows of x scaled by dt g) or H (dC, rows of dy scaled
    // by f); HG heads per round, their S staged at sS as [p][n] rows and read
    // transposed (XT), the rows in the matching k order.  The dC part also
    // forms u_t = f_t dy_t . (H C_t) of every head for the wave's two tiles as
    // rows, from the same staged H and loaded dy rows, into the fourth float of
    // the token's partials (H C_t with H read as rows, the C rows held as
    // operands: the same for every head).
    constexpr int HG = K::HG;
    constexpr int V_GT = (P * (N / VEC) + NTH - 1) / NTH;
    auto state_terms = [&](bool dB, T* sS, int lane2, int lr2, int lg2) {
        Frag cfr[2][KN];
        if (!dB && K::U_FIN) {
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int kn = 0; kn < KN; ++kn)
                    cfr[c][kn] = M::load(xc + (rb + t0 + (c == 0 ? j0 : j1) * 16 + lr2) * d.C + coff +
                                         kn * KS + SL * lg2);
        }
        for (int hf = 0; hf < hbs; hf += HG) {
            vt rs[HG][V_GT];
            Frag rr[HG][2][KP];
            float sc[HG][2];
            // Every load of the round first, then the row scales from the loaded
            // cumulative sums: computed under each head's branch, a scale waited
            // for its head's loads before the next head's were issued.  Slots past
            // the block's last head repeat it and are not used.
            float cse_r[HG], cst_r[HG][2], dt_r[HG][2];
#pragma unroll
            for (int q = 0; q < HG; ++q) {
                const int h = h0 + min(hf + q, hbs - 1);
                const int64_t hl = hl_of(h), so = st_of(h);
                const T* src = (dB ? gpn : hpn) + so;
#pragma unroll
                for (int v = 0; v < V_GT; ++v) {
                    const int idx = threadIdx.x + v * NTH;
                    if (idx < P * (N / VEC)) rs[q][v] = *(const vt*)(src + (int64_t)idx * VEC);
                }
                cse_r[q] = cs_ws[hl + Q - 1];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int t = (c == 0 ? j0 : j1) * 16 + lr2;
#pragma unroll
                    for (int kp = 0; kp < KP; ++kp)
                        rr[q][c][kp] = dB ? KPermRow<T>::load(xc + (rb + t0) * d.C + (int64_t)h * P,
                                                              (uint32_t)t * Cu + kp * KS, lg2)
                                          : KPermRow<T>::load(dy + (rb + t0) * HPd + (int64_t)h * P,
                                                              (uint32_t)(t * HPd + kp * KS), lg2);
                    cst_r[q][c] = cs_ws[hl + t];
                    dt_r[q][c] = dB ? dt_ws[hl + t] : 0.f;
                }
            }
#pragma unroll
            for (int q = 0; q < HG; ++q)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int t = (c == 0 ? j0 : j1) * 16 + lr2;
                    sc[q][c] = dB ? ((ssq[t] == seq_e) ? dt_r[q][c] * __expf(cse_r[q] - cst_r[q][c]) : 0.f)
                                  : ((ssq[t] == seq_refc) ? __expf(cst_r[q][c]) : 0.f);
                }
            __syncthreads();  // the previous round's products are done with sS
#pragma unroll
            for (int q = 0; q < HG; ++q) {
                if (hf + q < hbs) {
#pragma unroll
                    for (int v = 0; v < V_GT; ++v) {
                        const int idx = threadIdx.x + v * NTH;
                        if (idx < P * (N / VEC)) {
                            const int p = idx / (N / VEC), nv = idx % (N / VEC);
                            *(vt*)&sS[q * P * GR + p * GR + nv * VEC] = rs[q][v];
                        }
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < HG; ++q) {
                if (hf + q < hbs) {
                    const T* sq_ = sS + q * P * GR;
#pragma unroll
                    for (int kp = 0; kp < KP; ++kp) {
                        // both tiles from each S fragment read
                        Frag sf[2];
#pragma unroll
                        for (int c = 0; c < 2; ++c)
#pragma unroll
                            for (int e = 0; e < SL; ++e) sf[c][e] = (E)((float)rr[q][c][kp][e] * sc[q][c]);
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) {
                            const Frag xs = XT<T>::load(sq_, GR, kp * KS, nt * 16, lane2);
                            ab[0][nt] = M::mma(xs, sf[0], ab[0][nt]);
                            ab[1][nt] = M::mma(xs, sf[1], ab[1][nt]);
                        }
                    }
                    if (!dB && K::U_FIN) {
                        // (both tiles from each H fragment read)
                        f32x4 ys[2][PT];
#pragma unroll
                        for (int c = 0; c < 2; ++c)
#pragma unroll
                            for (int pt = 0; pt < PT; ++pt) ys[c][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kn = 0; kn < KN; ++kn)
#pragma unroll
                            for (int pt = 0; pt < PT; ++pt) {
                                const Frag hr = M::load(&sq_[(pt * 16 + lr2) * GR + kn * KS + SL * lg2]);
                                ys[0][pt] = M::mma(hr, cfr[0][kn], ys[0][pt]);
                                ys[1][pt] = M::mma(hr, cfr[1][kn], ys[1][pt]);
                            }
                        const int64_t hl = hl_of(h0 + hf + q);
#pragma unroll
                        for (int c = 0; c < 2; ++c) {
                            // dy element p = pt 16 + 4 lg2 + r of the row sits in
                            // slot (pt % TPK) 4 + r of block pt / TPK (KPermRow)
                            float up = 0.f;
#pragma unroll
                            for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    up += (float)rr[q][c][pt / TPK][(pt % TPK) * 4 + r] * ys[c][pt][r];
                            const float u = sc[q][c] * sum_groups(up);
                            if (lg2 == 0) tokp[(hl + (c == 0 ? j0 : j1) * 16 + lr2) * 4 + 3] = u;
                        }
                    }
                }
            }
        }
    };

    __syncthreads();  // every wave is done with the head loop's LDS
    // Z into LDS as natural rows (strip per row tile) for dC; C rows for dB
    auto zstore = [&](const f32x4 (&z)[TPK], int jc, int ks) {
#pragma unroll
        for (int it = 0; it < TPK; ++it) {
            const int a = ks * TPK + it;
            T* st = sZ + K::zoff(a) + 16 * jc + lr2;
            const int zp = K::zpitch(a);
#pragma unroll
            for (int r = 0; r < 4; ++r) st[(4 * lg2 + r) * zp] = (T)z[it][r];
        }
    };
#pragma unroll
    for (int m = 0; m < MAXA; ++m)
        if (m < n1) zstore(Z[m], j1, ks1 + m);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
        if (ks >= ks0) zstore(Z[ks + 1], j0, ks);
    stage_rows(coff);
    __syncthreads();

    auto zfrag = [&](const f32x4 (&z)[TPK]) {
        Frag f;
#pragma unroll
        for (int it = 0; it < TPK; ++it)
#pragma unroll
            for (int r = 0; r < 4; ++r) f[it * 4 + r] = (E)z[it][r];
        return f;
    };
    // ---- dB^T [n][j] = sum_i C^T[n][i] Z[i][j] + state terms (C^T read transposed)
    ab_zero();
#pragma unroll
    for (int m = 0; m < MAXA; ++m) {
        if (m < n1) {
            const Frag zf = zfrag(Z[m]);
            const int ks = ks1 + m;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                ab[1][nt] = M::mma(XT<T>::load(sBT, BR, ks * KS, nt * 16, lane2), zf, ab[1][nt]);
        }
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        if (ks >= ks0) {
            const Frag zf = zfrag(Z[ks + 1]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                ab[0][nt] = M::mma(XT<T>::load(sBT, BR, ks * KS, nt * 16, lane2), zf, ab[0][nt]);
        }
    }
    state_terms(true, sBT, lane2, lr2, lg2);  // G goes where the C rows were (the Z rows stay)
    ab_store(0, lr2, lg2);

    // ---- dC^T [n][i] = sum_j B^T[n][j] Z[i][j] + state terms (B^T read transposed)
    __syncthreads();  // every wave is done with sBT
    int opq3;
    asm volatile("s_mov_b32 %0, 0" : "=s"(opq3));
    {
    const int lane2 = threadIdx.x % 64 + opq3, lr2 = lane2 % 16, lg2 = lane2 / 16;
    stage_rows(boff);
    __syncthreads();
    ab_zero();
    {
        // the row tiles j0 < j1 over their k steps, both from each B^T fragment
        // read while both have the step
        auto zrow = [&](int a, int ks) {
            const T* zr = sZ + K::zoff(a) + lr2 * K::zpitch(a);
            Frag zf;
            if constexpr (TPK == 2) {
                const t4 lo = *(const t4*)&zr[ks * KS + 4 * lg2];
                const t4 hi = *(const t4*)&zr[ks * KS + 16 + 4 * lg2];
                zf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            } else {
                zf = *(const Frag*)&zr[ks * KS + 4 * lg2];
            }
            return zf;
        };
        for (int ks = 0; ks <= j1 / TPK; ++ks) {
            const bool both = ks <= j0 / TPK;  // wave-uniform
            const Frag zf1 = zrow(j1, ks);
            const Frag zf0 = both ? zrow(j0, ks) : zf1;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const Frag xs = XT<T>::load(sBT, BR, ks * KS, nt * 16, lane2);
                if (both) ab[0][nt] = M::mma(xs, zf0, ab[0][nt]);
                ab[1][nt] = M::mma(xs, zf1, ab[1][nt]);
            }
        }
    }
    state_terms(false, sZ, lane2, lr2, lg2);  // H^T goes where the Z rows were (after the first sync)
    ab_store(1, lr2, lg2);
    }
}

}  // namespace ssd
