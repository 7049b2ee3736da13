// Backward of the conv1d + SSD state-passing path (gfx950, wave64, MFMA).
//
// Megatron-LM #6808 (first commit): the backward mirrors the forward with a
// reverse boundary scan and recomputes every sequence-length-sized
// intermediate instead of saving it.  Here:
//
//   summary phase (ssd_segment_bwd_summary)
//     conv recompute -> xBC_conv (+ a chunk-transposed copy of the B and C
//     channels, k_bc_transpose), dt/cumsum recompute (k_dt_prep), and the
//     reverse chunk walk (k_state_walk, backward mode) that leaves, per
//     segment, dL/dS_in of the segment's own outputs and its block decay, in
//     the same packed layout as the forward summary.
//   reverse boundary scan (ssd_boundary_scan, reverse = 1) -> the gradient of
//     every segment's final state.
//     It also recomputes the zero-initial-state entering state of every chunk
//     (forward walk, stored transposed).
//   chunk phase (ssd_segment_bwd_chunks): k_chunk_bwd, per chunk and head:
//     dx, dB, dC and ddt with the true entering state H + decay S_in and the
//     true exit gradient G + decay dS_out, written into the buffers the conv
//     backward consumes.
//   conv phase (ssd_conv1d_bwd): k_conv_bwd (SiLU' and the transposed conv,
//     with a right halo from the causal successor segment) and k_bwd_reduce
//     (deterministic parameter gradients).
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

#include "ssd_internal.h"
#include "state_walk.h"

namespace ssd {

__device__ __forceinline__ float softplus_b(float z) {
    return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
}

template <typename T> struct KPermB;
template <> struct KPermB<bf16> {
    __device__ static __forceinline__ bf16x8 load(const bf16* p) {
        const bf16x4 lo = *(const bf16x4*)p;
        const bf16x4 hi = *(const bf16x4*)(p + 16);
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
};
template <> struct KPermB<float> {
    __device__ static __forceinline__ f32x4 load(const float* p) { return *(const f32x4*)p; }
};

template <typename T>
__device__ __forceinline__ void load4(const T* p, float* o) {
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = (float)p[r];
}

// Sum over the four lane groups (lanes l, l^16, l^32, l^48 share a column).
__device__ __forceinline__ float sum_groups(float v) {
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

// ---------------------------------------------------------------------------
// B and C channels of one chunk, transposed to [part][n][token] (part 0 = B,
// 1 = C), so that operands needing the token dimension as the MFMA k index
// read them with contiguous loads.
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
                for (int e = 0; e < VEC; ++e) tile[(nv * VEC + e) * QP + jj] = v[e];
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
// Per (chunk, head, tile group): every wave owns one 16-token tile and computes,
// for its tokens j as sources, dx_j and dB_j (outputs i >= j) and, for its
// tokens i as outputs, dC_i (sources j <= i).  Chunks with more tiles than
// waves are split over TG = Q / (16 NW) workgroups.  Per-token partial sums for
// ddt go to the workspace; k_ddt assembles ddt per chunk.
template <typename T, int P, int N, int Q, int NW>
__global__ void __launch_bounds__(NW * 64) k_chunk_bwd(
    Dims d, SegTab tab, const T* __restrict__ xc, const T* __restrict__ bct,
    const T* __restrict__ dy, const float* __restrict__ Dp, const float* __restrict__ dt_ws,
    const float* __restrict__ cs_ws, const float* __restrict__ ctot,
    const int32_t* __restrict__ seq, const T* __restrict__ hstT, const T* __restrict__ gst,
    const float* __restrict__ S_in, const float* __restrict__ dS_out, float* __restrict__ dv,
    T* __restrict__ dbc, float* __restrict__ rpart, float* __restrict__ tokp,
    float* __restrict__ dotgh, float* __restrict__ red4) {
    typedef Mma<T> M;
    typedef typename M::Frag Frag;
    constexpr int SL = M::SL, KS = M::KS;
    constexpr int VEC = 16 / sizeof(T);
    constexpr int QP = Q + VEC;  // pitch of dYt rows
    constexpr int PP = P + VEC;  // pitch of [n][p] tiles
    constexpr int NP = N + VEC;  // pitch of [p][n] tiles
    constexpr int PT = P / 16, NT = N / 16, QT = Q / 16, KP = P / KS, KN = N / KS;
    constexpr int TG = QT / NW;
    static_assert(TG * NW == QT, "tiles must split evenly over the waves");
    __shared__ __attribute__((aligned(16))) T dYt[P * QP];
    __shared__ __attribute__((aligned(16))) T HT[N * PP];
    __shared__ __attribute__((aligned(16))) T Gs[P * NP];
    __shared__ __attribute__((aligned(16))) T GT[N * PP];
    __shared__ float scs[Q], sdt[Q];
    __shared__ int ssq[Q];
    __shared__ float s_rw[NW][Q];  // per-wave row sums of F (summed in a fixed order)
    __shared__ float s_red[NW][2];
    // One KS-token block of operands shared by all waves, staged once per block:
    // phase 1: C rows, dy rows, transposed C; phase 2: x rows, transposed B.
    constexpr int RPN = N + VEC, RPP = P + VEC, TPK = KS + VEC;
    // Two buffers: block k+1 is loaded from global memory into registers while
    // block k is computed, then written to the other buffer.
    __shared__ __attribute__((aligned(16))) T sRowN[2][KS * RPN];
    __shared__ __attribute__((aligned(16))) T sRowP[2][KS * RPP];
    __shared__ __attribute__((aligned(16))) T sTr[2][N * TPK];
    // staging work per thread (vectors of VEC elements)
    constexpr int NTH = NW * 64;
    constexpr int V_RN = (KS * (N / VEC) + NTH - 1) / NTH;
    constexpr int V_RP = (KS * (P / VEC) + NTH - 1) / NTH;
    constexpr int V_TR = (N * (KS / VEC) + NTH - 1) / NTH;
    __shared__ float s_pre, s_post;
    typedef T vt __attribute__((ext_vector_type(VEC)));

    const int cm = blockIdx.x, h = blockIdx.y;
    const int64_t b = blockIdx.z / TG;
    const int tg = blockIdx.z % TG;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, lr = lane % 16, lg = lane / 16;
    const int g = h / d.hpg;
    const int64_t rb = b * d.L, t0 = (int64_t)cm * Q;
    const int64_t HPd = (int64_t)d.H * P;
    const int k = seg_of_chunk(tab, cm, Q);
    const int64_t s0 = tab.start[k];
    const int nc = (int)(tab.len[k] / Q);
    const int c = (int)((t0 - s0) / Q);
    const int cseg0 = (int)(s0 / Q);
    const bool first = c == 0, last = c == nc - 1;
    const int64_t pred = seg_pred_token(tab, k);
    const int64_t segref = pred >= 0 ? pred : s0;
    const int64_t refc = first ? segref : t0 - 1;
    const int64_t segend = s0 + tab.len[k] - 1;
    const int seq_segref = seq ? seq[rb + segref] : 0;
    const int seq_refc = seq ? seq[rb + refc] : 0;
    const int seq_e = seq ? seq[rb + t0 + Q - 1] : 0;
    const int seq_segend = seq ? seq[rb + segend] : 0;
    const int64_t xoff = (int64_t)h * P, boff = HPd + (int64_t)g * N;
    const int64_t coff = HPd + (int64_t)d.G * N + (int64_t)g * N;
    const T* bctB = bct + ((((int64_t)b * d.nchunk + cm) * d.G + g) * 2 + 0) * (int64_t)N * Q;
    const T* bctC = bctB + (int64_t)N * Q;
    const int64_t st_off = (((int64_t)b * d.nchunk + cm) * d.H + h) * (P * N);
    const int64_t sg_off = (((int64_t)k * d.batch + b) * d.H + h) * (P * N);
    const int64_t hl = ((int64_t)b * d.H + h) * d.L + t0;  // (row, head) token base

    if (threadIdx.x == 0) {
        const float* ct = ctot + ((int64_t)b * d.H + h) * d.nchunk;
        float pre = 0.f, post = 0.f;
        for (int cc = 0; cc < c; ++cc) pre += ct[cseg0 + cc];
        for (int cc = c + 1; cc < nc; ++cc) post += ct[cseg0 + cc];
        s_pre = pre;
        s_post = post;
    }
    for (int idx = threadIdx.x; idx < Q * (P / VEC); idx += blockDim.x) {
        const int jj = idx / (P / VEC), pv = idx % (P / VEC);
        const vt v = *(const vt*)(dy + (rb + t0 + jj) * HPd + xoff + pv * VEC);
#pragma unroll
        for (int e = 0; e < VEC; ++e) dYt[(pv * VEC + e) * QP + jj] = v[e];
    }
    for (int j = threadIdx.x; j < Q; j += blockDim.x) {
        scs[j] = cs_ws[hl + j];
        sdt[j] = dt_ws[hl + j];
        ssq[j] = seq ? seq[rb + t0 + j] : 0;
    }
    for (int j = threadIdx.x; j < NW * Q; j += blockDim.x) (&s_rw[0][0])[j] = 0.f;
    for (int idx = threadIdx.x; idx < N * (P / VEC); idx += blockDim.x) {
        const int n = idx / (P / VEC), pv = idx % (P / VEC);
        vt v;
        if (first) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] = (T)0.f;
        } else {
            v = *(const vt*)(hstT + st_off + (int64_t)n * P + pv * VEC);
        }
        *(vt*)&HT[n * PP + pv * VEC] = v;
    }
    __syncthreads();
    // True entering state H = H_zero + exp(pre) S_in (while no sequence starts
    // between the segment start and the chunk), true exit gradient
    // G = G_zero + exp(post) dS_out (while none starts after the chunk).
    // Vector loads along n: 4 (fp32) or 8 (bf16) entries per step.
    const float hs = (seq_refc == seq_segref) ? expf(s_pre) : 0.f;
    const float gs = (seq_e == seq_segend) ? expf(s_post) : 0.f;
    float dot = 0.f;
    for (int idx = threadIdx.x; idx < P * (N / VEC); idx += blockDim.x) {
        const int p = idx / (N / VEC), n0 = (idx % (N / VEC)) * VEC;
        const int64_t o = (int64_t)p * N + n0;
        vt gz;
        if (last) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) gz[e] = (T)0.f;
        } else {
            gz = *(const vt*)(gst + st_off + o);
        }
        float so[VEC], si[VEC];
#pragma unroll
        for (int q = 0; q < VEC / 4; ++q) {
            const f32x4 a4 = *(const f32x4*)(dS_out + sg_off + o + 4 * q);
            const f32x4 b4 = *(const f32x4*)(S_in + sg_off + o + 4 * q);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                so[4 * q + e] = a4[e];
                si[4 * q + e] = b4[e];
            }
        }
        vt gv;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int n = n0 + e;
            const float gt = (float)gz[e] + gs * so[e];
            const float ht = (float)HT[n * PP + p] + hs * si[e];
            HT[n * PP + p] = (T)ht;
            GT[n * PP + p] = (T)gt;
            gv[e] = (T)gt;
            dot += gt * ht;
        }
        *(vt*)&Gs[p * NP + n0] = gv;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
    if (lane == 0) s_red[wave][0] = dot;
    __syncthreads();
    if (threadIdx.x == 0 && tg == 0) {
        float t = 0.f;
        for (int w = 0; w < NW; ++w) t += s_red[w][0];
        dotgh[((int64_t)b * d.nchunk + cm) * d.H + h] = t;  // <G_exit, H_enter>
    }

    const float cs_e = scs[Q - 1];
    const float Dh = Dp[h];
    float dD_part = 0.f;
    {
        const int it = tg * NW + wave;
        const int j0T = it * 16;
        const int tj = j0T + lr;  // this lane's token (column of every output tile)
        const int64_t trow = rb + t0 + tj;
        const float cs_j = scs[tj], dt_j = sdt[tj];
        const int sq_j = ssq[tj];
        const float g_j = (sq_j == seq_e) ? expf(cs_e - cs_j) : 0.f;
        const float f_j = (sq_j == seq_refc) ? expf(cs_j) : 0.f;
        const T* xrow = xc + trow * d.C + xoff + 4 * lg;   // x of token tj at rows p of a tile
        const T* dyrow = dy + trow * HPd + xoff + 4 * lg;  // dy likewise

        // ---- dx and dB of the tile's tokens (as sources j) ----
        Frag Bn[KN], Xn[KP];
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) Bn[kn] = M::load(xc + trow * d.C + boff + kn * KS + SL * lg);
#pragma unroll
        for (int kp = 0; kp < KP; ++kp) Xn[kp] = M::load(xc + trow * d.C + xoff + kp * KS + SL * lg);
        f32x4 adx[PT], adb[NT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            adx[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kn = 0; kn < KN; ++kn)
                adx[pt] = M::mma(M::load(&Gs[(pt * 16 + lr) * NP + kn * KS + SL * lg]), Bn[kn],
                                 adx[pt]);
            adx[pt] *= g_j;
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            adb[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kp = 0; kp < KP; ++kp)
                adb[nt] = M::mma(M::load(&GT[(nt * 16 + lr) * PP + kp * KS + SL * lg]), Xn[kp],
                                 adb[nt]);
            adb[nt] *= g_j;
        }
        // v_j: what source j adds, through the exit state, to every decay inside the chunk
        float vpart = 0.f;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            float xv[4];
            load4(xrow + pt * 16, xv);
#pragma unroll
            for (int r = 0; r < 4; ++r) vpart += xv[r] * adx[pt][r];
        }
        const float v_j = dt_j * sum_groups(vpart);
        // F[i][j] = (C_i.B_j)(dy_i.x_j) exp(cs_i - cs_j) dt_j [same sequence, i >= j]:
        // row sums R_i (over this tile's j) go to s_rw, column sums K_j stay in kacc.
        // Both come from the same fp32 products, so sum_{i>=t}(R_i - K_i) cancels
        // in fp32 and equals sum_{i>=t} sum_{j<t} F[i][j].
        float kacc = 0.f;
        // Lockstep over the i-blocks this workgroup needs; a wave computes only
        // for blocks that reach its tile (i >= j).
        const int ib_lo = ((tg * NW * 16) / KS) * KS;
        // phase-1 block loads: C rows, dy rows, transposed C
        auto fetch1 = [&](int i0, vt (&rn)[V_RN], vt (&rp)[V_RP], vt (&tr)[V_TR]) {
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
            for (int q = 0; q < V_TR; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < N * (KS / VEC)) {
                    const int n = idx / (KS / VEC), kv = idx % (KS / VEC);
                    tr[q] = *(const vt*)(bctC + (int64_t)n * Q + i0 + kv * VEC);
                }
            }
        };
        auto store1 = [&](int buf, const vt (&rn)[V_RN], const vt (&rp)[V_RP], const vt (&tr)[V_TR]) {
#pragma unroll
            for (int q = 0; q < V_RN; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < KS * (N / VEC))
                    *(vt*)&sRowN[buf][(idx / (N / VEC)) * RPN + (idx % (N / VEC)) * VEC] = rn[q];
            }
#pragma unroll
            for (int q = 0; q < V_RP; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < KS * (P / VEC))
                    *(vt*)&sRowP[buf][(idx / (P / VEC)) * RPP + (idx % (P / VEC)) * VEC] = rp[q];
            }
#pragma unroll
            for (int q = 0; q < V_TR; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < N * (KS / VEC))
                    *(vt*)&sTr[buf][(idx / (KS / VEC)) * TPK + (idx % (KS / VEC)) * VEC] = tr[q];
            }
        };
        {
            vt rn[V_RN], rp[V_RP], tr[V_TR];
            fetch1(ib_lo, rn, rp, tr);
            store1(0, rn, rp, tr);
        }
        __syncthreads();
        int buf = 0;
#pragma unroll 1
        for (int i0 = ib_lo; i0 < Q; i0 += KS, buf ^= 1) {
            const bool more = i0 + KS < Q;
            vt rn[V_RN], rp[V_RP], tr[V_TR];
            if (more) fetch1(i0 + KS, rn, rp, tr);
            if (i0 + KS - 1 >= j0T) {  // the block reaches this wave's tile (i >= j)
            float uv[SL], wv[SL];
#pragma unroll
            for (int st = 0; st < KS / 16; ++st) {
                const int is = i0 + st * 16;
                f32x4 ut = f32x4{0.f, 0.f, 0.f, 0.f}, wt = f32x4{0.f, 0.f, 0.f, 0.f};
                if (is + 15 >= j0T) {
#pragma unroll
                    for (int kn = 0; kn < KN; ++kn)
                        ut = M::mma(M::load(&sRowN[buf][(st * 16 + lr) * RPN + kn * KS + SL * lg]),
                                    Bn[kn], ut);
#pragma unroll
                    for (int kp = 0; kp < KP; ++kp)
                        wt = M::mma(M::load(&sRowP[buf][(st * 16 + lr) * RPP + kp * KS + SL * lg]),
                                    Xn[kp], wt);
                }
                float fr[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = is + 4 * lg + r;
                    float m = 0.f;
                    if (i >= tj && ssq[i] == sq_j) m = expf(scs[i] - cs_j);
                    uv[st * 4 + r] = ut[r] * m;
                    wv[st * 4 + r] = wt[r] * m;
                    fr[r] = ut[r] * wt[r] * m * dt_j;
                    kacc += fr[r];
                }
                if (is + 15 >= j0T) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float x = fr[r];
                        x += __shfl_xor(x, 1, 64);
                        x += __shfl_xor(x, 2, 64);
                        x += __shfl_xor(x, 4, 64);
                        x += __shfl_xor(x, 8, 64);
                        if (lr == 0) s_rw[wave][is + 4 * lg + r] += x;
                    }
                }
            }
            const Frag uf = M::from_f(uv), wf = M::from_f(wv);
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
                adx[pt] = M::mma(KPermB<T>::load(&dYt[(pt * 16 + lr) * QP + i0 + 4 * lg]), uf,
                                 adx[pt]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                adb[nt] = M::mma(KPermB<T>::load(&sTr[buf][(nt * 16 + lr) * TPK + 4 * lg]), wf,
                                 adb[nt]);
            }
            if (more) store1(buf ^ 1, rn, rp, tr);
            __syncthreads();
        }
        float qpart = 0.f;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            float xv[4], dyv[4];
            load4(xrow + pt * 16, xv);
            load4(dyrow + pt * 16, dyv);
            f32x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                qpart += xv[r] * adx[pt][r];
                o[r] = dt_j * adx[pt][r] + Dh * dyv[r];
                dD_part += dyv[r] * xv[r];
            }
            *(f32x4*)(dv + trow * d.C + xoff + pt * 16 + 4 * lg) = o;
        }
        const float q_j = sum_groups(qpart);
        T* dbrow = dbc + (trow * d.H + h) * (2 * N);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) dbrow[nt * 16 + 4 * lg + r] = (T)(adb[nt][r] * dt_j);

        // ---- dC of the tile's tokens (as outputs i) ----
        Frag Dn[KP];
#pragma unroll
        for (int kp = 0; kp < KP; ++kp) Dn[kp] = M::load(dy + trow * HPd + xoff + kp * KS + SL * lg);
        f32x4 adc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            adc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kp = 0; kp < KP; ++kp)
                adc[nt] = M::mma(M::load(&HT[(nt * 16 + lr) * PP + kp * KS + SL * lg]), Dn[kp],
                                 adc[nt]);
            adc[nt] *= f_j;
        }
        // u_i = C_i . (entering-state part of dC_i): what the entering state adds to
        // output i, dotted with dy_i
        float upart = 0.f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            float cv[4];
            load4(xc + trow * d.C + coff + nt * 16 + 4 * lg, cv);
#pragma unroll
            for (int r = 0; r < 4; ++r) upart += cv[r] * adc[nt][r];
        }
        const float u_j = sum_groups(upart);
        // Lockstep over the j-blocks up to this workgroup's last tile.
        const int jb_hi = (tg + 1) * NW * 16 - 1;
        // phase-2 block loads: x rows, transposed B (reusing the row/transpose buffers)
        auto fetch2 = [&](int j0, vt (&rp)[V_RP], vt (&tr)[V_TR]) {
#pragma unroll
            for (int q = 0; q < V_RP; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < KS * (P / VEC)) {
                    const int jj = idx / (P / VEC), pv = idx % (P / VEC);
                    rp[q] = *(const vt*)(xc + (rb + t0 + j0 + jj) * d.C + xoff + pv * VEC);
                }
            }
#pragma unroll
            for (int q = 0; q < V_TR; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < N * (KS / VEC)) {
                    const int n = idx / (KS / VEC), kv = idx % (KS / VEC);
                    tr[q] = *(const vt*)(bctB + (int64_t)n * Q + j0 + kv * VEC);
                }
            }
        };
        auto store2 = [&](int bf, const vt (&rp)[V_RP], const vt (&tr)[V_TR]) {
#pragma unroll
            for (int q = 0; q < V_RP; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < KS * (P / VEC))
                    *(vt*)&sRowP[bf][(idx / (P / VEC)) * RPP + (idx % (P / VEC)) * VEC] = rp[q];
            }
#pragma unroll
            for (int q = 0; q < V_TR; ++q) {
                const int idx = threadIdx.x + q * NTH;
                if (idx < N * (KS / VEC))
                    *(vt*)&sTr[bf][(idx / (KS / VEC)) * TPK + (idx % (KS / VEC)) * VEC] = tr[q];
            }
        };
        {
            vt rp[V_RP], tr[V_TR];
            fetch2(0, rp, tr);
            store2(0, rp, tr);
        }
        __syncthreads();
        buf = 0;
#pragma unroll 1
        for (int j0 = 0; j0 <= jb_hi; j0 += KS, buf ^= 1) {
            const bool more = j0 + KS <= jb_hi;
            vt rp[V_RP], tr[V_TR];
            if (more) fetch2(j0 + KS, rp, tr);
            if (j0 <= j0T) {  // the block reaches back to this wave's tile (j <= i)
            float vv[SL];
#pragma unroll
            for (int st = 0; st < KS / 16; ++st) {
                const int js = j0 + st * 16;
                f32x4 vt4 = f32x4{0.f, 0.f, 0.f, 0.f};
                if (js <= j0T) {
#pragma unroll
                    for (int kp = 0; kp < KP; ++kp)
                        vt4 = M::mma(M::load(&sRowP[buf][(st * 16 + lr) * RPP + kp * KS + SL * lg]),
                                     Dn[kp], vt4);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = js + 4 * lg + r;
                    float m = 0.f;
                    if (j <= tj && ssq[j] == sq_j) m = expf(cs_j - scs[j]) * sdt[j];
                    vv[st * 4 + r] = vt4[r] * m;
                }
            }
            const Frag vf = M::from_f(vv);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                adc[nt] = M::mma(KPermB<T>::load(&sTr[buf][(nt * 16 + lr) * TPK + 4 * lg]), vf,
                                 adc[nt]);
            }
            if (more) store2(buf ^ 1, rp, tr);
            __syncthreads();
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) dbrow[N + nt * 16 + 4 * lg + r] = (T)adc[nt][r];
        const float K_j = sum_groups(kacc);
        if (lg == 0) {
            float* tp = tokp + (hl + tj) * 4;
            tp[0] = u_j - K_j;  // R_i is added by k_ddt from the row sums
            tp[1] = q_j;
            tp[2] = v_j;
        }
    }

#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dD_part += __shfl_xor(dD_part, off, 64);
    __syncthreads();
    if (lane == 0) s_red[wave][1] = dD_part;
    for (int t = threadIdx.x; t < Q; t += blockDim.x) {
        float rsum = 0.f;
        for (int w = 0; w < NW; ++w) rsum += s_rw[w][t];
        rpart[(hl + t) * TG + tg] = rsum;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float dd = 0.f;
        for (int w = 0; w < NW; ++w) dd += s_red[w][1];
        red4[(((int64_t)b * d.nchunk + cm) * d.H + h) * TG + tg] = dd;
    }
}

// ---------------------------------------------------------------------------
// ddt per chunk and head (one wave):
//   dL/d(dt_t A) = sum_{i >= t in t's sequence run} (R_i - K_i + u_i)
//                  + sum_{j < t} v_j + exp(cs_end) <G_exit, H_enter>,
// exactly 0 at a token that starts a packed sequence; then
// ddt_t = q_t + A dL/d(dt_t A) and the chain through clamp and softplus.
template <typename T>
__global__ void __launch_bounds__(64) k_ddt(Dims d, SegTab tab, int TG,
                                           const T* __restrict__ dt_raw,
                                           const float* __restrict__ dt_bias,
                                           const float* __restrict__ A_log,
                                           const float* __restrict__ dt_ws,
                                           const float* __restrict__ cs_ws,
                                           const int32_t* __restrict__ seq,
                                           const float* __restrict__ rpart,
                                           const float* __restrict__ tokp,
                                           const float* __restrict__ dotgh,
                                           const float* __restrict__ red4, T* __restrict__ ddt_raw,
                                           float* __restrict__ red) {
    const int cm = blockIdx.x, h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int lane = threadIdx.x;
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
    auto sq = [&](int t) { return seq ? seq[rb + t0 + t] : 0; };

    // segmented suffix of s (runs end where the sequence changes), lanes hold
    // tokens lane*E .. lane*E+E-1
    float sl[4], run = 0.f;
    bool rs[4], cut_any = false;
#pragma unroll
    for (int e = 3; e >= 0; --e) {
        if (e < E) {
            const int t = lane * E + e;
            const bool cut = t < Q - 1 && sq(t + 1) != sq(t);
            if (cut) run = 0.f;
            cut_any = cut_any || cut;
            float s = tokp[(hl + t) * 4 + 0];
            for (int g = 0; g < TG; ++g) s += rpart[(hl + t) * TG + g];
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
            vrun += tokp[(hl + lane * E + e) * 4 + 2];
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
            const bool starts = t > 0 ? sq(t) != sq(t - 1) : sq(0) != seq_refc;
            const float dl = starts ? 0.f : sl[e] + (rs[e] ? 0.f : carry) + vbefore + vl[e] + const4;
            const float ddt = tokp[(hl + t) * 4 + 1] + A * dl;
            const float z = (float)dt_raw[(rb + t0 + t) * d.H + h] + bias;
            const float sp = softplus_b(z);
            const bool pass = sp >= d.dt_min && sp <= d.dt_max;
            const float gr = pass ? ddt / (1.f + expf(-z)) : 0.f;
            ddt_raw[(rb + t0 + t) * d.H + h] = (T)gr;
            s_db += gr;
            s_da += dt_ws[hl + t] * dl;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        s_db += __shfl_xor(s_db, off, 64);
        s_da += __shfl_xor(s_da, off, 64);
    }
    if (lane == 0) {
        float dd = 0.f;
        for (int g = 0; g < TG; ++g) dd += red4[(((int64_t)b * d.nchunk + cm) * d.H + h) * TG + g];
        float* rp = red + (((int64_t)b * d.nchunk + cm) * d.H + h) * 3;
        rp[0] = s_db;
        rp[1] = s_da;
        rp[2] = dd;
    }
}

// ---------------------------------------------------------------------------
// dB and dC of a group are the sums of its heads' contributions; written into
// the B and C channels of dv (the conv output gradient), coalesced along n.
template <typename T>
__global__ void __launch_bounds__(256) k_bc_headsum(Dims d, const T* __restrict__ dbc,
                                                   float* __restrict__ dv) {
    const int GN2 = 2 * d.G * d.N;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= d.batch * d.L * GN2) return;
    const int64_t tok = idx / GN2;
    const int o = (int)(idx % GN2);
    const int part = o / (d.G * d.N), gn = o % (d.G * d.N), g = gn / d.N, n = gn % d.N;
    const T* src = dbc + (tok * d.H + (int64_t)g * d.hpg) * (2 * d.N) + part * d.N + n;
    float s = 0.f;
    for (int hh = 0; hh < d.hpg; ++hh) s += (float)src[(int64_t)hh * 2 * d.N];
    dv[tok * d.C + (int64_t)d.H * d.P + o] = s;
}

// ---------------------------------------------------------------------------
// SiLU' and the transposed causal conv.  A tile of 64 tokens needs du for its
// own tokens and the W-1 that follow in causal order (the right halo, from the
// causal successor segment), and xBC for W-1 tokens before those (to rebuild
// the pre-activation).  dv holds the gradient of every conv output channel.  dconv_w is written per tile and reduced later.
template <typename T, int W>
__global__ void __launch_bounds__(256) k_conv_bwd(Dims d, SegTab tab, const T* __restrict__ xBC,
                                                 const float* __restrict__ w,
                                                 const int32_t* __restrict__ seq,
                                                 const float* __restrict__ dvall,
                                                 T* __restrict__ dxBC, float* __restrict__ dwp) {
    constexpr int TT = 64, CT = 128, VEC = 8, CV = CT / VEC;
    constexpr int R = TT + 2 * (W - 1);   // xBC rows: causal offsets -(W-1) .. TT+W-2
    constexpr int RD = TT + W - 1;        // du rows: causal offsets 0 .. TT+W-2
    typedef T vec_t __attribute__((ext_vector_type(8)));
    __shared__ __attribute__((aligned(16))) T xt[R * CT];
    __shared__ __attribute__((aligned(16))) float dus[RD * CT];
    __shared__ int64_t rowmem[R];
    __shared__ int rowseq[R];
    __shared__ float wred[4][CV][VEC * W];

    const int64_t b = blockIdx.z;
    const int tt = blockIdx.y;
    const int64_t t0 = (int64_t)tt * TT;
    const int c0 = blockIdx.x * CT;
    const int64_t rb = b * d.L;
    int k = 0;
    for (int i = 0; i < tab.n; ++i)
        if (t0 >= tab.start[i] && t0 < tab.start[i] + tab.len[i]) k = i;
    const int64_t s0 = tab.start[k], s1 = s0 + tab.len[k];

    for (int r = threadIdx.x; r < R; r += blockDim.x) {
        const int64_t m = t0 - (W - 1) + r;
        int64_t mem;
        if (m >= s0 && m < s1) mem = m;
        else if (m < s0) mem = k > 0 ? tab.start[k - 1] + tab.len[k - 1] - (s0 - m) : -1;
        else mem = k + 1 < tab.n ? tab.start[k + 1] + (m - s1) : -1;
        rowmem[r] = mem;
        rowseq[r] = (mem >= 0 && seq) ? seq[rb + mem] : 0;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < R * CV; idx += blockDim.x) {
        const int r = idx / CV, v = idx % CV;
        const int c = c0 + v * VEC;
        vec_t val;
        if (c < d.C && rowmem[r] >= 0) {
            val = *(const vec_t*)(xBC + (rb + rowmem[r]) * d.C + c);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) val[e] = (T)0.f;
        }
        *(vec_t*)(xt + r * CT + v * VEC) = val;
    }
    __syncthreads();

    const int v = threadIdx.x % CV;
    const int c = c0 + v * VEC;
    const bool active = c < d.C;
    float wr[VEC][W];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int kk = 0; kk < W; ++kk) wr[e][kk] = active ? w[(c + e) * W + kk] : 0.f;

    // du for causal offsets 0 .. TT+W-2 (LDS rows W-1 .. R-1)
    for (int idx = threadIdx.x; idx < RD * CV; idx += blockDim.x) {
        const int o = idx / CV;
        const int r = o + W - 1;
        float dv8[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) dv8[e] = 0.f;
        const int64_t mem = rowmem[r];
        if (active && mem >= 0) {
            const f32x4* src = (const f32x4*)(dvall + (rb + mem) * d.C + c);
            const f32x4 lo = src[0], hi = src[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dv8[e] = lo[e];
                dv8[e + 4] = hi[e];
            }
        }
        const int sq = rowseq[r];
        float u[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) u[e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < W; ++kk) {
            const int rr = r - (W - 1) + kk;
            if (rowmem[rr] >= 0 && rowseq[rr] == sq) {
                const vec_t xv = *(const vec_t*)(xt + rr * CT + v * VEC);
#pragma unroll
                for (int e = 0; e < VEC; ++e) u[e] += wr[e][kk] * (float)xv[e];
            }
        }
        f32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float sg = 1.f / (1.f + expf(-u[e]));
            const float g = (mem >= 0) ? dv8[e] * sg * (1.f + u[e] * (1.f - sg)) : 0.f;
            if (e < 4) lo[e] = g;
            else hi[e - 4] = g;
        }
        *(f32x4*)&dus[o * CT + v * VEC] = lo;
        *(f32x4*)&dus[o * CT + v * VEC + 4] = hi;
    }
    __syncthreads();

    float dw[VEC][W];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int kk = 0; kk < W; ++kk) dw[e][kk] = 0.f;
    for (int idx = threadIdx.x; idx < TT * CV; idx += blockDim.x) {
        const int o = idx / CV;   // output token offset (source s of the forward taps)
        const int rs = o + W - 1;  // its LDS row
        const int sq = rowseq[rs];
        float acc[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < W; ++kk) {
            const int ot = o + (W - 1) - kk;  // forward output token that read s with tap kk
            const int rt = ot + W - 1;
            if (rowmem[rt] >= 0 && rowseq[rt] == sq) {
                const f32x4 lo = *(const f32x4*)&dus[ot * CT + v * VEC];
                const f32x4 hi = *(const f32x4*)&dus[ot * CT + v * VEC + 4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[e] += wr[e][kk] * lo[e];
                    acc[e + 4] += wr[e + 4][kk] * hi[e];
                }
            }
        }
        vec_t outv;
#pragma unroll
        for (int e = 0; e < VEC; ++e) outv[e] = (T)acc[e];
        // dconv_w: forward output o read source o-(W-1)+kk with tap kk
        const f32x4 dlo = *(const f32x4*)&dus[o * CT + v * VEC];
        const f32x4 dhi = *(const f32x4*)&dus[o * CT + v * VEC + 4];
#pragma unroll
        for (int kk = 0; kk < W; ++kk) {
            const int rr = o + kk;
            if (rowmem[rr] >= 0 && rowseq[rr] == sq) {
                const vec_t xv = *(const vec_t*)(xt + rr * CT + v * VEC);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dw[e][kk] += dlo[e] * (float)xv[e];
                    dw[e + 4][kk] += dhi[e] * (float)xv[e + 4];
                }
            }
        }
        if (active) *(vec_t*)(dxBC + (rb + t0 + o) * d.C + c) = outv;
    }
    // reduce dw over the 16 threads sharing this channel vector: lanes l, l^16,
    // l^32, l^48 of a wave by shuffles, then the four waves through LDS.
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int kk = 0; kk < W; ++kk) {
            float x = dw[e][kk];
            x += __shfl_xor(x, 16, 64);
            x += __shfl_xor(x, 32, 64);
            dw[e][kk] = x;
        }
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    if (lane < CV) {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
#pragma unroll
            for (int kk = 0; kk < W; ++kk) wred[wave][lane][e * W + kk] = dw[e][kk];
    }
    __syncthreads();
    for (int q = threadIdx.x; q < CV * VEC * W; q += blockDim.x) {
        const int vv = q / (VEC * W), j = q % (VEC * W);
        const float sum = wred[0][vv][j] + wred[1][vv][j] + wred[2][vv][j] + wred[3][vv][j];
        const int cc = c0 + vv * VEC + j / W;
        if (cc < d.C) dwp[(((int64_t)b * (d.L / TT) + tt) * d.C + cc) * W + (j % W)] = sum;
    }
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
    float s = 0.f;
    if (o < CW) {
        const int64_t ntot = d.batch * (d.L / 64);
        for (int64_t t = gq; t < ntot; t += 8) s += dwp[t * CW + o];
    } else if (o < nout) {
        const int j = o - CW, h = j / 3, q = j % 3;
        const int64_t ntot = d.batch * d.nchunk;
        for (int64_t bc = gq; bc < ntot; bc += 8) s += red[(bc * d.H + h) * 3 + q];
    }
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

template <typename T, int P, int N, int Q>
constexpr size_t chunk_bwd_lds() {
    constexpr size_t V = 16 / sizeof(T);
    constexpr size_t NW = Q >= 128 ? 8 : 4;
    constexpr size_t KS = sizeof(T) == 2 ? 32 : 16;
    return sizeof(T) * ((size_t)P * (Q + V) + 2 * (size_t)N * (P + V) + (size_t)P * (N + V) +
                        2 * (KS * (N + V) + KS * (P + V) + (size_t)N * (KS + V))) +
           (size_t)Q * 12 + NW * Q * 4 + 256;
}
constexpr size_t BWD_LDS_LIMIT = 160 * 1024;

template <typename T, int P, int N>
static bool bwd_shape_ok(int Q) {
    if (Q == 64) return chunk_bwd_lds<T, P, N, 64>() <= BWD_LDS_LIMIT;
    if (Q == 128) return chunk_bwd_lds<T, P, N, 128>() <= BWD_LDS_LIMIT;
    if (Q == 256) return chunk_bwd_lds<T, P, N, 256>() <= BWD_LDS_LIMIT;
    return false;
}

template <typename T, int P, int N, int Q>
static void launch_chunk_bwd(const Dims& d, const SegTab& t, const BwdArgs& a, const BwdWs& L,
                             char* ws, hipStream_t s) {
    if constexpr (chunk_bwd_lds<T, P, N, Q>() <= BWD_LDS_LIMIT) {
        constexpr int NW = Q >= 128 ? 8 : 4;
        constexpr int TG = Q / 16 / NW;
        hipLaunchKernelGGL((k_chunk_bwd<T, P, N, Q, NW>),
                           dim3((unsigned)d.nchunk, (unsigned)d.H, (unsigned)(d.batch * TG)),
                           dim3(NW * 64), 0, s, d, t, (const T*)(ws + L.xc),
                           (const T*)(ws + L.bct), (const T*)a.dy, a.D, (const float*)(ws + L.dt),
                           (const float*)(ws + L.cs), (const float*)(ws + L.ctot), a.seq,
                           (const T*)(ws + L.hstT), (const T*)(ws + L.gst), a.S_in, a.dS_out,
                           (float*)(ws + L.dv), (T*)(ws + L.dbc), (float*)(ws + L.rpart),
                           (float*)(ws + L.tokp), (float*)(ws + L.dotgh), (float*)(ws + L.red4));
        hipLaunchKernelGGL((k_ddt<T>),
                           dim3((unsigned)d.nchunk, (unsigned)d.H, (unsigned)d.batch), dim3(64), 0,
                           s, d, t, TG, (const T*)a.dt_raw, a.dt_bias, a.A_log,
                           (const float*)(ws + L.dt), (const float*)(ws + L.cs), a.seq,
                           (const float*)(ws + L.rpart), (const float*)(ws + L.tokp),
                           (const float*)(ws + L.dotgh), (const float*)(ws + L.red4),
                           (T*)a.ddt_raw, (float*)(ws + L.red));
    }
}

template <typename T, int W>
static void launch_conv_bwd_w(const Dims& d, const SegTab& t, const BwdArgs& a, const BwdWs& L,
                              char* ws, hipStream_t s) {
    dim3 grid((d.C + 127) / 128, (unsigned)(d.L / 64), (unsigned)d.batch);
    hipLaunchKernelGGL((k_conv_bwd<T, W>), grid, dim3(256), 0, s, d, t, (const T*)a.xBC, a.conv_w,
                       a.seq, (const float*)(ws + L.dv), (T*)a.dxBC,
                       (float*)(ws + L.dwp));
}

template <typename T>
static void launch_conv_bwd(const Dims& d, const SegTab& t, const BwdArgs& a, const BwdWs& L,
                            char* ws, hipStream_t s) {
    switch (d.W) {
        case 1: launch_conv_bwd_w<T, 1>(d, t, a, L, ws, s); break;
        case 2: launch_conv_bwd_w<T, 2>(d, t, a, L, ws, s); break;
        case 3: launch_conv_bwd_w<T, 3>(d, t, a, L, ws, s); break;
        case 4: launch_conv_bwd_w<T, 4>(d, t, a, L, ws, s); break;
        case 5: launch_conv_bwd_w<T, 5>(d, t, a, L, ws, s); break;
        case 6: launch_conv_bwd_w<T, 6>(d, t, a, L, ws, s); break;
        case 7: launch_conv_bwd_w<T, 7>(d, t, a, L, ws, s); break;
        default: launch_conv_bwd_w<T, 8>(d, t, a, L, ws, s); break;
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
    hipLaunchKernelGGL(k_bc_transpose<T>, dim3((unsigned)d.nchunk, (unsigned)d.G, (unsigned)d.batch),
                       dim3(256), 0, s, d, (const T*)xc, (T*)(ws + L.bct));
    launch_dt_prep(d, std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32, a.dt_raw, a.dt_bias,
                   a.A_log, a.seq, (float*)(ws + L.dt), (float*)(ws + L.cs),
                   (float*)(ws + L.ctot), s);
    hipLaunchKernelGGL((k_state_walk<T, P, N, WALK_FWD_NP>),
                       dim3((unsigned)d.H, (unsigned)d.nseg, (unsigned)d.batch), dim3(256), 0, s,
                       d, t, (const T*)xc, (int64_t)d.C, (const T*)xc, (int64_t)d.H * P,
                       (const float*)(ws + L.dt), (const float*)(ws + L.cs), a.seq,
                       (T*)(ws + L.hstT), (float*)nullptr);
    hipLaunchKernelGGL((k_state_walk<T, P, N, WALK_BWD_PN>),
                       dim3((unsigned)d.H, (unsigned)d.nseg, (unsigned)d.batch), dim3(256), 0, s,
                       d, t, (const T*)a.dy, (int64_t)d.H * P, (const T*)xc,
                       (int64_t)d.H * P + (int64_t)d.G * N, (const float*)(ws + L.dt),
                       (const float*)(ws + L.cs), a.seq, (T*)(ws + L.gst), summary);
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
static void conv_bwd_t(const Dims& d, const SegTab& t, const BwdArgs& a, void* ws_,
                       hipStream_t s) {
    const BwdWs L = bwd_ws_layout(d, std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32);
    char* ws = (char*)ws_;
    const int64_t nbc = d.batch * d.L * 2 * d.G * d.N;
    hipLaunchKernelGGL(k_bc_headsum<T>, dim3((unsigned)((nbc + 255) / 256)), dim3(256), 0, s, d,
                       (const T*)(ws + L.dbc), (float*)(ws + L.dv));
    launch_conv_bwd<T>(d, t, a, L, ws, s);
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

hipError_t launch_conv1d_bwd(const Dims& d, const SegTab& t, int act, const BwdArgs& a, void* ws,
                             hipStream_t s) {
    if (act == SSD_BF16) conv_bwd_t<bf16>(d, t, a, ws, s);
    else conv_bwd_t<float>(d, t, a, ws, s);
    return hipGetLastError();
}

}  // namespace ssd
