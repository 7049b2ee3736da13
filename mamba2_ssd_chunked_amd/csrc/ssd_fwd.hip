// Segment-local SSD forward and the correction pass (gfx950, wave64, MFMA).
//
// Kernels, in launch order:
//   k_dt_prep      dt = clamp(softplus(dt_raw + dt_bias)), l = dt*A, and the
//                  chunk-local inclusive cumsum cs of l, per (row, head, chunk).
//   k_walk_gram    (walk_gram.h) the state walk below and the group Gram tiles
//                  (gram.h) in one launch; shapes it does not fit launch the
//                  Gram tiles with dt prep (k_gram_dt), then k_state_walk.
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
//   k_chunk_y      one workgroup per (row, chunk, head): the intra-chunk term
//                  (C B^T masked by exp(cs_i - cs_j) dt_j, j <= i, same sequence)
//                  times X, plus the inter-chunk term exp(cs_i) C_i H_c.  Either
//                  into the zero-initial-state output y_zero (FP32), or, given
//                  the boundary scan's S_in, straight into y with the true
//                  entering state and D x (the correction folded in).
//   k_apply_init   y = y_zero + exp(cs_seg_i) C_i S_in^T + D x_i (the correction
//                  of #6808 once the boundary scan has produced S_in), for
//                  callers that keep y_zero.
#include <type_traits>

#include "conv_fused.h"
#include "dt_prep.h"
#include "gram.h"
#include "ssd_internal.h"
#include "state_walk.h"
#include "walk_gram.h"
#include "xt.h"

namespace ssd {

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
// dt prep on its own, DTB heads of one chunk per workgroup.
template <typename T>
__global__ void __launch_bounds__(256) k_dt_prep(Dims d, const T* __restrict__ dt_raw,
                                                const float* __restrict__ dt_bias,
                                                const float* __restrict__ A_log,
                                                const int32_t* __restrict__ seq,
                                                float* __restrict__ dt_ws, float* __restrict__ cs_ws,
                                                float* __restrict__ ctot) {
    __shared__ DtLds sm;
    dt_prep_block<T>(d, dt_raw, dt_bias, A_log, seq, dt_ws, cs_ws, ctot, blockIdx.x,
                     blockIdx.y * DTB, blockIdx.z, sm);
}

// ---------------------------------------------------------------------------
// Output pass, one workgroup per (row, chunk, head) with NW = Q/32 waves.  Wave
// w owns the 16-token output tiles a0 = w and a1 = QT-1-w, so every wave meets
// the same number of causal (source tile <= output tile) pairs.
//
// For output token i and source token j <= i of the same packed sequence the
// intra-chunk weight is (C_i . B_j) exp(cs_i - cs_j) dt_j.  C_i . B_j comes
// from the group's Gram tiles (gram.h); every load the workgroup needs (X of the
// head in its natural layout, the entering state, the Gram tiles of the wave's
// two output tiles, the decays) is issued up front, so one memory latency is
// paid per workgroup and about 58 KB of LDS lets two workgroups share a CU.
// In a chunk without a sequence start the decay is factored through the
// 16-token tiles a of i and b of j, with F and L the cumulative sums at a
// tile's first and last token:
//   exp(cs_i - cs_j) = exp(cs_i - F_a) exp(F_a - L_b) exp(L_b - cs_j),
// which needs no transcendental in the inner loop; chunks with a sequence start,
// or a tile whose decay span would leave the normal float range, take the exact
// per-element path.  The weighted Gram tile feeds the next MFMA as its k operand.
//
// FINAL = false: y_zero = intra-chunk term + exp(cs_i) C_i H_c^T with H_c the
//                zero-initial-state entering state (none for a segment's first
//                chunk), FP32, no D term.
// FINAL = true:  y = the same with H_c replaced by the true entering state
//                H_c + eps S_in (eps = exp(sum of dt A from the segment start to
//                the chunk), 0 once a packed sequence started in between), plus
//                D x, in the activation type.
// With spans (SpanPlan), H_c and eps run from the chunk's span start and S_st
// holds the state entering each span (zero-initial-state or true): the
// entering state is H_c + eps S_st[span].  This is the zero-state output and
//                the correction pass of #6808 in one pass: y_zero never goes to
//                memory and x and C are read once.  D is folded into the
//                diagonal of the weight matrix (j = i), so D x comes out of the
//                same MFMA.
template <typename T, int P, int N, int Q, bool FINAL, bool XC>
__global__ void __launch_bounds__(Q / 32 * 64, (P <= 64 ? 4 : 1)) k_chunk_y(Dims d, SegTab tab, const T* __restrict__ xc,
                                                        const T* __restrict__ bc, int64_t bstr,
                                                        const float* __restrict__ conv_w,
                                                        const T* __restrict__ gram,
                                                        const float* __restrict__ dt_ws,
                                                        const float* __restrict__ cs_ws,
                                                        const float* __restrict__ ctot,
                                                        const int32_t* __restrict__ seq,
                                                        const T* __restrict__ hst,
                                                        SpanPlan sp,
                                                        const float* __restrict__ S_st,
                                                        const float* __restrict__ Dp,
                                                        float* __restrict__ y_zero,
                                                        T* __restrict__ y) {
    typedef Mma<T> M;
    typedef typename M::Frag Frag;
    typedef typename M::Elem E;
    constexpr int SL = M::SL, KS = M::KS;
    constexpr int VEC = 16 / sizeof(T);
    constexpr int NW = Q / 32, NTH = NW * 64, QT = Q / 16;
    constexpr int PT = P / 16, NKF = N / KS;
    constexpr int XR = P + VEC;  // X row pitch (16-byte aligned rows for the vector stores)
    constexpr int HP = N + VEC;  // entering-state row pitch
    constexpr int YP = P + VEC;  // output staging pitch
    typedef T vt __attribute__((ext_vector_type(VEC)));
    typedef T t4 __attribute__((ext_vector_type(4)));
    // X [Q][XR] and the entering state [P][HP]; the output staging of the FINAL
    // variant reuses the same memory once the MFMAs are done
    constexpr int E_X = Q * XR, E_H = P * HP, E_Y = 2 * NW * 16 * YP;
    __shared__ __attribute__((aligned(16))) T U[E_X + E_H > E_Y ? E_X + E_H : E_Y];
    T* const sX = U;
    T* const sH = U + E_X;
    T* const sY = U;
    __shared__ __attribute__((aligned(16))) float scs[Q];
    __shared__ __attribute__((aligned(16))) float sdt[Q];
    __shared__ __attribute__((aligned(16))) float sea[Q];  // exp(cs_t - F(t))
    __shared__ __attribute__((aligned(16))) float seb[Q];  // exp(L(t) - cs_t) dt_t
    __shared__ __attribute__((aligned(16))) int ssq[Q];

    const ChunkHead ch = chunk_head_of_block(d);
    const int cm = ch.cm, h = ch.h;
    const int64_t b = ch.b;
    const int wave = wave_id(), lane = threadIdx.x % 64, lr = lane % 16, lg = lane / 16;
    const int g = h / d.hpg;
    const int64_t rb = b * d.L, t0 = (int64_t)cm * Q;
    const int k = seg_of_chunk(tab, cm, Q);
    const int64_t s0 = tab.start[k];
    const bool first = (t0 == s0);  // first chunk of the segment
    // the chunk's span (SpanPlan): the walk left the zero-state entering state of
    // every chunk but a span's first; S_st holds the state entering each span
    const int cseg0 = (int)(s0 / Q);
    const int jsp = (cm - cseg0) / sp.cps;
    const int cspan0 = cseg0 + jsp * sp.cps;
    const bool sfirst = (cm == cspan0);  // first chunk of its span
    const bool use_st = S_st != nullptr && (FINAL || jsp > 0);
    const int64_t pred = seg_pred_token(tab, k);
    // sequence of the state entering the segment, of the one entering the
    // chunk, and of the one entering the chunk's span
    const int seq_ref = seq ? seq[rb + (pred >= 0 ? pred : s0)] : 0;
    const int seq_prev = (seq && !first) ? seq[rb + t0 - 1] : seq_ref;
    const int seq_span = (seq && jsp > 0) ? seq[rb + (int64_t)cspan0 * Q - 1] : seq_ref;
    const bool split = seq && seq[rb + t0] != seq[rb + t0 + Q - 1];
    const int64_t xoff = (int64_t)h * P;
    const int64_t coff = (int64_t)d.G * N + (int64_t)g * N;  // C of group g in a bc row
    const int64_t hl = ((int64_t)b * d.H + h) * d.L + t0;
    const bool inter = FINAL || !first;
    const int a0 = wave, a1 = QT - 1 - wave;

    // ---- issue every global load of the workgroup.  First the C rows of the
    // wave's two output tiles for the inter-chunk term's first k step (each
    // later k step's are loaded a step ahead of their use)
    int i0[2];
    i0[0] = a0 * 16;
    i0[1] = a1 * 16;
    auto cload = [&](int it, int kn) {
        return M::load(bc + (rb + t0 + i0[it] + lr) * bstr + coff + kn * KS + SL * lg);
    };
    // every k step's C rows at once: each inter-chunk step would otherwise wait
    // a memory round trip for a few products (the conv-fused variant, whose
    // conv windows hold registers meanwhile, loads them one k step ahead)
    constexpr int CPRE = XC ? 1 : NKF;
    Frag cfc[2][NKF];
    if (inter) {
#pragma unroll
        for (int kn = 0; kn < CPRE; ++kn) {
            cfc[0][kn] = cload(0, kn);
            cfc[1][kn] = cload(1, kn);
        }
    }
    // the span's earlier chunk totals, for eps, reduced after the first barrier.
    // Lane l's first one (chunk cspan0 + l, clamped into the row and masked
    // later) is loaded with the workgroup's other rows, without a wait; spans
    // of more than 64 chunks add the rest after the barrier.  The conv-fused
    // variant, whose windows hold registers now, loads them all there.
    const float* ctb = ctot + ((int64_t)b * d.H + h) * d.nchunk;
    float ct_first = 0.f;
    if (!XC && use_st) ct_first = ctb[min(cspan0 + lane, d.nchunk - 1)];
    auto ct_sum = [&]() {
        float ctp = 0.f;
        if (use_st) {
            if constexpr (!XC) {
                if (cspan0 + lane < cm) ctp = ct_first;
                for (int c = cspan0 + 64 + lane; c < cm; c += 64) ctp += ctb[c];
            } else {
                for (int c = cspan0 + lane; c < cm; c += 64) ctp += ctb[c];
            }
        }
        return ctp;
    };
    constexpr int V_X = (Q * (P / VEC) + NTH - 1) / NTH;
    // XC (conv-fused): xc is the raw input; the thread owns column vector xpv of
    // rows xj0 .. xj0 + V_X - 1 and holds the conv window under them
    constexpr int CW = FUSED_CONV_W, RV = P / VEC;
    constexpr int NRW = XC ? V_X + CW - 1 : 1;
    static_assert(!XC || (FINAL && Q * RV % NTH == 0), "conv-fused output pass");
    const int xpv = threadIdx.x % RV, xj0 = (threadIdx.x / RV) * V_X;
    ConvWindow<T, VEC, NRW> xw;
    vt rx[XC ? 1 : V_X];
    if constexpr (XC) {
        load_window<T, VEC, CW, NRW>(xw, xc, seq, tab, k, rb, t0 + xj0, d.C, xoff + xpv * VEC);
    } else {
#pragma unroll
        for (int q = 0; q < V_X; ++q) {
            const int idx = threadIdx.x + q * NTH;
            if (idx < Q * (P / VEC)) {
                const int j = idx / (P / VEC), pv = idx % (P / VEC);
                rx[q] = *(const vt*)(xc + (rb + t0 + j) * d.C + xoff + pv * VEC);
            }
        }
    }
    constexpr int V_H = (P * (N / VEC) + NTH - 1) / NTH;
    vt rh[V_H];
    f32x4 rs[V_H][VEC / 4];
    const T* hp = hst + (((int64_t)b * d.nchunk + cm) * d.H + h) * (P * N);
    const float* stp = use_st ? S_st + (((int64_t)(sp.first[k] + jsp) * d.batch + b) * d.H + h) * (P * N)
                              : nullptr;
    if (inter) {
#pragma unroll
        for (int q = 0; q < V_H; ++q) {
            const int idx = threadIdx.x + q * NTH;
            if (idx < P * (N / VEC)) {
                const int p = idx / (N / VEC), nv = idx % (N / VEC);
                if (!sfirst) {
                    rh[q] = *(const vt*)(hp + (int64_t)p * N + nv * VEC);
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) rh[q][e] = (T)0.f;
                }
                if (use_st) {
#pragma unroll
                    for (int e = 0; e < VEC / 4; ++e)
                        rs[q][e] = *(const f32x4*)(stp + (int64_t)p * N + nv * VEC + 4 * e);
                }
            }
        }
    }
    // the chunk's cumulative sums, dt and sequence ids, one token per thread
    // (NTH = 2 Q), into registers first: a load followed by its LDS write here
    // would wait for every load issued before it.  (The conv-fused variant,
    // whose windows hold registers now, writes them to LDS straight away.)
    static_assert(NTH >= Q, "one token per thread");
    float rcs = 0.f, rdt = 0.f;
    int rsq = 0;
    if (threadIdx.x < Q) {
        rcs = cs_ws[hl + threadIdx.x];
        rdt = dt_ws[hl + threadIdx.x];
        if (seq) rsq = seq[rb + t0 + threadIdx.x];
        if constexpr (XC) {
            scs[threadIdx.x] = rcs;
            sdt[threadIdx.x] = rdt;
            ssq[threadIdx.x] = rsq;
        }
    }
    if constexpr (XC) {
        float taps[VEC][CW];
        load_taps<VEC, CW>(taps, conv_w, xoff + xpv * VEC);
        auto rows = [&](auto masked_tag) {
            constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
            for (int q = 0; q < V_X; ++q)
                *(vt*)&sX[(xj0 + q) * XR + xpv * VEC] = conv_silu<T, VEC, CW, NRW, MASKED>(xw, q, taps);
        };
        if (window_clean(xw)) rows(std::false_type{});
        else rows(std::true_type{});
    } else {
#pragma unroll
        for (int q = 0; q < V_X; ++q) {
            const int idx = threadIdx.x + q * NTH;
            if (idx < Q * (P / VEC)) *(vt*)&sX[(idx / (P / VEC)) * XR + (idx % (P / VEC)) * VEC] = rx[q];
        }
    }
    // the factored decay's token factors (unused on the exact path), from the
    // cumulative sums at the first and last token of the token's 16-token tile
    auto tables_lds = [&]() {  // from the cumulative sums in LDS
        for (int t = threadIdx.x; t < Q; t += NTH) {
            const int t16 = t & ~15;
            sea[t] = __expf(scs[t] - scs[t16]);
            seb[t] = __expf(scs[t16 + 15] - scs[t]) * sdt[t];
        }
    };
    if (!XC && threadIdx.x < Q) {
        scs[threadIdx.x] = rcs;
        sdt[threadIdx.x] = rdt;
        ssq[threadIdx.x] = rsq;
        // from registers: lanes of this wave hold the tile's first and last
        // token (Q = NTH / 2: whole waves take this branch)
        const float cf = __shfl(rcs, lane & ~15, 64), cl = __shfl(rcs, lane | 15, 64);
        sea[threadIdx.x] = __expf(rcs - cf);
        seb[threadIdx.x] = __expf(cl - rcs) * rdt;
    }
    auto stage_state = [&]() {
        // entering state [p][n]: zero-state part from the span's own chunks + eps
        // times the state entering the span; eps = exp(sum of the span's earlier
        // chunk totals), 0 if a sequence started between the span start and
        // this chunk (every wave reduces the totals itself)
        float eps = 0.f;
        if (use_st) {
            float part = ct_sum();
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
            eps = (seq_prev == seq_span) ? expf(part) : 0.f;
        }
#pragma unroll
        for (int q = 0; q < V_H; ++q) {
            const int idx = threadIdx.x + q * NTH;
            if (idx < P * (N / VEC)) {
                vt v = rh[q];
                if (use_st) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        v[e] = (T)((float)v[e] + eps * rs[q][e / 4][e % 4]);
                }
                *(vt*)&sH[(idx / (N / VEC)) * HP + (idx % (N / VEC)) * VEC] = v;
            }
        }
    };
    // The entering state goes to LDS before the barrier; the conv-fused variant
    // loads the chunk totals for eps only after it, and stages the state behind
    // a second barrier.
    if constexpr (!XC) {
        if (inter) stage_state();
    }
    __syncthreads();
    // The factored decay needs every tile's span cs(first) - cs(last) small
    // enough that its exponential stays a normal float; chunks with a sequence
    // start or a wider span take the exact per-element path.
    const bool exact = split || tile_span_wide<QT>(scs, lane);
    if constexpr (XC) {
        if (inter) stage_state();
        tables_lds();
        __syncthreads();
    }

    // Gram tiles of the wave's output tiles, DEPTH k steps ahead of their use
    // (the first ones overlap the inter-chunk term).  A source tile past the
    // output tile (not used: its weights are zero) loads the diagonal tile
    // instead, so the loads need no branch: under a branch a load might not have
    // been issued, and the wait for an older one would then also take the
    // loads issued after it.
    constexpr int TPK = KS / 16;  // source tiles per k step
    constexpr int NKS = Q / KS;
    constexpr int DEPTH = 3;
    const T* gb = gram + (((int64_t)b * d.nchunk + cm) * d.G + g) * (int64_t)gram_tiles(QT) * 256 + lane * 4;
    t4 cgr[DEPTH][2][TPK];
    auto fetch_gram = [&](int ks, t4 (&dst)[2][TPK]) {
#pragma unroll
        for (int st = 0; st < TPK; ++st) {
            const int bt = ks * TPK + st;
            dst[0][st] = *(const t4*)(gb + (int64_t)gram_index(a0, min(bt, a0)) * 256);
            dst[1][st] = *(const t4*)(gb + (int64_t)gram_index(a1, min(bt, a1)) * 256);
        }
    };
#pragma unroll
    for (int q = 0; q < DEPTH; ++q)
        if (q < NKS) fetch_gram(q, cgr[q]);

    // ---- inter-chunk term of the wave's two output tiles (C_i H^T, rows p, columns i)
    f32x4 acc[2][PT];
    float rsc_i[2], cs_i[2];
    int sq_i[2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int i = i0[it] + lr;
        cs_i[it] = scs[i];
        sq_i[it] = ssq[i];
        rsc_i[it] = exact ? 0.f : sea[i];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[it][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (inter) {
#pragma unroll
        for (int kn = 0; kn < NKF; ++kn) {
            if (kn + 1 >= CPRE && kn + 1 < NKF) {
                cfc[0][kn + 1] = cload(0, kn + 1);
                cfc[1][kn + 1] = cload(1, kn + 1);
            }
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const Frag hf = M::load(&sH[(pt * 16 + lr) * HP + kn * KS + SL * lg]);
                acc[0][pt] = M::mma(hf, cfc[0][kn], acc[0][pt]);
                acc[1][pt] = M::mma(hf, cfc[1][kn], acc[1][pt]);
            }
        }
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const float f = (sq_i[it] == seq_prev) ? expf(cs_i[it]) : 0.f;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[it][pt] *= f;
        }
    }
    const float Dh = FINAL ? Dp[h] : 0.f;

    // ---- intra-chunk term, one 32-token (KS = 32) or 16-token (KS = 16) k step at a time
    // the tile factor exp(F_a - L_b) of the wave's output tile a (it = 0, 1) and
    // source tile b <= a, held by lane b and read with readlane in the k steps
    // (a wave-uniform value: no LDS access per step)
    float stw[2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int at = it == 0 ? a0 : a1, l = lane < QT ? lane : 0;
        stw[it] = (!exact && l <= at) ? __expf(scs[16 * at] - scs[16 * l + 15]) : 0.f;
    }
    auto weight = [&](int it, int at, int bt, const t4& cgv, float (&vv)[4]) {
        const int js = bt * 16;
        const int i = i0[it] + lr;
        if (!exact) {
            const float rsc = rsc_i[it] * __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, stw[it]), bt));
            const f32x4 ej = *(const f32x4*)&seb[js + 4 * lg];
#pragma unroll
            for (int r = 0; r < 4; ++r) vv[r] = (float)cgv[r] * (rsc * ej[r]);
        } else {
            const f32x4 cj = *(const f32x4*)&scs[js + 4 * lg];
            const f32x4 dj = *(const f32x4*)&sdt[js + 4 * lg];
            const int4 sj = *(const int4*)&ssq[js + 4 * lg];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vv[r] = (sj[r] == sq_i[it] && js + 4 * lg + r <= i)
                            ? (float)cgv[r] * (__expf(cs_i[it] - cj[r]) * dj[r])
                            : 0.f;
        }
        if (bt == at) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = js + 4 * lg + r;
                if (j > i) vv[r] = 0.f;
                if (FINAL && j == i) vv[r] += Dh;
            }
        }
    };
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        const bool act0 = ks * TPK <= a0, act1 = ks * TPK <= a1;
        if (!act1) break;  // a1 >= a0: nothing left for either tile
        t4 cur[2][TPK];
#pragma unroll
        for (int st = 0; st < TPK; ++st) {
            cur[0][st] = cgr[ks % DEPTH][0][st];
            cur[1][st] = cgr[ks % DEPTH][1][st];
        }
        if (ks + DEPTH < NKS) fetch_gram(ks + DEPTH, cgr[ks % DEPTH]);
        Frag tb[2];
#pragma unroll
        for (int st = 0; st < TPK; ++st) {
            const int bt = ks * TPK + st;
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int at = it == 0 ? a0 : a1;
                float vv[4] = {0.f, 0.f, 0.f, 0.f};
                if (bt <= at) weight(it, at, bt, cur[it][st], vv);
#pragma unroll
                for (int r = 0; r < 4; ++r) tb[it][st * 4 + r] = (E)vv[r];
            }
        }
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const Frag xf = XT<T>::load(sX, XR, ks * KS, pt * 16, lane);
            if (act0) acc[0][pt] = M::mma(xf, tb[0], acc[0][pt]);
            acc[1][pt] = M::mma(xf, tb[1], acc[1][pt]);
        }
    }

    if (!FINAL) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            float* yo = y_zero + ((rb + t0 + i0[it] + lr) * d.H + h) * P;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) *(f32x4*)(yo + pt * 16 + 4 * lg) = acc[it][pt];
        }
        return;
    }
    // stage the wave's two [16 token][P] tiles in LDS, then store whole rows
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        T* st = sY + (wave * 2 + it) * 16 * YP;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
            *(t4*)&st[lr * YP + pt * 16 + 4 * lg] =
                t4{(T)acc[it][pt][0], (T)acc[it][pt][1], (T)acc[it][pt][2], (T)acc[it][pt][3]};
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const T* st = sY + (wave * 2 + it) * 16 * YP;
        for (int q = lane; q < 16 * RV; q += 64) {
            const int r = q / RV, v = q % RV;
            *(vt*)(y + ((rb + t0 + i0[it] + r) * d.H + h) * P + v * VEC) = *(const vt*)&st[r * YP + v * VEC];
        }
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

// LDS of k_chunk_y.
template <typename T, int P, int N, int Q>
constexpr size_t chunk_y_lds() {
    constexpr size_t V = 16 / sizeof(T), NW = Q / 32, QT = Q / 16;
    constexpr size_t main_ = (size_t)Q * (P + V) + (size_t)P * (N + V);
    constexpr size_t stage = 2 * NW * 16 * (P + V);
    return sizeof(T) * (main_ > stage ? main_ : stage) + Q * 20 + QT * QT * 4 + 16;
}
constexpr size_t LDS_LIMIT = 160 * 1024;

template <typename T, int P, int N>
static bool shape_ok(int Q) {
    if (Q == 64) return chunk_y_lds<T, P, N, 64>() <= LDS_LIMIT;
    if (Q == 128) return chunk_y_lds<T, P, N, 128>() <= LDS_LIMIT;
    if (Q == 256) return chunk_y_lds<T, P, N, 256>() <= LDS_LIMIT;
    return false;
}

// The B and C channels of the pass's inputs: bc + m * bstr for token row m.
template <typename T>
struct BCSrc {
    const T* bc;
    int64_t bstr;
};

template <typename T, int P, int N, int Q, bool FINAL>
static hipError_t launch_chunk_y(const Dims& d, const SegTab& t, const T* xc, BCSrc<T> bc,
                                 const float* conv_w, const T* gram, const float* dtw,
                                 const float* csw, const float* ctot, const int32_t* seq,
                                 const T* hst, const SpanPlan& sp, const float* S_st,
                                 const float* D, float* y_zero, T* y, hipStream_t s) {
    if constexpr (chunk_y_lds<T, P, N, Q>() <= LDS_LIMIT) {
        if constexpr (FINAL) {
            if (conv_w)
                return launch(k_chunk_y<T, P, N, Q, true, true>, chunk_head_grid(d),
                              dim3(Q / 32 * 64), s, d, t, xc, bc.bc, bc.bstr, conv_w, gram, dtw,
                              csw, ctot, seq, hst, sp, S_st, D, y_zero, y);
        }
        if (conv_w) return hipErrorInvalidValue;
        return launch(k_chunk_y<T, P, N, Q, FINAL, false>, chunk_head_grid(d), dim3(Q / 32 * 64),
                      s, d, t, xc, bc.bc, bc.bstr, conv_w, gram, dtw, csw, ctot, seq, hst, sp,
                      S_st, D, y_zero, y);
    }
    return hipErrorInvalidValue;
}

// conv_w null: xc_ is the conv output.  Otherwise (conv-fused) xc_ is the raw
// input: the B and C channels are convolved into the workspace first, and the
// walk convolves the x channels as it reads them.
template <typename T, int P, int N>
static hipError_t segment_states_t(const Dims& d, const SegTab& t, const void* xc_,
                                   const float* conv_w, const void* dt_raw, const float* dt_bias,
                                   const float* A_log, const int32_t* seq, float* summary,
                                   void* ws, hipStream_t s) {
    const T* xc = (const T*)xc_;
    constexpr int act = std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32;
    const bool xconv = conv_w != nullptr;
    const FwdWs L = fwd_ws_layout(d, t, act, xconv);
    char* w = (char*)ws;
    float* dtw = (float*)(w + L.dt);
    float* csw = (float*)(w + L.cs);
    float* ctot = (float*)(w + L.ctot);
    T* hst = (T*)(w + L.hst);
    BCSrc<T> bc = {xc + (int64_t)d.H * P, (int64_t)d.C};
    if (xconv) {
        bc = {(const T*)(w + L.bc), 2LL * d.G * N};
        SSD_TRY(launch_conv1d_channels(d, t, act, xc, conv_w, seq, d.H * P, 2 * d.G * N,
                                       bc.bstr, w + L.bc, s));
    }
    const SpanPlan sp = span_plan(d, t, true);
    const bool trivial = plan_trivial(sp, t);
    // long segments: walk their spans, then compose the span summaries
    const WalkArgs<T> wa = {xc,  nullptr, dtw, csw, seq, nullptr, hst,
                            trivial ? summary : (float*)(w + L.spsum),
                            sp,  bc.bc,   bc.bstr, conv_w};
    T* gram = (T*)(w + L.gram);
    if (!xconv && walk_gram_fits<T>(d)) {
        // dt prep first (the walk reads dt and the cumulative sums), then the
        // walk and the group Gram tiles the output pass reads in one launch
        SSD_TRY(launch_dt_prep(d, act, dt_raw, dt_bias, A_log, seq, dtw, csw, ctot, s));
        SSD_TRY(launch_walk_gram<T, P, N, false, false>(d, t, wa, bc.bc, bc.bstr, gram, s));
    } else {
        // the Gram tiles and dt prep share one launch (independent inputs); the
        // walk then needs dt and the cumulative sums
        SSD_TRY(launch_gram_dt<T, N>(d, bc.bc, bc.bstr, gram, dt_raw, dt_bias, A_log, seq, dtw,
                                     csw, ctot, s));
        if (xconv) SSD_TRY(launch_state_walk<T, P, N, false, true>(d, t, wa, s));
        else SSD_TRY(launch_state_walk<T, P, N, false>(d, t, wa, s));
    }
    if (trivial) return hipSuccess;
    return launch_span_combine(d, sp, (const float*)(w + L.spsum), summary, s);
}

// y_zero (FINAL = false) or the corrected y (FINAL = true), from the workspace
// that segment_states_t filled (decays, entering states, Gram tiles).
// conv_w as for segment_states_t (conv-fused: FINAL only).
template <typename T, int P, int N, bool FINAL>
static hipError_t segment_output_t(const Dims& d, const SegTab& t, const void* xc_,
                                   const float* conv_w, const int32_t* seq, void* ws,
                                   const float* S_in, const float* D, float* y_zero, void* y,
                                   hipStream_t s) {
    const T* xc = (const T*)xc_;
    const bool xconv = conv_w != nullptr;
    const FwdWs L =
        fwd_ws_layout(d, t, std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32, xconv);
    const BCSrc<T> bc = xconv ? BCSrc<T>{(const T*)((const char*)ws + L.bc), 2LL * d.G * N}
                              : BCSrc<T>{xc + (int64_t)d.H * P, (int64_t)d.C};
    char* w = (char*)ws;
    const float* dtw = (const float*)(w + L.dt);
    const float* csw = (const float*)(w + L.cs);
    const float* ctot = (const float*)(w + L.ctot);
    const T* hst = (const T*)(w + L.hst);
    const T* gram = (const T*)(w + L.gram);
    T* yo = (T*)y;
    const SpanPlan sp = span_plan(d, t, true);
    const float* S_st = FINAL ? S_in : nullptr;
    if (!plan_trivial(sp, t)) {
        // the state entering every span: from S_in (y) or from zero (y_zero)
        float* spst = (float*)(w + L.spst);
        SSD_TRY(launch_span_scan(d, sp, (const float*)(w + L.spsum), FINAL ? S_in : nullptr, spst, s));
        S_st = spst;
    }
    switch (d.Q) {
        case 64:
            return launch_chunk_y<T, P, N, 64, FINAL>(d, t, xc, bc, conv_w, gram, dtw, csw, ctot,
                                                      seq, hst, sp, S_st, D, y_zero, yo, s);
        case 128:
            return launch_chunk_y<T, P, N, 128, FINAL>(d, t, xc, bc, conv_w, gram, dtw, csw, ctot,
                                                       seq, hst, sp, S_st, D, y_zero, yo, s);
        case 256:
            return launch_chunk_y<T, P, N, 256, FINAL>(d, t, xc, bc, conv_w, gram, dtw, csw, ctot,
                                                       seq, hst, sp, S_st, D, y_zero, yo, s);
        default:
            return hipErrorInvalidValue;
    }
}

template <typename T, int P, int N>
static hipError_t apply_init_t(const Dims& d, const SegTab& t, const float* y_zero, const void* xc,
                               const float* D, const int32_t* seq, const float* S_in,
                               const void* ws, void* y, hipStream_t s) {
    const FwdWs L = fwd_ws_layout(d, t, std::is_same<T, bf16>::value ? SSD_BF16 : SSD_F32);
    const char* w = (const char*)ws;
    return launch(k_apply_init<T, P, N>, chunk_head_grid(d), dim3(256), s, d, t, y_zero,
                  (const T*)xc, D, seq, S_in, (const float*)(w + L.cs),
                  (const float*)(w + L.ctot), (T*)y);
}

hipError_t launch_dt_prep(const Dims& d, int act, const void* dt_raw, const float* dt_bias,
                          const float* A_log, const int32_t* seq, float* dt_ws, float* cs_ws,
                          float* ctot, hipStream_t s) {
    const dim3 grid((unsigned)d.nchunk, (unsigned)((d.H + DTB - 1) / DTB), (unsigned)d.batch);
    if (act == SSD_BF16)
        return launch(k_dt_prep<bf16>, grid, dim3(256), s, d, (const bf16*)dt_raw, dt_bias, A_log,
                      seq, dt_ws, cs_ws, ctot);
    return launch(k_dt_prep<float>, grid, dim3(256), s, d, (const float*)dt_raw, dt_bias, A_log,
                  seq, dt_ws, cs_ws, ctot);
}

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
        return segment_states_t<T, p, n>(d, t, xBC_conv, nullptr, dt_raw, dt_bias, A_log, seq, \
                                         summary, ws, s);                                      \
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
                                 const int32_t* seq, void* ws, float* y_zero, hipStream_t s) {
#define X(p, n)                                                                                 \
    if (d.P == p && d.N == n) {                                                                 \
        return segment_output_t<T, p, n, false>(d, t, xBC_conv, nullptr, seq, ws, nullptr,     \
                                                nullptr, y_zero, nullptr, s);                  \
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

hipError_t launch_segment_output_fused(const Dims& d, const SegTab& t, int act,
                                       const void* xBC_conv, const float* D, const int32_t* seq,
                                       const float* S_in, void* ws, void* y, hipStream_t s) {
#define X(p, n)                                                                                 \
    if (d.P == p && d.N == n) {                                                                 \
        return segment_output_t<T, p, n, true>(d, t, xBC_conv, nullptr, seq, ws, S_in, D,     \
                                               nullptr, y, s);                                 \
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

hipError_t launch_conv_segment_states(const Dims& d, const SegTab& t, int act, const void* xBC,
                                      const float* conv_w, const void* dt_raw,
                                      const float* dt_bias, const float* A_log,
                                      const int32_t* seq, float* summary, void* ws,
                                      hipStream_t s) {
    if (!conv_w || d.W != FUSED_CONV_W) return hipErrorInvalidValue;
#define X(p, n)                                                                           \
    if (d.P == p && d.N == n) {                                                           \
        return segment_states_t<T, p, n>(d, t, xBC, conv_w, dt_raw, dt_bias, A_log, seq,   \
                                         summary, ws, s);                                  \
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

hipError_t launch_conv_segment_output(const Dims& d, const SegTab& t, int act, const void* xBC,
                                      const float* conv_w, const float* D, const int32_t* seq,
                                      const float* S_in, void* ws, void* y, hipStream_t s) {
    if (!conv_w || d.W != FUSED_CONV_W) return hipErrorInvalidValue;
#define X(p, n)                                                                               \
    if (d.P == p && d.N == n) {                                                               \
        return segment_output_t<T, p, n, true>(d, t, xBC, conv_w, seq, ws, S_in, D, nullptr,   \
                                               y, s);                                          \
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
        return apply_init_t<T, p, n>(d, t, y_zero, xBC_conv, D, seq, S_in, ws, y, s); \
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
