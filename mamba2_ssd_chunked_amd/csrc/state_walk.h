// Per-segment walk of chunk states (forward) or state gradients (backward).
//
// One workgroup per (row, segment, head) visits the segment's chunks in causal
// order (forward) or reverse causal order (backward).  The running P x N
// matrix lives in MFMA accumulators (FP32).  For every chunk it first stores
// the running value, then applies the chunk's decay alpha_c = exp(cs_end)
// (exactly 0 when a packed sequence starts inside the chunk) and accumulates
// the chunk's own contribution A^T diag(w) B with MFMA:
//
//   forward : A = x, B = B channels, w_j = exp(cs_end - cs_j) dt_j [seq_j = seq_end];
//             the stored value is the state entering the chunk.
//   backward: A = dy, B = C channels, w_i = exp(cs_i) [seq_i = seq of the state
//             entering the chunk]; the stored value is the gradient of the
//             state leaving the chunk.
//
// A walk covers one span of a segment (a run of its chunks; see SpanPlan:
// the whole segment unless the forward walk splits long segments).  It starts
// from `init` ([S][b][H][P][N] FP32: S_in forward, dS_out backward, for walks
// with one span per segment) or from zero; from zero, the forward walk stores
// nothing for a span's first chunk (its entering state from the span's own
// chunks is zero).  The final value is the span's S_ext (forward) or dL/dS_in
// of the segment's own outputs (backward), and the product of the alphas its
// block decay, both written to `summary` (summary layout over spans) if given.
//
// This is the decay-weighted sum over earlier chunk states that
// state-spaces/mamba #482 (second comment) identifies as the part of the scan
// that must cross devices; Megatron-LM #6808 ships its segment-level result as
// the FP32 summary.
//
// A segment is read in slices of KT = 64 tokens (a chunk holds Q / KT of
// them).  Each slice passes through registers (loaded two slices ahead of its
// use, with the decay and sequence values of its chunk) into one of two LDS
// buffers: A rows scaled by w and B rows, both in their natural [token][.]
// layout, and both MFMA operands come from transposed LDS reads (XT).  While
// the waves multiply slice s from one buffer they write slice s + 1 into the
// other, so one barrier per slice suffices.
#pragma once

#include <type_traits>

#include "conv_fused.h"
#include "ssd_internal.h"
#include "xt.h"

namespace ssd {

// The pointers of one walk launch.
template <typename T>
struct WalkArgs {
    const T* xc;           // conv output [b][L][C]
    const T* dy;           // output gradient [b][L][H][P] (backward)
    const float* dt_ws;    // dt [b][H][L]
    const float* cs_ws;    // chunk-local cumulative sums [b][H][L]
    const int32_t* seq;    // packed sequence ids or null
    const float* init;     // starting value [S][b][H][P][N] or null (zero)
    T* store;              // value at every chunk start, or null
    float* summary;        // final value and block decay per span, or null
    SpanPlan sp;           // the runs of chunks walked (spans; one per segment
                           // unless the forward walk splits segments)
    // B and C channels of token row m at bc + m * bstr (B of group g at g N, C
    // at (G + g) N); null: inside xc's rows
    const T* bc = nullptr;
    int64_t bstr = 0;
    // conv-fused forward walk (XC): xc is the raw input and the x channels are
    // convolved here with these [C][W] taps
    const float* conv_w = nullptr;
};

constexpr int WALK_KT = 64;  // tokens per slice
// LDS of a walk block (elements of T): two slice buffers of HW heads' A rows
// and of the shared B rows.
template <typename T, int P, int N, int HW>
constexpr int walk_lds() {
    return 2 * HW * WALK_KT * (P + 16 / (int)sizeof(T)) + 2 * WALK_KT * (N + 16 / (int)sizeof(T));
}

// One walk block: block `blk` of `nblk` (the XCD-aware item mapping is over
// this range), its slice buffers at `lds`.  XC: the conv-fused forward walk,
// whose threads each own one column vector of VX consecutive x rows of a slice
// and the conv window under them (conv_fused.h).
template <typename T, int P, int N, bool BWD, bool SEQ, int HW, bool XC = false>
__device__ __forceinline__ void walk_block(const Dims& d, const SegTab& tab, const WalkArgs<T>& wa,
                                           T* lds, int64_t blk, int64_t nblk) {
    const T* __restrict__ xc = wa.xc;
    const T* __restrict__ dy = wa.dy;
    const float* __restrict__ dt_ws = wa.dt_ws;
    const float* __restrict__ cs_ws = wa.cs_ws;
    const int32_t* __restrict__ seq = wa.seq;
    const float* __restrict__ init = wa.init;
    T* __restrict__ store = wa.store;
    float* __restrict__ summary = wa.summary;
    typedef Mma<T> M;
    typedef typename M::Frag Frag;
    constexpr int KS = M::KS;
    constexpr int KT = WALK_KT;          // tokens per slice
    constexpr int NTH = 256 * HW, HTH = 256;  // threads of the block / of one head
    constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte load
    constexpr int XR = P + VEC, BR = N + VEC;
    constexpr int PT = P / 16, NTT = N / 16, NTW = (NTT + 3) / 4;
    constexpr int VX = (KT * (P / VEC) + HTH - 1) / HTH;  // A vectors per thread and slice
    constexpr int VB = (KT * (N / VEC) + NTH - 1) / NTH;  // B vectors per thread and slice
    // index checks that hold for every thread of the shape compile away (a
    // check the compiler cannot drop splits the loop body into small blocks
    // and forces full waits for the outstanding loads at their joins)
    constexpr bool XFULL = KT * (P / VEC) % HTH == 0, BFULL = KT * (N / VEC) % NTH == 0;
    constexpr bool NFULL = NTT % 4 == 0;
    constexpr int CW = FUSED_CONV_W, RV = P / VEC;
    constexpr int NRW = XC ? VX + CW - 1 : 1;  // conv window rows (XC)
    static_assert(!XC || (!BWD && XFULL), "the conv-fused walk is the forward walk");
    auto sX = reinterpret_cast<T(*)[HW][KT * XR]>(lds);
    auto sB = reinterpret_cast<T(*)[KT * BR]>(lds + 2 * HW * KT * XR);
    typedef T vt __attribute__((ext_vector_type(VEC)));

    // block -> (row, span, HW heads of one group): the walks of one (row,
    // span) are consecutive items and consecutive items go to one XCD, so
    // they share that XCD's L2 for the B (or C) rows they all read.  The HW
    // heads of a block share its B (or C) rows in LDS; threads hs*256 ..
    // hs*256+255 (four waves) walk head h0 + hs.  Span sg is span j of
    // segment k: its chunks j*cps .. of the segment.
    // head of the block this thread works on: whole waves per head (HTH = 256),
    // so it is the same for the wave; readfirstlane tells the compiler, which
    // keeps the per-head bases (rows, sums, state stores) in scalar registers
    const int hs = __builtin_amdgcn_readfirstlane(threadIdx.x / HTH);
    int h, k, sg;
    int64_t b;
    {
        constexpr int NXCD = 8;
        const int64_t n = nblk, i = blk;
        int64_t item = (n % NXCD == 0) ? (i % NXCD) * (n / NXCD) + i / NXCD : i;
        h = (int)(item % (d.H / HW)) * HW + hs;
        item /= d.H / HW;
        sg = (int)(item % wa.sp.n);
        b = item / wa.sp.n;
        k = 0;
        for (int q = 1; q < tab.n; ++q)
            if (sg >= wa.sp.first[q]) k = q;
    }
    const int jsp = sg - wa.sp.first[k];  // span index within the segment
    const int wave = wave_id() % 4, lane = threadIdx.x % 64, lr = lane % 16, lg = lane / 16;
    const int ht = threadIdx.x % HTH;  // thread index within the head
    const int g = h / d.hpg;
    const int Q = d.Q;
    const int64_t rb = b * d.L;
    const int nck = (int)(tab.len[k] / Q);
    const int64_t s0 = tab.start[k] + (int64_t)jsp * wa.sp.cps * Q;
    // the walk's first chunk (segment starts are whole chunks): chunk c of the
    // walk is cm0 + c, without a 64-bit division per chunk in the slice loop
    const int cm0 = (int)(s0 / Q);
    const int nc = min(wa.sp.cps, nck - jsp * wa.sp.cps);
    const int spc = Q / KT;  // slices per chunk
    const int ns = nc * spc;
    const int64_t pred = jsp > 0 ? s0 - 1 : seg_pred_token(tab, k);
    const float* dtp = dt_ws + ((int64_t)b * d.H + h) * d.L;
    const float* csp = cs_ws + ((int64_t)b * d.H + h) * d.L;
    const int64_t astr = BWD ? (int64_t)d.H * P : (int64_t)d.C;
    const T* arow = (BWD ? dy + rb * astr : xc + rb * astr) + (int64_t)h * P;
    const T* bsrc = wa.bc ? wa.bc : xc + (int64_t)d.H * P;
    const int64_t bstr = wa.bc ? wa.bstr : (int64_t)d.C;
    const T* brow = bsrc + rb * bstr + (BWD ? (int64_t)d.G * N : 0) + (int64_t)g * N;
    // XC: the thread's column vector and first row of a slice, and the taps
    const int xpv = ht % RV, xj0 = (ht / RV) * VX;
    float taps[XC ? VEC : 1][CW];
    if constexpr (XC) load_taps<VEC, CW>(taps, wa.conv_w, (int64_t)h * P + xpv * VEC);
    auto chunk_of = [&](int si) { return BWD ? nc - 1 - si / spc : si / spc; };

    // ---- one slice in registers, with the values of its chunk
    struct Slice {
        vt x[XC ? 1 : VX], b[VB];
        ConvWindow<T, VEC, NRW> win;  // XC: raw x rows xj0 - (W-1) .. xj0 + VX - 1
        float cs[VX], dt[VX];
        int sq[VX];
        float cse;       // cumulative log decay at the chunk's last token
        int seqe, seqr;  // sequence of the chunk's last token / of the state entering it
    };
    auto fetch = [&](Slice& r, int si) {
        const int c = chunk_of(si);
        const int64_t t0 = s0 + (int64_t)c * Q;
        const int64_t tb = t0 + (int64_t)(si % spc) * KT;
        r.cse = csp[t0 + Q - 1];
        // The state entering chunk c belongs to the sequence of the token just
        // before it; for a row's first segment that is the sequence of the
        // row's first token (an initial state feeds the first sequence).
        const int64_t ptok = c > 0 ? t0 - 1 : (pred >= 0 ? pred : s0);
        r.seqe = SEQ ? seq[rb + t0 + Q - 1] : 0;
        r.seqr = SEQ ? seq[rb + ptok] : 0;
        if constexpr (XC) {
            load_window<T, VEC, CW, NRW>(r.win, xc, SEQ ? seq : nullptr, tab, k, rb, tb + xj0,
                                         d.C, (int64_t)h * P + xpv * VEC);
#pragma unroll
            for (int q = 0; q < VX; ++q) {
                r.cs[q] = csp[tb + xj0 + q];
                r.dt[q] = dtp[tb + xj0 + q];
                r.sq[q] = r.win.sq[q + CW - 1];
            }
        } else {
#pragma unroll
            for (int q = 0; q < VX; ++q) {
                const int idx = ht + q * HTH;
                if (XFULL || idx < KT * (P / VEC)) {
                    const int jj = idx / (P / VEC), pv = idx % (P / VEC);
                    r.x[q] = *(const vt*)(arow + (tb + jj) * astr + pv * VEC);
                    r.cs[q] = csp[tb + jj];
                    r.dt[q] = BWD ? 0.f : dtp[tb + jj];
                    r.sq[q] = SEQ ? seq[rb + tb + jj] : 0;
                }
            }
        }
#pragma unroll
        for (int q = 0; q < VB; ++q) {
            const int idx = threadIdx.x + q * NTH;
            if (BFULL || idx < KT * (N / VEC)) {
                const int jj = idx / (N / VEC), nv = idx % (N / VEC);
                r.b[q] = *(const vt*)(brow + (tb + jj) * bstr + nv * VEC);
            }
        }
    };
    // A rows scaled by their weights, and B rows, into LDS buffer u; the weight
    // is zero for tokens of another sequence than seq_end (forward) or than the
    // entering state's (backward)
    auto stash = [&](const Slice& r, int u) {
        const int sref = BWD ? r.seqr : r.seqe;
        if constexpr (XC) {
            auto rows = [&](auto masked_tag) {
                constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
                for (int q = 0; q < VX; ++q) {
                    const float w = r.sq[q] != sref ? 0.f : __expf(r.cse - r.cs[q]) * r.dt[q];
                    const vt xv = conv_silu<T, VEC, CW, NRW, MASKED>(r.win, q, taps);
                    vt v;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) v[e] = (T)((float)xv[e] * w);
                    *(vt*)&sX[u][hs][(xj0 + q) * XR + xpv * VEC] = v;
                }
            };
            if (window_clean(r.win)) rows(std::false_type{});
            else rows(std::true_type{});
        }
#pragma unroll
        for (int q = 0; q < (XC ? 0 : VX); ++q) {
            const int idx = ht + q * HTH;
            if (XFULL || idx < KT * (P / VEC)) {
                const int jj = idx / (P / VEC), pv = idx % (P / VEC);
                const float w = r.sq[q] != sref ? 0.f
                                : BWD          ? __expf(r.cs[q])
                                               : __expf(r.cse - r.cs[q]) * r.dt[q];
                vt v;
#pragma unroll
                for (int e = 0; e < VEC; ++e) v[e] = (T)((float)r.x[q][e] * w);
                *(vt*)&sX[u][hs][jj * XR + pv * VEC] = v;
            }
        }
#pragma unroll
        for (int q = 0; q < VB; ++q) {
            const int idx = threadIdx.x + q * NTH;
            if (BFULL || idx < KT * (N / VEC)) {
                const int jj = idx / (N / VEC), nv = idx % (N / VEC);
                *(vt*)&sB[u][jj * BR + nv * VEC] = r.b[q];
            }
        }
    };

    const int64_t per = (int64_t)d.batch * d.H * P * N;
    const int64_t ig = ((int64_t)k * d.batch + b) * d.H + h;  // init walks: one span per segment
    f32x4 acc[PT][NTW];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int nt = wave + 4 * j;
            if (init && (NFULL || nt < NTT)) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[pt][j][r] = init[ig * (P * N) + (pt * 16 + 4 * lg + r) * N + nt * 16 + lr];
            } else {
                acc[pt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    float ablk = 1.f;

    // At a chunk's first slice (held by r): store the running value, then
    // apply the chunk's decay.
    auto chunk_start = [&](const Slice& r, int si) {
        const int c = chunk_of(si);
        const int cm = cm0 + c;
        const float alpha = (r.seqr == r.seqe) ? expf(r.cse) : 0.f;
        ablk *= alpha;
        if (store && (init || BWD || c > 0)) {
            T* hp = store + (((int64_t)b * d.nchunk + cm) * d.H + h) * (P * N);
            // lane ids from an opaque zero: the stores take the uniform base plus
            // a 32-bit lane offset recomputed here, instead of a 64-bit per-lane
            // address held (and spilled) across the slice loop
            int opq;
            asm volatile("s_mov_b32 %0, 0" : "=s"(opq));
            const int l2 = lane + opq, lr2 = l2 % 16, lg2 = l2 / 16;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    const int nt = wave + 4 * j;
                    if (NFULL || nt < NTT) {
                        const int n = nt * 16 + lr2;
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr)
                            *at32(hp, (uint32_t)((pt * 16 + 4 * lg2 + rr) * N + n)) = (T)acc[pt][j][rr];
                    }
                }
        }
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
            for (int j = 0; j < NTW; ++j) acc[pt][j] *= alpha;
    };
    // products of the slice in LDS buffer u
    auto multiply = [&](int u) {
#pragma unroll
        for (int kk = 0; kk < KT / KS; ++kk) {
            const int jb = kk * KS;
            Frag a[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) a[pt] = XT<T>::load(sX[u][hs], XR, jb, pt * 16, lane);
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int nt = wave + 4 * j;
                if (NFULL || nt < NTT) {
                    const Frag bb = XT<T>::load(sB[u], BR, jb, nt * 16, lane);
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) acc[pt][j] = M::mma(a[pt], bb, acc[pt][j]);
                }
            }
        }
    };
    // Slice si: `cur` holds it (already in LDS buffer u), `nxt` holds slice
    // si + 1 (not yet in LDS).  After the barrier every wave is done with the
    // products of slice si - 1, whose buffer 1 - u takes slice si + 1; `cur`
    // then takes slice si + 2.  Past the last slice the loads repeat it and its
    // copy goes to a buffer nobody reads any more: the loads and LDS writes of
    // every step are unconditional, so they stay in the step's straight-line
    // code, ahead of the products.
    Slice r0, r1;
    auto step = [&](Slice& cur, Slice& nxt, int si, int u, bool live) {
        __syncthreads();
        if (live && si % spc == 0) chunk_start(cur, si);
        fetch(cur, min(si + 2, ns - 1));
        // the loads stay ahead of the LDS writes, whose waits then cover only
        // the loads of the slice before
        __builtin_amdgcn_sched_barrier(0);
        stash(nxt, 1 - u);
        if (live) multiply(u);
    };

    if (ns > 0) {
        fetch(r0, 0);
        fetch(r1, min(1, ns - 1));
        stash(r0, 0);
    }
    for (int si = 0; si < ns; si += 2) {
        step(r0, r1, si, 0, true);
        step(r1, r0, si + 1, 1, si + 1 < ns);
    }

    if (!summary) return;
    float* sx = summary + (int64_t)sg * per + ((int64_t)b * d.H + h) * (P * N);
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int nt = wave + 4 * j;
            if (NFULL || nt < NTT) {
                const int n = nt * 16 + lr;
#pragma unroll
                for (int r = 0; r < 4; ++r) sx[(pt * 16 + 4 * lg + r) * N + n] = acc[pt][j][r];
            }
        }
    if (ht == 0)
        summary[(int64_t)wa.sp.n * per + ((int64_t)sg * d.batch + b) * d.H + h] = ablk;
}

// Two heads per block: four waves per SIMD, so that two blocks (of one walk or
// of the two walks of k_state_walk_pair) share a CU.  The conv-fused walk (XC)
// holds its conv windows and taps in registers and runs one block per CU.
template <typename T, int P, int N, bool BWD, bool SEQ, int HW, bool XC = false>
__global__ void __launch_bounds__(256 * HW, HW == 2 ? (XC ? 2 : 4) : 1) k_state_walk(Dims d, SegTab tab,
                                                                         WalkArgs<T> wa) {
    __shared__ __attribute__((aligned(16))) T lds[walk_lds<T, P, N, HW>()];
    walk_block<T, P, N, BWD, SEQ, HW, XC>(d, tab, wa, lds, blockIdx.x, gridDim.x);
}

// The reverse walk (blocks 0 .. n-1) and the forward walk (n .. 2n-1) in one
// launch: the two have no order between them, and their blocks share the CUs.
template <typename T, int P, int N, bool SEQ, int HW>
__global__ void __launch_bounds__(256 * HW, HW == 2 ? 4 : 1) k_state_walk_pair(Dims d, SegTab tab,
                                                                              WalkArgs<T> bwd,
                                                                              WalkArgs<T> fwd) {
    __shared__ __attribute__((aligned(16))) T lds[walk_lds<T, P, N, HW>()];
    const int64_t n = gridDim.x / 2;
    if ((int64_t)blockIdx.x < n)
        walk_block<T, P, N, true, SEQ, HW>(d, tab, bwd, lds, blockIdx.x, n);
    else
        walk_block<T, P, N, false, SEQ, HW>(d, tab, fwd, lds, blockIdx.x - n, n);
}

// One walk per (row, segment, head), see walk_block; A = x (forward) or dy
// (backward).  Two heads of a group per block where they exist (bf16: the
// float32 accumulators of two heads would not fit four waves per SIMD).
template <typename T>
inline int walk_heads(const Dims& d) {
    return (std::is_same<T, bf16>::value && d.hpg % 2 == 0) ? 2 : 1;
}

template <typename T, int P, int N, bool BWD, bool XC = false>
inline hipError_t launch_state_walk(const Dims& d, const SegTab& t, const WalkArgs<T>& wa,
                                    hipStream_t s) {
    const int hw = walk_heads<T>(d);
    const dim3 grid((unsigned)((int64_t)(d.H / hw) * wa.sp.n * d.batch));
    const dim3 block(256 * hw);
    if (XC && (!wa.conv_w || d.W != FUSED_CONV_W)) return hipErrorInvalidValue;
    if (hw == 2) {
        if (wa.seq) return launch(k_state_walk<T, P, N, BWD, true, 2, XC>, grid, block, s, d, t, wa);
        return launch(k_state_walk<T, P, N, BWD, false, 2, XC>, grid, block, s, d, t, wa);
    }
    if (wa.seq) return launch(k_state_walk<T, P, N, BWD, true, 1, XC>, grid, block, s, d, t, wa);
    return launch(k_state_walk<T, P, N, BWD, false, 1, XC>, grid, block, s, d, t, wa);
}

// The reverse and the forward walk of the backward pass in one launch.
template <typename T, int P, int N>
inline hipError_t launch_state_walk_pair(const Dims& d, const SegTab& t, const WalkArgs<T>& bwd,
                                         const WalkArgs<T>& fwd, hipStream_t s) {
    const int hw = walk_heads<T>(d);
    // both walks start from a state per segment: one span per segment
    if (bwd.sp.n != t.n || fwd.sp.n != t.n) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(2 * (int64_t)(d.H / hw) * d.nseg * d.batch));
    const dim3 block(256 * hw);
    if (hw == 2) {
        if (bwd.seq)
            return launch(k_state_walk_pair<T, P, N, true, 2>, grid, block, s, d, t, bwd, fwd);
        return launch(k_state_walk_pair<T, P, N, false, 2>, grid, block, s, d, t, bwd, fwd);
    }
    if (bwd.seq) return launch(k_state_walk_pair<T, P, N, true, 1>, grid, block, s, d, t, bwd, fwd);
    return launch(k_state_walk_pair<T, P, N, false, 1>, grid, block, s, d, t, bwd, fwd);
}

}  // namespace ssd
