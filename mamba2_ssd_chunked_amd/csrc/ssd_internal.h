// Internal types and device helpers shared by the gfx950 kernels of libssd.
//
// Everything here is wave64 CDNA4 code: MFMA fragments are built for
// v_mfma_f32_16x16x32_bf16 (bf16 activations) and v_mfma_f32_16x16x4_f32
// (float32 activations, four instructions per 16-deep k step).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <array>
#include <tuple>
#include <type_traits>
#include <utility>

#include "../../include/ssd.h"

namespace ssd {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// Problem sizes as the kernels see them (passed by value).
struct Dims {
    int64_t batch, L;  // rows, tokens per row
    int H, P, N, G, Q, W, C, hpg;
    int nchunk;        // L / Q
    int nseg;
    int act;           // ssd_dtype of the activations
    float dt_min, dt_max;
};
inline int act_of_dims(const Dims& d) { return d.act; }

// Kernel launch that returns the launch's own status (hipLaunchKernel), so a
// call made of several launches stops at the first that fails.  The arguments
// are converted to the kernel's parameter types first.
template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s,
                         Args&&... args) {
    std::tuple<KArgs...> a(std::forward<Args>(args)...);
    return std::apply(
        [&](auto&... v) {
            std::array<void*, sizeof...(KArgs) + 1> p = {(void*)&v..., nullptr};
            return hipLaunchKernel((const void*)kernel, grid, block, p.data(), 0, s);
        },
        a);
}

// Stops a host launcher at the first failed launch.
#define SSD_TRY(...)                              \
    do {                                          \
        const hipError_t ssd_e_ = (__VA_ARGS__);  \
        if (ssd_e_ != hipSuccess) return ssd_e_;  \
    } while (0)

// Segment table in causal order; start and len in tokens (memory offsets).
struct SegTab {
    int64_t start[SSD_MAX_SEGMENTS];
    int64_t len[SSD_MAX_SEGMENTS];
    int n;
};

// Segment holding memory chunk `cm` (chunk index = token offset / Q).
__device__ __forceinline__ int seg_of_chunk(const SegTab& t, int cm, int Q) {
    const int64_t tok = (int64_t)cm * Q;
    int k = 0;
    for (int i = 0; i < t.n; ++i)
        if (tok >= t.start[i] && tok < t.start[i] + t.len[i]) k = i;
    return k;
}

// Memory position of the token that causally precedes segment k's first token
// (-1 when k is the row's first segment).
__device__ __forceinline__ int64_t seg_pred_token(const SegTab& t, int k) {
    return k > 0 ? t.start[k - 1] + t.len[k - 1] - 1 : -1;
}

template <typename T>
__device__ __forceinline__ float to_f(T v) { return (float)v; }

// Conv tiling shared by the forward and backward conv kernels: a thread owns
// CONV_VEC channels and CONV_TPT tokens, a workgroup four token groups.
constexpr int CONV_VEC = 4;   // channels per thread
constexpr int CONV_TPT = 16;  // tokens per thread
constexpr int CONV_TT = 4 * CONV_TPT;  // tokens per workgroup (one group per wave)
// The conv width the conv-fused forward kernels are compiled for (Mamba2's
// d_conv).
constexpr int FUSED_CONV_W = 4;

template <typename T>
struct Vec4 {
    typedef T type __attribute__((ext_vector_type(4)));
};

// Memory position of the token `o` places after memory token t0 (o may be
// negative: causal predecessors), for t0 inside segment k; -1 when outside the
// row.  Callers keep |o| below a segment length.
__device__ __forceinline__ int64_t conv_row(const SegTab& tab, int k, int64_t t0, int o) {
    const int64_t s0 = tab.start[k], s1 = s0 + tab.len[k];
    const int64_t m = t0 + o;
    if (m >= s0 && m < s1) return m;
    if (m < s0) return k > 0 ? tab.start[k - 1] + tab.len[k - 1] - (s0 - m) : -1;
    return k + 1 < tab.n ? tab.start[k + 1] + (m - s1) : -1;
}

__device__ __forceinline__ int conv_seg(const SegTab& tab, int64_t t0) {
    int k = 0;
    for (int i = 0; i < tab.n; ++i)
        if (t0 >= tab.start[i] && t0 < tab.start[i] + tab.len[i]) k = i;
    return k;
}

// (chunk, head, row) of a workgroup in a 1-D grid of nchunk * H * batch
// workgroups.  The hardware hands workgroup i to XCD i % 8; giving each XCD one
// contiguous range of logical items, heads fastest, makes the workgroups that
// share a chunk's B and C channels (all heads of a group) run on one XCD at
// about the same time, so those channels are read into its L2 once.
struct ChunkHead {
    int cm, h;
    int64_t b;
};
__device__ __forceinline__ ChunkHead chunk_head_of_block(const Dims& d) {
    constexpr int NXCD = 8;
    const int64_t n = gridDim.x, i = blockIdx.x;
    const int64_t item = (n % NXCD == 0) ? (i % NXCD) * (n / NXCD) + i / NXCD : i;
    ChunkHead c;
    c.h = (int)(item % d.H);
    const int64_t rest = item / d.H;
    c.cm = (int)(rest % d.nchunk);
    c.b = rest / d.nchunk;
    return c;
}
inline dim3 chunk_head_grid(const Dims& d) {
    return dim3((unsigned)((int64_t)d.nchunk * d.H * d.batch));
}

// Index of the calling wave in its workgroup as a scalar (wave-uniform) value,
// so that branches on it compile to scalar branches rather than exec masks.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / 64));
}

// True if some 16-token tile's decay span (cumulative sum at its first token
// minus that at its last) exceeds 80, read from the chunk's cumulative sums in
// LDS.  Every wave evaluates all QT tiles itself (lane a takes tile a), so the
// workgroup agrees without a barrier.
template <int QT>
__device__ __forceinline__ bool tile_span_wide(const float* scs, int lane) {
    static_assert(QT <= 64, "one tile per lane");
    const bool w = lane < QT && (scs[16 * lane] - scs[16 * lane + 15] > 80.f);
    return __ballot(w) != 0ull;
}

// base + e elements with e a 32-bit lane offset.  With a base that is the same
// for the whole wave the compiler keeps the base in scalar registers and
// addresses the access with one vector register holding the byte offset (which
// must stay below 2^32), instead of a 64-bit address per lane.
template <typename T>
__device__ __forceinline__ T* at32(T* base, uint32_t e) {
    typedef typename std::conditional<std::is_const<T>::value, const char, char>::type B;
    return (T*)((B*)base + e * (uint32_t)sizeof(T));
}

// Raw buffer access (gfx9 resource word 3): a resource spans `bytes` bytes from
// `base`; a load at or past that end returns zeros and a store there is
// dropped by the hardware, so lanes outside a row's channels need no branch.
// Offsets are 32-bit: a resource covers one token row at a time.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
template <typename V>
__device__ __forceinline__ V buf_load(__amdgpu_buffer_rsrc_t r, int off) {
    static_assert(sizeof(V) == 4 || sizeof(V) == 8 || sizeof(V) == 16, "buffer access width");
    if constexpr (sizeof(V) == 4)
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    else if constexpr (sizeof(V) == 8)
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    else
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
template <typename V>
__device__ __forceinline__ void buf_store(V v, __amdgpu_buffer_rsrc_t r, int off) {
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    static_assert(sizeof(V) == 8 || sizeof(V) == 16, "buffer access width");
    if constexpr (sizeof(V) == 8)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, v), r, off, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// MFMA fragments.
//
// A 16x16 output tile lives in one wave: lane l holds column (l % 16) and rows
// 4*(l/16) + r, r = 0..3 (one f32x4).  For the operands, lane l holds row (A) or
// column (B) l % 16 and SL "slots" of the k dimension; the k index a slot stands
// for is the caller's choice, as long as A and B use the same map (the product
// sums over k, so any common bijection gives the same result).  The "natural"
// map is k = SL*(l/16) + s, i.e. SL consecutive k per lane (one 16-byte load).
template <typename T> struct Mma;

template <> struct Mma<bf16> {
    static constexpr int SL = 8;   // k slots per lane
    static constexpr int KS = 32;  // k consumed per mma()
    typedef bf16x8 Frag;
    typedef bf16 Elem;
    __device__ static __forceinline__ f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ Frag load(const bf16* p) { return *(const bf16x8*)p; }
    // Same as load, scaled by w[s] per slot (rounded to bf16 once).
    __device__ static __forceinline__ Frag load_scaled(const bf16* p, const float* w) {
        Frag v = *(const bf16x8*)p;
        Frag r;
#pragma unroll
        for (int s = 0; s < 8; ++s) r[s] = (bf16)((float)v[s] * w[s]);
        return r;
    }
    __device__ static __forceinline__ Frag from_f(const float* f) {
        Frag r;
#pragma unroll
        for (int s = 0; s < 8; ++s) r[s] = (bf16)f[s];
        return r;
    }
};

template <> struct Mma<float> {
    static constexpr int SL = 4;
    static constexpr int KS = 16;
    typedef f32x4 Frag;
    typedef float Elem;
    __device__ static __forceinline__ f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
        return c;
    }
    __device__ static __forceinline__ Frag load(const float* p) { return *(const f32x4*)p; }
    __device__ static __forceinline__ Frag load_scaled(const float* p, const float* w) {
        f32x4 v = *(const f32x4*)p;
        return f32x4{v[0] * w[0], v[1] * w[1], v[2] * w[2], v[3] * w[3]};
    }
    __device__ static __forceinline__ Frag from_f(const float* f) {
        return f32x4{f[0], f[1], f[2], f[3]};
    }
};

// (P, N) pairs with compiled kernels, per activation type.  bf16 needs
// N % 32 == 0 (one MFMA consumes 32 of k).  The chunk length and the backward
// narrow this further (chunk_supported, bwd_supported).
#define SSD_F32_SHAPES(X) X(16, 16) X(32, 32) X(64, 64) X(64, 128)
#define SSD_BF16_SHAPES(X) X(32, 64) X(64, 64) X(64, 128)

// Spans of the forward state walk.  One walk workgroup carries the running
// state through a run of chunks in causal order; a segment much longer than
// the others' total work would leave most CUs idle, so the forward walk splits
// each segment into spans of `cps` chunks (the last span of a segment may be
// shorter), walks every span from a zero state and composes the span
// summaries into the segment summary afterwards (the same affine composition
// as the boundary scan: S_out = a_span S_in + S_span).  cps is halved from the
// longest segment's chunk count while the walk grid has fewer than
// WALK_TARGET_BLOCKS workgroups (one per CU on the 256 CUs of an MI355X) and a
// span would keep at least WALK_MIN_SPAN_TOKENS tokens.  A plan with one span
// per segment ("trivial") needs no composition.
constexpr int WALK_TARGET_BLOCKS = 256;
constexpr int WALK_MIN_SPAN_TOKENS = 1024;
struct SpanPlan {
    int cps;                          // chunks per span
    int n;                            // spans over all segments
    int first[SSD_MAX_SEGMENTS + 1];  // first span of each segment; first[nseg] = n
};
// Heads per forward-walk workgroup (two heads of a group share B rows in bf16).
inline int walk_heads_of(const Dims& d, int act) {
    return (act == SSD_BF16 && d.hpg % 2 == 0) ? 2 : 1;
}
inline SpanPlan span_plan(const Dims& d, const SegTab& t, bool split) {
    SpanPlan p = {};
    int maxnc = 1;
    for (int k = 0; k < t.n; ++k) maxnc = (int)(t.len[k] / d.Q) > maxnc ? (int)(t.len[k] / d.Q) : maxnc;
    auto count = [&](int cps) {
        int64_t n = 0;
        for (int k = 0; k < t.n; ++k) n += (t.len[k] / d.Q + cps - 1) / cps;
        return n;
    };
    int cps = maxnc;
    if (split) {
        const int hw = walk_heads_of(d, act_of_dims(d));
        const int min_cps = WALK_MIN_SPAN_TOKENS / d.Q > 1 ? WALK_MIN_SPAN_TOKENS / d.Q : 1;
        while (cps > min_cps && count(cps) * (d.H / hw) * d.batch < WALK_TARGET_BLOCKS)
            cps = (cps + 1) / 2 > min_cps ? (cps + 1) / 2 : min_cps;
    }
    p.cps = cps;
    int n = 0;
    for (int k = 0; k < t.n; ++k) {
        p.first[k] = n;
        n += (int)((t.len[k] / d.Q + cps - 1) / cps);
    }
    p.first[t.n] = n;
    p.n = n;
    return p;
}
inline bool plan_trivial(const SpanPlan& p, const SegTab& t) { return p.n == t.n; }

// Size of the fixed device scratch of ssd_segment_fwd_noalloc (noalloc.hip),
// and its device address on the current device (taken once per device).
constexpr size_t SCRATCH_BYTES = SSD_SCRATCH_BYTES;
hipError_t scratch_address(void** out);

// Host-side launchers (defined in the .hip files).  Each returns hipSuccess or
// the launch error.
hipError_t launch_conv1d_fwd(const Dims& d, const SegTab& t, int act, const void* xBC,
                             const float* w, const int32_t* seq, void* out, hipStream_t s);
// conv + SiLU of channels c0 .. c0 + nc - 1 only, into columns 0 .. nc - 1 of
// `out` (token rows ostr elements apart)
hipError_t launch_conv1d_channels(const Dims& d, const SegTab& t, int act, const void* xBC,
                                  const float* w, const int32_t* seq, int c0, int nc,
                                  int64_t ostr, void* out, hipStream_t s);
// the whole conv pass and dt prep (dt, cumulative sums, chunk totals) in one launch
hipError_t launch_conv1d_dt(const Dims& d, const SegTab& t, int act, const void* xBC,
                            const float* w, const int32_t* seq, void* out, const void* dt_raw,
                            const float* dt_bias, const float* A_log, float* dt_ws, float* cs_ws,
                            float* ctot, hipStream_t s);
hipError_t launch_segment_states(const Dims& d, const SegTab& t, int act, const void* xBC_conv,
                                 const void* dt_raw, const float* dt_bias, const float* A_log,
                                 const int32_t* seq, float* summary, void* ws, hipStream_t s);
// The conv-fused forward: xBC is the raw input, conv_w its [C][W] taps; the B
// and C channels are convolved into the workspace, the x channels are
// recomputed by the walk and the output pass.
hipError_t launch_conv_segment_states(const Dims& d, const SegTab& t, int act, const void* xBC,
                                      const float* conv_w, const void* dt_raw,
                                      const float* dt_bias, const float* A_log,
                                      const int32_t* seq, float* summary, void* ws,
                                      hipStream_t s);
hipError_t launch_conv_segment_output(const Dims& d, const SegTab& t, int act, const void* xBC,
                                      const float* conv_w, const float* D, const int32_t* seq,
                                      const float* S_in, void* ws, void* y, hipStream_t s);
hipError_t launch_segment_output(const Dims& d, const SegTab& t, int act, const void* xBC_conv,
                                 const int32_t* seq, void* ws, float* y_zero, hipStream_t s);
hipError_t launch_segment_output_fused(const Dims& d, const SegTab& t, int act,
                                       const void* xBC_conv, const float* D, const int32_t* seq,
                                       const float* S_in, void* ws, void* y, hipStream_t s);
hipError_t launch_boundary_scan(const Dims& d, int nseg, const float* summary, const float* init,
                                int reverse, float* out, float* final_state, hipStream_t s);
hipError_t launch_apply_init_state(const Dims& d, const SegTab& t, int act, const float* y_zero,
                                   const void* xBC_conv, const float* D, const int32_t* seq,
                                   const float* S_in, const void* ws, void* y, hipStream_t s);
hipError_t launch_span_combine(const Dims& d, const SpanPlan& sp, const float* spsum,
                               float* summary, hipStream_t s);
hipError_t launch_span_scan(const Dims& d, const SpanPlan& sp, const float* spsum,
                            const float* S_in, float* spst, hipStream_t s);
bool kernels_supported(int P, int N, int act);
hipError_t launch_dt_prep(const Dims& d, int act, const void* dt_raw, const float* dt_bias,
                          const float* A_log, const int32_t* seq, float* dt_ws, float* cs_ws,
                          float* ctot, hipStream_t s);

// Arguments of the backward entry points (device pointers).
struct BwdArgs {
    const void* xBC;
    const float* conv_w;
    const void* dt_raw;
    const float* dt_bias;
    const float* A_log;
    const float* D;
    const int32_t* seq;
    const void* dy;
    const float* S_in;
    const float* dS_out;
    void* dxBC;
    void* ddt_raw;
    float* dconv_w;
    float* ddt_bias;
    float* dA_log;
    float* dD;
};
bool bwd_supported(int P, int N, int Q, int act);
bool chunk_supported(int P, int N, int Q, int act);

// Forward workspace layout (byte offsets), shared by the host code and launchers.
// With a non-trivial span plan it also holds the span summaries (S_span then
// a_span, the summary layout over spans) and the state entering every span
// (filled by the output calls).
struct FwdWs {
    size_t dt, cs, ctot, hst, gram, spsum, spst, bc, total;
};
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// The conv-fused forward (xconv) adds the convolved B and C channels,
// [b][L][2 G N] in the activation type, at `bc`.
inline FwdWs fwd_ws_layout(const Dims& d, const SegTab& t, int act, bool xconv = false) {
    FwdWs w;
    const size_t esz = act == SSD_BF16 ? 2 : 4;
    const size_t bhl = (size_t)d.batch * d.H * d.L;
    w.dt = 0;
    w.cs = align256(w.dt + bhl * 4);
    w.ctot = align256(w.cs + bhl * 4);
    w.hst = align256(w.ctot + (size_t)d.batch * d.H * d.nchunk * 4);
    w.gram = align256(w.hst + (size_t)d.batch * d.nchunk * d.H * d.P * d.N * esz);
    const size_t qt = (size_t)d.Q / 16;
    w.spsum = align256(w.gram + (size_t)d.batch * d.nchunk * d.G * (qt * (qt + 1) / 2) * 256 * esz);
    const SpanPlan sp = span_plan(d, t, true);
    const size_t bh = (size_t)d.batch * d.H;
    if (plan_trivial(sp, t)) {
        w.spst = w.spsum;
        w.total = w.spsum;
    } else {
        w.spst = align256(w.spsum + (size_t)sp.n * bh * ((size_t)d.P * d.N + 1) * 4);
        w.total = align256(w.spst + (size_t)sp.n * bh * d.P * d.N * 4);
    }
    w.bc = w.total;
    if (xconv) w.total = align256(w.bc + (size_t)d.batch * d.L * 2 * d.G * d.N * esz);
    return w;
}

// Heads per workgroup of the head-blocked chunk backward: the largest divisor of
// the heads per group up to eight.
inline int head_block(const Dims& d) {
    int hb = 1;
    for (int c = 1; c <= 8; ++c)
        if (d.hpg % c == 0) hb = c;
    return hb;
}

// Backward workspace layout (byte offsets).  The summary phase fills xc, gramt,
// dt, cs and ctot; the pass phase gpn and hpn; the chunk phase dv, dbc, rpart,
// tokp, dotgh and red4; the conv phase dbcs, red and dwp.
struct BwdWs {
    size_t xc, gramt, dt, cs, ctot, gpn, hpn, dv, dbc, dbcs, rpart, tokp, dotgh, red4, red, dwp,
        total;
};
inline BwdWs bwd_ws_layout(const Dims& d, int act) {
    BwdWs w;
    const size_t e = act == SSD_BF16 ? 2 : 4;
    const size_t BL = (size_t)d.batch * d.L;
    const size_t st = (size_t)d.batch * d.nchunk * d.H * d.P * d.N;
    const size_t bhl = (size_t)d.batch * d.H * d.L;
    size_t o = 0;
    w.xc = o;   o = align256(o + BL * d.C * e);
    // causal C_i . B_j tiles per (row, chunk, group), 256 elements each
    const size_t qt = (size_t)d.Q / 16;
    w.gramt = o; o = align256(o + (size_t)d.batch * d.nchunk * d.G * (qt * (qt + 1) / 2) * 256 * e);
    w.dt = o;   o = align256(o + bhl * 4);
    w.cs = o;   o = align256(o + bhl * 4);
    w.ctot = o; o = align256(o + (size_t)d.batch * d.H * d.nchunk * 4);
    w.gpn = o;  o = align256(o + st * e);  // exit gradient per chunk, [p][n]
    w.hpn = o;  o = align256(o + st * e);  // entering state per chunk, [p][n]
    w.dv = o;   o = align256(o + BL * d.H * d.P * e);  // d(conv output), x channels
    w.dbc = o;  o = align256(o + BL * (d.H / head_block(d)) * 2 * d.N * e);  // dB, dC per head block
    w.dbcs = o; o = align256(o + BL * d.G * 2 * d.N * e);  // the same, summed per group
    w.rpart = o; o = align256(o + bhl * 4);
    w.tokp = o; o = align256(o + bhl * 4 * 4);
    w.dotgh = o; o = align256(o + (size_t)d.batch * d.nchunk * d.H * 4);
    w.red4 = o; o = align256(o + (size_t)d.batch * d.nchunk * d.H * 4);
    w.red = o;  o = align256(o + (size_t)d.batch * d.nchunk * d.H * 3 * 4);
    w.dwp = o;  o = align256(o + (size_t)d.batch * (d.L / 64) * d.C * d.W * 4);
    w.total = o;
    return w;
}

hipError_t launch_bwd_summary(const Dims& d, const SegTab& t, int act, const BwdArgs& a,
                              float* summary, void* ws, hipStream_t s);
hipError_t launch_bwd_pass(const Dims& d, const SegTab& t, int act, const BwdArgs& a, void* ws,
                           hipStream_t s);
hipError_t launch_bwd_chunks(const Dims& d, const SegTab& t, int act, const BwdArgs& a, void* ws,
                             hipStream_t s);
hipError_t launch_conv1d_bwd(const Dims& d, const SegTab& t, int act, const BwdArgs& a, void* ws,
                             hipStream_t s);

}  // namespace ssd
