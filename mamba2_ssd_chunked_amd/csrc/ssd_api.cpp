// Host side of the C ABI declared in include/ssd.h: argument validation and
// kernel dispatch.  Every check runs before anything is enqueued, so an
// invalid call returns a negative ssd_status and leaves the stream untouched.
// Megatron-LM #6808 (description section "Not supported yet") likewise refuses
// unsupported configurations outright instead of computing something wrong.
#include <climits>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <utility>
#include <vector>

#include "ssd_internal.h"

using namespace ssd;

namespace {

bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

// Every launch grid of the library fits the dispatch limits: at most 2^32 - 1
// work-items and 2^31 - 1 workgroups along x, at most 65535 workgroups along y
// and z.  The grids are those of the launchers (conv1d.hip, gram.h, state_walk.h,
// ssd_fwd.hip, scan.hip, ssd_bwd.hip), computed here in 128-bit arithmetic so
// that no product overflows; a problem whose grids do not fit is rejected
// before anything is enqueued.
bool grids_fit(const ssd_problem* p, int64_t C) {
    typedef unsigned __int128 u128;
    const u128 b = (u128)p->batch, L = (u128)p->seqlen, H = (u128)p->nheads;
    const u128 G = (u128)p->ngroups, Q = (u128)p->chunk, nc = L / Q;
    const u128 nseg = SSD_MAX_SEGMENTS;
    const u128 PN = (u128)p->headdim * (u128)p->dstate, CC = (u128)C;
    auto x_ok = [](u128 blocks, u128 threads) {
        return blocks <= 0x7fffffffu && blocks * threads <= 0xffffffffu;
    };
    const u128 cx = (CC + 255) / 256;  // conv workgroups along channels
    bool ok = x_ok(cx, 256) && L / 64 <= 65535 && b <= 65535;                   // conv forward
    const u128 ty = L / 64 > 0 ? L / 64 : 1;
    ok = ok && x_ok(cx + (nc * ((H + 7) / 8) + ty - 1) / ty, 256);                // conv + dt prep
    ok = ok && x_ok(nc * G * b * (Q / 32), Q / 32 * 64);                           // Gram + dt prep
    ok = ok && x_ok(2 * H * nseg * b, 512);                                        // state walks
    ok = ok && x_ok(nc * H * b, 512);                                              // output passes
    ok = ok && x_ok((b * H * PN / 4 + 255) / 256, 256);                            // boundary scan
    ok = ok && nc <= 0x7fffffffu && (H + 7) / 8 <= 65535;                         // dt prep alone
    ok = ok && x_ok((b * L * G * 2 * (u128)p->dstate / 4 + 255) / 256, 256);       // dB, dC sums
    ok = ok && x_ok(cx * (L / 64) * b + (nc * H * b + 3) / 4, 256);                // conv backward
    ok = ok && x_ok((CC * (u128)p->conv_width + 3 * H + 31) / 32, 256);            // reductions
    return ok;
}

// Validates the problem and fills Dims.  Returns SSD_OK or an error.
int check_problem(const ssd_problem* p, Dims* d) {
    if (!p) return SSD_ERR_NULL;
    if (p->batch < 1 || p->seqlen < 1 || p->nheads < 1 || p->headdim < 1 || p->dstate < 1 ||
        p->ngroups < 1 || p->conv_width < 1)
        return SSD_ERR_SHAPE;
    if (p->nheads % p->ngroups != 0) return SSD_ERR_SHAPE;
    if (p->act_dtype != SSD_F32 && p->act_dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (!(p->dt_min >= 0.f) || !(p->dt_max >= p->dt_min)) return SSD_ERR_SHAPE;
    if (p->chunk != 64 && p->chunk != 128 && p->chunk != 256) return SSD_ERR_UNSUPPORTED;
    if (p->conv_width > 8) return SSD_ERR_UNSUPPORTED;
    if (p->seqlen % p->chunk != 0) return SSD_ERR_SHAPE;
    if (!kernels_supported(p->headdim, p->dstate, p->act_dtype)) return SSD_ERR_UNSUPPORTED;
    if (!chunk_supported(p->headdim, p->dstate, p->chunk, p->act_dtype)) return SSD_ERR_UNSUPPORTED;
    if (p->batch > 65535 || p->nheads > 65535 || p->seqlen > INT32_MAX) return SSD_ERR_SHAPE;
    const int64_t C = (int64_t)p->nheads * p->headdim + 2LL * p->ngroups * p->dstate;
    const int64_t esz = p->act_dtype == SSD_BF16 ? 2 : 4;
    // the token rows of one chunk of xBC must be addressable with 32-bit byte
    // offsets (the conv backward's buffer accesses, the chunk backward's lane
    // offsets), and every launch grid must fit
    if (C * esz * p->chunk > INT32_MAX) return SSD_ERR_SHAPE;
    if (!grids_fit(p, C)) return SSD_ERR_SHAPE;
    d->batch = p->batch;
    d->L = p->seqlen;
    d->H = p->nheads;
    d->P = p->headdim;
    d->N = p->dstate;
    d->G = p->ngroups;
    d->Q = p->chunk;
    d->W = p->conv_width;
    d->C = (int)C;
    d->hpg = p->nheads / p->ngroups;
    d->nchunk = (int)(p->seqlen / p->chunk);
    d->nseg = 0;
    d->act = p->act_dtype;
    d->dt_min = p->dt_min;
    d->dt_max = p->dt_max;
    return SSD_OK;
}

// Segments must tile [0, L) with chunk-aligned starts and lengths.
int check_segments(const ssd_segment* segs, int32_t nseg, Dims* d, SegTab* t) {
    if (!segs) return SSD_ERR_NULL;
    if (nseg < 1 || nseg > SSD_MAX_SEGMENTS) return SSD_ERR_SEGMENTS;
    std::vector<std::pair<int64_t, int64_t>> v;
    int64_t total = 0;
    std::memset(t, 0, sizeof(*t));
    for (int i = 0; i < nseg; ++i) {
        const int64_t s = segs[i].start, l = segs[i].len;
        if (l < 1 || s < 0 || s + l > d->L || s % d->Q != 0 || l % d->Q != 0)
            return SSD_ERR_SEGMENTS;
        v.emplace_back(s, l);
        total += l;
        t->start[i] = s;
        t->len[i] = l;
    }
    if (total != d->L) return SSD_ERR_SEGMENTS;
    std::sort(v.begin(), v.end());
    int64_t pos = 0;
    for (auto& e : v) {
        if (e.first != pos) return SSD_ERR_SEGMENTS;
        pos += e.second;
    }
    t->n = nseg;
    d->nseg = nseg;
    return SSD_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

}  // namespace

extern "C" {

const char* ssd_status_string(int status) {
    switch (status) {
        case SSD_OK: return "ok";
        case SSD_ERR_NULL: return "a required pointer is NULL";
        case SSD_ERR_SHAPE: return "inconsistent or out-of-range sizes";
        case SSD_ERR_UNSUPPORTED: return "no kernel for this (headdim, dstate, chunk, dtype, conv width)";
        case SSD_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case SSD_ERR_WORKSPACE: return "workspace missing or too small";
        case SSD_ERR_HIP: return "HIP launch error";
        case SSD_ERR_SEGMENTS: return "segment table does not tile the sequence in chunk units";
        case SSD_ERR_SCRATCH: return "problem needs more workspace than the fixed 64 MiB device scratch";
        default: return "unknown status";
    }
}

int32_t ssd_abi_version(void) { return 3; }

int32_t ssd_supported(int32_t headdim, int32_t dstate, int32_t act_dtype) {
    return kernels_supported(headdim, dstate, act_dtype) ? 1 : 0;
}

size_t ssd_workspace_bytes(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                           int32_t kind) {
    Dims d;
    SegTab t;
    if (check_problem(problem, &d) != SSD_OK) return 0;
    if (check_segments(segs, nseg, &d, &t) != SSD_OK) return 0;
    if (kind == SSD_WS_FORWARD) return fwd_ws_layout(d, t, problem->act_dtype).total;
    if (kind == SSD_WS_FORWARD_CONV) {
        if (d.W != FUSED_CONV_W) return 0;
        return fwd_ws_layout(d, t, problem->act_dtype, true).total;
    }
    if (kind == SSD_WS_BACKWARD) {
        if (!bwd_supported(d.P, d.N, d.Q, problem->act_dtype)) return 0;
        return bwd_ws_layout(d, problem->act_dtype).total;
    }
    return 0;
}

int ssd_conv1d_fwd(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                   const void* xBC, const float* conv_w, const int32_t* seq_idx, void* xBC_conv,
                   void* stream) {
    Dims d;
    SegTab t;
    int rc = check_problem(problem, &d);
    if (rc) return rc;
    if ((rc = check_segments(segs, nseg, &d, &t))) return rc;
    if (!xBC || !conv_w || !xBC_conv) return SSD_ERR_NULL;
    if (!aligned16(xBC) || !aligned16(conv_w) || !aligned16(seq_idx) || !aligned16(xBC_conv))
        return SSD_ERR_ALIGN;
    return hip_status(launch_conv1d_fwd(d, t, problem->act_dtype, xBC, conv_w, seq_idx, xBC_conv,
                                        (hipStream_t)stream));
}

namespace {
int check_states_args(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                      const void* xBC_conv, const void* dt_raw, const float* dt_bias,
                      const float* A_log, const int32_t* seq_idx, const float* summary,
                      const void* ws, size_t ws_bytes, Dims* d, SegTab* t) {
    int rc = check_problem(problem, d);
    if (rc) return rc;
    if ((rc = check_segments(segs, nseg, d, t))) return rc;
    if (!xBC_conv || !dt_raw || !dt_bias || !A_log || !summary) return SSD_ERR_NULL;
    if (!ws) return SSD_ERR_WORKSPACE;
    if (ws_bytes < fwd_ws_layout(*d, *t, problem->act_dtype).total) return SSD_ERR_WORKSPACE;
    if (!aligned16(xBC_conv) || !aligned16(dt_raw) || !aligned16(dt_bias) || !aligned16(A_log) ||
        !aligned16(seq_idx) || !aligned16(summary) || !aligned16(ws))
        return SSD_ERR_ALIGN;
    return SSD_OK;
}

int check_output_args(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                      const void* xBC_conv, const int32_t* seq_idx, const void* ws,
                      size_t ws_bytes, const float* y_zero, Dims* d, SegTab* t) {
    int rc = check_problem(problem, d);
    if (rc) return rc;
    if ((rc = check_segments(segs, nseg, d, t))) return rc;
    if (!xBC_conv || !y_zero) return SSD_ERR_NULL;
    if (!ws) return SSD_ERR_WORKSPACE;
    if (ws_bytes < fwd_ws_layout(*d, *t, problem->act_dtype).total) return SSD_ERR_WORKSPACE;
    if (!aligned16(xBC_conv) || !aligned16(seq_idx) || !aligned16(ws) || !aligned16(y_zero))
        return SSD_ERR_ALIGN;
    return SSD_OK;
}
}  // namespace

int ssd_segment_states(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                       const void* xBC_conv, const void* dt_raw, const float* dt_bias,
                       const float* A_log, const int32_t* seq_idx, float* summary, void* ws,
                       size_t ws_bytes, void* stream) {
    Dims d;
    SegTab t;
    int rc = check_states_args(problem, segs, nseg, xBC_conv, dt_raw, dt_bias, A_log, seq_idx,
                               summary, ws, ws_bytes, &d, &t);
    if (rc) return rc;
    return hip_status(launch_segment_states(d, t, problem->act_dtype, xBC_conv, dt_raw, dt_bias,
                                            A_log, seq_idx, summary, ws, (hipStream_t)stream));
}

int ssd_segment_output(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                       const void* xBC_conv, const int32_t* seq_idx, void* ws,
                       size_t ws_bytes, float* y_zero, void* stream) {
    Dims d;
    SegTab t;
    int rc = check_output_args(problem, segs, nseg, xBC_conv, seq_idx, ws, ws_bytes, y_zero, &d,
                               &t);
    if (rc) return rc;
    return hip_status(launch_segment_output(d, t, problem->act_dtype, xBC_conv, seq_idx, ws, y_zero,
                                            (hipStream_t)stream));
}

int ssd_segment_fwd(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                    const void* xBC_conv, const void* dt_raw, const float* dt_bias,
                    const float* A_log, const int32_t* seq_idx, float* y_zero, float* summary,
                    void* ws, size_t ws_bytes, void* stream) {
    Dims d;
    SegTab t;
    int rc = check_states_args(problem, segs, nseg, xBC_conv, dt_raw, dt_bias, A_log, seq_idx,
                               summary, ws, ws_bytes, &d, &t);
    if (rc) return rc;
    if ((rc = check_output_args(problem, segs, nseg, xBC_conv, seq_idx, ws, ws_bytes, y_zero, &d,
                                &t)))
        return rc;
    rc = hip_status(launch_segment_states(d, t, problem->act_dtype, xBC_conv, dt_raw, dt_bias,
                                          A_log, seq_idx, summary, ws, (hipStream_t)stream));
    if (rc) return rc;
    return hip_status(launch_segment_output(d, t, problem->act_dtype, xBC_conv, seq_idx, ws, y_zero,
                                            (hipStream_t)stream));
}

int ssd_segment_fwd_noalloc(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                            const void* xBC_conv, const void* dt_raw, const float* dt_bias,
                            const float* A_log, const int32_t* seq_idx, float* y_zero,
                            float* summary, void* stream) {
    Dims d;
    SegTab t;
    int rc = check_problem(problem, &d);
    if (rc) return rc;
    if ((rc = check_segments(segs, nseg, &d, &t))) return rc;
    if (!xBC_conv || !dt_raw || !dt_bias || !A_log || !summary || !y_zero) return SSD_ERR_NULL;
    if (!aligned16(xBC_conv) || !aligned16(dt_raw) || !aligned16(dt_bias) || !aligned16(A_log) ||
        !aligned16(seq_idx) || !aligned16(summary) || !aligned16(y_zero))
        return SSD_ERR_ALIGN;
    if (fwd_ws_layout(d, t, problem->act_dtype).total > SCRATCH_BYTES) return SSD_ERR_SCRATCH;
    void* ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return SSD_ERR_HIP;
    // every byte of the workspace the two phases read is written earlier in the
    // same call, so the scratch needs no clearing
    rc = hip_status(launch_segment_states(d, t, problem->act_dtype, xBC_conv, dt_raw, dt_bias,
                                          A_log, seq_idx, summary, ws, (hipStream_t)stream));
    if (rc) return rc;
    return hip_status(launch_segment_output(d, t, problem->act_dtype, xBC_conv, seq_idx, ws, y_zero,
                                            (hipStream_t)stream));
}

int ssd_boundary_scan(const ssd_problem* problem, int32_t nseg, const float* summary,
                      const float* init, int32_t reverse, float* out, float* final_state,
                      void* stream) {
    Dims d;
    int rc = check_problem(problem, &d);
    if (rc) return rc;
    if (nseg < 1 || nseg > SSD_MAX_SEGMENTS) return SSD_ERR_SEGMENTS;
    if (reverse != 0 && reverse != 1) return SSD_ERR_SHAPE;
    if (!summary || !out) return SSD_ERR_NULL;
    if (!aligned16(summary) || !aligned16(init) || !aligned16(out) || !aligned16(final_state))
        return SSD_ERR_ALIGN;
    return hip_status(
        launch_boundary_scan(d, nseg, summary, init, reverse, out, final_state, (hipStream_t)stream));
}

int ssd_apply_init_state(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                         const float* y_zero, const void* xBC_conv, const float* D,
                         const int32_t* seq_idx, const float* S_in, const void* ws,
                         size_t ws_bytes, void* y, void* stream) {
    Dims d;
    SegTab t;
    int rc = check_problem(problem, &d);
    if (rc) return rc;
    if ((rc = check_segments(segs, nseg, &d, &t))) return rc;
    if (!y_zero || !xBC_conv || !D || !S_in || !y) return SSD_ERR_NULL;
    if (!ws) return SSD_ERR_WORKSPACE;
    if (ws_bytes < fwd_ws_layout(d, t, problem->act_dtype).total) return SSD_ERR_WORKSPACE;
    if (!aligned16(y_zero) || !aligned16(xBC_conv) || !aligned16(D) || !aligned16(seq_idx) ||
        !aligned16(S_in) || !aligned16(ws) || !aligned16(y))
        return SSD_ERR_ALIGN;
    return hip_status(launch_apply_init_state(d, t, problem->act_dtype, y_zero, xBC_conv, D,
                                              seq_idx, S_in, ws, y, (hipStream_t)stream));
}

int ssd_segment_output_fused(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                             const void* xBC_conv, const float* D, const int32_t* seq_idx,
                             const float* S_in, void* ws, size_t ws_bytes, void* y,
                             void* stream) {
    Dims d;
    SegTab t;
    int rc = check_problem(problem, &d);
    if (rc) return rc;
    if ((rc = check_segments(segs, nseg, &d, &t))) return rc;
    if (!xBC_conv || !D || !S_in || !y) return SSD_ERR_NULL;
    if (!ws) return SSD_ERR_WORKSPACE;
    if (ws_bytes < fwd_ws_layout(d, t, problem->act_dtype).total) return SSD_ERR_WORKSPACE;
    if (!aligned16(xBC_conv) || !aligned16(D) || !aligned16(seq_idx) || !aligned16(S_in) ||
        !aligned16(ws) || !aligned16(y))
        return SSD_ERR_ALIGN;
    return hip_status(launch_segment_output_fused(d, t, problem->act_dtype, xBC_conv, D, seq_idx,
                                                  S_in, ws, y, (hipStream_t)stream));
}

int ssd_conv_segment_states(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                            const void* xBC, const float* conv_w, const void* dt_raw,
                            const float* dt_bias, const float* A_log, const int32_t* seq_idx,
                            float* summary, void* ws, size_t ws_bytes, void* stream) {
    Dims d;
    SegTab t;
    int rc = check_problem(problem, &d);
    if (rc) return rc;
    if ((rc = check_segments(segs, nseg, &d, &t))) return rc;
    if (d.W != FUSED_CONV_W) return SSD_ERR_UNSUPPORTED;
    if (!xBC || !conv_w || !dt_raw || !dt_bias || !A_log || !summary) return SSD_ERR_NULL;
    if (!ws) return SSD_ERR_WORKSPACE;
    if (ws_bytes < fwd_ws_layout(d, t, problem->act_dtype, true).total) return SSD_ERR_WORKSPACE;
    if (!aligned16(xBC) || !aligned16(conv_w) || !aligned16(dt_raw) || !aligned16(dt_bias) ||
        !aligned16(A_log) || !aligned16(seq_idx) || !aligned16(summary) || !aligned16(ws))
        return SSD_ERR_ALIGN;
    return hip_status(launch_conv_segment_states(d, t, problem->act_dtype, xBC, conv_w, dt_raw,
                                                 dt_bias, A_log, seq_idx, summary, ws,
                                                 (hipStream_t)stream));
}

int ssd_conv_segment_output(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                            const void* xBC, const float* conv_w, const float* D,
                            const int32_t* seq_idx, const float* S_in, void* ws,
                            size_t ws_bytes, void* y, void* stream) {
    Dims d;
    SegTab t;
    int rc = check_problem(problem, &d);
    if (rc) return rc;
    if ((rc = check_segments(segs, nseg, &d, &t))) return rc;
    if (d.W != FUSED_CONV_W) return SSD_ERR_UNSUPPORTED;
    if (!xBC || !conv_w || !D || !S_in || !y) return SSD_ERR_NULL;
    if (!ws) return SSD_ERR_WORKSPACE;
    if (ws_bytes < fwd_ws_layout(d, t, problem->act_dtype, true).total) return SSD_ERR_WORKSPACE;
    if (!aligned16(xBC) || !aligned16(conv_w) || !aligned16(D) || !aligned16(seq_idx) ||
        !aligned16(S_in) || !aligned16(ws) || !aligned16(y))
        return SSD_ERR_ALIGN;
    return hip_status(launch_conv_segment_output(d, t, problem->act_dtype, xBC, conv_w, D,
                                                 seq_idx, S_in, ws, y, (hipStream_t)stream));
}

int ssd_segment_bwd_summary(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                            const void* xBC, const float* conv_w, const void* dt_raw,
                            const float* dt_bias, const float* A_log, const int32_t* seq_idx,
                            const void* dy, float* summary, void* ws, size_t ws_bytes,
                            void* stream) {
    Dims d;
    SegTab t;
    int rc = check_problem(problem, &d);
    if (rc) return rc;
    if ((rc = check_segments(segs, nseg, &d, &t))) return rc;
    if (!bwd_supported(d.P, d.N, d.Q, problem->act_dtype)) return SSD_ERR_UNSUPPORTED;
    if (!xBC || !conv_w || !dt_raw || !dt_bias || !A_log || !dy || !summary) return SSD_ERR_NULL;
    if (!ws) return SSD_ERR_WORKSPACE;
    if (ws_bytes < bwd_ws_layout(d, problem->act_dtype).total) return SSD_ERR_WORKSPACE;
    if (!aligned16(xBC) || !aligned16(conv_w) || !aligned16(dt_raw) || !aligned16(dt_bias) ||
        !aligned16(A_log) || !aligned16(seq_idx) || !aligned16(dy) || !aligned16(summary) ||
        !aligned16(ws))
        return SSD_ERR_ALIGN;
    BwdArgs ar = {};
    ar.xBC = xBC;
    ar.conv_w = conv_w;
    ar.dt_raw = dt_raw;
    ar.dt_bias = dt_bias;
    ar.A_log = A_log;
    ar.seq = seq_idx;
    ar.dy = dy;
    return hip_status(launch_bwd_summary(d, t, problem->act_dtype, ar, summary, ws,
                                         (hipStream_t)stream));
}

namespace {
// Common checks of the chunk and conv phases of the backward.
int check_bwd(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg, Dims* d,
              SegTab* t, const void* ws, size_t ws_bytes) {
    int rc = check_problem(problem, d);
    if (rc) return rc;
    if ((rc = check_segments(segs, nseg, d, t))) return rc;
    if (!bwd_supported(d->P, d->N, d->Q, problem->act_dtype)) return SSD_ERR_UNSUPPORTED;
    if (!ws) return SSD_ERR_WORKSPACE;
    if (ws_bytes < bwd_ws_layout(*d, problem->act_dtype).total) return SSD_ERR_WORKSPACE;
    if (!aligned16(ws)) return SSD_ERR_ALIGN;
    return SSD_OK;
}
}  // namespace

int ssd_segment_bwd_pass(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                         const int32_t* seq_idx, const void* dy, const float* S_in,
                         const float* dS_out, void* ws, size_t ws_bytes, void* stream) {
    Dims d;
    SegTab t;
    int rc = check_bwd(problem, segs, nseg, &d, &t, ws, ws_bytes);
    if (rc) return rc;
    if (!dy || !S_in || !dS_out) return SSD_ERR_NULL;
    if (!aligned16(seq_idx) || !aligned16(dy) || !aligned16(S_in) || !aligned16(dS_out))
        return SSD_ERR_ALIGN;
    BwdArgs ar = {};
    ar.seq = seq_idx;
    ar.dy = dy;
    ar.S_in = S_in;
    ar.dS_out = dS_out;
    return hip_status(launch_bwd_pass(d, t, problem->act_dtype, ar, ws, (hipStream_t)stream));
}

int ssd_segment_bwd_chunks(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                           const float* D, const int32_t* seq_idx, const void* dy, void* ws,
                           size_t ws_bytes, void* stream) {
    Dims d;
    SegTab t;
    int rc = check_bwd(problem, segs, nseg, &d, &t, ws, ws_bytes);
    if (rc) return rc;
    if (!D || !dy) return SSD_ERR_NULL;
    if (!aligned16(D) || !aligned16(seq_idx) || !aligned16(dy)) return SSD_ERR_ALIGN;
    BwdArgs ar = {};
    ar.D = D;
    ar.seq = seq_idx;
    ar.dy = dy;
    return hip_status(launch_bwd_chunks(d, t, problem->act_dtype, ar, ws, (hipStream_t)stream));
}

int ssd_conv1d_bwd(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                   const void* xBC, const float* conv_w, const void* dt_raw, const float* dt_bias,
                   const float* A_log, const int32_t* seq_idx, void* ws, size_t ws_bytes,
                   void* dxBC, void* ddt_raw, float* dconv_w, float* ddt_bias, float* dA_log,
                   float* dD, void* stream) {
    Dims d;
    SegTab t;
    int rc = check_bwd(problem, segs, nseg, &d, &t, ws, ws_bytes);
    if (rc) return rc;
    if (!xBC || !conv_w || !dt_raw || !dt_bias || !A_log || !dxBC || !ddt_raw || !dconv_w ||
        !ddt_bias || !dA_log || !dD)
        return SSD_ERR_NULL;
    const void* ptrs[] = {xBC,  conv_w,  dt_raw,  dt_bias,  A_log,  seq_idx,
                          dxBC, ddt_raw, dconv_w, ddt_bias, dA_log, dD};
    for (const void* q : ptrs)
        if (!aligned16(q)) return SSD_ERR_ALIGN;
    BwdArgs ar = {};
    ar.xBC = xBC;
    ar.conv_w = conv_w;
    ar.dt_raw = dt_raw;
    ar.dt_bias = dt_bias;
    ar.A_log = A_log;
    ar.seq = seq_idx;
    ar.dxBC = dxBC;
    ar.ddt_raw = ddt_raw;
    ar.dconv_w = dconv_w;
    ar.ddt_bias = ddt_bias;
    ar.dA_log = dA_log;
    ar.dD = dD;
    return hip_status(launch_conv1d_bwd(d, t, problem->act_dtype, ar, ws, (hipStream_t)stream));
}

int ssd_segment_bwd(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                    const void* xBC, const float* conv_w, const void* dt_raw, const float* dt_bias,
                    const float* A_log, const float* D, const int32_t* seq_idx, const void* dy,
                    const float* S_in, const float* dS_out, void* ws, size_t ws_bytes, void* dxBC,
                    void* ddt_raw, float* dconv_w, float* ddt_bias, float* dA_log, float* dD,
                    void* stream) {
    Dims d;
    SegTab t;
    int rc = check_bwd(problem, segs, nseg, &d, &t, ws, ws_bytes);
    if (rc) return rc;
    if (!xBC || !conv_w || !dt_raw || !dt_bias || !A_log || !D || !dy || !S_in || !dS_out ||
        !dxBC || !ddt_raw || !dconv_w || !ddt_bias || !dA_log || !dD)
        return SSD_ERR_NULL;
    const void* ptrs[] = {xBC, conv_w, dt_raw, dt_bias, A_log, D, seq_idx, dy, S_in, dS_out,
                          dxBC, ddt_raw, dconv_w, ddt_bias, dA_log, dD};
    for (const void* q : ptrs)
        if (!aligned16(q)) return SSD_ERR_ALIGN;
    BwdArgs ar = {xBC, conv_w, dt_raw, dt_bias, A_log, D, seq_idx, dy, S_in, dS_out,
                  dxBC, ddt_raw, dconv_w, ddt_bias, dA_log, dD};
    rc = hip_status(launch_bwd_pass(d, t, problem->act_dtype, ar, ws, (hipStream_t)stream));
    if (rc) return rc;
    rc = hip_status(launch_bwd_chunks(d, t, problem->act_dtype, ar, ws, (hipStream_t)stream));
    if (rc) return rc;
    return hip_status(launch_conv1d_bwd(d, t, problem->act_dtype, ar, ws, (hipStream_t)stream));
}

}  // extern "C"
