/*
 * ssd.h - C ABI of the MI355X (gfx950) Mamba2 conv1d + SSD state-passing library.
 *
 * The operation (Megatron-LM pull request #6808, "Add state-passing context
 * parallelism for Mamba2", first commit message and the description section
 * "Mamba2 state-passing context parallelism"): a sequence is cut into causal
 * segments.  Each segment runs the causal depthwise conv (reading a halo of
 * W-1 tokens from its causal predecessor) and the SSD chunked scan under a zero
 * initial state, and emits an FP32 summary (final state S_ext, block decay
 * a_block).  Because a segment's SSD map is affine in its initial state,
 * S_out = a_block * S_in + S_ext, an exclusive causal scan over the summaries
 * recovers every segment's true initial state S_in, after which the term
 * C_t * decay_t * S_in is added to that segment's outputs.  The backward pass
 * mirrors this with a reverse scan and recomputes sequence-length-sized
 * intermediates instead of storing them.  On one GPU the segments are the
 * shards one device would hold, at their real shape.
 *
 * Model (per row b, head h, token t in causal order; the Mamba-2 selective SSM):
 *   v      = SiLU(causal depthwise conv(xBC))        channels [x (H*P) | B (G*N) | C (G*N)]
 *   dt_t   = clamp(softplus(dt_raw[t,h] + dt_bias[h]), dt_min, dt_max)
 *   A      = -exp(A_log[h]);  head h reads group g = h / (H/G)
 *   h_t    = exp(dt_t A) h_{t-1} + dt_t x_t B_t^T     (decay exactly 0 where a packed
 *   y_t    = h_t C_t + D[h] x_t                        sequence starts: seq_idx changes)
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is a device pointer to contiguous memory, 16-byte
 *    aligned, owned by the caller.  The library never allocates, frees or
 *    synchronises; all work is enqueued on `stream` (a hipStream_t, NULL = the
 *    default stream) and the call returns without waiting.
 *  - Token arrays are [batch][seqlen][...] in *memory order*.  The segment table
 *    lists segments in causal order; `start` is the segment's memory offset.
 *    Segments must tile [0, seqlen): disjoint, every `start` and `len` a
 *    multiple of `chunk`, lengths summing to seqlen.  The same table applies to
 *    every row.  This covers contiguous shards and the "virtual" front/back
 *    layout in which memory order differs from causal order (description
 *    section "Why virtual is the mode to prefer").
 *  - seq_idx (optional, int32 [batch][seqlen], memory order) must be
 *    non-decreasing along each row in causal order.  Token t starts a new packed
 *    sequence when seq_idx differs from its causal predecessor's; conv taps and
 *    state decays never cross such a start (they are exactly zero).  This is
 *    the seq_idx-from-cu_seqlens reset of NeMo Automodel pull request #1441,
 *    "Key changes"; Megatron-LM #6808 rejects packing ("Not supported yet"),
 *    this library supports it.
 *  - Activation tensors (xBC, xBC_conv, dt_raw, y, dy, dxBC, ddt_raw) use
 *    problem->act_dtype; parameters, states, summaries, y_zero and every
 *    parameter gradient are float32.
 *  - Outputs are overwritten, never accumulated.
 *  - Errors: all arguments, and every launch grid the call will need, are
 *    checked on the host before anything is enqueued; on such an error the
 *    function returns a negative ssd_status and enqueues nothing.  A launch
 *    that the HIP runtime refuses returns SSD_ERR_HIP.  A call made of several
 *    launches stops at the first refused one: the launches before it stay
 *    enqueued, so the outputs are then undefined.
 *  - Calls are re-entrant and hold no global state.
 */
#ifndef MI355X_SSD_H
#define MI355X_SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_MAX_SEGMENTS 64

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL = -1,        /* a required pointer is NULL                       */
    SSD_ERR_SHAPE = -2,       /* inconsistent sizes                               */
    SSD_ERR_UNSUPPORTED = -3, /* valid problem the library has no kernel for      */
    SSD_ERR_ALIGN = -4,       /* a tensor pointer is not 16-byte aligned           */
    SSD_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required        */
    SSD_ERR_HIP = -6,         /* the HIP runtime reported an error at launch       */
    SSD_ERR_SEGMENTS = -7,    /* the segment table does not tile the sequence      */
    SSD_ERR_SCRATCH = -8      /* the problem needs more than the fixed scratch     */
} ssd_status;

typedef struct {
    int64_t batch;      /* rows; a packed (THD) batch is one row                 */
    int64_t seqlen;     /* tokens per row (THD: total tokens)                    */
    int32_t nheads;     /* H                                                     */
    int32_t headdim;    /* P                                                     */
    int32_t dstate;     /* N                                                     */
    int32_t ngroups;    /* G, H % G == 0                                         */
    int32_t chunk;      /* Q: SSD chunk length, 64, 128 or 256                   */
    int32_t conv_width; /* W, 1..8                                               */
    int32_t act_dtype;  /* ssd_dtype of the activation tensors                   */
    float dt_min;       /* clamp bounds of dt, 0 <= dt_min <= dt_max             */
    float dt_max;
} ssd_problem;
/* Size limits (SSD_ERR_SHAPE beyond them): with C = nheads * headdim + 2 *
 * ngroups * dstate channels, chunk * C * sizeof(activation) < 2^31 bytes;
 * batch and nheads <= 65535; seqlen <= 2^31 - 1; and every launch grid within
 * the hardware's limits. */

typedef struct {
    int64_t start; /* memory offset of the segment's first token            */
    int64_t len;   /* tokens                                                 */
} ssd_segment;

/* Workspace kinds for ssd_workspace_bytes. */
enum { SSD_WS_FORWARD = 0, SSD_WS_BACKWARD = 1, SSD_WS_FORWARD_CONV = 2 };

/* Human-readable text for an ssd_status value (static storage). */
const char* ssd_status_string(int status);

/* Library ABI version (increments on incompatible changes). */
int32_t ssd_abi_version(void);

/* Returns 1 when (headdim, dstate, act_dtype) has compiled kernels, else 0:
 * float32 (16, 16), (32, 32), (64, 64), (64, 128); bf16 (32, 64), (64, 64),
 * (64, 128).  Every chunk length runs the forward; the backward runs every
 * bf16 pair at every chunk length and the float32 pairs at chunks 64 and 128
 * (ssd_workspace_bytes(..., SSD_WS_BACKWARD) is 0 for the rest, and the
 * backward calls return SSD_ERR_UNSUPPORTED). */
int32_t ssd_supported(int32_t headdim, int32_t dstate, int32_t act_dtype);

/* Bytes of device workspace the forward (SSD_WS_FORWARD: ssd_segment_fwd, read
 * again by ssd_apply_init_state), conv-fused forward (SSD_WS_FORWARD_CONV:
 * ssd_conv_segment_states and ssd_conv_segment_output) or backward
 * (SSD_WS_BACKWARD) calls need for this problem.  Returns 0 for an invalid
 * problem or kind, and for SSD_WS_FORWARD_CONV when conv_width is not 4. */
size_t ssd_workspace_bytes(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                           int32_t kind);

/* Causal depthwise conv1d + SiLU over every channel of xBC.
 * Each segment's first W-1 taps read the last W-1 tokens of its causal
 * predecessor segment (the conv halo exchanged between shards in #6808's first commit); the
 * first segment sees zeros before the row start.
 *   xBC       [batch][seqlen][C] act_dtype, C = H*P + 2*G*N   (in)
 *   conv_w    [C][W] float32; conv_w[c][W-1] multiplies the current token (in)
 *   seq_idx   [batch][seqlen] int32 or NULL                     (in)
 *   xBC_conv  [batch][seqlen][C] act_dtype                      (out)        */
int ssd_conv1d_fwd(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                   const void* xBC, const float* conv_w, const int32_t* seq_idx,
                   void* xBC_conv, void* stream);

/* Segment-local SSD under a zero initial state, plus each segment's summary.
 * Computes, per chunk, the intra-chunk term (C B^T masked by the segment-sum
 * decay, times dt x), the chunk states B^T (decay * dt * x), the FP32 walk of
 * states across the chunks of a segment (the decay-weighted sum of all earlier
 * chunk states that state-spaces/mamba issue #482 singles out as the part that
 * must cross devices), and the inter-chunk output term.
 *   xBC_conv  [batch][seqlen][C] act_dtype (output of ssd_conv1d_fwd)   (in)
 *   dt_raw    [batch][seqlen][H] act_dtype                               (in)
 *   dt_bias, A_log  [H] float32                                          (in)
 *   seq_idx   [batch][seqlen] int32 or NULL                              (in)
 *   y_zero    [batch][seqlen][H][P] float32: SSM output with every
 *             segment started from a zero state, without D*x             (out)
 *   summary   float32: S_ext [nseg][batch][H][P][N] (segment index in
 *             causal order) followed by a_block [nseg][batch][H]         (out)
 *   ws        ssd_workspace_bytes(..., SSD_WS_FORWARD) bytes; keeps dt and
 *             cumulative decays that ssd_apply_init_state reads again    (out)  */
int ssd_segment_fwd(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                    const void* xBC_conv, const void* dt_raw, const float* dt_bias,
                    const float* A_log, const int32_t* seq_idx, float* y_zero, float* summary,
                    void* ws, size_t ws_bytes, void* stream);

/* ssd_segment_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same outputs from the same kernels, with the workspace in a fixed device
 * array of the library (SSD_SCRATCH_BYTES = 64 MiB per GPU, held until the
 * process ends) instead of a `ws` argument.  The call allocates nothing.
 * Problems whose forward workspace (ssd_workspace_bytes(..., SSD_WS_FORWARD))
 * exceeds SSD_SCRATCH_BYTES return SSD_ERR_SCRATCH before anything is enqueued.
 * Every call on one GPU uses that GPU's one array: calls that overlap on a GPU
 * (on different streams, or from different threads) race and give wrong
 * results.  The scratch keeps the last call's contents; nothing in it needs
 * clearing, since each call reads only what it wrote.  The workspace stays
 * internal, so ssd_apply_init_state cannot follow this call (the fused output
 * path or ssd_segment_fwd serve callers that need the corrected y).
 * Arguments as for ssd_segment_fwd, without ws and ws_bytes. */
#define SSD_SCRATCH_BYTES (64u << 20)
int ssd_segment_fwd_noalloc(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                            const void* xBC_conv, const void* dt_raw, const float* dt_bias,
                            const float* A_log, const int32_t* seq_idx, float* y_zero,
                            float* summary, void* stream);

/* The two phases of ssd_segment_fwd, for callers that overlap the summary
 * exchange with the local intra-chunk work (#6808's first commit issues the
 * summary gather asynchronously and hides it behind the local C*B^T work).
 * ssd_segment_states computes dt, the cumulative decays, every chunk's entering
 * state, the segment summaries (into `summary` and `ws`) and the causal C B^T
 * Gram tiles of every chunk and group (into `ws`); ssd_segment_output then
 * computes y_zero from the same inputs and `ws`.  Calling both in this
 * order is the same as ssd_segment_fwd.  When the state walk splits long
 * segments into spans (see ssd_workspace_bytes), ssd_segment_output also
 * writes the states entering the spans into `ws`, so the output calls take a
 * writable workspace.  */
int ssd_segment_states(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                       const void* xBC_conv, const void* dt_raw, const float* dt_bias,
                       const float* A_log, const int32_t* seq_idx, float* summary, void* ws,
                       size_t ws_bytes, void* stream);
int ssd_segment_output(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                       const void* xBC_conv, const int32_t* seq_idx, void* ws,
                       size_t ws_bytes, float* y_zero, void* stream);

/* Affine scan over segment summaries, in causal segment order (#6808's first
 * commit: an exclusive scan, in causal order, over the gathered summaries).
 * summary holds M[k] = [nseg][batch][H][P*N] followed by a[k] = [nseg][batch][H].
 *  reverse = 0:  out[0] = init (zeros if NULL); out[k+1] = a[k] out[k] + M[k].
 *                out is S_in, the true initial state of every segment.
 *                final_state (optional) = a[nseg-1] out[nseg-1] + M[nseg-1].
 *  reverse = 1:  out[nseg-1] = init (zeros if NULL); out[k-1] = a[k] out[k] + M[k].
 *                With M = dL/dS_in local terms this gives each segment's
 *                final-state gradient; final_state (optional) = a[0] out[0] + M[0].
 *  out, final_state: [nseg][batch][H][P][N] and [batch][H][P][N] float32.   */
int ssd_boundary_scan(const ssd_problem* problem, int32_t nseg, const float* summary,
                      const float* init, int32_t reverse, float* out, float* final_state,
                      void* stream);

/* Correction and output pass: y = y_zero + decay_t * C_t S_in^T + D x_t, the
 * correction of Megatron-LM #6808's first commit (a segment's outputs gain the
 * term C_t * decay * S_in once the boundary scan has produced its S_in).
 * decay_t = exp(sum of dt*A from the segment start through t), and 0 once a
 * packed sequence starts inside the segment; for the first segment of a row,
 * S_in is the state before the row's first token.
 *   y_zero    float32 from ssd_segment_fwd                                  (in)
 *   xBC_conv  as for ssd_segment_fwd                                        (in)
 *   D         [H] float32                                                   (in)
 *   seq_idx   as for ssd_segment_fwd                                        (in)
 *   S_in      [nseg][batch][H][P][N] float32 (ssd_boundary_scan output)     (in)
 *   ws        the workspace ssd_segment_fwd filled for the same problem,
 *             segments and inputs (read only)                               (in)
 *   y         [batch][seqlen][H][P] act_dtype                               (out) */
int ssd_apply_init_state(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                         const float* y_zero, const void* xBC_conv, const float* D,
                         const int32_t* seq_idx, const float* S_in, const void* ws,
                         size_t ws_bytes, void* y, void* stream);

/* ssd_segment_output and ssd_apply_init_state in one pass, for callers that run
 * the boundary scan between ssd_segment_states and the output pass (the
 * summaries of #6808 depend only on the chunk states, so the scan can precede
 * the output work).  Every chunk's output uses its true entering state (the
 * zero-state walk plus decay * S_in) and D x is added in the same pass, so
 * y_zero is never written and x and C are read once.  Same result as
 * ssd_segment_output followed by ssd_apply_init_state, up to rounding.
 *   xBC_conv, D, seq_idx   as for ssd_apply_init_state                         (in)
 *   S_in      [nseg][batch][H][P][N] float32 (ssd_boundary_scan output)         (in)
 *   ws        the workspace ssd_segment_states filled for the same problem,
 *             segments and inputs; the states entering the spans of long
 *             segments are written into it                                      (in/out)
 *   y         [batch][seqlen][H][P] act_dtype                                   (out) */
int ssd_segment_output_fused(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                             const void* xBC_conv, const float* D, const int32_t* seq_idx,
                             const float* S_in, void* ws, size_t ws_bytes, void* y,
                             void* stream);

/* The conv-fused forward: ssd_conv1d_fwd folded into the two forward phases,
 * so the convolved x channels never go to memory (#6808's first commit names
 * the conv halo as part of the fused Conv1d + SSD function; state-spaces/mamba
 * #482, second comment, puts the conv before the scan).  Both calls take the
 * raw xBC and the conv taps instead of xBC_conv.  ssd_conv_segment_states
 * convolves the B and C channels into `ws` and then does what
 * ssd_segment_states does, its state walk convolving the x channels as it
 * reads them (each segment's first W-1 taps read its causal predecessor's
 * last tokens, as in ssd_conv1d_fwd); after the boundary scan,
 * ssd_conv_segment_output does what ssd_segment_output_fused does, again
 * convolving the x channels itself.  The results equal ssd_conv1d_fwd
 * followed by ssd_segment_states, ssd_boundary_scan and
 * ssd_segment_output_fused: the conv arithmetic is the same, operation for
 * operation.  Compiled for conv_width 4 only (SSD_ERR_UNSUPPORTED otherwise).
 *   xBC, conv_w   as for ssd_conv1d_fwd                                     (in)
 *   dt_raw, dt_bias, A_log, seq_idx, summary   as for ssd_segment_states
 *   D, S_in, y    as for ssd_segment_output_fused
 *   ws    ssd_workspace_bytes(..., SSD_WS_FORWARD_CONV) bytes: filled by the
 *         states call, read (and for long segments written) by the output
 *         call for the same problem, segments and inputs                 (in/out) */
int ssd_conv_segment_states(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                            const void* xBC, const float* conv_w, const void* dt_raw,
                            const float* dt_bias, const float* A_log, const int32_t* seq_idx,
                            float* summary, void* ws, size_t ws_bytes, void* stream);
int ssd_conv_segment_output(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                            const void* xBC, const float* conv_w, const float* D,
                            const int32_t* seq_idx, const float* S_in, void* ws,
                            size_t ws_bytes, void* y, void* stream);

/* Backward, summary phase (Megatron-LM #6808, first commit: the backward
 * mirrors the forward, each segment summarising the gradient its own outputs
 * send to its initial state, gathered and reverse-scanned like the forward
 * summaries; sequence-length-sized intermediates are recomputed, not stored).
 * Recomputes the conv output, dt and the
 * cumulative decays into `ws` (sequence-length-sized intermediates are
 * recomputed, never saved from the forward), then walks every segment's chunks
 * in reverse causal order carrying the state gradient.  Writes, in the summary
 * layout of ssd_segment_fwd:
 *   M[k] = dL/dS_in[k] caused by segment k's own outputs   [nseg][batch][H][P][N]
 *   a[k] = segment k's block decay                          [nseg][batch][H]
 * ssd_boundary_scan(reverse = 1) over this summary then yields every segment's
 * final-state gradient dS_out.
 *   xBC, conv_w, dt_raw, dt_bias, A_log, seq_idx   forward inputs           (in)
 *   dy        [batch][seqlen][H][P] act_dtype                                (in)
 *   summary   float32, summary layout                                        (out)
 *   ws        ssd_workspace_bytes(..., SSD_WS_BACKWARD) bytes                (out) */
int ssd_segment_bwd_summary(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                            const void* xBC, const float* conv_w, const void* dt_raw,
                            const float* dt_bias, const float* A_log, const int32_t* seq_idx,
                            const void* dy, float* summary, void* ws, size_t ws_bytes,
                            void* stream);

/* Backward, segment phase: every gradient of the path (Megatron-LM #6808,
 * first commit: with its initial state from the forward scan and its
 * final-state gradient from the reverse scan, each segment runs the SSD
 * backward locally and writes its gradients straight into the buffers the
 * convolution backward consumes).
 *   S_in      [nseg][batch][H][P][N] float32: initial states from the forward
 *             boundary scan (segment-count sized, so it may be kept)         (in)
 *   dS_out    [nseg][batch][H][P][N] float32: final-state gradients from the
 *             reverse boundary scan                                          (in)
 *   ws        the workspace ssd_segment_bwd_summary filled                   (in/out)
 *   dxBC      [batch][seqlen][C] act_dtype                                   (out)
 *   ddt_raw   [batch][seqlen][H] act_dtype                                   (out)
 *   dconv_w   [C][W], ddt_bias [H], dA_log [H], dD [H] float32, summed over
 *             every row and segment of this call                             (out) */
int ssd_segment_bwd(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                    const void* xBC, const float* conv_w, const void* dt_raw, const float* dt_bias,
                    const float* A_log, const float* D, const int32_t* seq_idx, const void* dy,
                    const float* S_in, const float* dS_out, void* ws, size_t ws_bytes, void* dxBC,
                    void* ddt_raw, float* dconv_w, float* ddt_bias, float* dA_log, float* dD,
                    void* stream);

/* The three phases of ssd_segment_bwd, in this order (calling them is the same
 * as ssd_segment_bwd; each reads the workspace ssd_segment_bwd_summary filled):
 *  ssd_segment_bwd_pass    walks every segment's chunks from S_in forward and
 *                          from dS_out backward (reading dy for the chunks'
 *                          gradient contributions), leaving in `ws` the true
 *                          entering state and exit-state gradient of every chunk.
 *  ssd_segment_bwd_chunks  per chunk and head: dx, dB, dC (into `ws`, the
 *                          buffers the conv backward consumes, as #6808's first
 *                          commit does) and the per-token and per-chunk partial
 *                          sums of d(dt), dA and dD.
 *  ssd_conv1d_bwd          assembles ddt_raw per token (the chain through the dt
 *                          clamp and softplus), sums dB and dC over each group's
 *                          heads, applies SiLU' and the transposed causal conv
 *                          (its right halo read from the causal successor
 *                          segment) to give dxBC, and reduces dconv_w, ddt_bias,
 *                          dA_log and dD (fixed order, deterministic).
 * Arguments mean what they mean for ssd_segment_bwd. */
int ssd_segment_bwd_pass(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                         const int32_t* seq_idx, const void* dy, const float* S_in,
                         const float* dS_out, void* ws, size_t ws_bytes, void* stream);
int ssd_segment_bwd_chunks(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                           const float* D, const int32_t* seq_idx, const void* dy, void* ws,
                           size_t ws_bytes, void* stream);
int ssd_conv1d_bwd(const ssd_problem* problem, const ssd_segment* segs, int32_t nseg,
                   const void* xBC, const float* conv_w, const void* dt_raw, const float* dt_bias,
                   const float* A_log, const int32_t* seq_idx, void* ws, size_t ws_bytes,
                   void* dxBC, void* ddt_raw, float* dconv_w, float* ddt_bias, float* dA_log,
                   float* dD, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MI355X_SSD_H */
