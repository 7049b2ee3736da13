/*
 * CPU oracle for the Mamba2 causal conv1d + SSD mixer core, in float64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU path shares no code,
 * header, table or helper with it, and nothing here knows about chunks,
 * segments, summaries or scans: it runs the plain recurrence token by token over
 * the whole (unsegmented) sequence in causal order.  Chunking and segment-local
 * state passing only reassociate these sums, which the Megatron-LM pull request
 * "Add state-passing context parallelism for Mamba2" (#6808) states in its
 * description, section "Testing": re-association changes bf16 rounding but not
 * the mathematics.  That is why this definition is the one every GPU result is
 * compared against.
 *
 * Definitions followed (notation of the Mamba-2 selective state space model the
 * pages build on; the issue "Sequence parallelism in the mixer" on
 * state-spaces/mamba #482 points to its chunked algorithm):
 *   u[t,c]  = sum_k w[c,k] * xBC[t-(W-1)+k, c]     causal depthwise conv, taps
 *             that fall before the row start or across a sequence reset are 0
 *   v       = u * sigmoid(u)                       SiLU on every conv channel
 *   channels of v: [ x (H*P) | B (G*N) | C (G*N) ], head h uses group h/(H/G)
 *   dt_t    = clamp(softplus(dt_raw[t,h] + dt_bias[h]), dt_min, dt_max)
 *   A       = -exp(A_log[h])
 *   a_t     = exp(dt_t * A), or exactly 0 when token t starts a new packed
 *             sequence (seq_idx[t] != seq_idx[t-1]); the NeMo Automodel pull
 *             request #1441 (context parallelism for Nemotron v3, section Key
 *             changes) derives seq_idx from cu_seqlens for exactly these resets
 *   h_t     = a_t * h_{t-1} + dt_t * x_t (outer) B_t          h_{-1} = init (0)
 *   y_t     = h_t C_t + D[h] * x_t
 *
 * The backward entry points are the exact adjoint of the above, written out
 * term by term (reverse-time recurrence of G_t = dL/dh_t).
 *
 * Inputs are the stored values (bf16-exact or fp32) passed as float and upcast;
 * every accumulation is float64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double sigm(double z) { return 1.0 / (1.0 + exp(-z)); }

/* log(1 + e^z), written so that it neither overflows nor loses small values. */
static double softplus(double z) { return (z > 0 ? z : 0.0) + log1p(exp(-fabs(z))); }

static double clampd(double v, double lo, double hi) { return v < lo ? lo : (v > hi ? hi : v); }

/* Causal depthwise conv followed by SiLU.
 *   xBC [batch][L][C], w [C][W], seq_idx [batch][L] or NULL.
 *   u_out (optional) receives the pre-activation, v_out the SiLU output. */
void oracle_conv_silu(int64_t batch, int64_t L, int64_t C, int64_t W, const float* xBC,
                      const float* w, const int32_t* seq_idx, double* u_out, double* v_out) {
#pragma omp parallel for schedule(static)
    for (int64_t bt = 0; bt < batch * L; ++bt) {
        const int64_t b = bt / L, t = bt % L;
        for (int64_t c = 0; c < C; ++c) {
            double u = 0.0;
            for (int64_t k = 0; k < W; ++k) {
                const int64_t s = t - (W - 1) + k;
                if (s < 0) continue;
                if (seq_idx && seq_idx[b * L + s] != seq_idx[b * L + t]) continue;
                u += (double)w[c * W + k] * (double)xBC[(b * L + s) * C + c];
            }
            if (u_out) u_out[bt * C + c] = u;
            v_out[bt * C + c] = u * sigm(u);
        }
    }
}

/* Adjoint of oracle_conv_silu: given dv = dL/dv, returns dL/dxBC and dL/dw. */
void oracle_conv_silu_bwd(int64_t batch, int64_t L, int64_t C, int64_t W, const float* xBC,
                          const float* w, const int32_t* seq_idx, const double* dv,
                          double* dxBC, double* dw) {
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < C; ++c) {
        for (int64_t k = 0; k < W; ++k) dw[c * W + k] = 0.0;
        for (int64_t b = 0; b < batch; ++b) {
            for (int64_t t = 0; t < L; ++t) dxBC[(b * L + t) * C + c] = 0.0;
            for (int64_t t = 0; t < L; ++t) {
                double u = 0.0;
                for (int64_t k = 0; k < W; ++k) {
                    const int64_t s = t - (W - 1) + k;
                    if (s < 0) continue;
                    if (seq_idx && seq_idx[b * L + s] != seq_idx[b * L + t]) continue;
                    u += (double)w[c * W + k] * (double)xBC[(b * L + s) * C + c];
                }
                const double sg = sigm(u);
                const double du = dv[(b * L + t) * C + c] * sg * (1.0 + u * (1.0 - sg));
                for (int64_t k = 0; k < W; ++k) {
                    const int64_t s = t - (W - 1) + k;
                    if (s < 0) continue;
                    if (seq_idx && seq_idx[b * L + s] != seq_idx[b * L + t]) continue;
                    dxBC[(b * L + s) * C + c] += (double)w[c * W + k] * du;
                    dw[c * W + k] += du * (double)xBC[(b * L + s) * C + c];
                }
            }
        }
    }
}

/* Token-by-token SSD forward.
 *   v        [batch][L][C]   post-conv activations, C = H*P + 2*G*N
 *   dt_raw   [batch][L][H]
 *   dt_bias, A_log, D [H]
 *   seq_idx  [batch][L] or NULL
 *   init     [batch][H][P][N] or NULL (state before the row's first token)
 *   y        [batch][L][H][P]
 *   final_state [batch][H][P][N] or NULL */
void oracle_ssd_fwd(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                    const double* v, const float* dt_raw, const float* dt_bias,
                    const float* A_log, const float* D, double dt_min, double dt_max,
                    const int32_t* seq_idx, const double* init, double* y,
                    double* final_state) {
    const int64_t C = H * P + 2 * G * N;
    const int64_t hpg = H / G;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < batch * H; ++bh) {
        const int64_t b = bh / H, h = bh % H, g = h / hpg;
        const double A = -exp((double)A_log[h]);
        double* st = (double*)malloc(sizeof(double) * P * N);
        for (int64_t i = 0; i < P * N; ++i) st[i] = init ? init[bh * P * N + i] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const double* row = v + (b * L + t) * C;
            const double* x = row + h * P;
            const double* Bv = row + H * P + g * N;
            const double* Cv = row + H * P + G * N + g * N;
            const int reset = (t > 0 && seq_idx && seq_idx[b * L + t] != seq_idx[b * L + t - 1]);
            const double dt = clampd(softplus((double)dt_raw[(b * L + t) * H + h] + (double)dt_bias[h]),
                                     dt_min, dt_max);
            const double a = reset ? 0.0 : exp(dt * A);
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n)
                    st[p * N + n] = a * st[p * N + n] + dt * x[p] * Bv[n];
            double* yo = y + ((b * L + t) * H + h) * P;
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) acc += st[p * N + n] * Cv[n];
                yo[p] = acc + (double)D[h] * x[p];
            }
        }
        if (final_state)
            for (int64_t i = 0; i < P * N; ++i) final_state[bh * P * N + i] = st[i];
        free(st);
    }
}

/* Adjoint of oracle_ssd_fwd.
 *   dy        [batch][L][H][P]
 *   dv        [batch][L][C]      dL/dv (x, B and C channels)
 *   ddt_raw   [batch][L][H]      dL/d dt_raw (through clamp and softplus)
 *   ddt_bias, dA_log, dD [H]
 *   dinit     [batch][H][P][N] or NULL
 * The clamp passes the gradient when dt_min <= softplus(.) <= dt_max. */
void oracle_ssd_bwd(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                    const double* v, const float* dt_raw, const float* dt_bias,
                    const float* A_log, const float* D, double dt_min, double dt_max,
                    const int32_t* seq_idx, const double* init, const float* dy,
                    double* dv, double* ddt_raw, double* ddt_bias, double* dA_log,
                    double* dD, double* dinit) {
    const int64_t C = H * P + 2 * G * N;
    const int64_t hpg = H / G;
    double* dBh = (double*)calloc((size_t)(batch * H * L * N), sizeof(double));
    double* dCh = (double*)calloc((size_t)(batch * H * L * N), sizeof(double));
    double* part = (double*)calloc((size_t)(batch * H * 3), sizeof(double));

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < batch * H; ++bh) {
        const int64_t b = bh / H, h = bh % H, g = h / hpg;
        const double A = -exp((double)A_log[h]);
        double* states = (double*)malloc(sizeof(double) * (size_t)(L * P * N));
        double* dts = (double*)malloc(sizeof(double) * (size_t)L);
        double* as = (double*)malloc(sizeof(double) * (size_t)L);
        double* Gs = (double*)malloc(sizeof(double) * (size_t)(P * N));
        /* forward, keeping every state */
        for (int64_t t = 0; t < L; ++t) {
            const double* row = v + (b * L + t) * C;
            const double* x = row + h * P;
            const double* Bv = row + H * P + g * N;
            const int reset = (t > 0 && seq_idx && seq_idx[b * L + t] != seq_idx[b * L + t - 1]);
            const double dt = clampd(softplus((double)dt_raw[(b * L + t) * H + h] + (double)dt_bias[h]),
                                     dt_min, dt_max);
            const double a = reset ? 0.0 : exp(dt * A);
            dts[t] = dt;
            as[t] = a;
            double* cur = states + t * P * N;
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n) {
                    const double prev = t > 0 ? states[(t - 1) * P * N + p * N + n]
                                              : (init ? init[bh * P * N + p * N + n] : 0.0);
                    cur[p * N + n] = a * prev + dt * x[p] * Bv[n];
                }
        }
        /* reverse sweep: Gs holds dL/dh_t */
        for (int64_t i = 0; i < P * N; ++i) Gs[i] = 0.0;
        double s_dA = 0.0, s_dD = 0.0, s_db = 0.0;
        for (int64_t t = L - 1; t >= 0; --t) {
            const double* row = v + (b * L + t) * C;
            const double* x = row + h * P;
            const double* Bv = row + H * P + g * N;
            const double* Cv = row + H * P + G * N + g * N;
            const float* dyt = dy + ((b * L + t) * H + h) * P;
            const double dt = dts[t], a = as[t];
            const double* cur = states + t * P * N;
            const double* prev = t > 0 ? states + (t - 1) * P * N : (init ? init + bh * P * N : NULL);
            /* y_t = h_t C_t: dL/dh_t gains dy_t (outer) C_t */
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n) Gs[p * N + n] += (double)dyt[p] * Cv[n];
            /* dC_t = h_t^T dy_t */
            for (int64_t n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int64_t p = 0; p < P; ++p) acc += cur[p * N + n] * (double)dyt[p];
                dCh[(bh * L + t) * N + n] = acc;
            }
            /* dx_t = dt G B_t + D dy_t ; dB_t = dt G^T x_t */
            double* dvx = dv + (b * L + t) * C + h * P;
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) acc += Gs[p * N + n] * Bv[n];
                dvx[p] = dt * acc + (double)D[h] * (double)dyt[p];
            }
            for (int64_t n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int64_t p = 0; p < P; ++p) acc += Gs[p * N + n] * x[p];
                dBh[(bh * L + t) * N + n] = dt * acc;
            }
            /* d dt_t: through the input term and through a_t = exp(dt_t A) */
            double gx = 0.0, gh = 0.0;
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n) {
                    gx += Gs[p * N + n] * x[p] * Bv[n];
                    if (prev) gh += Gs[p * N + n] * prev[p * N + n];
                }
            const double dl = a * gh; /* dL/d(dt_t A); zero across a reset since a = 0 */
            const double ddt = gx + A * dl;
            s_dA += dt * dl;
            double dd = 0.0;
            for (int64_t p = 0; p < P; ++p) dd += (double)dyt[p] * x[p];
            s_dD += dd;
            const double z = (double)dt_raw[(b * L + t) * H + h] + (double)dt_bias[h];
            const double sp = softplus(z);
            const double g_raw = (sp >= dt_min && sp <= dt_max) ? ddt * sigm(z) : 0.0;
            ddt_raw[(b * L + t) * H + h] = g_raw;
            s_db += g_raw;
            /* carry to t-1 */
            for (int64_t i = 0; i < P * N; ++i) Gs[i] *= a;
        }
        if (dinit)
            for (int64_t i = 0; i < P * N; ++i) dinit[bh * P * N + i] = Gs[i];
        part[bh * 3 + 0] = s_dA * A; /* dA/dA_log = -exp(A_log) = A */
        part[bh * 3 + 1] = s_dD;
        part[bh * 3 + 2] = s_db;
        free(states);
        free(dts);
        free(as);
        free(Gs);
    }

    for (int64_t h = 0; h < H; ++h) {
        dA_log[h] = 0.0;
        dD[h] = 0.0;
        ddt_bias[h] = 0.0;
        for (int64_t b = 0; b < batch; ++b) {
            dA_log[h] += part[(b * H + h) * 3 + 0];
            dD[h] += part[(b * H + h) * 3 + 1];
            ddt_bias[h] += part[(b * H + h) * 3 + 2];
        }
    }
    /* B and C channels are shared by the heads of a group: sum per group */
#pragma omp parallel for schedule(static)
    for (int64_t bt = 0; bt < batch * L; ++bt) {
        const int64_t b = bt / L, t = bt % L;
        double* row = dv + bt * C;
        for (int64_t g = 0; g < G; ++g)
            for (int64_t n = 0; n < N; ++n) {
                double sb = 0.0, sc = 0.0;
                for (int64_t h = g * hpg; h < (g + 1) * hpg; ++h) {
                    sb += dBh[((b * H + h) * L + t) * N + n];
                    sc += dCh[((b * H + h) * L + t) * N + n];
                }
                row[H * P + g * N + n] = sb;
                row[H * P + G * N + g * N + n] = sc;
            }
    }
    free(dBh);
    free(dCh);
    free(part);
}

/* Number of OpenMP threads the oracle will use (reported with CPU timings). */
int oracle_num_threads(void) {
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
