/* The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every
 * entry point on a small packed problem with an initial state (the oracle's
 * own arithmetic is pinned elsewhere; this checks memory safety and finite
 * results).  Exits 0 when every output is finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_conv_silu(int64_t, int64_t, int64_t, int64_t, const float*, const float*,
                      const int32_t*, double*, double*);
void oracle_conv_silu_bwd(int64_t, int64_t, int64_t, int64_t, const float*, const float*,
                          const int32_t*, const double*, double*, double*);
void oracle_ssd_fwd(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, const double*,
                    const float*, const float*, const float*, const float*, double, double,
                    const int32_t*, const double*, double*, double*);
void oracle_ssd_bwd(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, const double*,
                    const float*, const float*, const float*, const float*, double, double,
                    const int32_t*, const double*, const float*, double*, double*, double*,
                    double*, double*, double*);

static float frand(unsigned* s) {
    *s = *s * 1664525u + 1013904223u;
    return ((*s >> 8) & 0xffff) / 32768.0f - 1.0f;
}

static int finite_all(const double* a, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) return 0;
    return 1;
}

int main(void) {
    const int64_t b = 2, L = 40, H = 4, P = 3, N = 4, G = 2, W = 4;
    const int64_t C = H * P + 2 * G * N;
    unsigned s = 12345u;
    float* xBC = malloc(sizeof(float) * b * L * C);
    float* w = malloc(sizeof(float) * C * W);
    float* dtr = malloc(sizeof(float) * b * L * H);
    float dtb[4], alog[4], D[4];
    float* dy = malloc(sizeof(float) * b * L * H * P);
    int32_t* seq = malloc(sizeof(int32_t) * b * L);
    for (int64_t i = 0; i < b * L * C; ++i) xBC[i] = frand(&s);
    for (int64_t i = 0; i < C * W; ++i) w[i] = 0.5f * frand(&s);
    for (int64_t i = 0; i < b * L * H; ++i) dtr[i] = frand(&s);
    for (int64_t i = 0; i < b * L * H * P; ++i) dy[i] = frand(&s);
    for (int h = 0; h < 4; ++h) {
        dtb[h] = -2.5f + frand(&s);
        alog[h] = 0.5f + 0.5f * frand(&s);
        D[h] = frand(&s);
    }
    for (int64_t r = 0; r < b; ++r)
        for (int64_t t = 0; t < L; ++t) seq[r * L + t] = t < 13 ? 0 : (t < 14 ? 1 : 2);
    double* u = malloc(sizeof(double) * b * L * C);
    double* v = malloc(sizeof(double) * b * L * C);
    double* init = malloc(sizeof(double) * b * H * P * N);
    double* y = malloc(sizeof(double) * b * L * H * P);
    double* fin = malloc(sizeof(double) * b * H * P * N);
    double* dv = malloc(sizeof(double) * b * L * C);
    double* ddt = malloc(sizeof(double) * b * L * H);
    double ddb[4], dal[4], dD[4];
    double* dinit = malloc(sizeof(double) * b * H * P * N);
    double* dx = malloc(sizeof(double) * b * L * C);
    double* dw = malloc(sizeof(double) * C * W);
    for (int64_t i = 0; i < b * H * P * N; ++i) init[i] = frand(&s);
    oracle_conv_silu(b, L, C, W, xBC, w, seq, u, v);
    oracle_ssd_fwd(b, L, H, P, N, G, v, dtr, dtb, alog, D, 1e-3, 0.1, seq, init, y, fin);
    oracle_ssd_bwd(b, L, H, P, N, G, v, dtr, dtb, alog, D, 1e-3, 0.1, seq, init, dy, dv, ddt,
                   ddb, dal, dD, dinit);
    oracle_conv_silu_bwd(b, L, C, W, xBC, w, seq, dv, dx, dw);
    /* and without packing or an initial state */
    oracle_ssd_fwd(b, L, H, P, N, G, v, dtr, dtb, alog, D, 1e-3, 0.1, NULL, NULL, y, NULL);
    int ok = finite_all(v, b * L * C) && finite_all(y, b * L * H * P) && finite_all(fin, b * H * P * N) &&
             finite_all(dv, b * L * C) && finite_all(ddt, b * L * H) && finite_all(dinit, b * H * P * N) &&
             finite_all(dx, b * L * C) && finite_all(dw, C * W) && finite_all(ddb, 4) &&
             finite_all(dal, 4) && finite_all(dD, 4);
    printf("oracle outputs finite: %d\n", ok);
    free(xBC); free(w); free(dtr); free(dy); free(seq); free(u); free(v); free(init); free(y);
    free(fin); free(dv); free(ddt); free(dinit); free(dx); free(dw);
    return ok ? 0 : 1;
}
