/* Host validation of the C ABI under AddressSanitizer and UndefinedBehavior-
 * Sanitizer (host code only; no GPU is touched: every call below is refused by
 * validation before anything is launched, or is a pure host query).  Exits 0
 * when every status is the expected one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ssd.h"

static int fails = 0;
#define EXPECT(expr, want)                                                           \
    do {                                                                             \
        long got_ = (long)(expr);                                                    \
        if (got_ != (long)(want)) {                                                  \
            fprintf(stderr, "line %d: %s = %ld, expected %ld\n", __LINE__, #expr,    \
                    got_, (long)(want));                                             \
            ++fails;                                                                 \
        }                                                                            \
    } while (0)

int main(void) {
    ssd_problem p = {2, 8192, 32, 64, 128, 1, 256, 4, SSD_BF16, 1e-3f, 0.1f};
    ssd_segment segs[SSD_MAX_SEGMENTS + 1];
    for (int i = 0; i < 8; ++i) {
        segs[i].start = i * 1024;
        segs[i].len = 1024;
    }
    void* F = (void*)0x100000;                   /* never dereferenced */
    const float* Ff = (const float*)0x100000;
    const int32_t* mis = (const int32_t*)0x100004; /* misaligned */

    /* workspace queries over a grid of shapes, dtypes, chunks and segment tables */
    size_t total = 0;
    for (int act = 0; act < 2; ++act)
        for (int P = 8; P <= 256; P *= 2)
            for (int N = 8; N <= 256; N *= 2)
                for (int Q = 32; Q <= 512; Q *= 2) {
                    ssd_problem q = {1, 16 * 1024, 8, P, N, 2, Q, 4, act, 1e-3f, 0.1f};
                    ssd_segment s[4] = {{0, 4096}, {4096, 4096}, {8192, 4096}, {12288, 4096}};
                    total += ssd_workspace_bytes(&q, s, 4, SSD_WS_FORWARD);
                    total += ssd_workspace_bytes(&q, s, 4, SSD_WS_BACKWARD);
                    total += ssd_workspace_bytes(&q, s, 1, SSD_WS_FORWARD); /* does not tile */
                    total += ssd_workspace_bytes(&q, s, 4, SSD_WS_FORWARD_CONV);
                }
    printf("workspace sum %zu\n", total);
    EXPECT(ssd_workspace_bytes(&p, segs, 8, SSD_WS_FORWARD) > 0, 1);
    EXPECT(ssd_workspace_bytes(&p, segs, 8, 7), 0);

    /* argument checks of every entry point */
    EXPECT(ssd_conv1d_fwd(NULL, segs, 8, F, Ff, NULL, F, NULL), SSD_ERR_NULL);
    EXPECT(ssd_conv1d_fwd(&p, segs, 8, F, Ff, mis, F, NULL), SSD_ERR_ALIGN);
    EXPECT(ssd_conv1d_fwd(&p, segs, 0, F, Ff, NULL, F, NULL), SSD_ERR_SEGMENTS);
    EXPECT(ssd_conv1d_fwd(&p, segs, SSD_MAX_SEGMENTS + 1, F, Ff, NULL, F, NULL), SSD_ERR_SEGMENTS);
    EXPECT(ssd_segment_fwd(&p, segs, 8, F, F, Ff, Ff, NULL, (float*)F, (float*)F, F, 1, NULL),
           SSD_ERR_WORKSPACE);
    EXPECT(ssd_segment_fwd_noalloc(&p, segs, 8, F, F, Ff, Ff, mis, (float*)F, (float*)F, NULL),
           SSD_ERR_ALIGN);
    EXPECT(ssd_segment_states(&p, segs, 8, NULL, F, Ff, Ff, NULL, (float*)F, F, 1 << 30, NULL),
           SSD_ERR_NULL);
    EXPECT(ssd_segment_output(&p, segs, 8, F, NULL, NULL, 1 << 30, (float*)F, NULL),
           SSD_ERR_WORKSPACE);
    EXPECT(ssd_boundary_scan(&p, 8, Ff, NULL, 2, (float*)F, NULL, NULL), SSD_ERR_SHAPE);
    EXPECT(ssd_apply_init_state(&p, segs, 8, Ff, F, Ff, NULL, Ff, F, 1, F, NULL),
           SSD_ERR_WORKSPACE);
    EXPECT(ssd_segment_output_fused(&p, segs, 8, F, NULL, NULL, Ff, F, 1 << 30, F, NULL),
           SSD_ERR_NULL);
    EXPECT(ssd_conv_segment_states(&p, segs, 8, F, NULL, F, Ff, Ff, NULL, (float*)F, F,
                                   1 << 30, NULL),
           SSD_ERR_NULL);
    EXPECT(ssd_conv_segment_output(&p, segs, 8, F, Ff, Ff, mis, Ff, F, (size_t)1 << 40, F, NULL),
           SSD_ERR_ALIGN);
    EXPECT(ssd_conv_segment_output(&p, segs, 8, F, Ff, Ff, NULL, Ff, F, 1, F, NULL),
           SSD_ERR_WORKSPACE);
    EXPECT(ssd_segment_bwd_summary(&p, segs, 8, F, Ff, F, Ff, Ff, mis, F, (float*)F, F,
                                   (size_t)1 << 40, NULL),
           SSD_ERR_ALIGN);
    EXPECT(ssd_segment_bwd_pass(&p, segs, 8, NULL, F, Ff, Ff, F, 16, NULL), SSD_ERR_WORKSPACE);
    EXPECT(ssd_segment_bwd_chunks(&p, segs, 8, NULL, NULL, F, F, (size_t)1 << 40, NULL),
           SSD_ERR_NULL);
    EXPECT(ssd_conv1d_bwd(&p, segs, 8, F, Ff, F, Ff, Ff, NULL, F, (size_t)1 << 40, F, F,
                          (float*)F, (float*)F, (float*)F, NULL, NULL),
           SSD_ERR_NULL);
    EXPECT(ssd_segment_bwd(&p, segs, 8, F, Ff, F, Ff, Ff, Ff, NULL, F, Ff, Ff, F, 0, F, F,
                           (float*)F, (float*)F, (float*)F, (float*)F, NULL),
           SSD_ERR_WORKSPACE);

    /* segment tables that do not tile the row */
    ssd_segment bad[3] = {{0, 1024}, {512, 1024}, {2048, 6144}};
    EXPECT(ssd_conv1d_fwd(&p, bad, 3, F, Ff, NULL, F, NULL), SSD_ERR_SEGMENTS);
    ssd_segment neg[1] = {{-256, 8192}};
    EXPECT(ssd_conv1d_fwd(&p, neg, 1, F, Ff, NULL, F, NULL), SSD_ERR_SEGMENTS);

    /* extreme sizes: over-long row, grid overflow, huge products */
    ssd_problem L = p;
    L.batch = 1;
    L.seqlen = (int64_t)1 << 23;
    ssd_segment whole = {0, L.seqlen};
    EXPECT(ssd_conv1d_fwd(&L, &whole, 1, F, Ff, NULL, F, NULL), SSD_ERR_SHAPE);
    ssd_problem G = p;
    G.batch = 4096;
    G.nheads = 4096;
    G.seqlen = 256;
    ssd_segment g1 = {0, 256};
    EXPECT(ssd_conv1d_fwd(&G, &g1, 1, F, Ff, NULL, F, NULL), SSD_ERR_SHAPE);
    ssd_problem X = p;
    X.batch = 65535;
    X.nheads = 65535;
    X.ngroups = 65535;
    X.seqlen = ((int64_t)1 << 31) - 256;
    ssd_segment x1 = {0, X.seqlen};
    EXPECT(ssd_workspace_bytes(&X, &x1, 1, SSD_WS_FORWARD), 0);
    ssd_problem Z = p;
    Z.seqlen = INT64_MAX;
    EXPECT(ssd_workspace_bytes(&Z, segs, 8, SSD_WS_FORWARD), 0);
    Z.seqlen = 8192;
    Z.dt_max = -1.f;
    EXPECT(ssd_conv1d_fwd(&Z, segs, 8, F, Ff, NULL, F, NULL), SSD_ERR_SHAPE);

    for (int code = -9; code <= 1; ++code)
        if (!ssd_status_string(code) || strlen(ssd_status_string(code)) == 0) ++fails;
    EXPECT(ssd_supported(64, 128, SSD_BF16), 1);
    EXPECT(ssd_supported(128, 128, SSD_BF16), 0);
    printf("%d failed checks\n", fails);
    return fails == 0 ? 0 : 1;
}
