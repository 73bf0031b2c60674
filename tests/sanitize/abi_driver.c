/* Drives the host side of the C ABI (argument validation, size helpers and
 * the dry run of the product dispatch) over valid, invalid and extreme
 * arguments, for a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * on the host code. No GPU is needed: calls with valid arguments stop at the
 * device check (BL_ERR_DEVICE) before any launch. Exits non-zero when a call
 * returns an unexpected status; the sanitizers abort on their own findings. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "bitlinear.h"

static int fails = 0;
#define EXPECT(cond)                                                         \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
            ++fails;                                                         \
        }                                                                    \
    } while (0)

int main(int argc, char **argv) {
    const int have_gpu = argc > 1 && strcmp(argv[1], "gpu") == 0;
    void *P = (void *)(uintptr_t)0x10000; /* aligned stand-in, never dereferenced */
    char buf[4096];
    /* pure helpers */
    const int64_t ks[] = {1, 3, 15, 16, 17, 63, 64, 65, 127, 128, 129, 4095, 4096, 4099, 11008,
                          16909320, 16909321, INT64_MAX / 2};
    for (size_t i = 0; i < sizeof ks / sizeof ks[0]; ++i)
        for (int l = -1; l < 4; ++l) (void)bitlinear_packed_row_bytes(ks[i], l);
    EXPECT(bitlinear_packed_row_bytes(0, 0) == -1);
    EXPECT(bitlinear_pack_workspace_bytes(INT64_MAX, INT64_MAX) == 0);
    EXPECT(bitlinear_pack_workspace_bytes(4096, 4096) > 0);
    for (int s = -1; s < 5; ++s) EXPECT(bitlinear_status_string(s) != NULL);
    EXPECT(bitlinear_version() >> 16 == 1);
    EXPECT(strlen(bitlinear_source_hash()) > 0);
    EXPECT(bitlinear_pack_noalloc_max_scratch_bytes() == 16384);

    /* dispatch dry runs over many shapes, layouts and output types */
    const int64_t ms[] = {0, 1, 2, 4, 5, 16, 17, 33, 48, 96, 128, 129, 255, 256, 511, 512, 1000,
                          2048, 4096, 65600, 70000, 65535LL * 128};
    const int64_t ns[] = {0, 1, 7, 16, 200, 256, 4096, 11008, 12288, 32768, 100000};
    const int64_t kk[] = {1, 17, 64, 256, 4096, 4176, 5000, 11008, 16909320};
    long launches = 0;
    for (size_t a = 0; a < sizeof ms / sizeof ms[0]; ++a)
        for (size_t b = 0; b < sizeof ns / sizeof ns[0]; ++b)
            for (size_t c = 0; c < sizeof kk / sizeof kk[0]; ++c)
                for (int l = 0; l < 3; ++l)
                    for (int yd = 0; yd < 2; ++yd) {
                        const int n = bitlinear_forward_plan(ms[a], ns[b], kk[c], l, yd, 0, buf,
                                                             sizeof buf);
                        EXPECT(n >= 0);
                        if (ms[a] > 0 && ns[b] > 0) EXPECT(n >= 1);
                        launches += n;
                        if (ms[a] <= 4) {
                            const int f = bitlinear_forward_plan(ms[a], ns[b], kk[c], l, yd, 1, buf,
                                                                 sizeof buf);
                            EXPECT(f >= 0);
                        }
                    }
    EXPECT(bitlinear_forward_plan(5, 8, 8, 0, 0, 1, buf, sizeof buf) == -1);
    EXPECT(bitlinear_forward_plan(1, 8, 0, 0, 0, 0, buf, sizeof buf) == -1);
    EXPECT(bitlinear_forward_plan(1, 8, 8, 9, 0, 0, buf, sizeof buf) == -1);
    EXPECT(bitlinear_forward_plan(1, 8, 8, 0, 0, 0, NULL, 0) == 1);
    EXPECT(bitlinear_forward_plan(2048, 11008, 4096, 0, 1, 0, buf, 8) == 1 && strlen(buf) == 7);

    /* argument errors come back before any device call */
    EXPECT(bitlinear_pack_weights(NULL, 0, 4, 64, 0, 0, 1e-5f, P, P, P, 1 << 20, NULL) ==
           BL_ERR_INVALID_ARG);
    EXPECT(bitlinear_pack_weights(P, 0, 4, 64, 0, 2, 1e-5f, P, P, P, 1 << 20, NULL) ==
           BL_ERR_INVALID_ARG);
    EXPECT(bitlinear_pack_weights(P, 0, INT64_MAX, 64, 0, 0, 1e-5f, P, P, P, 1 << 20, NULL) ==
           BL_ERR_INVALID_ARG);
    EXPECT(bitlinear_pack_weights(P, 0, 4, 64, 0, 0, 1e-5f, P, P, P, 0, NULL) == BL_ERR_INVALID_ARG);
    EXPECT(bitlinear_pack_weights_noalloc(P, 0, 4, 64, 0, 0, -1.f, P, P, NULL) ==
           BL_ERR_INVALID_ARG);
    EXPECT(bitlinear_quant_acts(P, 0, -1, 64, P, P, NULL) == BL_ERR_INVALID_ARG);
    EXPECT(bitlinear_quant_acts(P, 7, 1, 64, P, P, NULL) == BL_ERR_INVALID_ARG);
    EXPECT(bitlinear_forward(P, P, P, 0, P, 1, 1, 16909321, P, 0, NULL, NULL) == BL_ERR_INVALID_ARG);
    EXPECT(bitlinear_forward(P, P, (uint8_t *)P + 4, 0, P, 1, 1, 64, P, 0, NULL, NULL) ==
           BL_ERR_INVALID_ARG);
    EXPECT(bitlinear_linear(P, 1, P, 0, P, 5, 8, 64, P, 0, NULL, NULL) == BL_ERR_UNSUPPORTED);
    const int64_t segs_bad[] = {4, 0};
    EXPECT(bitlinear_forward_segmented(P, P, P, 0, P, segs_bad, 2, 1, 64, P, 0, NULL, NULL) ==
           BL_ERR_INVALID_ARG);
    const int64_t segs_big[] = {INT64_MAX, INT64_MAX};
    EXPECT(bitlinear_forward_segmented(P, P, P, 0, P, segs_big, 2, 1, 64, P, 0, NULL, NULL) ==
           BL_ERR_INVALID_ARG);
    EXPECT(bitlinear_forward_lut(P, P, P, 0, P, 1, 8, 64, P, 0, NULL, NULL) == BL_ERR_UNSUPPORTED);
    EXPECT(bitlinear_backward_input(P, 1, P, 0, P, 4, 12, 64, P, NULL) == BL_ERR_UNSUPPORTED);
    EXPECT(bitlinear_backward_weight(P, P, 1, 4, 8, 12, P, NULL) == BL_ERR_UNSUPPORTED);
    /* empty problems are no-ops */
    EXPECT(bitlinear_forward(P, P, P, 0, P, 0, 8, 64, P, 0, NULL, NULL) == BL_OK);
    EXPECT(bitlinear_quant_acts(P, 0, 0, 64, P, P, NULL) == BL_OK);
    if (!have_gpu) {
        /* valid arguments, no gfx950 device: refused at the device check */
        EXPECT(bitlinear_pack_weights(P, 0, 4, 64, 0, 0, 1e-5f, P, P, P, 1 << 20, NULL) ==
               BL_ERR_DEVICE);
        EXPECT(bitlinear_pack_weights_noalloc(P, 0, 4, 64, 0, 0, 1e-5f, P, P, NULL) ==
               BL_ERR_DEVICE);
        EXPECT(bitlinear_quant_acts(P, 0, 4, 64, P, P, NULL) == BL_ERR_DEVICE);
        EXPECT(bitlinear_forward(P, P, P, 0, P, 4, 8, 64, P, 0, NULL, NULL) == BL_ERR_DEVICE);
        EXPECT(bitlinear_linear(P, 1, P, 0, P, 1, 8, 64, P, 0, NULL, NULL) == BL_ERR_DEVICE);
    }
    if (fails) {
        fprintf(stderr, "abi driver: %d FAILED checks\n", fails);
        return 1;
    }
    printf("abi driver: ok (%ld planned launches)\n", launches);
    return 0;
}
