/* Drives every function of the CPU oracle over ragged shapes so that a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer can catch out-of-range
 * accesses and undefined arithmetic. Exits non-zero on a failed round trip;
 * the sanitizers abort on their own findings. Test infrastructure: it links
 * the oracle only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

float orc_absmean(const float *w, int64_t count, double *mean64);
float orc_mean(const float *w, int64_t count, double *mean64);
int64_t orc_ternary_codes(const float *w, int64_t count, float gamma, float eps, double gamma64,
                          int8_t *codes, uint8_t *flag);
int64_t orc_binary_codes(const float *w, int64_t count, float alpha, double alpha64,
                         int8_t *codes, uint8_t *flag);
int64_t orc_row_bytes_2bit(int64_t K);
void orc_pack_2bit(const int8_t *codes, int64_t N, int64_t K, uint8_t *packed);
int64_t orc_unpack_2bit(const uint8_t *packed, int64_t N, int64_t K, int8_t *codes);
int64_t orc_row_bytes_base3(int64_t K);
void orc_pack_base3(const int8_t *codes, int64_t N, int64_t K, uint8_t *packed);
int64_t orc_unpack_base3(const uint8_t *packed, int64_t N, int64_t K, int8_t *codes);
int64_t orc_row_bytes_1bit(int64_t K);
int64_t orc_pack_1bit(const int8_t *codes, int64_t N, int64_t K, uint8_t *packed);
int64_t orc_unpack_1bit(const uint8_t *packed, int64_t N, int64_t K, int8_t *codes);
int64_t orc_quant_acts(const float *x, int64_t M, int64_t K, int8_t *xq, float *scale,
                       uint8_t *flag);
int64_t orc_int_product(const int8_t *xq, const int8_t *codes, int64_t M, int64_t N, int64_t K,
                        int32_t *acc);
void orc_epilogue(const int32_t *acc, float gamma, const float *scale, int64_t M, int64_t N,
                  double *y);
uint16_t orc_bf16_rne(float f);
void orc_bf16_rne_array(const float *f, int64_t count, uint16_t *out);
void orc_ste_grad_x(const float *grad_y, const int8_t *codes, float gamma, int64_t M, int64_t N,
                    int64_t K, double *grad_x);
void orc_ste_grad_w(const float *grad_y, const float *x, int64_t M, int64_t N, int64_t K,
                    double *grad_w);

static uint64_t rng = 88172645463325252ull;
static float urand(void) { /* xorshift64, uniform in [-1, 1) */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (float)((rng >> 11) * (1.0 / 9007199254740992.0)) * 2.f - 1.f;
}

static int check_layout(const char *name, int8_t *codes, int64_t N, int64_t K,
                        int64_t (*rb)(int64_t), void (*pack)(const int8_t *, int64_t, int64_t, uint8_t *),
                        int64_t (*unpack)(const uint8_t *, int64_t, int64_t, int8_t *)) {
    const int64_t bytes = N * rb(K);
    uint8_t *p = malloc((size_t)bytes);
    int8_t *back = malloc((size_t)(N * K));
    pack(codes, N, K, p);
    const int64_t bad = unpack(p, N, K, back);
    int fail = bad != 0;
    for (int64_t i = 0; i < N * K; ++i) fail |= back[i] != codes[i];
    if (fail) fprintf(stderr, "%s round trip failed N=%lld K=%lld\n", name, (long long)N, (long long)K);
    free(p);
    free(back);
    return fail;
}

int main(void) {
    const int64_t shapes[][3] = {{1, 1, 1}, {3, 5, 7}, {8, 256, 256}, {2, 17, 129}, {5, 33, 4099},
                                 {1, 7, 80}, {4, 3, 64}};
    int fail = 0;
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
        const int64_t M = shapes[s][0], N = shapes[s][1], K = shapes[s][2];
        float *w = malloc(sizeof(float) * (size_t)(N * K));
        float *x = malloc(sizeof(float) * (size_t)(M * K));
        float *gy = malloc(sizeof(float) * (size_t)(M * N));
        for (int64_t i = 0; i < N * K; ++i) w[i] = 0.02f * urand();
        for (int64_t i = 0; i < M * K; ++i) x[i] = urand();
        for (int64_t i = 0; i < M * N; ++i) gy[i] = 1e-3f * urand();
        int8_t *codes = malloc((size_t)(N * K)), *bcodes = malloc((size_t)(N * K));
        uint8_t *flag = malloc((size_t)(N * K));
        double g64, a64;
        const float g = orc_absmean(w, N * K, &g64);
        const float a = orc_mean(w, N * K, &a64);
        orc_ternary_codes(w, N * K, g, 1e-5f, g64, codes, flag);
        orc_binary_codes(w, N * K, a, a64, bcodes, flag);
        fail |= check_layout("2bit", codes, N, K, orc_row_bytes_2bit, orc_pack_2bit, orc_unpack_2bit);
        fail |= check_layout("base3", codes, N, K, orc_row_bytes_base3, orc_pack_base3,
                             orc_unpack_base3);
        {
            uint8_t *p = malloc((size_t)(N * orc_row_bytes_1bit(K)));
            int8_t *back = malloc((size_t)(N * K));
            fail |= orc_pack_1bit(bcodes, N, K, p) != 0;
            fail |= orc_unpack_1bit(p, N, K, back) != 0;
            for (int64_t i = 0; i < N * K; ++i) fail |= back[i] != bcodes[i];
            free(p);
            free(back);
        }
        int8_t *xq = malloc((size_t)(M * K));
        float *sc = malloc(sizeof(float) * (size_t)M);
        uint8_t *xf = malloc((size_t)(M * K));
        orc_quant_acts(x, M, K, xq, sc, xf);
        int32_t *acc = malloc(sizeof(int32_t) * (size_t)(M * N));
        fail |= orc_int_product(xq, codes, M, N, K, acc) != 0;
        double *y = malloc(sizeof(double) * (size_t)(M * N));
        orc_epilogue(acc, g, sc, M, N, y);
        float *yf = malloc(sizeof(float) * (size_t)(M * N));
        uint16_t *yb = malloc(sizeof(uint16_t) * (size_t)(M * N));
        for (int64_t i = 0; i < M * N; ++i) yf[i] = (float)y[i];
        orc_bf16_rne_array(yf, M * N, yb);
        double *gx = malloc(sizeof(double) * (size_t)(M * K));
        double *gw = malloc(sizeof(double) * (size_t)(N * K));
        orc_ste_grad_x(gy, codes, g, M, N, K, gx);
        orc_ste_grad_w(gy, x, M, N, K, gw);
        for (int64_t i = 0; i < M * K; ++i) fail |= !isfinite(gx[i]);
        free(w); free(x); free(gy); free(codes); free(bcodes); free(flag); free(xq); free(sc);
        free(xf); free(acc); free(y); free(yf); free(yb); free(gx); free(gw);
    }
    fail |= orc_bf16_rne(1.0f) != 0x3F80;
    if (fail) {
        fprintf(stderr, "oracle driver: FAILED\n");
        return 1;
    }
    printf("oracle driver: ok\n");
    return 0;
}
