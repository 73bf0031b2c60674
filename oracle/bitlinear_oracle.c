/*
 * BitLinear oracle: a plain, slow, scalar CPU implementation of the BitNet
 * b1.58 BitLinear forward pass (and its 1-bit and training-step relatives).
 *
 * THIS IS TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it. The GPU library never calls,
 * links or includes anything here, and this file includes nothing of the GPU
 * library: the two share no code, headers, tables or constants.
 *
 * Sources (web pages, cited by title and section):
 *   [QAT-zh]   "QAT与BitNet：1-bit及1.58-bit量化训练解析" (kongchang.com, zh)
 *   [QAT-en]   "QAT and BitNet: A Deep Dive into 1-bit and 1.58-bit
 *               Quantization-Aware Training" (kongchang.com, en)
 *   [b158]     "BitNet b1.58深度解析：三值权重如何重塑大模型推理" (0539edu.com)
 *
 * Every floating-point step that decides an integer (a weight code, an
 * activation code) is taken in IEEE fp32, as the pages' PyTorch code does
 * (default dtype float32). Build with -ffp-contract=off so no step is fused.
 * Reductions that the pages write as a mean are accumulated in fp64 and
 * rounded once to fp32. Products are brute force in int64.
 *
 * Parity pins: every function here is pinned by tests under tests/ that do
 * not call back into this file for the expected value (worked examples the
 * pages print, exact rational arithmetic, brute force, closed forms).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

/* ------------------------------------------------------------------------ */
/* Weight scale: gamma = mean(|W|) over the whole matrix.
 * [QAT-en] "The Ternary Weight Recipe", step 1 and its ternary_weights code
 * (w.abs().mean()); [b158] §3.1 first step (gamma = mean(|W|)); [b158] §5.2
 * ternary_weight_quantize reduces the whole tensor, so the mean is per matrix.
 * Accumulated in fp64 in row-major order, divided in fp64, rounded once.
 * *mean64 (may be NULL) receives the unrounded fp64 mean. */
float orc_absmean(const float *w, int64_t count, double *mean64)
{
    double s = 0.0;
    for (int64_t i = 0; i < count; ++i)
        s += fabs((double)w[i]);
    double m = s / (double)count;
    if (mean64) *mean64 = m;
    return (float)m;
}

/* alpha = mean(W) (signed) for the 1-bit BitNet weights.
 * [QAT-en] "The BitLinear Recipe" step 2 (take the mean alpha of the weights).
 * Same accumulation rule as orc_absmean. */
float orc_mean(const float *w, int64_t count, double *mean64)
{
    double s = 0.0;
    for (int64_t i = 0; i < count; ++i)
        s += (double)w[i];
    double m = s / (double)count;
    if (mean64) *mean64 = m;
    return (float)m;
}

/* Ternary codes: c = clamp(round(w / (gamma + eps)), -1, 1).
 * [QAT-en] "The Ternary Weight Recipe" code: (w / (gamma + eps)).round()
 * .clamp(-1, 1) with eps = 1e-5; [b158] §3.1 steps 2-3.
 * fp32: d = gamma + eps, r = w / d (IEEE division), rintf = round half to
 * even (torch.round). flag[i] = 1 when the fp64 quotient w/(gamma64+eps) lies
 * within 1e-6 relative of the only boundary that survives the clamp, |r|=0.5.
 * flag may be NULL. Returns the number of flagged elements. */
int64_t orc_ternary_codes(const float *w, int64_t count, float gamma, float eps,
                          double gamma64, int8_t *codes, uint8_t *flag)
{
    const float d = gamma + eps;
    const double d64 = gamma64 + (double)eps;
    int64_t nflag = 0;
    for (int64_t i = 0; i < count; ++i) {
        float r = w[i] / d;
        float q = rintf(r);
        if (q > 1.0f) q = 1.0f;
        if (q < -1.0f) q = -1.0f;
        codes[i] = (int8_t)q;
        double r64 = fabs((double)w[i] / d64);
        int f = fabs(r64 - 0.5) <= 1e-6 * 0.5;
        if (flag) flag[i] = (uint8_t)f;
        nflag += f;
    }
    return nflag;
}

/* 1-bit codes: +1 where w > alpha, else -1.
 * [QAT-en] "The BitLinear Recipe" step 2 (values above alpha become +1,
 * values below become -1). A weight exactly equal to alpha is not covered by
 * the page; it maps to -1 here. Compared in fp32. flag[i] = 1 when
 * |w - alpha64| <= 1e-6 |alpha64|. */
int64_t orc_binary_codes(const float *w, int64_t count, float alpha,
                         double alpha64, int8_t *codes, uint8_t *flag)
{
    int64_t nflag = 0;
    for (int64_t i = 0; i < count; ++i) {
        codes[i] = (int8_t)(w[i] > alpha ? 1 : -1);
        int f = fabs((double)w[i] - alpha64) <= 1e-6 * fabs(alpha64);
        if (flag) flag[i] = (uint8_t)f;
        nflag += f;
    }
    return nflag;
}

/* ------------------------------------------------------------------------ */
/* Storage. [b158] §2.3 and §6.3: two bits per weight with the three patterns
 * 00, 01, 10 (four weights per byte), or five ternary values per byte since
 * 3^5 = 243 <= 256; [QAT-en] "Why Is It Called 1.58 Bits?".
 *
 * 2-bit layout (bit placement is not fixed by the pages; this is the reading
 * adopted): the stored value is u = c + 1, so 00 = -1, 01 = 0, 10 = +1 and 11
 * is never written. A row of K codes occupies row_bytes =
 * roundup(ceil(K/4), 16) bytes. Codes are grouped by 16 (one 32-bit
 * little-endian word per group); code k of the row lives in
 *     byte  4*(k/16) + (k%4),   bits  2*((k%16)/4) .. +1.
 * Padding codes are 0 (u = 1).                                              */
int64_t orc_row_bytes_2bit(int64_t K)
{
    int64_t b = (K + 3) / 4;
    return (b + 15) / 16 * 16;
}

void orc_pack_2bit(const int8_t *codes, int64_t N, int64_t K, uint8_t *packed)
{
    const int64_t rb = orc_row_bytes_2bit(K);
    for (int64_t n = 0; n < N; ++n) {
        uint8_t *row = packed + n * rb;
        for (int64_t j = 0; j < rb; ++j) row[j] = 0;
        for (int64_t k = 0; k < rb * 4; ++k) {
            int u = (k < K) ? codes[n * K + k] + 1 : 1;
            int64_t byte = 4 * (k / 16) + (k % 4);
            int shift = 2 * (int)((k % 16) / 4);
            row[byte] = (uint8_t)(row[byte] | (u << shift));
        }
    }
}

/* Returns the number of invalid fields (pattern 11) met; such codes are
 * written as 0. */
int64_t orc_unpack_2bit(const uint8_t *packed, int64_t N, int64_t K, int8_t *codes)
{
    const int64_t rb = orc_row_bytes_2bit(K);
    int64_t bad = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t byte = 4 * (k / 16) + (k % 4);
            int shift = 2 * (int)((k % 16) / 4);
            int u = (packed[n * rb + byte] >> shift) & 3;
            if (u == 3) { ++bad; u = 1; }
            codes[n * K + k] = (int8_t)(u - 1);
        }
    }
    return bad;
}

/* Base-3 layout (reading adopted): t = c + 1 in {0,1,2}; byte j of a row
 * holds codes 5j..5j+4 as the base-3 number t0 + 3 t1 + 9 t2 + 27 t3 + 81 t4
 * (first code in the least significant trit), values 0..242. row_bytes =
 * roundup(ceil(K/5), 16); padding trits are t = 1 (code 0).                 */
int64_t orc_row_bytes_base3(int64_t K)
{
    int64_t b = (K + 4) / 5;
    return (b + 15) / 16 * 16;
}

void orc_pack_base3(const int8_t *codes, int64_t N, int64_t K, uint8_t *packed)
{
    const int64_t rb = orc_row_bytes_base3(K);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < rb; ++j) {
            int v = 0, p = 1;
            for (int i = 0; i < 5; ++i) {
                int64_t k = 5 * j + i;
                int t = (k < K) ? codes[n * K + k] + 1 : 1;
                v += t * p;
                p *= 3;
            }
            packed[n * rb + j] = (uint8_t)v;
        }
    }
}

/* Returns the number of invalid bytes (243..255) met; their codes are 0. */
int64_t orc_unpack_base3(const uint8_t *packed, int64_t N, int64_t K, int8_t *codes)
{
    const int64_t rb = orc_row_bytes_base3(K);
    int64_t bad = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; 5 * j < K; ++j) {
            int v = packed[n * rb + j];
            int valid = v < 243;
            if (!valid) ++bad;
            for (int i = 0; i < 5; ++i) {
                int64_t k = 5 * j + i;
                int t = v % 3;
                v /= 3;
                if (k < K) codes[n * K + k] = (int8_t)(valid ? t - 1 : 0);
            }
        }
    }
    return bad;
}

/* 1-bit layout, for the binary (1-bit BitLinear) codes only: [QAT-en] "What
 * Does BitLinear Change?" stores each +-1 weight in one bit. Bit placement is
 * not fixed by the pages; reading adopted: bit 1 = +1, bit 0 = -1; codes are
 * grouped by 32 (one 32-bit little-endian word per group) and code k of the
 * row lives in
 *     byte  4*(k/32) + (k%4),   bit  (k%32)/4.
 * A row occupies roundup(ceil(K/8), 16) bytes; padding bits are 0.          */
int64_t orc_row_bytes_1bit(int64_t K)
{
    int64_t b = (K + 7) / 8;
    return (b + 15) / 16 * 16;
}

/* Returns the number of codes that are not +-1 (a ternary 0 has no 1-bit
 * encoding); they are written as bit 0. */
int64_t orc_pack_1bit(const int8_t *codes, int64_t N, int64_t K, uint8_t *packed)
{
    const int64_t rb = orc_row_bytes_1bit(K);
    int64_t bad = 0;
    for (int64_t n = 0; n < N; ++n) {
        uint8_t *row = packed + n * rb;
        for (int64_t j = 0; j < rb; ++j) row[j] = 0;
        for (int64_t k = 0; k < K; ++k) {
            int c = codes[n * K + k];
            if (c != 1 && c != -1) ++bad;
            if (c == 1) {
                int64_t byte = 4 * (k / 32) + (k % 4);
                int bit = (int)((k % 32) / 4);
                row[byte] = (uint8_t)(row[byte] | (1 << bit));
            }
        }
    }
    return bad;
}

/* Every bit pattern is valid; returns 0. */
int64_t orc_unpack_1bit(const uint8_t *packed, int64_t N, int64_t K, int8_t *codes)
{
    const int64_t rb = orc_row_bytes_1bit(K);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t byte = 4 * (k / 32) + (k % 4);
            int bit = (int)((k % 32) / 4);
            codes[n * K + k] = (int8_t)(((packed[n * rb + byte] >> bit) & 1) ? 1 : -1);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Per-token symmetric absmax INT8 activations.
 * [b158] §3.2: scale = max(|x|) per token, x_q = clamp(round(x / scale *
 * 127), -127, 127); [b158] §5.2 activation_quantize_int8 clamps the scale
 * below at 1e-6. fp32 steps in the written order: division, then * 127, then
 * round half to even, then clamp. flag[m*K+k] = 1 when the fp64 value
 * |x/s*127| is within 1e-6 relative of a half-integer (a rounding boundary).
 * Returns the number of flagged elements. */
int64_t orc_quant_acts(const float *x, int64_t M, int64_t K,
                       int8_t *xq, float *scale, uint8_t *flag)
{
    int64_t nflag = 0;
    for (int64_t m = 0; m < M; ++m) {
        const float *row = x + m * K;
        float s = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(row[k]);
            if (a > s) s = a;
        }
        if (s < 1e-6f) s = 1e-6f;
        scale[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            float t = row[k] / s;
            t = t * 127.0f;
            float q = rintf(t);
            if (q > 127.0f) q = 127.0f;
            if (q < -127.0f) q = -127.0f;
            xq[m * K + k] = (int8_t)q;
            double q64 = fabs((double)row[k] / (double)s * 127.0);
            double h = floor(q64) + 0.5;
            int f = fabs(q64 - h) <= 1e-6 * h;
            if (flag) flag[m * K + k] = (uint8_t)f;
            nflag += f;
        }
    }
    return nflag;
}

/* ------------------------------------------------------------------------ */
/* Integer product acc[m,n] = sum_k xq[m,k] * c[n,k] (y = x W^T, W is
 * [out, in]). [b158] §4.2: y_i = sum_j w_ij x_j, where w = +1 adds, w = -1
 * subtracts and w = 0 skips; [b158] §3.3: INT32 accumulator. Brute force in
 * int64 with no ternary shortcut, then narrowed. Returns the number of
 * outputs whose |acc| exceeds 2^31 - 1 (0 for every K <= 16909320). */
int64_t orc_int_product(const int8_t *xq, const int8_t *codes, int64_t M,
                        int64_t N, int64_t K, int32_t *acc)
{
    int64_t overflow = 0;
#pragma omp parallel for reduction(+ : overflow) schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const int8_t *c = codes + n * K;
        for (int64_t m = 0; m < M; ++m) {
            const int8_t *q = xq + m * K;
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)q[k] * (int64_t)c[k];
            if (s > 2147483647LL || s < -2147483647LL) ++overflow;
            acc[m * N + n] = (int32_t)s;
        }
    }
    return overflow;
}

/* Dequant epilogue: y[m,n] = acc[m,n] * gamma * scale[m] / 127.
 * [b158] §5.2-5.3: x_deq = x_q / 127 * scale and out * gamma (the weight
 * scale is gamma, not gamma + eps); [QAT-en] "What Does BitLinear Change?":
 * the two scaling factors stretch the result back. One fp64 evaluation per
 * element; y64 receives it unrounded. */
void orc_epilogue(const int32_t *acc, float gamma, const float *scale,
                  int64_t M, int64_t N, double *y64)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y64[m * N + n] = (double)acc[m * N + n] * (double)gamma *
                             (double)scale[m] / 127.0;
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs only). */
uint16_t orc_bf16_rne(float f)
{
    union { float f; uint32_t u; } v;
    v.f = f;
    uint32_t lsb = (v.u >> 16) & 1u;
    return (uint16_t)((v.u + 0x7FFFu + lsb) >> 16);
}

void orc_bf16_rne_array(const float *f, int64_t count, uint16_t *out)
{
    for (int64_t i = 0; i < count; ++i) out[i] = orc_bf16_rne(f[i]);
}

/* ------------------------------------------------------------------------ */
/* Training step with the straight-through estimator (identity STE).
 * [QAT-en] "How Gradients Flow" (backward pretends rounding is the
 * identity); [b158] §5.3 (W_effective = W_ternary + W - W.detach()).
 * The quantised forward is y = gamma * (x W_q^T); under the identity STE the
 * gradients are grad_x = grad_y (gamma W_q) and grad_W = grad_y^T x, with the
 * scales held constant. fp64 accumulation, written out as fp64. */
void orc_ste_grad_x(const float *grad_y, const int8_t *codes, float gamma,
                    int64_t M, int64_t N, int64_t K, double *grad_x)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            double s = 0.0;
            for (int64_t n = 0; n < N; ++n)
                s += (double)grad_y[m * N + n] * (double)codes[n * K + k];
            grad_x[m * K + k] = s * (double)gamma;
        }
}

void orc_ste_grad_w(const float *grad_y, const float *x, int64_t M, int64_t N,
                    int64_t K, double *grad_w)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            double s = 0.0;
            for (int64_t m = 0; m < M; ++m)
                s += (double)grad_y[m * N + n] * (double)x[m * K + k];
            grad_w[n * K + k] = s;
        }
}

/* Number of OpenMP threads the product loops would use (1 without OpenMP). */
/* Threads the OpenMP loops above use from now on (the CPU baseline times
 * the oracle on one thread and on all host threads). */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
