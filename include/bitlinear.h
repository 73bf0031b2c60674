/*
 * bitlinear.h — C ABI of the MI355X (gfx950) BitLinear library.
 *
 * The library computes the BitNet b1.58 BitLinear forward pass in five steps:
 * absmean ternarisation of a weight matrix, packing of the codes, per-token
 * symmetric absmax INT8 activation quantisation, an integer product of INT8
 * activations against {-1, 0, +1} codes with INT32 accumulation, and the
 * gamma * scale / 127 dequant epilogue. Sources, cited by page title and
 * section:
 *   [QAT-en] "QAT and BitNet: A Deep Dive into 1-bit and 1.58-bit
 *            Quantization-Aware Training" (kongchang.com)
 *   [QAT-zh] "QAT与BitNet：1-bit及1.58-bit量化训练解析" (kongchang.com)
 *   [b158]   "BitNet b1.58深度解析：三值权重如何重塑大模型推理" (0539edu.com)
 *
 * Conventions for every call:
 *  - Shapes: W is [N, K] row-major (out_features x in_features), x is [M, K]
 *    row-major (M tokens), y is [M, N] row-major: y = x W^T ([b158] §4.2,
 *    y_i = sum_j w_ij x_j).
 *  - Every array argument is a DEVICE pointer, owned and allocated by the
 *    caller, 16-byte aligned, except the weight scales (gamma, gammas), which
 *    need only 4-byte alignment so that a stack of matrices can keep its
 *    scales in consecutive floats. The library never allocates, frees or
 *    synchronises: each call only enqueues kernels on `stream` (a hipStream_t
 *    passed as void*, NULL = the default stream) and returns.
 *  - Argument errors are detected before any HIP call; the call then returns
 *    BL_ERR_INVALID_ARG with no side effect. Bad arguments are: a NULL
 *    required pointer, a misaligned pointer, a negative size, K < 1,
 *    K > 16909320 (127*K must fit in INT32), an unknown dtype / layout /
 *    scheme, a too-small workspace. M = 0 or N = 0 is an empty problem and
 *    returns BL_OK without launching anything (pack_weights needs N >= 1).
 *  - If the current device is not a gfx950 GPU, or a launch fails, the call
 *    returns BL_ERR_DEVICE (the HIP error is consumed). Kernels that fault
 *    later surface at the caller's next synchronisation.
 *  - Non-finite inputs (NaN, Inf) are outside the contract.
 *  - Calls may come from several host threads and streams. The library's
 *    only process-wide state is per-device and set once: the result of the
 *    architecture check, the compute-unit count and the raised LDS limit of
 *    kernels that use more than 64 KiB, all kept in atomics. Concurrent calls
 *    that write the same output buffers race like any other GPU work.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BL_OK = 0,
    BL_ERR_INVALID_ARG = 1,
    BL_ERR_UNSUPPORTED = 2,
    BL_ERR_DEVICE = 3
} bl_status;

/* Element types of floating-point inputs and outputs. bf16 values are
 * widened exactly to fp32 before any arithmetic. */
typedef enum { BL_F32 = 0, BL_BF16 = 1 } bl_dtype;

/* Packed weight layouts ([b158] §2.3 and §6.3: two bits per weight with the
 * patterns 00, 01, 10, four weights per byte; or five ternary values per
 * byte since 3^5 = 243 <= 256, 1.6 bits per weight).
 *
 * BL_PACK_2BIT: the stored field is u = c + 1 (00 = -1, 01 = 0, 10 = +1; 11
 *   is never written). A row takes row_bytes = roundup(ceil(K/4), 16) bytes.
 *   Codes are grouped by 16 into one little-endian 32-bit word; code k of a
 *   row sits in byte 4*(k/16) + (k%4) at bits 2*((k%16)/4)..+1, so that
 *   (word >> 2j) & 0x03030303 holds codes 4j..4j+3 of the group in its four
 *   bytes. Padding codes (k >= K) are 0.
 * BL_PACK_BASE3: byte j of a row holds codes 5j..5j+4 as the base-3 number
 *   t0 + 3 t1 + 9 t2 + 27 t3 + 81 t4 with t = c + 1 (first code in the least
 *   significant trit; values 0..242). row_bytes = roundup(ceil(K/5), 16);
 *   padding trits are t = 1 (code 0).
 * BL_PACK_1BIT: binary codes only (BL_BINARY), one bit per weight as in the
 *   1-bit BitLinear ([QAT-en] "What Does BitLinear Change?": +-1 weights at
 *   1 bit each). Bit 1 = +1, bit 0 = -1. Codes are grouped by 32 into one
 *   little-endian 32-bit word; code k of a row sits in byte 4*(k/32) + (k%4)
 *   at bit (k%32)/4, so that (word >> j) & 0x01010101 holds codes 4j..4j+3 in
 *   its four bytes. row_bytes = roundup(ceil(K/8), 16); padding bits are 0
 *   (the products never read them). Every bit pattern is a valid matrix. */
typedef enum { BL_PACK_2BIT = 0, BL_PACK_BASE3 = 1, BL_PACK_1BIT = 2 } bl_layout;

/* Weight quantisers.
 * BL_TERNARY (b1.58): gamma = mean|W|; c = clamp(round(W / (gamma + eps)),
 *   -1, 1), round half to even ([QAT-en] "The Ternary Weight Recipe" and its
 *   ternary_weights code; [b158] §3.1).
 * BL_BINARY (1-bit BitNet): alpha = mean(W); c = +1 where W > alpha, else -1;
 *   the weight scale is beta = mean|W| ([QAT-en] "The BitLinear Recipe",
 *   steps 2 and 4). */
typedef enum { BL_TERNARY = 0, BL_BINARY = 1 } bl_scheme;

/* Bytes one packed row of K codes occupies in `layout`; -1 for K < 1 or an
 * unknown layout. Host-only, pure. */
int64_t bitlinear_packed_row_bytes(int64_t K, int layout);

/* Device workspace (bytes) bitlinear_pack_weights needs for an N x K matrix:
 * it holds the per-block partial sums of the two-pass mean reduction. 0 for
 * N < 1, K < 1 or an N * K past the int64 range (shapes the pack refuses). */
size_t bitlinear_pack_workspace_bytes(int64_t N, int64_t K);

/* Quantise and pack a latent weight matrix ([QAT-en] "The Ternary Weight
 * Recipe"; [b158] §3.1 and §6.3; [QAT-en] "The BitLinear Recipe" for
 * BL_BINARY).
 *   W         [N, K] w_dtype (BL_F32 or BL_BF16), read only.
 *   eps       added to gamma before the division (1e-5 in the pages' code);
 *             ignored by BL_BINARY. Must be finite and >= 0.
 *   packed    out: [N, bitlinear_packed_row_bytes(K, layout)] uint8.
 *   gamma     out: 1 float, the weight scale the epilogue multiplies by
 *             (gamma = mean|W| for BL_TERNARY; beta = mean|W| for BL_BINARY).
 *             It stays on the device; no host synchronisation happens.
 *   workspace device scratch of at least bitlinear_pack_workspace_bytes(N, K)
 *             bytes; its contents are overwritten.
 * The mean is accumulated in fp64 and rounded once to fp32. Layout
 * BL_PACK_1BIT holds binary codes only: BL_TERNARY with it returns
 * BL_ERR_INVALID_ARG. */
bl_status bitlinear_pack_weights(const void *W, int w_dtype, int64_t N, int64_t K,
                                 int scheme, int layout, float eps,
                                 uint8_t *packed, float *gamma,
                                 void *workspace, size_t workspace_bytes,
                                 void *stream);

/* Allocation-free variant of bitlinear_pack_weights, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same quantisation and packing, with
 * the same arguments and results, but the mean's partial sums live in the
 * library's own scratch array of bitlinear_pack_noalloc_max_scratch_bytes()
 * bytes (16 KiB), held by every GPU the library runs on until the process
 * ends, instead of in a caller workspace. Nothing is allocated or freed, by
 * the library or by any routine it calls. Every call on one GPU shares that
 * GPU's scratch: calls that overlap on one GPU (concurrent streams, threads
 * or graph replays) race and may produce wrong scales; serialise them. Each
 * call rewrites every partial it reads, so nothing needs clearing between
 * calls. Shapes whose partial sums would not fit return BL_ERR_INVALID_ARG
 * (the mean uses at most 1024 partials, so every accepted shape fits); a
 * failed look-up of the scratch's device address returns BL_ERR_DEVICE. */
bl_status bitlinear_pack_weights_noalloc(const void *W, int w_dtype, int64_t N, int64_t K,
                                         int scheme, int layout, float eps,
                                         uint8_t *packed, float *gamma, void *stream);

/* Bytes of the allocation-free pack's scratch array (per GPU). Host-only. */
size_t bitlinear_pack_noalloc_max_scratch_bytes(void);

/* Per-token symmetric absmax INT8 quantisation ([b158] §3.2 and §5.2):
 * s_m = max(max_k |x[m,k]|, 1e-6); xq = clamp(round(x / s_m * 127), -127, 127)
 * with fp32 division, then * 127, then round half to even.
 *   x      [M, K] x_dtype (BL_F32 or BL_BF16), read only.
 *   xq     out: [M, K] int8 codes (never -128).
 *   scale  out: [M] float, the s_m above. */
bl_status bitlinear_quant_acts(const void *x, int x_dtype, int64_t M, int64_t K,
                               int8_t *xq, float *scale, void *stream);

/* Integer product and dequant epilogue ([b158] §4.2: +1 adds, -1 subtracts,
 * 0 skips; §3.3: INT32 accumulator; §5.2-5.3: x_q / 127 * scale and
 * out * gamma):
 *   acc[m,n] = sum_k xq[m,k] * c[n,k]             (exact INT32)
 *   y[m,n]   = acc[m,n] * gamma * scale[m] / 127  (fp32, then y_dtype)
 *   xq, scale  from bitlinear_quant_acts ([M, K] int8, [M] float).
 *   packed     [N, row_bytes] in `layout`; gamma: 1 float (device).
 *   y          out: [M, N], y_dtype BL_F32 or BL_BF16 (round to nearest even).
 *   acc        optional out: [M, N] int32 accumulators, or NULL.
 * Dispatch on M: small batches (M <= 16) stream the packed weights once;
 * medium batches stream them once per 16-token chunk (all chunks in one
 * launch) while that is measured faster, i.e. for a few chunks and moderate
 * N; larger M runs the tiled INT8 matrix-core product. Results do not depend
 * on the path (the INT32 sums are exact). */
bl_status bitlinear_forward(const int8_t *xq, const float *scale,
                            const uint8_t *packed, int layout, const float *gamma,
                            int64_t M, int64_t N, int64_t K,
                            void *y, int y_dtype, int32_t *acc, void *stream);

/* Fused decode step: per-token INT8 quantisation of x (exactly as
 * bitlinear_quant_acts) and the product with its epilogue (exactly as
 * bitlinear_forward) in one launch, for the latency-bound decode regime.
 *   x       [M, K] x_dtype (BL_F32 or BL_BF16), read only.
 *   packed  [N, row_bytes] in `layout`; gamma: 1 float (device).
 *   y       out: [M, N] y_dtype; acc: optional out [M, N] int32, or NULL.
 * Only 1 <= M <= 4 is supported: every workgroup re-derives the token scales
 * from x, which pays off only for a handful of tokens. Larger M returns
 * BL_ERR_UNSUPPORTED (use bitlinear_quant_acts + bitlinear_forward).
 * Sources as for bitlinear_quant_acts and bitlinear_forward. */
bl_status bitlinear_linear(const void *x, int x_dtype, const uint8_t *packed, int layout,
                           const float *gamma, int64_t M, int64_t N, int64_t K,
                           void *y, int y_dtype, int32_t *acc, void *stream);

/* Stacked matrices: several weight matrices that share an input (the Q, K and
 * V projections of an attention block) stored as consecutive row segments of
 * one packed matrix, each segment quantised on its own with its own gamma, so
 * one launch serves all of them (launch latency dominates the decode regime).
 * Per segment the result is exactly that of bitlinear_forward /
 * bitlinear_linear on the segment alone; y holds the segments' outputs side by
 * side along its columns.
 *   packed    [N, row_bytes] with N = sum(seg_rows): segment s occupies the
 *             seg_rows[s] rows after segments 0..s-1 (pack each segment with
 *             bitlinear_pack_weights into its row range, and its gamma into
 *             gammas + s).
 *   gammas    device array of nseg floats.
 *   seg_rows  HOST array of nseg row counts, each >= 1; 1 <= nseg <= 8.
 *   y, acc    [M, N].
 * Other arguments, limits and errors as for bitlinear_forward /
 * bitlinear_linear; a bad segment table returns BL_ERR_INVALID_ARG. */
bl_status bitlinear_forward_segmented(const int8_t *xq, const float *scale, const uint8_t *packed,
                                      int layout, const float *gammas, const int64_t *seg_rows,
                                      int nseg, int64_t M, int64_t K, void *y, int y_dtype,
                                      int32_t *acc, void *stream);
bl_status bitlinear_linear_segmented(const void *x, int x_dtype, const uint8_t *packed, int layout,
                                     const float *gammas, const int64_t *seg_rows, int nseg,
                                     int64_t M, int64_t K, void *y, int y_dtype, int32_t *acc,
                                     void *stream);

/* Alternative decode scheme for the base-3 layout, one token: instead of
 * expanding each weight byte into five codes, the workgroup tabulates, for
 * every group of five activations, the partial sums of the first two and the
 * last three trits (9 + 27 entries) and reads two entries per weight byte
 * ([b158] §2.3 and §6.3: five weights per byte are unpacked by table lookup
 * or bit operations). Same arguments and result as bitlinear_forward (acc
 * bit-identical); kept to compare the lookup scheme with the in-register
 * decode. Only layout BL_PACK_BASE3 and M = 1 are supported (else
 * BL_ERR_UNSUPPORTED); M = 0 or N = 0 is a no-op. */
bl_status bitlinear_forward_lut(const int8_t *xq, const float *scale, const uint8_t *packed,
                                int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                                void *y, int y_dtype, int32_t *acc, void *stream);

/* Backward products of the straight-through estimator, for training with the
 * codes the forward pass used ([QAT-en] "How Gradients Flow: Fake Quantization
 * and STE": the backward pass treats rounding as the identity, so gradients
 * reach the latent weights; [b158] §5.3, the BitLinear layer with the
 * straight-through estimator). With y = x W_q^T and W_q = gamma * c:
 *   grad_x = grad_y W_q   and   grad_W = grad_y^T x.
 * Both run on the bf16 matrix cores with fp32 accumulation (fp32 operands
 * as exact bf16 pieces, below).
 *
 * bitlinear_backward_input: grad_x[m,k] = gamma * sum_n grad_y[m,n] * c[n,k].
 *   grad_y  [M, N], gy_dtype BL_BF16 or BL_F32. fp32 values are split exactly
 *           into three bf16 pieces (hi + mid + lo, 8 significant bits each) and
 *           the contraction runs over all three into one fp32 sum, so each
 *           product term is still exact (for |grad_y| >= 2^-110; smaller
 *           values may lose bits below 2^-133). Three times the matrix-core
 *           work of bf16 grad_y.
 *   packed  [N, row_bytes] codes in `layout` (BL_PACK_2BIT, BL_PACK_BASE3 or
 *           BL_PACK_1BIT: the forward's own matrix; no transposed copy is
 *           needed); gamma: 1 float (device).
 *   grad_x  out: [M, K] fp32.
 * Requires N % 8 == 0 (else BL_ERR_UNSUPPORTED).
 * Dimensions above 2^24 return BL_ERR_INVALID_ARG.
 * M = 0 is a no-op; N = 0 writes zeros. */
bl_status bitlinear_backward_input(const void *grad_y, int gy_dtype, const uint8_t *packed,
                                   int layout, const float *gamma, int64_t M, int64_t N,
                                   int64_t K, float *grad_x, void *stream);

/* bitlinear_backward_weight: grad_w[n,k] = sum_m grad_y[m,n] * x[m,k].
 *   grad_y  [M, N]; x [M, K] (the layer input); both of `dtype`: BL_BF16
 *           (products exact in fp32, fp32 sums), or BL_F32: each value is
 *           split exactly into three bf16 pieces, and the six piece products
 *           other than mid.lo, lo.mid and lo.lo are summed in fp32 (6M
 *           terms), so each product is exact to within 2^-20 of its
 *           magnitude (for values >= 2^-110; see backward_input). Six times
 *           the matrix-core work of bf16.
 *   grad_w  out: [N, K] fp32.
 * Requires N % 8 == 0 and K % 8 == 0 (else BL_ERR_UNSUPPORTED). N = 0 is a
 * no-op; M = 0 writes zeros. */
bl_status bitlinear_backward_weight(const void *grad_y, const void *x, int dtype, int64_t M,
                                    int64_t N, int64_t K, float *grad_w, void *stream);

/* Dry run of the product dispatch: describes, without launching anything or
 * touching device memory, the kernel launches bitlinear_forward (fused = 0)
 * or bitlinear_linear with bf16 x (fused = 1) would enqueue for an M x N x K
 * product in `layout` with output type y_dtype. The stacked (segmented)
 * variants dispatch exactly as the plain calls with N = sum of the segments.
 * One line per launch: the kernel instantiation as the profiler names it,
 * then "grid=GXxGY block=THREADS lds=BYTES". Writes at most len - 1
 * characters and a terminating NUL into buf (buf may be NULL when len is 0).
 * Returns the number of launches (0 for M = 0 or N = 0), or -1 for arguments
 * the call itself would refuse. Launch shapes that depend on the device's
 * compute-unit count use the current device's, and assume none without a GPU.
 * For tests and profiling: it lets a caller check which kernel configuration
 * serves a shape. Host-only; safe to call from several threads. */
int bitlinear_forward_plan(int64_t M, int64_t N, int64_t K, int layout, int y_dtype, int fused,
                           char *buf, size_t len);

/* Human-readable name of a status code (static string). */
const char *bitlinear_status_string(int status);

/* Library version, (major << 16) | minor. */
int bitlinear_version(void);

/* Digest of the source files the library was built from (32 hex digits; a
 * static string), so that a binding can refuse a library built from other
 * sources than the ones beside it. "unknown" if the build did not set it. */
const char *bitlinear_source_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
