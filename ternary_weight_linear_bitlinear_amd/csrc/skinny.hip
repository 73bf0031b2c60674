// Decode-side product for small batches (1 <= M <= 16 tokens): the packed
// weights are streamed from HBM exactly once with 16-byte loads, expanded in
// registers to signed code bytes, and multiplied on the INT8 matrix cores
// (v_mfma_i32_16x16x64_i8) with the batch in the 16-column operand. A
// weight of +1 adds the activation, -1 subtracts it and 0 contributes
// nothing ([b158] "BitNet b1.58深度解析" §4.2); the sums are exact INT32
// ([b158] §3.3), then scaled by gamma * scale[m] / 127 ([b158] §5.2-5.3).
//
// Work split: a block owns 16 consecutive weight rows; its KS waves split the
// row length K. One "super-step" of a wave covers four 16-byte units of
// packed codes per row (64 codes per unit in the 2-bit layout, 80 in base-3),
// one unit per 16-lane group; the matrix-core k slots of lane group g are
// mapped to that unit's codes and the activation operand is read with the
// same mapping, so every instruction sums over real codes only. A wave
// issues the loads of all NSS super-steps of a round before consuming any,
// so each lane keeps NSS 16-byte weight loads in flight, while the block
// stages the round's slice of the activations in LDS. The KS partial 16x16
// tiles are added through LDS.
#include "bl_internal.hpp"
#include "device_util.hpp"

namespace bl {
namespace {

template <int LAYOUT>
struct SkinnyCfg {
    static constexpr int kUnitCodes = LAYOUT == kLayout2Bit ? 64 : 80;
    static constexpr int kSteps = kUnitCodes / 16;  // MFMA instructions per unit
};

// Decode one 16-byte unit into signed code bytes (natural k order).
template <int LAYOUT>
__device__ __forceinline__ void decode_unit(const uint4 wv, const uint64_t *lut, int c[20]) {
    if (LAYOUT == kLayout2Bit) {
        expand_2bit_word(wv.x, c + 0);
        expand_2bit_word(wv.y, c + 4);
        expand_2bit_word(wv.z, c + 8);
        expand_2bit_word(wv.w, c + 12);
    } else {
        uint32_t d[20];
#pragma unroll
        for (int i = 0; i < 20; ++i) d[i] = 0u;
        const uint32_t w[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t v = (w[j / 4] >> (8 * (j % 4))) & 0xFFu;
            const uint64_t e = lut[(j % 4) * 256 + v];
            const int dw = (5 * j) / 4;
            d[dw] |= (uint32_t)e;
            d[dw + 1] |= (uint32_t)(e >> 32);
        }
#pragma unroll
        for (int i = 0; i < 20; ++i) c[i] = (int)d[i];
    }
}

template <int LAYOUT, int KS, int NSS, typename YT>
__global__ __launch_bounds__(64 * KS) void skinny_kernel(
    const int8_t *__restrict__ xq, const float *__restrict__ scale,
    const uint8_t *__restrict__ packed, const float *__restrict__ gamma_p, int M, int64_t N,
    int64_t K, int64_t rb, YT *__restrict__ y, int32_t *__restrict__ acc_out) {
    using C = SkinnyCfg<LAYOUT>;
    constexpr int kRoundUnits = KS * NSS * 4;                 // units per round
    constexpr int kRoundK = kRoundUnits * C::kUnitCodes;       // codes per round
    constexpr int kActStride = kRoundK + 16;                   // LDS row stride (bytes)
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint64_t *lut = reinterpret_cast<uint64_t *>(smem);                 // base-3 only
    int8_t *act = reinterpret_cast<int8_t *>(smem + (LAYOUT == kLayoutBase3 ? 8192 : 0));
    v4i *part = reinterpret_cast<v4i *>(smem + (LAYOUT == kLayoutBase3 ? 8192 : 0));

    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    const int r = lane % 16;  // weight row within the block (A) / token (B)
    const int g = lane / 16;  // lane group = unit within the super-step
    const int64_t n0 = (int64_t)blockIdx.x * 16;

    if (LAYOUT == kLayoutBase3) {
        for (int i = threadIdx.x; i < 4 * 256; i += 64 * KS)
            lut[i] = base3_entry((uint32_t)(i % 256)) << (8 * (i / 256));
    }

    const int64_t units = rb / 16;
    const bool row_ok = n0 + r < N;
    const uint8_t *wrow = packed + (n0 + r) * rb;
    const bool aligned = (K % 16) == 0;

    v4i acc = {0, 0, 0, 0};
    for (int64_t u0 = 0; u0 < units; u0 += kRoundUnits) {
        // 1. issue every weight load of this round
        uint4 wv[NSS];
#pragma unroll
        for (int s = 0; s < NSS; ++s) {
            const int64_t unit = u0 + (int64_t)(s * KS + wave) * 4 + g;
            const bool ok = row_ok && unit < units;
            // out-of-range lanes read a valid address and are zeroed (no branch)
            const uint4 v = *reinterpret_cast<const uint4 *>(ok ? wrow + unit * 16 : packed);
            wv[s] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
        }
        // 2. stage activations xq[0:M, k0 : k0 + kRoundK] in LDS (zero past K)
        const int64_t k0 = u0 * C::kUnitCodes;
        __syncthreads();  // previous round's readers are done
        const int chunks = M * (kRoundK / 16);
        for (int q = threadIdx.x; q < chunks; q += 64 * KS) {
            const int t = q / (kRoundK / 16), cc = q % (kRoundK / 16);
            const int64_t k = k0 + cc * 16;
            const int8_t *src = xq + (int64_t)t * K;
            v4i v = {0, 0, 0, 0};
            if (aligned) {
                const bool ok = k < K;  // K % 16 == 0: a chunk is all in or all out
                const v4i a = *reinterpret_cast<const v4i *>(ok ? src + k : xq);
                v = ok ? a : v4i{0, 0, 0, 0};
            } else if (k < K) {
                uint32_t d[4] = {0u, 0u, 0u, 0u};
                for (int e = 0; e < 16; ++e)
                    if (k + e < K) d[e / 4] |= (uint32_t)(uint8_t)src[k + e] << (8 * (e % 4));
                v = v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
            }
            *reinterpret_cast<v4i *>(act + t * kActStride + cc * 16) = v;
        }
        __syncthreads();
        // 3. expand and multiply
#pragma unroll
        for (int s = 0; s < NSS; ++s) {
            int c[20];
            decode_unit<LAYOUT>(wv[s], lut, c);
            const int ul = (s * KS + wave) * 4 + g;  // unit within the round
#pragma unroll
            for (int st = 0; st < C::kSteps; ++st) {
                v4i b = {0, 0, 0, 0};
                if (r < M)
                    b = *reinterpret_cast<const v4i *>(act + r * kActStride +
                                                       ul * C::kUnitCodes + 16 * st);
                const v4i a = {c[4 * st], c[4 * st + 1], c[4 * st + 2], c[4 * st + 3]};
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
            }
        }
    }

    __syncthreads();
    part[wave * 64 + lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    v4i tot = part[lane];
#pragma unroll
    for (int w = 1; w < KS; ++w) tot += part[w * 64 + lane];

    // lane holds D[4g + i][r]: weight rows n0 + 4g + i, token r
    const int t = r;
    if (t >= M) return;
    const float f = gamma_p[0] * scale[t] / 127.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t n = n0 + 4 * g + i;
        if (n >= N) continue;
        const int32_t a = tot[i];
        const float v = (float)a * f;
        if constexpr (sizeof(YT) == 4)
            y[(int64_t)t * N + n] = v;
        else
            y[(int64_t)t * N + n] = (YT)f32_to_bf16_rne(v);
        if (acc_out) acc_out[(int64_t)t * N + n] = a;
    }
}

template <int LAYOUT, int KS, int NSS, typename YT>
hipError_t launch_skinny_t(const int8_t *xq, const float *scale, const uint8_t *packed,
                           const float *gamma, int64_t M, int64_t N, int64_t K, YT *y,
                           int32_t *acc, hipStream_t s) {
    const int64_t rb = LAYOUT == kLayout2Bit ? row_bytes_2bit(K) : row_bytes_base3(K);
    // the partial-tile buffer aliases the activation area (needs KS*1 KiB)
    const size_t act = (size_t)M * (KS * NSS * 4 * SkinnyCfg<LAYOUT>::kUnitCodes + 16);
    const size_t smem = (LAYOUT == kLayoutBase3 ? 8192 : 0) +
                        (act > (size_t)KS * 1024 ? act : (size_t)KS * 1024);
    dim3 grid((unsigned)((N + 15) / 16)), block(64 * KS);
    auto kern = skinny_kernel<LAYOUT, KS, NSS, YT>;
    static int lds_raised = 0;  // one flag per instantiation of this launcher
    hipError_t e = allow_dynamic_lds(kern, smem, &lds_raised);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, block, smem, s, xq, scale, packed, gamma, (int)M, N, K, rb, y,
                       acc);
    return hipGetLastError();
}

template <int LAYOUT, typename YT>
hipError_t launch_skinny_l(const int8_t *xq, const float *scale, const uint8_t *packed,
                           const float *gamma, int64_t M, int64_t N, int64_t K, YT *y,
                           int32_t *acc, hipStream_t s) {
    // one round of 4 waves x 4 super-steps covers 4096 codes (2-bit) / 5120
    // (base-3): 64 (80) KiB of activations at M = 16
    return launch_skinny_t<LAYOUT, 4, 4, YT>(xq, scale, packed, gamma, M, N, K, y, acc, s);
}

// ---------------------------------------------------------------------------
// Fused decode (1 <= M <= 4 tokens): per-token absmax INT8 quantisation of x
// inside every block, then the same weight-streaming product. Each block
// issues its weight loads first, derives the token scales s_m = max(max|x|,
// 1e-6) from a full pass over x (from L2), quantises the round's slice of x
// straight into LDS with quant1() (the same fp32 steps as the stand-alone
// quantiser, so codes are identical), and multiplies. One launch instead of
// two on the latency-bound decode path.
constexpr int kFusedMaxM = 4;

template <int LAYOUT, int KS, int NSS, int MAXM, typename XT, typename YT>
__global__ __launch_bounds__(64 * KS) void linear_decode_kernel(
    const XT *__restrict__ x, const uint8_t *__restrict__ packed,
    const float *__restrict__ gamma_p, int M, int64_t N, int64_t K, int64_t rb,
    YT *__restrict__ y, int32_t *__restrict__ acc_out) {
    using C = SkinnyCfg<LAYOUT>;
    constexpr int kThreads = 64 * KS;
    constexpr int kRoundUnits = KS * NSS * 4;
    constexpr int kRoundK = kRoundUnits * C::kUnitCodes;
    constexpr int kActStride = kRoundK + 16;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint64_t *lut = reinterpret_cast<uint64_t *>(smem);
    int8_t *act = reinterpret_cast<int8_t *>(smem + (LAYOUT == kLayoutBase3 ? 8192 : 0));
    v4i *part = reinterpret_cast<v4i *>(act);
    __shared__ float red[kFusedMaxM][KS];
    __shared__ float tok_scale[kFusedMaxM];

    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    const int r = lane % 16;
    const int g = lane / 16;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t units = rb / 16;
    const bool row_ok = n0 + r < N;
    const uint8_t *wrow = packed + (n0 + r) * rb;
    const bool vec = (K % 8) == 0;

    uint4 wv[NSS];
    auto issue = [&](int64_t u0) {
#pragma unroll
        for (int s = 0; s < NSS; ++s) {
            const int64_t unit = u0 + (int64_t)(s * KS + wave) * 4 + g;
            const bool ok = row_ok && unit < units;
            // out-of-range lanes read a valid address and are zeroed
            const uint8_t *src = ok ? wrow + unit * 16 : packed;
            const uint4 v = *reinterpret_cast<const uint4 *>(src);
            wv[s] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    issue(0);

    if (LAYOUT == kLayoutBase3) {
        for (int i = threadIdx.x; i < 4 * 256; i += kThreads)
            lut[i] = base3_entry((uint32_t)(i % 256)) << (8 * (i / 256));
    }

    // token scales: s_m = max(max_k |x[m, k]|, 1e-6), a block-wide max per
    // token. When the row fits one round, each thread loads its 16-element
    // chunks of x once and keeps them for the quantisation below.
    constexpr int kChunksPerTok = kRoundK / 16;
    constexpr int kMaxQ = (MAXM * kChunksPerTok + kThreads - 1) / kThreads;
    const bool one_round = units <= kRoundUnits;
    float xv[kMaxQ][16];
    float amax[kFusedMaxM] = {0.f, 0.f, 0.f, 0.f};
    auto load_chunk = [&](int t, int64_t k, float *v) {
        const XT *row = x + (int64_t)t * K;
        if (vec && k + 16 <= K) {
            load8(row + k, v);
            load8(row + k + 8, v + 8);
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = k + e < K ? Elem<XT>::get(row, k + e) : 0.f;
        }
    };
    if (one_round) {
#pragma unroll
        for (int i = 0; i < kMaxQ; ++i) {
            const int q = threadIdx.x + i * kThreads;
            const int t = q / kChunksPerTok;
            if (t < M) {
                load_chunk(t, (int64_t)(q % kChunksPerTok) * 16, xv[i]);
                float m = 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(xv[i][e]));
#pragma unroll
                for (int tt = 0; tt < kFusedMaxM; ++tt)
                    amax[tt] = tt == t ? fmaxf(amax[tt], m) : amax[tt];
            }
        }
    } else {
        for (int t = 0; t < M; ++t) {
            const XT *row = x + (int64_t)t * K;
            float am = 0.f;
            if (vec) {
                for (int64_t k = (int64_t)threadIdx.x * 8; k < K; k += (int64_t)kThreads * 8) {
                    float v[8];
                    load8(row + k, v);
#pragma unroll
                    for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(v[e]));
                }
            } else {
                for (int64_t k = threadIdx.x; k < K; k += kThreads)
                    am = fmaxf(am, fabsf(Elem<XT>::get(row, k)));
            }
#pragma unroll
            for (int tt = 0; tt < kFusedMaxM; ++tt) amax[tt] = tt == t ? am : amax[tt];
        }
    }
#pragma unroll
    for (int t = 0; t < kFusedMaxM; ++t) {
        if (t >= M) break;
        const float m = wave_max(amax[t]);
        if (lane == 0) red[t][wave] = m;
    }
    __syncthreads();
    if (threadIdx.x < M) {
        float m = red[threadIdx.x][0];
#pragma unroll
        for (int w = 1; w < KS; ++w) m = fmaxf(m, red[threadIdx.x][w]);
        tok_scale[threadIdx.x] = fmaxf(m, 1e-6f);
    }
    __syncthreads();

    auto store_codes = [&](int t, int cc, const float *v) {
        const float sc = tok_scale[t];
        uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 16; ++e)
            d[e / 4] |= (uint32_t)(uint8_t)quant1(v[e], sc) << (8 * (e % 4));
        *reinterpret_cast<v4i *>(act + t * kActStride + cc * 16) =
            v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
    };

    v4i acc = {0, 0, 0, 0};
    for (int64_t u0 = 0; u0 < units; u0 += kRoundUnits) {
        if (u0 > 0) {
            issue(u0);
            __syncthreads();  // previous round's readers are done
        }
        // quantise x[0:M, k0 : k0 + kRoundK] into LDS (zero past K)
        const int64_t k0 = u0 * C::kUnitCodes;
        if (one_round) {
#pragma unroll
            for (int i = 0; i < kMaxQ; ++i) {
                const int q = threadIdx.x + i * kThreads;
                if (q < M * kChunksPerTok) store_codes(q / kChunksPerTok, q % kChunksPerTok, xv[i]);
            }
        } else {
            for (int q = threadIdx.x; q < M * kChunksPerTok; q += kThreads) {
                const int t = q / kChunksPerTok, cc = q % kChunksPerTok;
                float v[16];
                load_chunk(t, k0 + cc * 16, v);
                store_codes(t, cc, v);
            }
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < NSS; ++s) {
            int c[20];
            decode_unit<LAYOUT>(wv[s], lut, c);
            const int ul = (s * KS + wave) * 4 + g;
#pragma unroll
            for (int st = 0; st < C::kSteps; ++st) {
                v4i b = {0, 0, 0, 0};
                if (r < M)
                    b = *reinterpret_cast<const v4i *>(act + r * kActStride +
                                                       ul * C::kUnitCodes + 16 * st);
                const v4i a = {c[4 * st], c[4 * st + 1], c[4 * st + 2], c[4 * st + 3]};
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
            }
        }
    }

    __syncthreads();
    part[wave * 64 + lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    v4i tot = part[lane];
#pragma unroll
    for (int w = 1; w < KS; ++w) tot += part[w * 64 + lane];
    const int t = r;
    if (t >= M) return;
    const float f = gamma_p[0] * tok_scale[t] / 127.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t n = n0 + 4 * g + i;
        if (n >= N) continue;
        const int32_t a = tot[i];
        const float v = (float)a * f;
        if constexpr (sizeof(YT) == 4)
            y[(int64_t)t * N + n] = v;
        else
            y[(int64_t)t * N + n] = (YT)f32_to_bf16_rne(v);
        if (acc_out) acc_out[(int64_t)t * N + n] = a;
    }
}

template <int LAYOUT, int MAXM, typename XT, typename YT>
hipError_t launch_linear_m(const XT *x, const uint8_t *packed, const float *gamma, int64_t M,
                           int64_t N, int64_t K, YT *y, int32_t *acc, hipStream_t s) {
    constexpr int KS = 4, NSS = 4;
    const int64_t rb = LAYOUT == kLayout2Bit ? row_bytes_2bit(K) : row_bytes_base3(K);
    const size_t act = (size_t)MAXM * (KS * NSS * 4 * SkinnyCfg<LAYOUT>::kUnitCodes + 16);
    const size_t smem = (LAYOUT == kLayoutBase3 ? 8192 : 0) +
                        (act > (size_t)KS * 1024 ? act : (size_t)KS * 1024);
    auto kern = linear_decode_kernel<LAYOUT, KS, NSS, MAXM, XT, YT>;
    static int lds_raised = 0;
    hipError_t e = allow_dynamic_lds(kern, smem, &lds_raised);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)((N + 15) / 16)), dim3(64 * KS), smem, s, x, packed,
                       gamma, (int)M, N, K, rb, y, acc);
    return hipGetLastError();
}

// A one-token specialisation keeps only 16 values of x per thread, which
// leaves registers for more resident workgroups per CU.
template <int LAYOUT, typename XT, typename YT>
hipError_t launch_linear_t(const XT *x, const uint8_t *packed, const float *gamma, int64_t M,
                           int64_t N, int64_t K, YT *y, int32_t *acc, hipStream_t s) {
    if (M == 1) return launch_linear_m<LAYOUT, 1>(x, packed, gamma, M, N, K, y, acc, s);
    return launch_linear_m<LAYOUT, kFusedMaxM>(x, packed, gamma, M, N, K, y, acc, s);
}

template <int LAYOUT, typename XT>
hipError_t launch_linear_x(const XT *x, const uint8_t *packed, const float *gamma, int64_t M,
                           int64_t N, int64_t K, void *y, int y_dtype, int32_t *acc,
                           hipStream_t s) {
    if (y_dtype == kF32)
        return launch_linear_t<LAYOUT>(x, packed, gamma, M, N, K, static_cast<float *>(y), acc, s);
    return launch_linear_t<LAYOUT>(x, packed, gamma, M, N, K, static_cast<uint16_t *>(y), acc, s);
}

}  // namespace

hipError_t launch_forward_skinny(const int8_t *xq, const float *scale, const uint8_t *packed,
                                 int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                                 void *y, int y_dtype, int32_t *acc, hipStream_t stream) {
    if (layout == kLayout2Bit) {
        if (y_dtype == kF32)
            return launch_skinny_l<kLayout2Bit>(xq, scale, packed, gamma, M, N, K,
                                                static_cast<float *>(y), acc, stream);
        return launch_skinny_l<kLayout2Bit>(xq, scale, packed, gamma, M, N, K,
                                            static_cast<uint16_t *>(y), acc, stream);
    }
    if (y_dtype == kF32)
        return launch_skinny_l<kLayoutBase3>(xq, scale, packed, gamma, M, N, K,
                                             static_cast<float *>(y), acc, stream);
    return launch_skinny_l<kLayoutBase3>(xq, scale, packed, gamma, M, N, K,
                                         static_cast<uint16_t *>(y), acc, stream);
}

}  // namespace bl

namespace bl {

int64_t fused_decode_max_m() { return kFusedMaxM; }

hipError_t launch_linear_decode(const void *x, int x_dtype, const uint8_t *packed, int layout,
                                const float *gamma, int64_t M, int64_t N, int64_t K, void *y,
                                int y_dtype, int32_t *acc, hipStream_t stream) {
    if (layout == kLayout2Bit) {
        if (x_dtype == kF32)
            return launch_linear_x<kLayout2Bit>(static_cast<const float *>(x), packed, gamma, M,
                                                N, K, y, y_dtype, acc, stream);
        return launch_linear_x<kLayout2Bit>(static_cast<const uint16_t *>(x), packed, gamma, M, N,
                                            K, y, y_dtype, acc, stream);
    }
    if (x_dtype == kF32)
        return launch_linear_x<kLayoutBase3>(static_cast<const float *>(x), packed, gamma, M, N,
                                             K, y, y_dtype, acc, stream);
    return launch_linear_x<kLayoutBase3>(static_cast<const uint16_t *>(x), packed, gamma, M, N, K,
                                         y, y_dtype, acc, stream);
}

}  // namespace bl
