// Decode-side product for small batches (1 <= M <= 16 tokens): the packed
// weights are streamed from HBM exactly once with 16-byte loads, expanded in
// registers to signed code bytes, and multiplied on the INT8 matrix cores
// (v_mfma_i32_16x16x64_i8) with the batch in the 16-column operand. A
// weight of +1 adds the activation, -1 subtracts it and 0 contributes
// nothing ([b158] "BitNet b1.58深度解析" §4.2); the sums are exact INT32
// ([b158] §3.3), then scaled by gamma * scale[m] / 127 ([b158] §5.2-5.3).
//
// Work split: a block owns 16 consecutive weight rows; its KS waves split the
// row length K and their 16x16 partial tiles are added through LDS. In one
// "super-step" the four 16-lane groups of a wave each take one 16-byte unit
// of packed codes per row (64 codes in the 2-bit layout, 80 in base-3); the
// matrix-core k slots of lane group g are mapped to that unit's codes, and
// the activation operand is loaded with the same mapping, so the sum over
// the 64 k slots of one instruction is a sum over real codes only.
#include "bl_internal.hpp"
#include "device_util.hpp"

namespace bl {
namespace {

// Load 16 activation bytes xq[t, k .. k+15], zero past K.
__device__ __forceinline__ v4i load_act16(const int8_t *__restrict__ row, int64_t K,
                                          int64_t k, bool aligned) {
    v4i r = {0, 0, 0, 0};
    if (k + 16 <= K && aligned) {
        r = *reinterpret_cast<const v4i *>(row + k);
    } else if (k < K) {
        uint32_t d[4] = {0u, 0u, 0u, 0u};
        for (int e = 0; e < 16; ++e)
            if (k + e < K) d[e / 4] |= (uint32_t)(uint8_t)row[k + e] << (8 * (e % 4));
        r = v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
    }
    return r;
}

template <int LAYOUT, int KS, typename YT>
__global__ __launch_bounds__(64 * KS) void skinny_kernel(
    const int8_t *__restrict__ xq, const float *__restrict__ scale,
    const uint8_t *__restrict__ packed, const float *__restrict__ gamma_p, int M, int64_t N,
    int64_t K, int64_t rb, YT *__restrict__ y, int32_t *__restrict__ acc_out) {
    constexpr int kUnitCodes = LAYOUT == kLayout2Bit ? 64 : 80;
    constexpr int kSteps = kUnitCodes / 16;  // MFMA instructions per unit
    __shared__ uint64_t lut[LAYOUT == kLayoutBase3 ? 4 * 256 : 1];
    __shared__ v4i part[KS][64];

    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    const int r = lane % 16;  // weight row within the block / token index
    const int g = lane / 16;  // lane group = unit within the super-step
    const int64_t n0 = (int64_t)blockIdx.x * 16;

    if (LAYOUT == kLayoutBase3) {
        // four copies of the decode table, shifted by 0..3 bytes
        for (int i = threadIdx.x; i < 4 * 256; i += 64 * KS) {
            const int a = i / 256, v = i % 256;
            lut[i] = base3_entry((uint32_t)v) << (8 * a);
        }
        __syncthreads();
    }

    const int64_t units = rb / 16;
    const int64_t supers = (units + 3) / 4;
    const bool row_ok = n0 + r < N;
    const uint8_t *wrow = packed + (n0 + r) * rb;
    const bool tok_ok = r < M;
    const int8_t *xrow = xq + (int64_t)r * K;
    const bool aligned = (K % 16) == 0;

    v4i acc = {0, 0, 0, 0};
    for (int64_t ss = wave; ss < supers; ss += KS) {
        const int64_t unit = ss * 4 + g;
        const bool unit_ok = unit < units;
        uint4 wv = make_uint4(0u, 0u, 0u, 0u);
        if (unit_ok && row_ok) wv = *reinterpret_cast<const uint4 *>(wrow + unit * 16);
        int c[kSteps * 4];
        if (LAYOUT == kLayout2Bit) {
            expand_2bit_word(wv.x, c + 0);
            expand_2bit_word(wv.y, c + 4);
            expand_2bit_word(wv.z, c + 8);
            expand_2bit_word(wv.w, c + 12);
        } else {
            uint32_t d[20];
#pragma unroll
            for (int i = 0; i < 20; ++i) d[i] = 0u;
            const uint32_t bytes[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const uint32_t v = (bytes[j / 4] >> (8 * (j % 4))) & 0xFFu;
                const uint64_t e = lut[(j % 4) * 256 + v];
                const int dw = (5 * j) / 4;
                d[dw] |= (uint32_t)e;
                d[dw + 1] |= (uint32_t)(e >> 32);
            }
#pragma unroll
            for (int i = 0; i < 20; ++i) c[i] = (int)d[i];
        }
        const int64_t kbase = unit * kUnitCodes;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            v4i b = {0, 0, 0, 0};
            if (tok_ok && unit_ok) b = load_act16(xrow, K, kbase + 16 * s, aligned);
            const v4i a = {c[4 * s], c[4 * s + 1], c[4 * s + 2], c[4 * s + 3]};
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
        }
    }

    part[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    v4i tot = part[0][lane];
#pragma unroll
    for (int w = 1; w < KS; ++w) tot += part[w][lane];

    // lane holds D[4g + i][r]: weight rows n0 + 4g + i, token r
    const int t = r;
    if (t >= M) return;
    const float gs = gamma_p[0] * scale[t];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t n = n0 + 4 * g + i;
        if (n >= N) continue;
        const int32_t a = tot[i];
        const float v = ((float)a * gs) / 127.0f;
        if constexpr (sizeof(YT) == 4)
            y[(int64_t)t * N + n] = v;
        else
            y[(int64_t)t * N + n] = (YT)f32_to_bf16_rne(v);
        if (acc_out) acc_out[(int64_t)t * N + n] = a;
    }
}

template <int LAYOUT, typename YT>
hipError_t launch_skinny_t(const int8_t *xq, const float *scale, const uint8_t *packed,
                           const float *gamma, int64_t M, int64_t N, int64_t K, YT *y,
                           int32_t *acc, hipStream_t s) {
    const int64_t rb = LAYOUT == kLayout2Bit ? row_bytes_2bit(K) : row_bytes_base3(K);
    constexpr int KS = 4;
    dim3 grid((unsigned)((N + 15) / 16)), block(64 * KS);
    hipLaunchKernelGGL((skinny_kernel<LAYOUT, KS, YT>), grid, block, 0, s, xq, scale, packed,
                       gamma, (int)M, N, K, rb, y, acc);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_skinny(const int8_t *xq, const float *scale, const uint8_t *packed,
                                 int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                                 void *y, int y_dtype, int32_t *acc, hipStream_t stream) {
    if (layout == kLayout2Bit) {
        if (y_dtype == kF32)
            return launch_skinny_t<kLayout2Bit>(xq, scale, packed, gamma, M, N, K,
                                                static_cast<float *>(y), acc, stream);
        return launch_skinny_t<kLayout2Bit>(xq, scale, packed, gamma, M, N, K,
                                            static_cast<uint16_t *>(y), acc, stream);
    }
    if (y_dtype == kF32)
        return launch_skinny_t<kLayoutBase3>(xq, scale, packed, gamma, M, N, K,
                                             static_cast<float *>(y), acc, stream);
    return launch_skinny_t<kLayoutBase3>(xq, scale, packed, gamma, M, N, K,
                                         static_cast<uint16_t *>(y), acc, stream);
}

}  // namespace bl
