// Prefill-side product (M > 16 tokens): a tiled INT8 matrix-core GEMM.
// Activations (int8) and weight codes are staged through LDS per k-tile; the
// packed weights are expanded to signed code bytes once per block and k-tile
// on their way into LDS, then consumed by v_mfma_i32_32x32x32_i8. Every
// product term is an INT8 activation times a code in {-1, 0, +1}, summed
// exactly in INT32 ([b158] "BitNet b1.58深度解析" §3.3 and §4.2), then
// scaled by gamma * scale[m] / 127 in the epilogue ([b158] §5.2-5.3).
//
// Tile: BM = 128 tokens x BN = 128 weight rows per block, four waves in a
// 2 x 2 arrangement, each wave owning a 64 x 64 sub-tile (2 x 2 fragments of
// 32 x 32). A k-tile is two 16-byte units of packed codes per weight row:
// 128 codes in the 2-bit layout, 160 in base-3, i.e. 4 or 5 MFMA k-steps.
#include "bl_internal.hpp"
#include "device_util.hpp"

namespace bl {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int kThreads = 256;

template <int LAYOUT>
struct GemmCfg {
    static constexpr int kUnitCodes = LAYOUT == kLayout2Bit ? 64 : 80;
    static constexpr int BK = 2 * kUnitCodes;  // codes per k-tile
    static constexpr int LDSK = BK + 16;       // padded LDS row (bank spread)
    static constexpr int KSTEPS = BK / 32;
    static constexpr int ACHUNKS = BM * BK / 16 / kThreads;  // 16B A chunks per thread
};

template <int LAYOUT, typename YT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const int8_t *__restrict__ xq, const float *__restrict__ scale,
    const uint8_t *__restrict__ packed, const float *__restrict__ gamma_p, int64_t M,
    int64_t N, int64_t K, int64_t rb, YT *__restrict__ y, int32_t *__restrict__ acc_out) {
    using C = GemmCfg<LAYOUT>;
    __shared__ __attribute__((aligned(16))) int8_t As[BM * C::LDSK];
    __shared__ __attribute__((aligned(16))) int8_t Bs[BN * C::LDSK];
    __shared__ uint64_t lut[LAYOUT == kLayoutBase3 ? 4 * 256 : 1];

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    const int wm = wave / 2, wn = wave % 2;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;

    if (LAYOUT == kLayoutBase3) {
        for (int i = tid; i < 4 * 256; i += kThreads)
            lut[i] = base3_entry((uint32_t)(i % 256)) << (8 * (i / 256));
        __syncthreads();
    }

    const int64_t units = rb / 16;
    const int64_t ktiles = (units + 1) / 2;
    const bool a_aligned = (K % 16) == 0;

    // B: thread -> (weight row, unit) = one 16-byte packed load per k-tile
    const int b_row = tid / 2, b_unit = tid % 2;
    const bool b_row_ok = n0 + b_row < N;

    v4i a_reg[C::ACHUNKS];
    uint4 b_reg;

    auto load_tile = [&](int64_t kt) {
        const int64_t kc0 = kt * C::BK;
#pragma unroll
        for (int i = 0; i < C::ACHUNKS; ++i) {
            const int q = tid + i * kThreads;
            const int row = q / (C::BK / 16), col = q % (C::BK / 16);
            const int64_t m = m0 + row, k = kc0 + col * 16;
            v4i v = {0, 0, 0, 0};
            if (m < M) {
                const int8_t *p = xq + m * K;
                if (a_aligned && k + 16 <= K) {
                    v = *reinterpret_cast<const v4i *>(p + k);
                } else if (k < K) {
                    uint32_t d[4] = {0u, 0u, 0u, 0u};
                    for (int e = 0; e < 16; ++e)
                        if (k + e < K) d[e / 4] |= (uint32_t)(uint8_t)p[k + e] << (8 * (e % 4));
                    v = v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
                }
            }
            a_reg[i] = v;
        }
        const int64_t unit = kt * 2 + b_unit;
        b_reg = make_uint4(0u, 0u, 0u, 0u);
        if (b_row_ok && unit < units)
            b_reg = *reinterpret_cast<const uint4 *>(packed + (n0 + b_row) * rb + unit * 16);
    };

    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < C::ACHUNKS; ++i) {
            const int q = tid + i * kThreads;
            const int row = q / (C::BK / 16), col = q % (C::BK / 16);
            *reinterpret_cast<v4i *>(As + row * C::LDSK + col * 16) = a_reg[i];
        }
        int8_t *dst = Bs + b_row * C::LDSK + b_unit * C::kUnitCodes;
        if (LAYOUT == kLayout2Bit) {
            const uint32_t w[4] = {b_reg.x, b_reg.y, b_reg.z, b_reg.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                int c[4];
                expand_2bit_word(w[q], c);
                *reinterpret_cast<v4i *>(dst + 16 * q) = v4i{c[0], c[1], c[2], c[3]};
            }
        } else {
            uint32_t d[20];
#pragma unroll
            for (int i = 0; i < 20; ++i) d[i] = 0u;
            const uint32_t w[4] = {b_reg.x, b_reg.y, b_reg.z, b_reg.w};
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const uint32_t v = (w[j / 4] >> (8 * (j % 4))) & 0xFFu;
                const uint64_t e = lut[(j % 4) * 256 + v];
                const int dw = (5 * j) / 4;
                d[dw] |= (uint32_t)e;
                d[dw + 1] |= (uint32_t)(e >> 32);
            }
#pragma unroll
            for (int q = 0; q < 5; ++q)
                *reinterpret_cast<v4i *>(dst + 16 * q) =
                    v4i{(int)d[4 * q], (int)d[4 * q + 1], (int)d[4 * q + 2], (int)d[4 * q + 3]};
        }
    };

    v16i acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int frow = lane % 32;        // fragment row (A) / column (B)
    const int fk = 16 * (lane / 32);   // byte offset of this lane's k slots

    if (ktiles > 0) load_tile(0);
    for (int64_t kt = 0; kt < ktiles; ++kt) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (kt + 1 < ktiles) load_tile(kt + 1);
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            v4i a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const v4i *>(
                    As + (wm * 64 + i * 32 + frow) * C::LDSK + ks * 32 + fk);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = *reinterpret_cast<const v4i *>(
                    Bs + (wn * 64 + j * 32 + frow) * C::LDSK + ks * 32 + fk);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0,
                                                                      0, 0);
        }
    }

    // Epilogue. Fragment register r of lane l holds D[i][j] with
    // j = l % 32 (weight row), i = 8 (r / 4) + 4 (l / 32) + r % 4 (token).
    const float gamma = gamma_p[0];
#pragma unroll
    for (int fi = 0; fi < 2; ++fi) {
#pragma unroll
        for (int fj = 0; fj < 2; ++fj) {
            const int64_t n = n0 + wn * 64 + fj * 32 + (lane % 32);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * 64 + fi * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
                if (m >= M || n >= N) continue;
                const int32_t a = acc[fi][fj][r];
                const float v = ((float)a * (gamma * scale[m])) / 127.0f;
                if constexpr (sizeof(YT) == 4)
                    y[m * N + n] = v;
                else
                    y[m * N + n] = (YT)f32_to_bf16_rne(v);
                if (acc_out) acc_out[m * N + n] = a;
            }
        }
    }
}

template <int LAYOUT, typename YT>
hipError_t launch_gemm_t(const int8_t *xq, const float *scale, const uint8_t *packed,
                         const float *gamma, int64_t M, int64_t N, int64_t K, YT *y,
                         int32_t *acc, hipStream_t s) {
    const int64_t rb = LAYOUT == kLayout2Bit ? row_bytes_2bit(K) : row_bytes_base3(K);
    dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM)), block(kThreads);
    hipLaunchKernelGGL((gemm_kernel<LAYOUT, YT>), grid, block, 0, s, xq, scale, packed, gamma,
                       M, N, K, rb, y, acc);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_gemm(const int8_t *xq, const float *scale, const uint8_t *packed,
                               int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                               void *y, int y_dtype, int32_t *acc, hipStream_t stream) {
    if (layout == kLayout2Bit) {
        if (y_dtype == kF32)
            return launch_gemm_t<kLayout2Bit>(xq, scale, packed, gamma, M, N, K,
                                              static_cast<float *>(y), acc, stream);
        return launch_gemm_t<kLayout2Bit>(xq, scale, packed, gamma, M, N, K,
                                          static_cast<uint16_t *>(y), acc, stream);
    }
    if (y_dtype == kF32)
        return launch_gemm_t<kLayoutBase3>(xq, scale, packed, gamma, M, N, K,
                                           static_cast<float *>(y), acc, stream);
    return launch_gemm_t<kLayoutBase3>(xq, scale, packed, gamma, M, N, K,
                                       static_cast<uint16_t *>(y), acc, stream);
}

}  // namespace bl
