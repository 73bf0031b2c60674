// Prefill-side product (M > 16 tokens): a tiled INT8 matrix-core GEMM.
// Activations (int8) and weight codes are staged through LDS per k-tile; the
// packed weights are expanded to signed code bytes once per block and k-tile
// on their way into LDS, then consumed by v_mfma_i32_32x32x32_i8. Every
// product term is an INT8 activation times a code in {-1, 0, +1}, summed
// exactly in INT32 ([b158] "BitNet b1.58深度解析" §3.3 and §4.2), then
// scaled by gamma * scale[m] / 127 in the epilogue ([b158] §5.2-5.3).
//
// Block tile BM tokens x BN weight rows, WM x WN waves, each owning
// (BM/WM) x (BN/WN) outputs as 32 x 32 fragments. A k-tile is two 16-byte
// units of packed codes per weight row: 128 codes in the 2-bit layout, 160
// in base-3, i.e. 4 or 5 MFMA k-steps. LDS is double buffered and the global
// loads run two k-tiles ahead through two register sets: while tile k is
// multiplied, tile k+1 (already in registers) is written to the other LDS
// buffer and tile k+2 is in flight; one barrier per k-tile. Blocks are
// mapped to tiles so that each of the eight XCDs (dispatched round-robin by
// block id) works on a contiguous run of tiles, which shares activation rows
// in that XCD's L2.
#include "bl_internal.hpp"
#include "device_util.hpp"

namespace bl {
namespace {

constexpr int kXcds = 8;

template <int LAYOUT, int BM_, int BN_, int WM_, int WN_>
struct GemmCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int THREADS = 64 * WM * WN;
    static constexpr int UC = LAYOUT == kLayout2Bit ? 64 : 80;  // codes per 16-byte unit
    static constexpr int UNITS = 2;                               // units per row per k-tile
    static constexpr int BK = UNITS * UC;                         // codes per k-tile
    static constexpr int LDSK = BK + 16;                          // padded LDS row (bytes)
    static constexpr int KSTEPS = BK / 32;
    static constexpr int ACH = BM * BK / 16 / THREADS;            // A 16B chunks per thread
    static constexpr int BUNITS = BN * UNITS;                     // B units per k-tile
    static constexpr int FI = BM / WM / 32, FJ = BN / WN / 32;    // fragments per wave
    static constexpr int STAGE = (BM + BN) * LDSK;
    static constexpr int LUT = LAYOUT == kLayoutBase3 ? 8192 : 0;
    static constexpr int SMEM = LUT + 2 * STAGE;
    static_assert(BM * BK % (16 * THREADS) == 0, "A tile must split evenly");
    static_assert(BUNITS <= THREADS, "one B unit per thread at most");
    static_assert(FI >= 1 && FJ >= 1, "wave tile of at least one fragment");
};

template <int LAYOUT, int BM, int BN, int WM, int WN, typename YT>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(
    const int8_t *__restrict__ xq, const float *__restrict__ scale,
    const uint8_t *__restrict__ packed, const float *__restrict__ gamma_p, int64_t M,
    int64_t N, int64_t K, int64_t rb, int tiles_m, int tiles_n, YT *__restrict__ y,
    int32_t *__restrict__ acc_out) {
    using C = GemmCfg<LAYOUT, BM, BN, WM, WN>;
    constexpr int kThreads = C::THREADS;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint64_t *lut = reinterpret_cast<uint64_t *>(smem);
    int8_t *stage0 = reinterpret_cast<int8_t *>(smem + C::LUT);

    // XCD-aware tile mapping
    const int ntiles = tiles_m * tiles_n;
    const int per_xcd = (ntiles + kXcds - 1) / kXcds;
    const int b = blockIdx.x;
    const int t = (b % kXcds) * per_xcd + b / kXcds;
    if (t >= ntiles) return;
    const int64_t m0 = (int64_t)(t / tiles_n) * BM;
    const int64_t n0 = (int64_t)(t % tiles_n) * BN;

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    const int wm = wave / WN, wn = wave % WN;

    if (LAYOUT == kLayoutBase3) {
        for (int i = tid; i < 4 * 256; i += kThreads)
            lut[i] = base3_entry((uint32_t)(i % 256)) << (8 * (i / 256));
    }

    const int64_t units = rb / 16;
    const int64_t ktiles = (units + C::UNITS - 1) / C::UNITS;
    const bool a_aligned = (K % 16) == 0;
    const bool has_b = tid < C::BUNITS;
    const int b_row = tid / C::UNITS, b_unit = tid % C::UNITS;
    const bool b_row_ok = has_b && n0 + b_row < N;
    const uint8_t *b_src = packed + (n0 + b_row) * rb;

    v4i a_regs[2][C::ACH];
    uint4 b_regs[2];

    auto load_tile = [&](int64_t kt, v4i *a_reg, uint4 &b_reg) {
        const int64_t kc0 = kt * C::BK;
#pragma unroll
        for (int i = 0; i < C::ACH; ++i) {
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
        const int64_t unit = kt * C::UNITS + b_unit;
        b_reg = make_uint4(0u, 0u, 0u, 0u);
        if (b_row_ok && unit < units) b_reg = *reinterpret_cast<const uint4 *>(b_src + unit * 16);
    };

    auto store_tile = [&](int8_t *st, const v4i *a_reg, const uint4 b_reg) {
        int8_t *As = st;
        int8_t *Bs = st + BM * C::LDSK;
#pragma unroll
        for (int i = 0; i < C::ACH; ++i) {
            const int q = tid + i * kThreads;
            const int row = q / (C::BK / 16), col = q % (C::BK / 16);
            *reinterpret_cast<v4i *>(As + row * C::LDSK + col * 16) = a_reg[i];
        }
        if (!has_b) return;
        int8_t *dst = Bs + b_row * C::LDSK + b_unit * C::UC;
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

    v16i acc[C::FI][C::FJ];
#pragma unroll
    for (int i = 0; i < C::FI; ++i)
#pragma unroll
        for (int j = 0; j < C::FJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int frow = lane % 32;       // fragment row (A) / column (B)
    const int fk = 16 * (lane / 32);  // byte offset of this lane's k slots

    if (LAYOUT == kLayoutBase3) __syncthreads();  // decode table ready
    // Pipeline: LDS holds tiles kt (being multiplied) and kt+1 (being
    // written); registers hold tile kt+1 (arrived) and kt+2 (in flight).
    if (ktiles > 0) load_tile(0, a_regs[0], b_regs[0]);
    if (ktiles > 1) load_tile(1, a_regs[1], b_regs[1]);
    if (ktiles > 0) store_tile(stage0, a_regs[0], b_regs[0]);
    __syncthreads();
    for (int64_t kt = 0; kt < ktiles; ++kt) {
        const int cur_i = (int)(kt & 1);
        int8_t *cur = stage0 + cur_i * C::STAGE;
        int8_t *nxt = stage0 + (cur_i ^ 1) * C::STAGE;
        if (kt + 2 < ktiles) {
            if (cur_i == 0) load_tile(kt + 2, a_regs[0], b_regs[0]);
            else load_tile(kt + 2, a_regs[1], b_regs[1]);
        }
        const int8_t *As = cur;
        const int8_t *Bs = cur + BM * C::LDSK;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            v4i a[C::FI], bb[C::FJ];
#pragma unroll
            for (int i = 0; i < C::FI; ++i)
                a[i] = *reinterpret_cast<const v4i *>(
                    As + (wm * (BM / WM) + i * 32 + frow) * C::LDSK + ks * 32 + fk);
#pragma unroll
            for (int j = 0; j < C::FJ; ++j)
                bb[j] = *reinterpret_cast<const v4i *>(
                    Bs + (wn * (BN / WN) + j * 32 + frow) * C::LDSK + ks * 32 + fk);
#pragma unroll
            for (int i = 0; i < C::FI; ++i)
#pragma unroll
                for (int j = 0; j < C::FJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], bb[j], acc[i][j], 0,
                                                                      0, 0);
        }
        if (kt + 1 < ktiles) {
            if (cur_i == 0) store_tile(nxt, a_regs[1], b_regs[1]);
            else store_tile(nxt, a_regs[0], b_regs[0]);
        }
        __syncthreads();
    }

    // Epilogue. Fragment register r of lane l holds D[i][j] with
    // j = l % 32 (weight row), i = 8 (r / 4) + 4 (l / 32) + r % 4 (token).
    const float gamma = gamma_p[0];
#pragma unroll
    for (int fi = 0; fi < C::FI; ++fi) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m =
                m0 + wm * (BM / WM) + fi * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
            if (m >= M) continue;
            const float f = gamma * scale[m] / 127.0f;
#pragma unroll
            for (int fj = 0; fj < C::FJ; ++fj) {
                const int64_t n = n0 + wn * (BN / WN) + fj * 32 + (lane % 32);
                if (n >= N) continue;
                const int32_t a = acc[fi][fj][r];
                const float v = (float)a * f;
                if constexpr (sizeof(YT) == 4)
                    y[m * N + n] = v;
                else
                    y[m * N + n] = (YT)f32_to_bf16_rne(v);
                if (acc_out) acc_out[m * N + n] = a;
            }
        }
    }
}

template <int LAYOUT, int BM, int BN, int WM, int WN, typename YT>
hipError_t launch_gemm_tile(const int8_t *xq, const float *scale, const uint8_t *packed,
                            const float *gamma, int64_t M, int64_t N, int64_t K, YT *y,
                            int32_t *acc, hipStream_t s) {
    using C = GemmCfg<LAYOUT, BM, BN, WM, WN>;
    const int64_t rb = LAYOUT == kLayout2Bit ? row_bytes_2bit(K) : row_bytes_base3(K);
    const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
    const int64_t ntiles = (int64_t)tm * tn;
    const int64_t blocks = (ntiles + kXcds - 1) / kXcds * kXcds;
    auto kern = gemm_kernel<LAYOUT, BM, BN, WM, WN, YT>;
    static int lds_raised = 0;
    hipError_t e = allow_dynamic_lds(kern, C::SMEM, &lds_raised);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(C::THREADS), C::SMEM, s, xq, scale,
                       packed, gamma, M, N, K, rb, tm, tn, y, acc);
    return hipGetLastError();
}

template <int LAYOUT, typename YT>
hipError_t launch_gemm_t(const int8_t *xq, const float *scale, const uint8_t *packed,
                         const float *gamma, int64_t M, int64_t N, int64_t K, YT *y,
                         int32_t *acc, hipStream_t s) {
    // the largest tile that still gives every CU about two tiles
    auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    if (tiles(256, 128) >= 512)
        return launch_gemm_tile<LAYOUT, 256, 128, 4, 2>(xq, scale, packed, gamma, M, N, K, y, acc,
                                                        s);
    if (tiles(128, 128) >= 256)
        return launch_gemm_tile<LAYOUT, 128, 128, 2, 2>(xq, scale, packed, gamma, M, N, K, y, acc,
                                                        s);
    return launch_gemm_tile<LAYOUT, 128, 64, 2, 2>(xq, scale, packed, gamma, M, N, K, y, acc, s);
}

}  // namespace

hipError_t launch_forward_gemm(const int8_t *xq, const float *scale, const uint8_t *packed,
                               int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                               void *y, int y_dtype, int32_t *acc, hipStream_t stream) {
    if (M > (int64_t)2147483647 || N > (int64_t)2147483647) return hipErrorInvalidValue;
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
