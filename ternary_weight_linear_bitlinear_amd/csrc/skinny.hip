// Decode-side product for small batches (1 <= M <= 16 tokens): the packed
// weights are streamed from HBM exactly once with 16-byte loads, expanded in
// registers to code bytes (the stored 2-bit / 1-bit fields, corrected
// exactly afterwards; signed codes for base-3), and multiplied on the INT8
// matrix cores (v_mfma_i32_16x16x64_i8) with the batch in the 16-column
// operand. A
// weight of +1 adds the activation, -1 subtracts it and 0 contributes
// nothing ([b158] "BitNet b1.58深度解析" §4.2); the sums are exact INT32
// ([b158] §3.3), then scaled by gamma * scale[m] / 127 ([b158] §5.2-5.3).
//
// Work split: a block owns 16 consecutive weight rows (16 * RG for batches);
// its KS waves split the row length K. One "super-step" of a wave covers four 16-byte units of
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

// Launch shapes (measured on MI355X with the weights streamed from HBM):
// eight waves per workgroup, each keeping two 16-byte weight loads per lane
// in flight, beat four waves with four loads when there are few workgroups
// per CU (shorter serial expand/multiply chain per wave once the data lands;
// long rows). From kWideN rows on (at least four workgroups per CU) four waves
// with four loads keep more bytes in flight per CU and stream faster.
// Batches at N >= 8192 put three (up to 12288 rows: one round of at most
// 256 workgroups) or two row groups in a workgroup, cutting the activation
// staging per weight byte. A batch of one 16-token chunk with one or three
// row groups, and one token over rows longer than a round with at most one
// tile per CU, run sixteen waves with one load per lane: each wave's
// expand-and-multiply chain after the weights land is half as long (2-bit
// 16 x 4096 x 4096 4.6 -> 4.4 us, base-3 5.7 -> 5.2 us, base-3 16 x 12288 x
// 4096 8.9 -> 8.5 us, one token over 4096 x 11008 8.9 -> 8.4 us); with two
// row groups or several chunks they were slower (2-bit 16 x 16384 x 4096
// 8.5 -> 9.6 us, 40 x 4096 x 4096 7.4 -> 8.2 us). One token over one-round
// rows with more tiles than CUs runs four waves with four loads, which keep
// more blocks resident (8192 x 4096 5.8 -> 4.7 us, 11008 x 4096 6.8 -> 6.0
// us; at 4096 rows the same as eight waves).
constexpr int kSkKS = 8, kSkNSS = 2, kSkRG2MinN = 8192;
constexpr int kFdKS = 8, kFdNSS = 2;
constexpr int kOneKS = 16, kOneNSS = 1;
static_assert(kOneKS * kOneNSS == kFdKS * kFdNSS && kFdKS * kFdNSS == 4 * 4,
              "every one-token launch shape covers 64 units per round");
constexpr int64_t kWideN = 16384;

// 16 elements of x held as raw 16-byte pieces (two for bf16, four for fp32),
// widened to fp32.
__device__ __forceinline__ void unpack_raw(const uint4 (&p)[2], float v[16]) {
    const uint32_t w[8] = {p[0].x, p[0].y, p[0].z, p[0].w, p[1].x, p[1].y, p[1].z, p[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void unpack_raw(const uint4 (&p)[4], float v[16]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[4 * i] = __uint_as_float(p[i].x);
        v[4 * i + 1] = __uint_as_float(p[i].y);
        v[4 * i + 2] = __uint_as_float(p[i].z);
        v[4 * i + 3] = __uint_as_float(p[i].w);
    }
}

// A unit is what one lane loads per row: 16 bytes of 2-bit (64 codes) or
// base-3 (80 codes) codes, 8 bytes of 1-bit codes (64 codes), so that every
// layout feeds the same 16-code matrix-core steps.
template <int LAYOUT>
struct SkinnyCfg {
    static constexpr int kUnitCodes = LAYOUT == kLayoutBase3 ? 80 : 64;
    static constexpr int kUnitBytes = LAYOUT == kLayout1Bit ? 8 : 16;
    static constexpr int kSteps = kUnitCodes / 16;  // MFMA instructions per unit
};

template <int LAYOUT>
__device__ __forceinline__ uint4 load_unit(const uint8_t *p) {
    if constexpr (LAYOUT == kLayout1Bit) {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        return make_uint4(v.x, v.y, 0u, 0u);
    } else {
        return *reinterpret_cast<const uint4 *>(p);
    }
}

// 2-bit and 1-bit units are multiplied as their stored fields (u = c + 1,
// or b = (c + 1) / 2), two instructions per four codes instead of three; one
// more matrix-core instruction per k-step, with every weight byte 1, gives
// each wave the sum of the activations it multiplied, and the exact INT32
// correction follows the last round: acc = sum u x - sum x (2-bit) or
// 2 sum b x - sum x (1-bit). Base-3 units decode to signed codes through the
// table. The correction's bound: each wave sums K / KS codes, so every
// partial stays within 2 * 127 * K / KS (well inside INT32 for K < 2^31 / 127).
template <int LAYOUT>
constexpr bool kFieldCodes = LAYOUT != kLayoutBase3;
constexpr int kOnes = 0x01010101;

template <int LAYOUT>
__device__ __forceinline__ v4i field_correction(const v4i acc, const v4i ones) {
    if constexpr (LAYOUT == kLayout1Bit) return acc + acc - ones;
    return acc - ones;
}

// Decode one unit into code bytes (natural k order): stored fields for 2-bit
// and 1-bit (see above), signed codes for base-3.
template <int LAYOUT>
__device__ __forceinline__ void decode_unit(const uint4 wv, const uint64_t *lut, int c[20]) {
    if constexpr (LAYOUT == kLayout2Bit) {
        fields_2bit_word(wv.x, c + 0);
        fields_2bit_word(wv.y, c + 4);
        fields_2bit_word(wv.z, c + 8);
        fields_2bit_word(wv.w, c + 12);
    } else if constexpr (LAYOUT == kLayout1Bit) {
        fields_1bit_half(wv.x, 0, c + 0);
        fields_1bit_half(wv.x, 1, c + 4);
        fields_1bit_half(wv.y, 0, c + 8);
        fields_1bit_half(wv.y, 1, c + 12);
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

// The activation operands of one unit's matrix-core steps (16 bytes each, one
// token row of the staged tile), read back to back so that their LDS
// latencies overlap.
//
// Both decode kernels feed the matrix cores without masking. Lanes of tokens
// past M read token M - 1's row (`tok` below), so their output columns hold
// copies that are never stored. Weight loads that fall outside the matrix
// (rows past N, units past the row) read a valid address and are not zeroed:
// rows past N only reach outputs that are never stored, and units past the
// row meet activations that are staged as zero past K, so they add nothing.
template <int STEPS>
__device__ __forceinline__ void read_act_unit(const int8_t *p, v4i (&b)[STEPS]) {
#pragma unroll
    for (int st = 0; st < STEPS; ++st) b[st] = *reinterpret_cast<const v4i *>(p + 16 * st);
}

// Epilogue of the decode products: four consecutive outputs n .. n + 3 of one
// token (row pointers yt, acct) from their INT32 sums, y = acc * gamma *
// scale / 127. A single matrix takes one factor; stacked segments pick each
// row's own (a wave-uniform branch, so the common case skips the selection).
template <typename YT>
__device__ __forceinline__ void store_outputs(const GammaMap &gm,
                                              const float (&gs)[kMaxSegments], float scale,
                                              const v4i tot, int64_t n, int64_t N, YT *yt,
                                              int32_t *acct) {
    float f[4];
    if (gm.nseg == 1) {
        const float f0 = gs[0] * scale / 127.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = f0;
    } else {
        float fs[kMaxSegments];
        seg_factors(gm, gs, scale, fs);
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = seg_pick(gm, fs, n + i);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (n + i >= N) continue;
        const float v = (float)tot[i] * f[i];
        if constexpr (sizeof(YT) == 4)
            yt[n + i] = v;
        else
            yt[n + i] = (YT)f32_to_bf16_rne(v);
        if (acct) acct[n + i] = tot[i];
    }
}

// RG row groups of 16 weight rows per workgroup share every activation read
// from LDS (one operand load feeds RG matrix-core instructions); RG > 1 pays
// off for batches, where activations outweigh the packed weights per row.
// MAXM bounds the batch, so the registers that carry a round's activation
// slice into LDS are sized at compile time.
//
// Order within a round: the activation slice (L2-resident, small) is loaded
// into registers first, then the weight loads are issued. Vector-memory
// counters complete in issue order, so the wait for the activations leaves
// every weight load in flight, and the LDS staging overlaps the HBM latency.
// MR: rows longer than one round (a separate instantiation, so one-round rows
// keep the registers the next round's requests would take).
template <int LAYOUT, int KS, int NSS, int RG, int MAXM, bool MR, typename YT>
__global__ __launch_bounds__(64 * KS) void skinny_kernel(
    const int8_t *__restrict__ xq, const float *__restrict__ scale,
    const uint8_t *__restrict__ packed, const GammaMap gm, int M, int64_t N,
    int64_t K, int64_t rb, YT *__restrict__ y, int32_t *__restrict__ acc_out) {
    using C = SkinnyCfg<LAYOUT>;
    constexpr int kThreads = 64 * KS;
    constexpr int kRoundUnits = KS * NSS * 4;                 // units per round
    constexpr int kRoundK = kRoundUnits * C::kUnitCodes;       // codes per round
    constexpr int kActStride = kRoundK + 16;                   // LDS row stride (bytes)
    constexpr int kChunksPerTok = kRoundK / 16;
    constexpr int kMaxQ = (MAXM * kChunksPerTok + kThreads - 1) / kThreads;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint64_t *lut = reinterpret_cast<uint64_t *>(smem);                 // base-3 only
    int8_t *act = reinterpret_cast<int8_t *>(smem + (LAYOUT == kLayoutBase3 ? 8192 : 0));
    v4i *part = reinterpret_cast<v4i *>(smem + (LAYOUT == kLayoutBase3 ? 8192 : 0));

    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    const int r = lane % 16;  // weight row within a row group (A) / token (B)
    const int g = lane / 16;  // lane group = unit within the super-step
    const int64_t n0 = (int64_t)blockIdx.x * 16 * RG;
    // larger batches run as chunks of MAXM tokens, one per grid row
    {
        const int64_t t0 = (int64_t)blockIdx.y * MAXM;
        xq += t0 * K;
        scale += t0;
        y += t0 * N;
        if (acc_out) acc_out += t0 * N;
        M = M - (int)t0 < MAXM ? M - (int)t0 : MAXM;
    }
    float gs[kMaxSegments];
    load_gammas(gm, gs);
    // batches of up to 16 tokens load this lane's token scale (token r) before
    // any activation or weight, so that its latency overlaps theirs instead of
    // following the reduction (measured slower for the 4-token variants)
    float sc_early = 0.f;
    if constexpr (MAXM > 4) sc_early = r < M ? scale[r] : 0.f;

    if (LAYOUT == kLayoutBase3) {  // visible after the first round's barriers
        for (int i = threadIdx.x; i < 4 * 256; i += kThreads)
            lut[i] = base3_entry((uint32_t)(i % 256)) << (8 * (i / 256));
    }

    const int64_t units = rb / C::kUnitBytes;
    const bool aligned = (K % 16) == 0;
    const int chunks = M * kChunksPerTok;
    const uint8_t *wrow[RG];
    bool row_ok[RG];
#pragma unroll
    for (int q = 0; q < RG; ++q) {
        row_ok[q] = n0 + 16 * q + r < N;
        wrow[q] = packed + (n0 + 16 * q + r) * rb;
    }

    const int tok = r < M ? r : M - 1;  // token row this lane's activation operand reads
    v4i acc[RG];
#pragma unroll
    for (int q = 0; q < RG; ++q) acc[q] = v4i{0, 0, 0, 0};
    v4i ones = {0, 0, 0, 0};  // field layouts: sum of the activations multiplied

    // every weight load of the round starting at unit u0. Out-of-range units
    // load a valid address and are used as loaded (see read_act_unit): a
    // select right at the load would make the compiler wait for it there.
    uint4 wv[RG][NSS];
    auto issue_w = [&](int64_t u0) {
#pragma unroll
        for (int q = 0; q < RG; ++q)
#pragma unroll
            for (int s = 0; s < NSS; ++s) {
                const int64_t unit = u0 + (int64_t)(s * KS + wave) * 4 + g;
                const bool ok = row_ok[q] && unit < units;
                wv[q][s] = load_unit<LAYOUT>(ok ? wrow[q] + unit * C::kUnitBytes : packed);
            }
    };
    // chunks of K % 16 != 0 rows, byte by byte (zero past K)
    auto stage_bytes = [&](int64_t k0) {
        for (int q = threadIdx.x; q < chunks; q += kThreads) {
            const int t = q / kChunksPerTok, cc = q % kChunksPerTok;
            const int64_t k = k0 + cc * 16;
            const int8_t *src = xq + (int64_t)t * K;
            uint32_t d[4] = {0u, 0u, 0u, 0u};
            for (int e = 0; e < 16; ++e)
                if (k + e < K) d[e / 4] |= (uint32_t)(uint8_t)src[k + e] << (8 * (e % 4));
            *reinterpret_cast<v4i *>(act + t * kActStride + cc * 16) =
                v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
        }
    };
    // expand and multiply one round; one activation read feeds RG instructions
    auto multiply = [&]() {
        v4i b[NSS][C::kSteps];
#pragma unroll
        for (int s = 0; s < NSS; ++s)
            read_act_unit<C::kSteps>(
                act + tok * kActStride + ((s * KS + wave) * 4 + g) * C::kUnitCodes, b[s]);
#pragma unroll
        for (int s = 0; s < NSS; ++s) {
            int c[RG][20];
#pragma unroll
            for (int q = 0; q < RG; ++q) decode_unit<LAYOUT>(wv[q][s], lut, c[q]);
#pragma unroll
            for (int st = 0; st < C::kSteps; ++st) {
#pragma unroll
                for (int q = 0; q < RG; ++q) {
                    const v4i a = {c[q][4 * st], c[q][4 * st + 1], c[q][4 * st + 2],
                                   c[q][4 * st + 3]};
                    acc[q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[s][st], acc[q], 0, 0, 0);
                }
                if constexpr (kFieldCodes<LAYOUT>)
                    ones = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4i{kOnes, kOnes, kOnes, kOnes},
                                                                 b[s][st], ones, 0, 0, 0);
            }
        }
    };

    if constexpr (!MR) {
        // One round: this thread's chunks of xq[0:M, 0:K] (16 bytes each; with
        // K % 16 == 0 a chunk is entirely inside or outside the row) go
        // straight into LDS (16-byte direct-to-LDS loads, no registers) ahead
        // of the weights: vector-memory counters complete in issue order, so
        // the wait for them leaves every weight load in flight. A wave's 64
        // chunks are consecutive in one token row (64 divides the chunks per
        // row), so its LDS offset is uniform. Chunks past K read a placeholder
        // address and are zeroed once they have landed.
        if (aligned) {
#pragma unroll
            for (int i = 0; i < kMaxQ; ++i) {
                const int qw = __builtin_amdgcn_readfirstlane(threadIdx.x - lane + i * kThreads);
                const int t = qw / kChunksPerTok;
                if (t < M) {  // wave-uniform
                    const int64_t k = (qw % kChunksPerTok + lane) * 16;
                    const int8_t *src = k < K ? xq + (int64_t)t * K + k : xq;
                    __builtin_amdgcn_global_load_lds(
                        src, to_lds(act + t * kActStride + (qw % kChunksPerTok) * 16), 16, 0, 0);
                }
            }
        }
        issue_w(0);
        if (aligned) {
            __builtin_amdgcn_s_waitcnt(vmcnt_only(RG * NSS));
            if (kRoundK > K) {
#pragma unroll
                for (int i = 0; i < kMaxQ; ++i) {
                    const int q = threadIdx.x + i * kThreads;
                    const int64_t k = (q % kChunksPerTok) * 16;
                    if (q < chunks && k >= K)
                        *reinterpret_cast<v4i *>(act + (q / kChunksPerTok) * kActStride +
                                                 (q % kChunksPerTok) * 16) = v4i{0, 0, 0, 0};
                }
            }
        } else {
            stage_bytes(0);
        }
        lds_barrier();
        multiply();
    } else {
        // Several rounds: each round's activation chunks are loaded into
        // registers ahead of its weights, before the barrier that lets the
        // tile be rewritten, so both overlap the previous round's tail.
        for (int64_t u0 = 0; u0 < units; u0 += kRoundUnits) {
            const int64_t k0 = u0 * C::kUnitCodes;
            v4i xa[kMaxQ];
            bool xok[kMaxQ];
            if (aligned) {
#pragma unroll
                for (int i = 0; i < kMaxQ; ++i) {
                    const int q = threadIdx.x + i * kThreads;
                    const int t = q / kChunksPerTok;
                    const int64_t k = k0 + (q % kChunksPerTok) * 16;
                    xok[i] = q < chunks && k < K;
                    xa[i] = *reinterpret_cast<const v4i *>(xok[i] ? xq + (int64_t)t * K + k : xq);
                }
            }
            issue_w(u0);
            lds_barrier();  // the previous round's readers are done
            if (aligned) {
#pragma unroll
                for (int i = 0; i < kMaxQ; ++i) {
                    const int q = threadIdx.x + i * kThreads;
                    if (q < chunks)
                        *reinterpret_cast<v4i *>(act + (q / kChunksPerTok) * kActStride +
                                                 (q % kChunksPerTok) * 16) =
                            xok[i] ? xa[i] : v4i{0, 0, 0, 0};
                }
            } else {
                stage_bytes(k0);
            }
            lds_barrier();
            multiply();
        }
    }

    if constexpr (kFieldCodes<LAYOUT>) {
#pragma unroll
        for (int q = 0; q < RG; ++q) acc[q] = field_correction<LAYOUT>(acc[q], ones);
    }
    lds_barrier();
#pragma unroll
    for (int q = 0; q < RG; ++q) part[(q * KS + wave) * 64 + lane] = acc[q];
    lds_barrier();
    const int t = r;
    if (t >= M) return;
    const float sc = MAXM > 4 ? sc_early : scale[t];
    for (int q = wave; q < RG; q += KS) {  // wave q finishes row group q
        v4i tot = part[(q * KS) * 64 + lane];
#pragma unroll
        for (int w = 1; w < KS; ++w) tot += part[(q * KS + w) * 64 + lane];
        // lane holds D[4g + i][r]: weight rows n0 + 16q + 4g + i, token r
        store_outputs(gm, gs, sc, tot, n0 + 16 * q + 4 * g, N, y + (int64_t)t * N,
                      acc_out ? acc_out + (int64_t)t * N : nullptr);
    }
}

template <int LAYOUT, int KS, int NSS, int RG, int MAXM, typename YT>
hipError_t launch_skinny_t(const int8_t *xq, const float *scale, const uint8_t *packed,
                           const GammaMap &gamma, int64_t M, int64_t N, int64_t K, YT *y,
                           int32_t *acc, hipStream_t s) {
    const int64_t rb = row_bytes_of(LAYOUT, K);
    // the partial-tile buffer aliases the activation area (needs KS*RG KiB)
    const int64_t chunk_m = M < MAXM ? M : MAXM;
    const int64_t round_units = (int64_t)KS * NSS * 4;
    const size_t lut = LAYOUT == kLayoutBase3 ? 8192 : 0;
    const size_t act = (size_t)chunk_m * (KS * NSS * 4 * SkinnyCfg<LAYOUT>::kUnitCodes + 16);
    const size_t part = (size_t)KS * RG * 1024;
    const size_t smem = lut + (act > part ? act : part);
    dim3 grid((unsigned)((N + 16 * RG - 1) / (16 * RG)), (unsigned)((M + MAXM - 1) / MAXM)),
        block(64 * KS);
    const bool mr = rb / SkinnyCfg<LAYOUT>::kUnitBytes > round_units;
    if (t_plan) {
        plan_note(grid.x, grid.y, block.x, smem, "skinny_kernel<%d, %d, %d, %d, %d, %s, %s>",
                  LAYOUT, KS, NSS, RG, MAXM, mr ? "true" : "false", type_name<YT>());
        return hipSuccess;
    }
    auto go = [&](auto kern, LdsFlag *flag) {
        hipError_t e = allow_dynamic_lds(kern, smem, flag);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, grid, block, smem, s, xq, scale, packed, gamma, (int)M, N, K, rb,
                           y, acc);
        return hipGetLastError();
    };
    static LdsFlag lds_raised[2];  // one flag per kernel of this launcher
    if (mr) return go(skinny_kernel<LAYOUT, KS, NSS, RG, MAXM, true, YT>, &lds_raised[1]);
    return go(skinny_kernel<LAYOUT, KS, NSS, RG, MAXM, false, YT>, &lds_raised[0]);
}

template <int LAYOUT, typename YT>
hipError_t launch_skinny_l(const int8_t *xq, const float *scale, const uint8_t *packed,
                           const GammaMap &gamma, int64_t M, int64_t N, int64_t K, YT *y,
                           int32_t *acc, hipStream_t s) {
    // eight waves x two super-steps: one round covers 4096 codes (2-bit) or
    // 5120 (base-3); at M = 16 that is 64 (80) KiB of staged activations
    if (M <= 4 && N >= kWideN)
        return launch_skinny_t<LAYOUT, 4, 4, 1, 4, YT>(xq, scale, packed, gamma, M, N, K, y, acc,
                                                      s);
    if (M <= 4)
        return launch_skinny_t<LAYOUT, kSkKS, kSkNSS, 1, 4, YT>(xq, scale, packed, gamma, M, N, K,
                                                               y, acc, s);
    // up to 16 x 256 x 3 rows: three row groups, so that one round of
    // workgroups (at most one per compute unit) covers the matrix
    const bool one_chunk = M <= 16;  // larger batches run as several 16-token chunks
    if (N >= kSkRG2MinN && N <= 16 * 256 * 3) {
        if (one_chunk)
            return launch_skinny_t<LAYOUT, kOneKS, kOneNSS, 3, 16, YT>(xq, scale, packed, gamma, M,
                                                                     N, K, y, acc, s);
        return launch_skinny_t<LAYOUT, kSkKS, kSkNSS, 3, 16, YT>(xq, scale, packed, gamma, M, N, K,
                                                               y, acc, s);
    }
    if (N >= kSkRG2MinN)
        return launch_skinny_t<LAYOUT, kSkKS, kSkNSS, 2, 16, YT>(xq, scale, packed, gamma, M, N, K,
                                                               y, acc, s);
    if (one_chunk)
        return launch_skinny_t<LAYOUT, kOneKS, kOneNSS, 1, 16, YT>(xq, scale, packed, gamma, M, N,
                                                                 K, y, acc, s);
    return launch_skinny_t<LAYOUT, kSkKS, kSkNSS, 1, 16, YT>(xq, scale, packed, gamma, M, N, K,
                                                           y, acc, s);
}

// ---------------------------------------------------------------------------
// Fused decode (1 <= M <= 4 tokens): per-token absmax INT8 quantisation of x
// inside every block, then the same weight-streaming product. Each block
// loads its chunks of x (from L2), issues its weight loads, derives the token
// scales s_m = max(max|x|, 1e-6) and quantises the round's slice of x into
// LDS with quant4() (the same fp32 steps as the stand-alone quantiser, so
// codes are identical) while the weights are still in flight, then
// multiplies. One launch instead of two on the latency-bound decode path.
constexpr int kFusedMaxM = 4;
// Streaming variant (several tokens, many tiles): grid capped at two blocks per
// compute unit, 8 waves of 2 units each, one tile of weights in flight ahead
// (one, three or four blocks per unit, 4-wave blocks and two tiles ahead were
// all slower on MI355X at N = 6144 .. 22016).
constexpr int kFusedBlocksPerCu = 2;
constexpr int kFsKS = 8, kFsNSS = 2;

template <int LAYOUT, int KS, int NSS, int MAXM, bool STREAM, int RG, typename XT, typename YT>
__global__ __launch_bounds__(64 * KS) void linear_decode_kernel(
    const XT *__restrict__ x, const uint8_t *__restrict__ packed,
    const GammaMap gm, int M, int64_t N, int64_t K, int64_t rb,
    YT *__restrict__ y, int32_t *__restrict__ acc_out) {
    using C = SkinnyCfg<LAYOUT>;
    constexpr int kThreads = 64 * KS;
    constexpr int kRoundUnits = KS * NSS * 4;
    constexpr int kRoundK = kRoundUnits * C::kUnitCodes;
    constexpr int kActStride = kRoundK + 16;
    // STREAM: the block streams tiles (see below); otherwise it owns one tile
    // and keeps the register count that lets more blocks stay resident. A
    // tile is RG groups of 16 weight rows that share every activation read.
    static_assert(!STREAM || RG == 1, "streaming blocks take one row group per tile");
    // LDS: [base-3 table] [activation tile, MAXM rows] [two partial-sum areas]
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint64_t *lut = reinterpret_cast<uint64_t *>(smem);
    int8_t *act = reinterpret_cast<int8_t *>(smem + (LAYOUT == kLayoutBase3 ? 8192 : 0));
    v4i *part = reinterpret_cast<v4i *>(act + MAXM * kActStride);
    __shared__ float red[kFusedMaxM][KS];
    __shared__ float tok_scale[kFusedMaxM];

    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    const int r = lane % 16;
    const int g = lane / 16;
    const int64_t tiles = (N + 16 * RG - 1) / (16 * RG);
    const int64_t units = rb / C::kUnitBytes;
    const bool vec = (K % 8) == 0;

    float gs[kMaxSegments];
    load_gammas(gm, gs);
    // this lane's weight units of tile `tile`, round starting at unit u0
    uint4 wv[RG][NSS], wn[RG][NSS];
    bool wok[RG][NSS], wnok[RG][NSS];
    auto issue = [&](int64_t tile, int64_t u0, uint4 (&w)[RG][NSS], bool (&ok)[RG][NSS]) {
#pragma unroll
        for (int q = 0; q < RG; ++q) {
            const int64_t n = (tile * RG + q) * 16 + r;
            const uint8_t *wrow = packed + n * rb;
#pragma unroll
            for (int s = 0; s < NSS; ++s) {
                const int64_t unit = u0 + (int64_t)(s * KS + wave) * 4 + g;
                ok[q][s] = n < N && unit < units;
                // out-of-range lanes read a valid address; the value is zeroed
                // where it is consumed, so no wait is forced here
                w[q][s] = load_unit<LAYOUT>(ok[q][s] ? wrow + unit * C::kUnitBytes : packed);
            }
        }
    };

    // token scales: s_m = max(max_k |x[m, k]|, 1e-6), a block-wide max per
    // token. When the row fits one round, each thread loads its 16-element
    // chunks of x once and keeps them for the quantisation below. With
    // K % 16 == 0 those loads are issued before the weight loads: memory
    // counters complete in issue order, so the scale and quantisation work
    // then overlaps the weights' HBM latency instead of following it.
    constexpr int kChunksPerTok = kRoundK / 16;
    constexpr int kMaxQ = (MAXM * kChunksPerTok + kThreads - 1) / kThreads;
    constexpr int kRaw = (int)sizeof(XT);  // 16-byte pieces per 16-element chunk
    const bool one_round = units <= kRoundUnits;
    const bool early = one_round && (K % 16) == 0;
    // (out-of-range chunks load a valid address unconditionally and are
    // zeroed only after the weight loads are issued: a select right at the
    // load would make the compiler wait for it there)
    uint4 xr[kMaxQ][kRaw];
    bool xok[kMaxQ];
    if (early) {
#pragma unroll
        for (int i = 0; i < kMaxQ; ++i) {
            const int q = threadIdx.x + i * kThreads;
            const int t = q / kChunksPerTok;
            const int64_t k = (int64_t)(q % kChunksPerTok) * 16;
            xok[i] = t < M && k < K;
            const uint4 *src =
                reinterpret_cast<const uint4 *>(xok[i] ? x + (int64_t)t * K + k : x);
#pragma unroll
            for (int j = 0; j < kRaw; ++j) xr[i][j] = src[j];
        }
    }
    const int64_t tile0 = blockIdx.x;
    issue(tile0, 0, wv, wok);
    // streaming (rows that fit one round): x is quantised once per block and
    // the block takes tiles tile0, tile0 + gridDim.x, ...; the next tile's
    // weights are always in flight while the current one is multiplied
    if (STREAM && one_round && tile0 + gridDim.x < tiles) issue(tile0 + gridDim.x, 0, wn, wnok);

    if (LAYOUT == kLayoutBase3) {
        for (int i = threadIdx.x; i < 4 * 256; i += kThreads)
            lut[i] = base3_entry((uint32_t)(i % 256)) << (8 * (i / 256));
    }

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
    auto track_max = [&](int t, const float *v) {
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[e]));
#pragma unroll
        for (int tt = 0; tt < kFusedMaxM; ++tt) amax[tt] = tt == t ? fmaxf(amax[tt], m) : amax[tt];
    };
    if (early) {
#pragma unroll
        for (int i = 0; i < kMaxQ; ++i) {
            const int q = threadIdx.x + i * kThreads;
            const int t = q / kChunksPerTok;
            unpack_raw(xr[i], xv[i]);
#pragma unroll
            for (int e = 0; e < 16; ++e) xv[i][e] = xok[i] ? xv[i][e] : 0.f;
            if (t < M) track_max(t, xv[i]);
        }
    } else if (one_round) {
#pragma unroll
        for (int i = 0; i < kMaxQ; ++i) {
            const int q = threadIdx.x + i * kThreads;
            const int t = q / kChunksPerTok;
            if (t < M) {
                load_chunk(t, (int64_t)(q % kChunksPerTok) * 16, xv[i]);
                track_max(t, xv[i]);
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
    lds_barrier();
    if (threadIdx.x < M) {
        float m = red[threadIdx.x][0];
#pragma unroll
        for (int w = 1; w < KS; ++w) m = fmaxf(m, red[threadIdx.x][w]);
        tok_scale[threadIdx.x] = fmaxf(m, 1e-6f);
    }
    lds_barrier();

    auto store_codes = [&](int t, int cc, const float *v) {
        const float sc = tok_scale[t];
        const float rc = 1.0f / sc;
        v4i d;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            d[i] = (int)quant4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3], sc, rc);
        *reinterpret_cast<v4i *>(act + t * kActStride + cc * 16) = d;
    };

    if (one_round) {
#pragma unroll
        for (int i = 0; i < kMaxQ; ++i) {
            const int q = threadIdx.x + i * kThreads;
            if (q < M * kChunksPerTok) store_codes(q / kChunksPerTok, q % kChunksPerTok, xv[i]);
        }
        lds_barrier();
    }

    const int tok = r < M ? r : M - 1;  // token row this lane's activation operand reads
    int buf = 0;
    for (int64_t tile = tile0; tile < tiles; tile += gridDim.x) {
        v4i acc[RG];
#pragma unroll
        for (int q = 0; q < RG; ++q) acc[q] = v4i{0, 0, 0, 0};
        v4i ones = {0, 0, 0, 0};  // field layouts: sum of the activations multiplied
        for (int64_t u0 = 0; u0 < units; u0 += kRoundUnits) {
            if (!one_round) {
                if (u0 > 0 || tile != tile0) {
                    issue(tile, u0, wv, wok);
                    lds_barrier();  // previous round's readers are done
                }
                // quantise x[0:M, k0 : k0 + kRoundK] into LDS (zero past K)
                const int64_t k0 = u0 * C::kUnitCodes;
                for (int q = threadIdx.x; q < M * kChunksPerTok; q += kThreads) {
                    const int t = q / kChunksPerTok, cc = q % kChunksPerTok;
                    float v[16];
                    load_chunk(t, k0 + cc * 16, v);
                    store_codes(t, cc, v);
                }
                lds_barrier();
            }
#pragma unroll
            for (int s = 0; s < NSS; ++s) {
                const int ul = (s * KS + wave) * 4 + g;
                v4i b[C::kSteps];
                read_act_unit<C::kSteps>(act + tok * kActStride + ul * C::kUnitCodes, b);
                int c[RG][20];
#pragma unroll
                for (int q = 0; q < RG; ++q) decode_unit<LAYOUT>(wv[q][s], lut, c[q]);
#pragma unroll
                for (int st = 0; st < C::kSteps; ++st) {
#pragma unroll
                    for (int q = 0; q < RG; ++q) {
                        const v4i a = {c[q][4 * st], c[q][4 * st + 1], c[q][4 * st + 2],
                                       c[q][4 * st + 3]};
                        acc[q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[st], acc[q], 0, 0,
                                                                       0);
                    }
                    if constexpr (kFieldCodes<LAYOUT>)
                        ones = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                            v4i{kOnes, kOnes, kOnes, kOnes}, b[st], ones, 0, 0, 0);
                }
            }
        }
        if (STREAM && one_round) {
            const int64_t ahead = tile + 2 * (int64_t)gridDim.x;
#pragma unroll
            for (int q = 0; q < RG; ++q)
#pragma unroll
                for (int s = 0; s < NSS; ++s) {
                    wv[q][s] = wn[q][s];
                    wok[q][s] = wnok[q][s];
                }
            if (ahead < tiles) issue(ahead, 0, wn, wnok);
        }

        // sum over the waves through LDS; two areas, so one barrier per tile
        // suffices (an area is rewritten only after the next tile's barrier,
        // which the reducing waves reach after their reads of this one)
        if constexpr (kFieldCodes<LAYOUT>) {
#pragma unroll
            for (int q = 0; q < RG; ++q) acc[q] = field_correction<LAYOUT>(acc[q], ones);
        }
        v4i *pb = part + buf * (RG * KS * 64);
        buf ^= 1;
#pragma unroll
        for (int q = 0; q < RG; ++q) pb[(q * KS + wave) * 64 + lane] = acc[q];
        lds_barrier();
        const int t = r;
        if (t < M) {
            for (int q = wave; q < RG; q += KS) {  // wave q finishes row group q
                v4i tot = pb[(q * KS) * 64 + lane];
#pragma unroll
                for (int w = 1; w < KS; ++w) tot += pb[(q * KS + w) * 64 + lane];
                store_outputs(gm, gs, tok_scale[t], tot, (tile * RG + q) * 16 + 4 * g, N,
                              y + (int64_t)t * N, acc_out ? acc_out + (int64_t)t * N : nullptr);
            }
        }
        if constexpr (!STREAM) break;  // one tile per block
    }
}

template <int LAYOUT, int MAXM, int KS, int NSS, bool STREAM, typename XT, typename YT,
          int RG = 1>
hipError_t launch_linear_m(const XT *x, const uint8_t *packed, const GammaMap &gamma, int64_t M,
                           int64_t N, int64_t K, int64_t grid, YT *y, int32_t *acc,
                           hipStream_t s) {
    const int64_t rb = row_bytes_of(LAYOUT, K);
    constexpr int64_t kRoundK = (int64_t)KS * NSS * 4 * SkinnyCfg<LAYOUT>::kUnitCodes;
    const size_t smem = (LAYOUT == kLayoutBase3 ? 8192 : 0) + (size_t)MAXM * (kRoundK + 16) +
                        2 * (size_t)RG * KS * 1024;
    auto kern = linear_decode_kernel<LAYOUT, KS, NSS, MAXM, STREAM, RG, XT, YT>;
    if (t_plan) {
        plan_note((unsigned)grid, 1, 64 * KS, smem,
                  "linear_decode_kernel<%d, %d, %d, %d, %s, %d, %s, %s>", LAYOUT, KS, NSS, MAXM,
                  STREAM ? "true" : "false", RG, type_name<XT>(), type_name<YT>());
        return hipSuccess;
    }
    static LdsFlag lds_raised{0};
    hipError_t e = allow_dynamic_lds(kern, smem, &lds_raised);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * KS), smem, s, x, packed, gamma,
                       (int)M, N, K, rb, y, acc);
    return hipGetLastError();
}

// Launch shapes, measured on MI355X. Below kWideN rows: one 16-row tile per
// block, except for several tokens whose rows fit one round (K % 16 == 0)
// when the tiles outnumber kFusedBlocksPerCu blocks per compute unit:
// quantising x in every block would then dominate, so the grid is capped and
// each block streams several tiles. From kWideN rows on: 4-wave blocks of two
// row groups (four for several tokens from 2 kWideN rows on), which cut the
// same per-block work while every weight load stays in flight. A one-token
// specialisation keeps only 16 values of x per thread, which leaves registers
// for more resident blocks.
template <int LAYOUT, typename XT, typename YT>
hipError_t launch_linear_t(const XT *x, const uint8_t *packed, const GammaMap &gamma, int64_t M,
                           int64_t N, int64_t K, YT *y, int32_t *acc, hipStream_t s) {
    const int64_t tiles = (N + 15) / 16;
    if (M > 1 && N >= kWideN) {
        // several tokens, many rows: 2 (from 32768 rows on 4) row groups per
        // block instead of a capped grid (M=2, 16384 rows: 10.7 -> 9.0 us;
        // 32768 rows: 16.2 -> 14.3 us)
        if (N >= 2 * kWideN)
            return launch_linear_m<LAYOUT, kFusedMaxM, 4, 4, false, XT, YT, 4>(
                x, packed, gamma, M, N, K, (N + 63) / 64, y, acc, s);
        return launch_linear_m<LAYOUT, kFusedMaxM, 4, 4, false, XT, YT, 2>(
            x, packed, gamma, M, N, K, (N + 31) / 32, y, acc, s);
    }
    if (M > 1 && K % 16 == 0 &&
        K <= (int64_t)kFsKS * kFsNSS * 4 * SkinnyCfg<LAYOUT>::kUnitCodes) {
        const int64_t cap = (int64_t)kFusedBlocksPerCu * device_cu_count();
        if (cap > 0 && tiles > cap)
            return launch_linear_m<LAYOUT, kFusedMaxM, kFsKS, kFsNSS, true>(x, packed, gamma, M, N,
                                                                          K, cap, y, acc, s);
    }
    if (N >= kWideN) {
        // one token: two row groups per block halve the per-block work of
        // reading and quantising x (32768 x 4096: 11.4 -> 10.8 us 2-bit,
        // 11.3 -> 9.9 us 1-bit; four groups or eight waves were slower)
        return launch_linear_m<LAYOUT, 1, 4, 4, false, XT, YT, 2>(x, packed, gamma, M, N, K,
                                                                  (N + 31) / 32, y, acc, s);
    }
    if (M == 1) {
        // a round is 64 units for every launch shape below (KS * NSS = 16)
        const bool one_round =
            row_bytes_of(LAYOUT, K) / SkinnyCfg<LAYOUT>::kUnitBytes <= (int64_t)kFdKS * kFdNSS * 4;
        const int64_t cus = device_cu_count();
        if (one_round && cus > 0 && tiles > cus)
            return launch_linear_m<LAYOUT, 1, 4, 4, false>(x, packed, gamma, M, N, K, tiles, y,
                                                           acc, s);
        if (!one_round && cus > 0 && tiles <= cus)
            return launch_linear_m<LAYOUT, 1, kOneKS, kOneNSS, false>(x, packed, gamma, M, N, K,
                                                                      tiles, y, acc, s);
        return launch_linear_m<LAYOUT, 1, kFdKS, kFdNSS, false>(x, packed, gamma, M, N, K, tiles,
                                                                y, acc, s);
    }
    return launch_linear_m<LAYOUT, kFusedMaxM, kFdKS, kFdNSS, false>(x, packed, gamma, M, N, K,
                                                                     tiles, y, acc, s);
}

template <int LAYOUT, typename XT>
hipError_t launch_linear_x(const XT *x, const uint8_t *packed, const GammaMap &gamma, int64_t M,
                           int64_t N, int64_t K, void *y, int y_dtype, int32_t *acc,
                           hipStream_t s) {
    if (y_dtype == kF32)
        return launch_linear_t<LAYOUT>(x, packed, gamma, M, N, K, static_cast<float *>(y), acc, s);
    return launch_linear_t<LAYOUT>(x, packed, gamma, M, N, K, static_cast<uint16_t *>(y), acc, s);
}

template <int LAYOUT>
hipError_t skinny_y(const int8_t *xq, const float *scale, const uint8_t *packed,
                    const GammaMap &gamma, int64_t M, int64_t N, int64_t K, void *y, int y_dtype,
                    int32_t *acc, hipStream_t stream) {
    if (y_dtype == kF32)
        return launch_skinny_l<LAYOUT>(xq, scale, packed, gamma, M, N, K, static_cast<float *>(y),
                                       acc, stream);
    return launch_skinny_l<LAYOUT>(xq, scale, packed, gamma, M, N, K, static_cast<uint16_t *>(y),
                                   acc, stream);
}

template <int LAYOUT>
hipError_t linear_xy(const void *x, int x_dtype, const uint8_t *packed, const GammaMap &gamma,
                     int64_t M, int64_t N, int64_t K, void *y, int y_dtype, int32_t *acc,
                     hipStream_t stream) {
    if (x_dtype == kF32)
        return launch_linear_x<LAYOUT>(static_cast<const float *>(x), packed, gamma, M, N, K, y,
                                       y_dtype, acc, stream);
    return launch_linear_x<LAYOUT>(static_cast<const uint16_t *>(x), packed, gamma, M, N, K, y,
                                   y_dtype, acc, stream);
}

}  // namespace

hipError_t launch_forward_skinny(const int8_t *xq, const float *scale, const uint8_t *packed,
                                 int layout, const GammaMap &gamma, int64_t M, int64_t N, int64_t K,
                                 void *y, int y_dtype, int32_t *acc, hipStream_t stream) {
    switch (layout) {
        case kLayout2Bit:
            return skinny_y<kLayout2Bit>(xq, scale, packed, gamma, M, N, K, y, y_dtype, acc,
                                         stream);
        case kLayoutBase3:
            return skinny_y<kLayoutBase3>(xq, scale, packed, gamma, M, N, K, y, y_dtype, acc,
                                          stream);
        default:
            return skinny_y<kLayout1Bit>(xq, scale, packed, gamma, M, N, K, y, y_dtype, acc,
                                         stream);
    }
}

int64_t fused_decode_max_m() { return kFusedMaxM; }

// Batches above 16 tokens stream the weights once per 16-token chunk (all
// chunks in one launch). That beats the tiled GEMM for a few chunks: with few
// token tiles the GEMM keeps few blocks busy, each walking all of K, and long
// rows (K >= 8192) favour the chunks further. Crossovers measured on MI355X
// with the weights streamed from HBM (K = 4096 and 11008, N = 4096 to 32768):
// 2-bit and 1-bit up to 3 chunks at any N, 6 at N <= 8192, 8 for long rows at
// N <= 16384; base-3, whose decode costs more per byte, up to 3 chunks at
// N <= 16384 and 5 at N <= 4096.
bool skinny_handles(int64_t M, int64_t N, int64_t K, int layout) {
    if (M <= kSkinnyMaxM) return true;
    const int64_t chunks = (M + kSkinnyMaxM - 1) / kSkinnyMaxM;
    if (layout == kLayoutBase3) return (N <= 4096 && chunks <= 5) || (N <= 16384 && chunks <= 3);
    return chunks <= 3 || (N <= 8192 && chunks <= 6) || (K >= 8192 && N <= 16384 && chunks <= 8);
}

hipError_t launch_linear_decode(const void *x, int x_dtype, const uint8_t *packed, int layout,
                                const GammaMap &gamma, int64_t M, int64_t N, int64_t K, void *y,
                                int y_dtype, int32_t *acc, hipStream_t stream) {
    switch (layout) {
        case kLayout2Bit:
            return linear_xy<kLayout2Bit>(x, x_dtype, packed, gamma, M, N, K, y, y_dtype, acc,
                                          stream);
        case kLayoutBase3:
            return linear_xy<kLayoutBase3>(x, x_dtype, packed, gamma, M, N, K, y, y_dtype, acc,
                                           stream);
        default:
            return linear_xy<kLayout1Bit>(x, x_dtype, packed, gamma, M, N, K, y, y_dtype, acc,
                                          stream);
    }
}

}  // namespace bl
