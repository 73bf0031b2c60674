// Prefill-side product (M > 16 tokens): a tiled INT8 matrix-core GEMM.
// Every product term is an INT8 activation times a code in {-1, 0, +1},
// summed exactly in INT32 ([b158] "BitNet b1.58深度解析" §3.3 and §4.2), then
// scaled by gamma * scale[m] / 127 in the epilogue ([b158] §5.2-5.3). The
// instruction is v_mfma_i32_32x32x32_i8.
//
// Data flow. Activations (int8) are staged through LDS, double buffered.
// Packed weight codes never touch LDS: each wave loads the packed units of
// its own fragment columns straight from global memory (L2) and expands them
// in registers to signed code bytes. A unit is 16 bytes (64 codes in the
// 2-bit layout, 80 in base-3) or 8 bytes (64 codes in the 1-bit layout). The
// k slots of an MFMA are a free choice as long as both operands agree, so
// within one k-tile of two units per weight row (128 or 160 codes) lane group
// g (lanes 32g..32g+31) takes unit g, and MFMA k-step s takes codes
// [UC*g + 16 s, +16) of the tile for that lane group (UC = codes per unit);
// one load then feeds all 4 (5) k-steps of the tile, and the activation
// operand is read from LDS at the same offsets.
//
// Block tile BM tokens x BN weight rows, WM x WN waves, each owning
// (BM/WM) x (BN/WN) outputs as 32 x 32 fragments. Loads run two k-tiles ahead
// through two register sets; one barrier per k-tile. For long rows over few
// tiles, KG groups of WM x WN waves split a tile's k-tiles and add their
// INT32 sums through LDS before the epilogue. Blocks are mapped to
// tiles so that each of the eight XCDs (dispatched round-robin by block id)
// works on a contiguous run of tiles sharing activation rows in its L2.
#include "bl_internal.hpp"
#include "device_util.hpp"

#include <type_traits>

namespace bl {
namespace {

constexpr int kXcds = 8;

// How a launch treats the ends of its rows, fixed per launch:
//  kWholeK   K % 16 == 0, every k-tile holds two whole units and (1-bit)
//            rows carry no padding codes: loads need no guard;
//  kGuardedK K % 16 == 0 otherwise: the last k-tile's data past K is zeroed
//            where it is consumed;
//  kRaggedK  K % 16 != 0: activation rows are read byte-wise.
constexpr int kWholeK = 0, kGuardedK = 1, kRaggedK = 2;
inline int gemm_k_mode(int layout, int64_t K) {
    if (K % 16 != 0) return kRaggedK;
    const int64_t units = row_bytes_of(layout, K) / (layout == kLayout1Bit ? 8 : 16);
    const int64_t unit_codes = layout == kLayoutBase3 ? 80 : 64;
    if (units % 2 != 0 || (layout == kLayout1Bit && K != units * unit_codes)) return kGuardedK;
    return kWholeK;
}

template <int LAYOUT, int BM_, int BN_, int WM_, int WN_, int DIST_, int KG_ = 1>
struct GemmCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int DIST = DIST_;  // k-tiles the global loads run ahead (1, 2 or 4)
    static constexpr int KG = KG_;      // k-groups: wave groups splitting the k-tiles
    static constexpr int kGroupThreads = 64 * WM * WN;
    static constexpr int kThreads = kGroupThreads * KG;
    static constexpr int UC = LAYOUT == kLayoutBase3 ? 80 : 64;  // codes per unit
    static constexpr int LB = LAYOUT == kLayout1Bit ? 8 : 16;     // bytes per unit
    static constexpr int BK = 2 * UC;                             // codes per k-tile
    static constexpr int LDSK = BK + 16;                          // padded LDS row (bytes)
    static constexpr int KSTEPS = UC / 16;                        // MFMA k-steps per tile
    // A tile in 16-byte chunks, dealt round-robin over the group's threads;
    // when they do not divide evenly the last chunk slot of some threads is
    // empty (base-3's 160-code k-tile over one row of waves)
    static constexpr int ACHUNKS = BM * BK / 16;
    static constexpr int ACH = (ACHUNKS + kGroupThreads - 1) / kGroupThreads;
    static constexpr bool A_EVEN = ACHUNKS % kGroupThreads == 0;
    static constexpr int FI = BM / WM / 32, FJ = BN / WN / 32;    // fragments per wave
    static constexpr int STAGE = BM * LDSK;
    static constexpr int LUT = LAYOUT == kLayoutBase3 ? 8192 : 0;
    // each k-group stages its own tiles; afterwards groups 1..KG-1 hand their
    // INT32 tile to group 0 through the same memory
    static constexpr int STAGES = KG * 2 * STAGE, RED = (KG - 1) * BM * BN * 4;
    // bf16 tiles leave through LDS one row of waves at a time (BM / WM rows)
    static constexpr int OUT = (BM / WM) * (BN * 2 + 16);
    static constexpr int SMEM0 = STAGES > RED ? STAGES : RED;
    static constexpr int SMEM = LUT + (SMEM0 > OUT ? SMEM0 : OUT);
    static_assert(DIST == 1 || DIST == 2 || DIST == 4, "register sets: 1, 2 or 4");
};

// Expand one packed 16-byte unit into UC code bytes (natural order).
template <int LAYOUT>
__device__ __forceinline__ void expand_unit(const uint4 wv, const uint64_t *lut, int c[20]) {
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

// One unit of packed codes (16 bytes; 8 bytes in the 1-bit layout).
template <int LAYOUT>
__device__ __forceinline__ uint4 load_b(const uint8_t *p) {
    if constexpr (LAYOUT == kLayout1Bit) {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        return make_uint4(v.x, v.y, 0u, 0u);
    } else {
        return *reinterpret_cast<const uint4 *>(p);
    }
}

// One product over a column range of the packed matrix: y[:, 0:N] (row stride
// ldy) from packed rows 0..N-1.
template <typename YT>
struct GemmArgs {
    const int8_t *xq;
    const float *scale;
    const uint8_t *packed;
    GammaMap gm;
    int64_t M, N, K, rb;
    int tiles_m, tiles_n;
    YT *y;
    int64_t ldy;
    int32_t *acc_out;
    int band;  // row tiles per band of the tile order (tile_band); 0 or 1: row by row
};

// Tile order: bands of `band` row tiles, each band walked column by column
// (band 1 is plain row order). The 32 CUs of an XCD run up to 32
// consecutive tiles at once; in bands of a row tiles those cover a row tiles
// by run / a column tiles. For tiles that read a_bytes of activations and
// b_bytes of weights, the band (1, 2, 4 or 8) that minimises the bytes
// such a run reads through the XCD's L2 is taken (ties keep the smaller
// band). Measured on MI355X: 512 x 4096 x 4096 in 64 x 64 tiles 17.4 ->
// 16.0 us, 256 x 11008 x 4096 25.1 -> 23.7 us, the base-3 prefill GEMM
// 136 -> 132 us; the 2-bit prefill unchanged.
inline int tile_band(int tm, int tn, int64_t a_bytes, int64_t b_bytes) {
    constexpr int64_t kCusPerXcd = 32;
    const int64_t share = ((int64_t)tm * tn + kXcds - 1) / kXcds;
    const int64_t run = share < kCusPerXcd ? share : kCusPerXcd;
    int best = 1;
    int64_t best_cost = INT64_MAX;
    for (int a = 1; a <= tm && a <= 8; a *= 2) {
        int64_t rows, cols;
        if (run <= (int64_t)a * tn) {
            rows = run < a ? run : a;
            cols = (run + a - 1) / a;
        } else {
            rows = (run + tn - 1) / tn;
            cols = tn;
        }
        const int64_t cost = rows * a_bytes + cols * b_bytes;
        if (cost < best_cost) best_cost = cost, best = a;
    }
    return best;
}

// Block b of nblocks -> tile index: each of the eight XCDs (dispatched
// round-robin by block id) gets a contiguous run of tiles in the tile order
// above, which share activation rows and weight rows in its L2. -1 past the
// last tile.
__device__ __forceinline__ int xcd_tile(int b, int ntiles) {
    const int per_xcd = (ntiles + kXcds - 1) / kXcds;
    const int t = (b % kXcds) * per_xcd + b / kXcds;
    return t < ntiles ? t : -1;
}

template <int LAYOUT, int BM, int BN, int WM, int WN, int DIST, int KG, int KMODE,
          typename YT>
__device__ __forceinline__ void gemm_tile(const GemmArgs<YT> &g, int t) {
    using C = GemmCfg<LAYOUT, BM, BN, WM, WN, DIST, KG>;
    constexpr bool EVEN_K = KMODE != kRaggedK;  // K % 16 == 0
    constexpr int kThreads = C::kThreads;
    constexpr int kGT = C::kGroupThreads;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint64_t *lut = reinterpret_cast<uint64_t *>(smem);
    const int8_t *__restrict__ xq = g.xq;
    const float *__restrict__ scale = g.scale;
    const uint8_t *__restrict__ packed = g.packed;
    const GammaMap &gm = g.gm;
    const int64_t M = g.M, N = g.N, K = g.K, rb = g.rb, ldy = g.ldy;
    const int tiles_n = g.tiles_n;
    YT *__restrict__ y = g.y;
    int32_t *__restrict__ acc_out = g.acc_out;

    int tr = t / tiles_n, tc = t % tiles_n;
    if (g.band > 1) {
        // bands of g.band row tiles, each walked column by column
        const int per_band = g.band * tiles_n;
        const int b0 = t / per_band, idx = t - b0 * per_band;
        const int rows = min(g.band, g.tiles_m - b0 * g.band);
        tr = b0 * g.band + idx % rows;
        tc = idx / rows;
    }
    const int64_t m0 = (int64_t)tr * BM;
    const int64_t n0 = (int64_t)tc * BN;

    const int tid = threadIdx.x;
    // k-group kg (a run of whole waves, so kg is wave-uniform) and the
    // thread's place within its group
    const int kg = KG == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid / kGT);
    const int gtid = KG == 1 ? tid : tid % kGT;
    const int wave = gtid / 64, lane = tid % 64;
    const int wm = wave / WN, wn = wave % WN;
    int8_t *stage0 = reinterpret_cast<int8_t *>(smem + C::LUT) + kg * 2 * C::STAGE;
    const int frow = lane % 32;  // fragment row (A) / column (B)
    const int lg = lane / 32;    // lane group: packed unit within the k-tile

    if (LAYOUT == kLayoutBase3) {
        for (int i = tid; i < 4 * 256; i += kThreads)
            lut[i] = base3_entry((uint32_t)(i % 256)) << (8 * (i / 256));
    }

    const int64_t units = rb / C::LB;
    const int64_t ktiles = (units + 1) / 2;
    // this lane's weight rows (one per fragment column block)
    const uint8_t *b_src[C::FJ];
#pragma unroll
    for (int j = 0; j < C::FJ; ++j) {
        const int64_t n = n0 + wn * (BN / WN) + j * 32 + frow;
        b_src[j] = packed + (n < N ? n : 0) * rb;
    }

    v4i a_regs[DIST][C::ACH];
    uint4 b_regs[DIST][C::FJ];

    // Launches whose rows hold whole k-tiles (k-mode kWholeK, see
    // gemm_k_mode) load without guards: the k-tile index is clamped, so the
    // prefetches past the last tile re-read a valid tile whose data is never
    // used, and token rows past M re-read row M - 1 (weight rows past N read
    // row 0): each output depends only on its own token and weight row, so
    // those rows only feed outputs that are never stored. Guarded launches
    // (data past K in the last k-tile) read the same valid addresses and zero
    // what lies past K where it is consumed, so no branch or select splits the
    // load stream and the compiler keeps all of a tile's loads in flight. Rows
    // that are not a multiple of 16 bytes load dwords (K % 4 == 0) or bytes.
    auto load_tile = [&](int64_t kt, v4i *a_reg, uint4 *b_reg, auto guard_c) {
        constexpr bool G = decltype(guard_c)::value;
        if (!G) kt = kt < ktiles ? kt : ktiles - 1;
        const int64_t kc0 = kt * C::BK;
#pragma unroll
        for (int i = 0; i < C::ACH; ++i) {
            const int q = gtid + i * kGT;
            if (!C::A_EVEN && i == C::ACH - 1 && q >= C::ACHUNKS) continue;
            const int row = q / (C::BK / 16), col = q % (C::BK / 16);
            const int64_t m = m0 + row, k = kc0 + col * 16;
            if (!G || EVEN_K) {
                // (a chunk is wholly below or above K: K % 16 == 0 here;
                // guarded tiles zero the chunks past K in store_a)
                const int64_t mr = m < M ? m : M - 1;
                a_reg[i] = *reinterpret_cast<const v4i *>(xq + mr * K + (k < K ? k : 0));
            } else if (K % 4 == 0) {
                // rows 4-byte aligned: four dword loads; dwords past K read
                // the row's first one and are zeroed in store_a
                const int64_t mr = m < M ? m : M - 1;
                const int32_t *p = reinterpret_cast<const int32_t *>(xq + mr * K);
                v4i v;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const int64_t kd = k + 4 * d;
                    v[d] = p[(kd < K ? kd : 0) / 4];
                }
                a_reg[i] = v;
            } else {
                v4i v = {0, 0, 0, 0};
                if (m < M && k < K) {
                    const int8_t *p = xq + m * K;
                    uint32_t d[4] = {0u, 0u, 0u, 0u};
                    for (int e = 0; e < 16; ++e)
                        if (k + e < K) d[e / 4] |= (uint32_t)(uint8_t)p[k + e] << (8 * (e % 4));
                    v = v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
                }
                a_reg[i] = v;
            }
        }
        const int64_t unit = kt * 2 + lg;
#pragma unroll
        for (int j = 0; j < C::FJ; ++j) {
            // guarded tiles read the row's first unit in place of units past
            // the end and zero them before the multiply
            const int64_t u = G && unit >= units ? 0 : unit;
            b_reg[j] = load_b<LAYOUT>(b_src[j] + u * C::LB);
        }
    };

    // Stage the activation registers of k-tile kt in LDS. Guarded tiles zero
    // the chunks (dwords, for 4-byte rows) past K here, where the values are
    // consumed (a select at the load would make the compiler wait for it).
    auto store_a = [&](int8_t *As, const v4i *a_reg, int64_t kt, auto guard_c) {
        constexpr bool Z = decltype(guard_c)::value && EVEN_K;
#pragma unroll
        for (int i = 0; i < C::ACH; ++i) {
            const int q = gtid + i * kGT;
            if (!C::A_EVEN && i == C::ACH - 1 && q >= C::ACHUNKS) continue;
            const int row = q / (C::BK / 16), col = q % (C::BK / 16);
            v4i v = a_reg[i];
            const int64_t kb = kt * C::BK + col * 16;
            if constexpr (Z) {
                if (kb >= K) v = v4i{0, 0, 0, 0};
            }
            if constexpr (KMODE == kRaggedK) {  // the dword path of load_tile
                if (K % 4 == 0) {
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        if (kb + 4 * d >= K) v[d] = 0;
                }
            }
            *reinterpret_cast<v4i *>(As + row * C::LDSK + col * 16) = v;
        }
    };
    // Guarded tiles: weight units past the row's end multiply as zero codes.
    auto zero_units = [&](uint4 (&bu)[C::FJ], int64_t kt, auto guard_c) {
        if constexpr (decltype(guard_c)::value) {
            if (kt * 2 + lg >= units) {
#pragma unroll
                for (int j = 0; j < C::FJ; ++j) bu[j] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };

    v16i acc[C::FI][C::FJ];
#pragma unroll
    for (int i = 0; i < C::FI; ++i)
#pragma unroll
        for (int j = 0; j < C::FJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    // The loop is unrolled by U steps so that LDS buffers and register sets
    // are static and the compiler can wait for exactly the loads a step
    // consumes. With one group the body is free of branches: pairs of steps,
    // then one last step when the k-tile count is odd. Loads of tiles past
    // the end read valid addresses and are never multiplied.
    //
    // With k-groups, group kg takes the k-tiles [k_lo, k_hi) of an equal
    // share. Every group runs the same number of steps, so the barriers
    // match; steps past a group's share (and, with four register sets, past
    // the end) skip the multiply, a wave-uniform branch, and their loads read
    // valid addresses.
    constexpr int U = DIST > 2 ? DIST : 2;
    constexpr bool kSkip = KG > 1 || DIST > 2;
    int64_t k_lo = 0, k_hi = ktiles, kt_end = ktiles;
    if constexpr (kSkip) {
        const int64_t share = (ktiles + KG - 1) / KG;
        k_lo = kg * share;
        k_hi = k_lo + share < ktiles ? k_lo + share : ktiles;
        kt_end = k_lo + (share + U - 1) / U * U;
    }

    // Multiply the k-tile in LDS buffer As by the weight units bu (one per
    // fragment column block). 2-bit: k-step ks consumes exactly word ks of a
    // unit, expanded just before use (4 live registers per column block).
    // Base-3: a unit's five trits per byte straddle k-steps, so the whole
    // unit is expanded first.
    auto mma = [&](const int8_t *As, const uint4 (&bu)[C::FJ]) {
        int cb[LAYOUT == kLayoutBase3 ? C::FJ : 1][20];
        if constexpr (LAYOUT == kLayoutBase3) {
#pragma unroll
            for (int j = 0; j < C::FJ; ++j) expand_unit<LAYOUT>(bu[j], lut, cb[j]);
        }
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            v4i a[C::FI];
#pragma unroll
            for (int i = 0; i < C::FI; ++i)
                a[i] = *reinterpret_cast<const v4i *>(
                    As + (wm * (BM / WM) + i * 32 + frow) * C::LDSK + lg * C::UC + ks * 16);
#pragma unroll
            for (int j = 0; j < C::FJ; ++j) {
                v4i bj;
                if constexpr (LAYOUT == kLayout2Bit) {
                    const uint32_t w = ks == 0 ? bu[j].x : ks == 1 ? bu[j].y : ks == 2 ? bu[j].z
                                                                                     : bu[j].w;
                    int c[4];
                    expand_2bit_word(w, c);
                    bj = v4i{c[0], c[1], c[2], c[3]};
                } else if constexpr (LAYOUT == kLayout1Bit) {
                    // k-step ks: codes 16 ks .. +15 of the unit = half ks % 2
                    // of word ks / 2
                    int c[4];
                    expand_1bit_half(ks < 2 ? bu[j].x : bu[j].y, ks % 2, c);
                    bj = v4i{c[0], c[1], c[2], c[3]};
                } else {
                    bj = v4i{cb[j][4 * ks], cb[j][4 * ks + 1], cb[j][4 * ks + 2],
                             cb[j][4 * ks + 3]};
                }
                // weights as the row operand: D[n][m], so each lane ends up
                // holding four consecutive output columns per register quad
#pragma unroll
                for (int i = 0; i < C::FI; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bj, a[i], acc[i][j], 0, 0,
                                                                      0);
            }
        }
    };

    auto run = [&](auto guard_c) {
        if constexpr (DIST >= 2) {
            // LDS holds tiles kt and kt+1; registers hold kt+1 (arrived) up to
            // kt+DIST (in flight). Register set S = (kt - k_lo) % DIST holds
            // tile kt, LDS buffer S % 2.
#pragma unroll
            for (int d = 0; d < DIST; ++d) load_tile(k_lo + d, a_regs[d], b_regs[d], guard_c);
            store_a(stage0, a_regs[0], k_lo, guard_c);
            __syncthreads();  // tile k_lo (and the decode table) ready
            auto step = [&](int64_t kt, auto set_c) {
                constexpr int S = decltype(set_c)::value;
                constexpr int L = S % 2;
                uint4 bu[C::FJ];
    #pragma unroll
                for (int j = 0; j < C::FJ; ++j) bu[j] = b_regs[S][j];
                load_tile(kt + DIST, a_regs[S], b_regs[S], guard_c);
                zero_units(bu, kt, guard_c);
                if (!kSkip || kt < k_hi) mma(stage0 + L * C::STAGE, bu);
                store_a(stage0 + (L ^ 1) * C::STAGE, a_regs[(S + 1) % DIST], kt + 1, guard_c);
                lds_barrier();
            };
            if constexpr (kSkip) {
                for (int64_t kt = k_lo; kt < kt_end; kt += U) {
                    step(kt, std::integral_constant<int, 0>{});
                    step(kt + 1, std::integral_constant<int, 1 % DIST>{});
                    if constexpr (U == 4) {
                        step(kt + 2, std::integral_constant<int, 2 % DIST>{});
                        step(kt + 3, std::integral_constant<int, 3 % DIST>{});
                    }
                }
            } else {
                int64_t kt = k_lo;
                for (; kt + 1 < k_hi; kt += 2) {
                    step(kt, std::integral_constant<int, 0>{});
                    step(kt + 1, std::integral_constant<int, 1>{});
                }
                if (kt < k_hi) step(kt, std::integral_constant<int, 0>{});
            }
        } else {
            // LDS holds tiles kt and kt+1; one register set carries tile kt+1.
            load_tile(k_lo, a_regs[0], b_regs[0], guard_c);
            store_a(stage0, a_regs[0], k_lo, guard_c);
            __syncthreads();
            auto step = [&](int64_t kt, auto buf_c) {
                constexpr int S = decltype(buf_c)::value;
                uint4 bu[C::FJ];
    #pragma unroll
                for (int j = 0; j < C::FJ; ++j) bu[j] = b_regs[0][j];
                load_tile(kt + 1, a_regs[0], b_regs[0], guard_c);
                zero_units(bu, kt, guard_c);
                if (!kSkip || kt < k_hi) mma(stage0 + S * C::STAGE, bu);
                store_a(stage0 + (S ^ 1) * C::STAGE, a_regs[0], kt + 1, guard_c);
                lds_barrier();
            };
            if constexpr (kSkip) {
                for (int64_t kt = k_lo; kt < kt_end; kt += 2) {
                    step(kt, std::integral_constant<int, 0>{});
                    step(kt + 1, std::integral_constant<int, 1>{});
                }
            } else {
                int64_t kt = k_lo;
                for (; kt + 1 < k_hi; kt += 2) {
                    step(kt, std::integral_constant<int, 0>{});
                    step(kt + 1, std::integral_constant<int, 1>{});
                }
                if (kt < k_hi) step(kt, std::integral_constant<int, 0>{});
            }
        }

    };
    // The k-mode is fixed per launch (gemm_k_mode), so each kernel holds one
    // load path and its registers are allocated for that path alone.
    run(std::integral_constant<bool, KMODE != kWholeK>{});

    if constexpr (KG > 1) {
        // Groups 1..KG-1 hand their INT32 sums to group 0 through LDS (free
        // again: the last step ended on a barrier), one 64-lane row per
        // accumulator register, so the accesses are conflict-free. The sums
        // are exact, so the split does not change any result.
        constexpr int kRegs = C::FI * C::FJ * 16;
        int32_t *red = reinterpret_cast<int32_t *>(smem + C::LUT);
        if (kg > 0) {
            int32_t *dst = red + ((kg - 1) * (WM * WN) + wave) * kRegs * 64 + lane;
#pragma unroll
            for (int i = 0; i < C::FI; ++i)
#pragma unroll
                for (int j = 0; j < C::FJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) dst[((i * C::FJ + j) * 16 + r) * 64] = acc[i][j][r];
        }
        lds_barrier();
        if (kg > 0) return;
        for (int h = 1; h < KG; ++h) {
            const int32_t *src = red + ((h - 1) * (WM * WN) + wave) * kRegs * 64 + lane;
#pragma unroll
            for (int i = 0; i < C::FI; ++i)
#pragma unroll
                for (int j = 0; j < C::FJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] += src[((i * C::FJ + j) * 16 + r) * 64];
        }
    }

    // Epilogue. Fragment (i, j) register r of lane l holds D[n][m] with
    // m = l % 32 (token within fragment i) and n = 8 (r / 4) + 4 (l / 32) +
    // r % 4 (weight row within fragment j): registers 4q..4q+3 are four
    // consecutive outputs of one token, written with one 8- or 16-byte store.
    // One matrix: f = gamma * scale[m] / 127 per token. Stacked segments:
    // each output scales by its row's gamma times scale[m] / 127.
    float gs[kMaxSegments];
    load_gammas(gm, gs);
    const bool one = gm.nseg == 1;
    const bool full = m0 + BM <= M && n0 + BN <= N && (ldy % 4) == 0;
    if constexpr (sizeof(YT) == 2 && KG == 1 && BN >= 128) {
        if (full && one && (ldy % 8) == 0) {
            // Whole bf16 tiles of one matrix leave through LDS, one row of
            // waves at a time:
            // those waves write their outputs into the (now free) staging
            // memory, then every thread stores 16-byte pieces of whole output
            // rows, so each global store fills complete cache lines instead of
            // scattering 8-byte pieces over 32 rows. Values and rounding are
            // those of the direct stores. (Measured: 4096^3 68.7 -> 64.7 us;
            // the narrow 128 x 64 tiles were slower this way and keep the
            // direct stores.)
            constexpr int RS = BN * 2 + 16;  // LDS bytes per output row (padded)
            static_assert((BM / WM) * RS <= C::SMEM - C::LUT, "half tile fits the staging LDS");
            uint8_t *ot = smem + C::LUT;
            for (int h = 0; h < WM; ++h) {
                if (wm == h) {
#pragma unroll
                    for (int i = 0; i < C::FI; ++i) {
                        const int64_t m = m0 + wm * (BM / WM) + i * 32 + frow;
                        const float f1 = gs[0] * scale[m] / 127.0f;
#pragma unroll
                        for (int j = 0; j < C::FJ; ++j) {
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const int nl = wn * (BN / WN) + j * 32 + 8 * q + 4 * lg;
                                const int64_t n = n0 + nl;
                                const int32_t a0 = acc[i][j][4 * q], a1 = acc[i][j][4 * q + 1];
                                const int32_t a2 = acc[i][j][4 * q + 2], a3 = acc[i][j][4 * q + 3];
                                const bf16x2 lo = {(__bf16)((float)a0 * f1), (__bf16)((float)a1 * f1)};
                                const bf16x2 hi = {(__bf16)((float)a2 * f1), (__bf16)((float)a3 * f1)};
                                *reinterpret_cast<uint2 *>(ot + (i * 32 + frow) * RS + nl * 2) =
                                    make_uint2(__builtin_bit_cast(uint32_t, lo),
                                               __builtin_bit_cast(uint32_t, hi));
                                if (acc_out)
                                    *reinterpret_cast<int4 *>(acc_out + m * ldy + n) =
                                        make_int4(a0, a1, a2, a3);
                            }
                        }
                    }
                }
                lds_barrier();
                constexpr int kPieces = (BM / WM) * (BN / 8);  // 16-byte pieces
                for (int c = tid; c < kPieces; c += kThreads) {
                    const int row = c / (BN / 8), pc = c % (BN / 8);
                    const uint4 v = *reinterpret_cast<const uint4 *>(ot + row * RS + pc * 16);
                    *reinterpret_cast<uint4 *>(y + (m0 + h * (BM / WM) + row) * ldy + n0 +
                                               pc * 8) = v;
                }
                lds_barrier();  // the next row of waves reuses the memory
            }
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < C::FI; ++i) {
        const int64_t m = m0 + wm * (BM / WM) + i * 32 + frow;
        const float sm = scale[m < M ? m : 0];
        const float f1 = gs[0] * sm / 127.0f;
        const float sm127 = sm / 127.0f;
#pragma unroll
        for (int j = 0; j < C::FJ; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = n0 + wn * (BN / WN) + j * 32 + 8 * q + 4 * lg;
                const int32_t a0 = acc[i][j][4 * q], a1 = acc[i][j][4 * q + 1];
                const int32_t a2 = acc[i][j][4 * q + 2], a3 = acc[i][j][4 * q + 3];
                float f[4] = {f1, f1, f1, f1};
                if (!one) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) f[e] = seg_gamma(gm, gs, n + e) * sm127;
                }
                const float v0 = (float)a0 * f[0], v1 = (float)a1 * f[1];
                const float v2 = (float)a2 * f[2], v3 = (float)a3 * f[3];
                if (full) {
                    if constexpr (sizeof(YT) == 4) {
                        *reinterpret_cast<float4 *>(y + m * ldy + n) = make_float4(v0, v1, v2, v3);
                    } else {
                        const bf16x2 lo = {(__bf16)v0, (__bf16)v1};
                        const bf16x2 hi = {(__bf16)v2, (__bf16)v3};
                        *reinterpret_cast<uint2 *>(y + m * ldy + n) =
                            make_uint2(__builtin_bit_cast(uint32_t, lo),
                                       __builtin_bit_cast(uint32_t, hi));
                    }
                    if (acc_out)
                        *reinterpret_cast<int4 *>(acc_out + m * ldy + n) = make_int4(a0, a1, a2, a3);
                } else if (m < M) {
                    const int32_t av[4] = {a0, a1, a2, a3};
                    const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (n + e >= N) continue;
                        if constexpr (sizeof(YT) == 4)
                            y[m * ldy + n + e] = vv[e];
                        else
                            y[m * ldy + n + e] = (YT)f32_to_bf16_rne(vv[e]);
                        if (acc_out) acc_out[m * ldy + n + e] = av[e];
                    }
                }
            }
        }
    }
}

template <int LAYOUT, int BM, int BN, int WM, int WN, int DIST, int KG, int KMODE,
          typename YT>
__global__ __launch_bounds__(64 * WM * WN * KG) void gemm_kernel(const GemmArgs<YT> g) {
    const int t = xcd_tile(blockIdx.x, g.tiles_m * g.tiles_n);
    if (t < 0) return;
    gemm_tile<LAYOUT, BM, BN, WM, WN, DIST, KG, KMODE, YT>(g, t);
}

// BM x 256 tiles (BM = 256, 128 or 96) of 2-bit or 1-bit rows of whole k-tiles,
// bf16 out, tiles whole in N: the activation tile reaches LDS by direct-to-LDS
// loads (16 bytes a lane, no staging registers), three k-tiles deep, and the
// registers this frees hold the next k-step's activation fragments while the
// current one is multiplied. One row of eight waves as in gemm_tile (BM x 32
// each), weights expanded in registers the same way; the sums are identical.
//
// - Three LDS stages, each its own array (dma_lds). The compiler waits for
//   every outstanding direct-to-LDS load before an LDS read that may alias it;
//   reads of one array are not held up by loads into another. Every kernel
//   that runs these tiles shares the same arrays (the one-launch pair runs two
//   tile heights).
// - A wave's direct-to-LDS write is 1 KiB contiguous (lane l at 16 l), i.e.
//   eight activation rows of 128 bytes with no padding. To keep the fragment
//   reads free of bank conflicts, lane l loads chunk (l % 8) ^ ((row / 2) % 8)
//   of its row, and readers look a chunk up at the same swizzled slot. Each
//   wave loads 32 rows (BM = 256) or 16 rows (BM <= 128; for BM = 96 the
//   last two waves load rows 96..127, which are never read). Rows past M
//   re-read row M - 1 and feed only outputs that are not stored.
// - Each step issues J direct-to-LDS loads and one weight load (J = 4 or 2),
//   after its first fragment reads and weight word. Before the step's barrier
//   a wave waits until at most J + 2 vector-memory operations are
//   outstanding: the weight load of the next k-tile and the J + 1 operations
//   of this step. That leaves the next k-tile's own activation loads done, so
//   the barrier publishes them to the other waves.
// - The output tile leaves through a fourth array, 64 rows at a time.
constexpr int kDmaStage = 256 * 128;  // one k-tile of activations, bytes
constexpr int kDmaOutRow = 256 * 2 + 16;
struct DmaLds {
    int8_t *s0, *s1, *s2;
    uint8_t *out;
};
// The arrays of the stages and the output staging, declared once (not per tile
// height) so that every kernel running these tiles shares them.
__device__ __forceinline__ DmaLds dma_lds() {
    __shared__ __attribute__((aligned(16))) int8_t s0[kDmaStage];
    __shared__ __attribute__((aligned(16))) int8_t s1[kDmaStage];
    __shared__ __attribute__((aligned(16))) int8_t s2[kDmaStage];
    __shared__ __attribute__((aligned(16))) uint8_t out[64 * kDmaOutRow];
    return DmaLds{s0, s1, s2, out};
}

template <int LAYOUT, int BM, bool SEG, typename YT>
__device__ __forceinline__ void gemm_tile_dma(const GemmArgs<YT> &g, int t) {
    static_assert(LAYOUT != kLayoutBase3 && sizeof(YT) == 2, "2-bit and 1-bit rows, bf16 out");
    static_assert(BM == 256 || BM == 128 || BM == 96, "tile heights");
    using C = GemmCfg<LAYOUT, BM, 256, 1, 8, 2>;
    constexpr int FI = BM / 32;              // fragments per wave
    constexpr int RPW = BM == 256 ? 32 : 16; // activation rows each wave loads
    constexpr int J = RPW / 8;               // direct-to-LDS loads per wave and k-tile
    const DmaLds lds = dma_lds();
    int8_t *const dma_s0 = lds.s0, *const dma_s1 = lds.s1, *const dma_s2 = lds.s2;
    uint8_t *const dma_out = lds.out;
    const int8_t *__restrict__ xq = g.xq;
    const float *__restrict__ scale = g.scale;
    const GammaMap &gm = g.gm;
    const int64_t M = g.M, K = g.K, rb = g.rb, ldy = g.ldy;
    const int tiles_n = g.tiles_n;
    YT *__restrict__ y = g.y;
    int32_t *__restrict__ acc_out = g.acc_out;

    int tr = t / tiles_n, tc = t % tiles_n;
    if (g.band > 1) {
        const int per_band = g.band * tiles_n;
        const int b0 = t / per_band, idx = t - b0 * per_band;
        const int rows = min(g.band, g.tiles_m - b0 * g.band);
        tr = b0 * g.band + idx % rows;
        tc = idx / rows;
    }
    const int64_t m0 = (int64_t)tr * BM, n0 = (int64_t)tc * 256;
    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int frow = lane % 32, lg = lane / 32;
    const int64_t ktiles = rb / C::LB / 2;  // whole k-tiles (the caller checks)

    // this lane's weight row and activation rows
    const uint8_t *bsrc = g.packed + (n0 + wave * 32 + frow) * rb;
    // (sized for the largest J: an array sized by J would make the load builtin's
    // arguments depend on BM, which the host compilation pass rejects)
    const int8_t *asrc[4];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int row = RPW * wave + 8 * j + lane / 8;
        const int64_t m = m0 + row;
        asrc[j] = xq + (m < M ? m : M - 1) * K + ((lane % 8) ^ ((row / 2) % 8)) * 16;
    }
    // k-tiles past the last re-read it (valid addresses; never multiplied)
    auto load_a = [&](int64_t kt, int8_t *S) {
        kt = kt < ktiles ? kt : ktiles - 1;
#pragma unroll
        for (int j = 0; j < J; ++j)
            __builtin_amdgcn_global_load_lds(asrc[j] + kt * 128,
                                             to_lds(S + (RPW * wave + 8 * j) * 128), 16, 0, 0);
    };
    uint4 breg[3];
    auto load_w = [&](int64_t kt, uint4 &r) {
        kt = kt < ktiles ? kt : ktiles - 1;
        r = load_b<LAYOUT>(bsrc + (kt * 2 + lg) * C::LB);
    };

    v16i acc[FI];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0;

    // fragment i, k-step ks of this lane: row 32 i + frow, chunk 4 lg + ks,
    // at the swizzled slot ((row / 2) % 8 does not depend on i)
    const int xs = (frow / 2) % 8;
    auto frag = [&](const int8_t *S, int i, int ks) {
        return *reinterpret_cast<const v4i *>(S + (i * 32 + frow) * 128 + ((4 * lg + ks) ^ xs) * 16);
    };
    auto expand = [&](const uint4 &bu, int ks, int (&c)[4]) {
        if constexpr (LAYOUT == kLayout2Bit) {
            expand_2bit_word(ks == 0 ? bu.x : ks == 1 ? bu.y : ks == 2 ? bu.z : bu.w, c);
        } else {
            expand_1bit_half(ks < 2 ? bu.x : bu.y, ks % 2, c);
        }
    };
    // One k-tile from stage S; `issue` sends the loads of k-tile kt + 2 after
    // the first fragment reads and weight word (a wait the compiler places
    // before those then covers only loads of earlier steps).
    auto step = [&](const int8_t *S, const uint4 &bu, auto issue) {
        v4i a[2][FI];
#pragma unroll
        for (int i = 0; i < FI; ++i) a[0][i] = frag(S, i, 0);
        int c0[4];
        expand(bu, 0, c0);
        __builtin_amdgcn_sched_barrier(0);
        issue();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4) {
#pragma unroll
                for (int i = 0; i < FI; ++i) a[(ks + 1) & 1][i] = frag(S, i, ks + 1);
            }
            // keeps the next k-step's reads ahead of this k-step's multiplies
            __builtin_amdgcn_sched_barrier(0);
            int c[4] = {c0[0], c0[1], c0[2], c0[3]};
            if (ks > 0) expand(bu, ks, c);
            const v4i bj = v4i{c[0], c[1], c[2], c[3]};
#pragma unroll
            for (int i = 0; i < FI; ++i)
                acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bj, a[ks & 1][i], acc[i], 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_only(J + 2));
        lds_barrier();
    };

    load_a(0, dma_s0);
    load_w(0, breg[0]);
    load_a(1, dma_s1);
    load_w(1, breg[1]);
    __builtin_amdgcn_s_waitcnt(vmcnt_only(J + 2));  // k-tile 0's activations
    lds_barrier();
    // k-tile kt sits in stage kt % 3 and weight set kt % 3
    int64_t kt = 0;
    for (; kt + 3 <= ktiles; kt += 3) {
        step(dma_s0, breg[0], [&]() { load_a(kt + 2, dma_s2); load_w(kt + 2, breg[2]); });
        step(dma_s1, breg[1], [&]() { load_a(kt + 3, dma_s0); load_w(kt + 3, breg[0]); });
        step(dma_s2, breg[2], [&]() { load_a(kt + 4, dma_s1); load_w(kt + 4, breg[1]); });
    }
    if (kt < ktiles)
        step(dma_s0, breg[0], [&]() { load_a(kt + 2, dma_s2); load_w(kt + 2, breg[2]); });
    if (kt + 1 < ktiles)
        step(dma_s1, breg[1], [&]() { load_a(kt + 3, dma_s0); load_w(kt + 3, breg[0]); });
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));  // no direct-to-LDS load outlives the block

    // Epilogue: y = acc * f as bf16; one matrix: f = gamma * scale[m] / 127;
    // stacked segments (SEG): f = gamma(n) * (scale[m] / 127). Rows 64 p ..
    // 64 p + 63 (fragments 2 p and 2 p + 1 of every wave) per pass. (A single
    // matrix has its own instantiation: the segment selection's registers
    // cost the main loop 2-3% at 4096^3.)
    float gs[SEG ? kMaxSegments : 1];
    if constexpr (SEG) load_gammas(gm, gs);
    else gs[0] = gm.g[0];
#pragma unroll
    for (int p = 0; p < (FI + 1) / 2; ++p) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int i = 2 * p + ii;
            if (i >= FI) break;
            const int64_t m = m0 + i * 32 + frow;
            const float sm = scale[m < M ? m : M - 1];
            const float f1 = gs[0] * sm / 127.0f;
            const float sm127 = sm / 127.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = wave * 32 + 8 * q + 4 * lg;
                const int32_t a0 = acc[i][4 * q], a1 = acc[i][4 * q + 1];
                const int32_t a2 = acc[i][4 * q + 2], a3 = acc[i][4 * q + 3];
                float f[4] = {f1, f1, f1, f1};
                if constexpr (SEG) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) f[e] = seg_gamma(gm, gs, n0 + nl + e) * sm127;
                }
                const bf16x2 lo = {(__bf16)((float)a0 * f[0]), (__bf16)((float)a1 * f[1])};
                const bf16x2 hi = {(__bf16)((float)a2 * f[2]), (__bf16)((float)a3 * f[3])};
                *reinterpret_cast<uint2 *>(dma_out + (ii * 32 + frow) * kDmaOutRow + nl * 2) =
                    make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
                if (acc_out && m < M)
                    *reinterpret_cast<int4 *>(acc_out + m * ldy + n0 + nl) = make_int4(a0, a1, a2, a3);
            }
        }
        lds_barrier();
        const int rows = FI - 2 * p >= 2 ? 64 : 32;
        for (int c = tid; c < rows * 32; c += 512) {  // 16-byte pieces of the pass's rows
            const int row = c / 32, pc = c % 32;
            const int64_t m = m0 + 64 * p + row;
            if (m < M) {
                const uint4 v = *reinterpret_cast<const uint4 *>(dma_out + row * kDmaOutRow + pc * 16);
                *reinterpret_cast<uint4 *>(y + m * ldy + n0 + pc * 8) = v;
            }
        }
        lds_barrier();
    }
}

template <int LAYOUT, int BM, bool SEG, typename YT>
__global__ __launch_bounds__(512) void gemm_dma_kernel(const GemmArgs<YT> g) {
    const int t = xcd_tile(blockIdx.x, g.tiles_m * g.tiles_n);
    if (t < 0) return;
    gemm_tile_dma<LAYOUT, BM, SEG, YT>(g, t);
}

// The prefill shape in one launch with the direct-to-LDS tiles: 256 x 256
// tiles over whole rounds, then BM2 x 256 tiles over the leftover columns.
template <int LAYOUT, int BM2, bool SEG, typename YT>
__global__ __launch_bounds__(512) void gemm_dma_pair_kernel(const GemmArgs<YT> g1, int blocks1,
                                                            const GemmArgs<YT> g2) {
    const int b = blockIdx.x;
    if (b < blocks1) {
        const int t = xcd_tile(b, g1.tiles_m * g1.tiles_n);
        if (t >= 0) gemm_tile_dma<LAYOUT, 256, SEG, YT>(g1, t);
    } else {
        const int t = xcd_tile(b - blocks1, g2.tiles_m * g2.tiles_n);
        if (t >= 0) gemm_tile_dma<LAYOUT, BM2, SEG, YT>(g2, t);
    }
}

// The direct-to-LDS tiles serve a launch when its columns are whole 256-wide
// tiles, the rows hold whole k-tiles (2-bit, or 1-bit without padding codes)
// and the output is bf16 with rows of whole 16-byte pieces.
template <int LAYOUT, typename YT>
bool gemm_dma_fits(int64_t N, int64_t K, int64_t ldy) {
    if constexpr (LAYOUT == kLayoutBase3 || sizeof(YT) != 2) {
        return false;
    } else {
        return N % 256 == 0 && ldy % 8 == 0 && gemm_k_mode(LAYOUT, K) == kWholeK;
    }
}

template <int LAYOUT, int BM, typename YT>
hipError_t launch_gemm_dma(const int8_t *xq, const float *scale, const uint8_t *packed,
                           const GammaMap &gamma, int64_t M, int64_t N, int64_t K, YT *y,
                           int64_t ldy, int32_t *acc, hipStream_t s) {
    const int64_t rb = row_bytes_of(LAYOUT, K);
    const int tm = (int)((M + BM - 1) / BM), tn = (int)(N / 256);
    GemmArgs<YT> g{xq, scale, packed, gamma, M, N, K, rb, tm, tn, y, ldy, acc};
    g.band = tile_band(tm, tn, (int64_t)BM * K, (int64_t)256 * rb);
    const unsigned blocks = (unsigned)((tm * tn + kXcds - 1) / kXcds * kXcds);
    if (t_plan) {
        // (static LDS: three stages and the output staging)
        plan_note(blocks, 1, 512, 3 * kDmaStage + 64 * kDmaOutRow,
                  "gemm_dma_kernel<%d, %d, %s, %s>", LAYOUT, BM,
                  gamma.nseg > 1 ? "true" : "false", type_name<YT>());
        return hipSuccess;
    }
    if constexpr (LAYOUT != kLayoutBase3 && sizeof(YT) == 2)
        if (gamma.nseg > 1)
            hipLaunchKernelGGL((gemm_dma_kernel<LAYOUT, BM, true, YT>), dim3(blocks), dim3(512), 0,
                               s, g);
        else
            hipLaunchKernelGGL((gemm_dma_kernel<LAYOUT, BM, false, YT>), dim3(blocks), dim3(512), 0,
                               s, g);
    return hipGetLastError();
}

template <int LAYOUT, int BM2, typename YT>
hipError_t launch_gemm_dma_pair(const int8_t *xq, const float *scale, const uint8_t *packed,
                                const GammaMap &gamma, int64_t M, int64_t N, int64_t K,
                                int64_t n_main, YT *y, int32_t *acc, hipStream_t s) {
    const int64_t rb = row_bytes_of(LAYOUT, K);
    const int tm = (int)((M + 255) / 256), tm2 = (int)((M + BM2 - 1) / BM2);
    const int tn1 = (int)(n_main / 256), tn2 = (int)((N - n_main) / 256);
    GemmArgs<YT> g1{xq, scale, packed, gamma, M, n_main, K, rb, tm, tn1, y, N, acc};
    GemmArgs<YT> g2{xq, scale, packed + n_main * rb, gamma.from_row(n_main), M, N - n_main,
                    K, rb, tm2, tn2, y + n_main, N, acc ? acc + n_main : nullptr};
    g1.band = tile_band(tm, tn1, 256 * K, 256 * rb);
    g2.band = tile_band(tm2, tn2, BM2 * K, 256 * rb);
    const int blocks1 = (tm * tn1 + kXcds - 1) / kXcds * kXcds;
    const int blocks2 = (tm2 * tn2 + kXcds - 1) / kXcds * kXcds;
    if (t_plan) {
        plan_note((unsigned)(blocks1 + blocks2), 1, 512, 3 * kDmaStage + 64 * kDmaOutRow,
                  "gemm_dma_pair_kernel<%d, %d, %s, %s> (%d tiles 256x256 + %d tiles %dx256)",
                  LAYOUT, BM2, gamma.nseg > 1 ? "true" : "false", type_name<YT>(), tm * tn1,
                  tm2 * tn2, BM2);
        return hipSuccess;
    }
    if constexpr (LAYOUT != kLayoutBase3 && sizeof(YT) == 2) {
        const dim3 grid((unsigned)(blocks1 + blocks2));
        if (gamma.nseg > 1)
            hipLaunchKernelGGL((gemm_dma_pair_kernel<LAYOUT, BM2, true, YT>), grid, dim3(512), 0, s,
                               g1, blocks1, g2);
        else
            hipLaunchKernelGGL((gemm_dma_pair_kernel<LAYOUT, BM2, false, YT>), grid, dim3(512), 0,
                               s, g1, blocks1, g2);
    }
    return hipGetLastError();
}

// The prefill shape in one launch: the first blocks cover the columns that
// fill whole rounds of 256 x 256 tiles, the rest the leftover columns in
// BM2 x 256 tiles (BM2 = 128, or 96 when those still make one round).
// Leftover tiles start as soon as CUs free up, so their start-up overlaps the
// output writes of the large tiles (and no second launch is waited for).
template <int LAYOUT, int KMODE, typename YT, int BM2>
__global__ __launch_bounds__(512) void gemm_pair_kernel(const GemmArgs<YT> g1, int blocks1,
                                                        const GemmArgs<YT> g2) {
    const int b = blockIdx.x;
    if (b < blocks1) {
        const int t = xcd_tile(b, g1.tiles_m * g1.tiles_n);
        if (t >= 0) gemm_tile<LAYOUT, 256, 256, 1, 8, 2, 1, KMODE, YT>(g1, t);
    } else {
        const int t = xcd_tile(b - blocks1, g2.tiles_m * g2.tiles_n);
        if (t >= 0) gemm_tile<LAYOUT, BM2, 256, 1, 8, 2, 1, KMODE, YT>(g2, t);
    }
}

template <int LAYOUT, int BM, int BN, int WM, int WN, int DIST, int KG = 1, typename YT>
hipError_t launch_gemm_tile(const int8_t *xq, const float *scale, const uint8_t *packed,
                            const GammaMap &gamma, int64_t M, int64_t N, int64_t K, YT *y,
                            int64_t ldy, int32_t *acc, hipStream_t s) {
    using C = GemmCfg<LAYOUT, BM, BN, WM, WN, DIST, KG>;
    const int64_t rb = row_bytes_of(LAYOUT, K);
    const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
    const int64_t ntiles = (int64_t)tm * tn;
    const int64_t blocks = (ntiles + kXcds - 1) / kXcds * kXcds;
    GemmArgs<YT> g{xq, scale, packed, gamma, M, N, K, rb, tm, tn, y, ldy, acc};
    // (128 x 64 tiles keep row order: banded, they measured 2-4% slower)
    g.band = BM == 128 && BN == 64 ? 1 : tile_band(tm, tn, (int64_t)BM * K, (int64_t)BN * rb);
    auto launch = [&](auto kern, LdsFlag *flag) {
        hipError_t e = allow_dynamic_lds(kern, C::SMEM, flag);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(C::kThreads), C::SMEM, s, g);
        return hipGetLastError();
    };
    if (t_plan) {
        plan_note((unsigned)blocks, 1, C::kThreads, C::SMEM,
                  "gemm_kernel<%d, %d, %d, %d, %d, %d, %d, %d, %s>", LAYOUT, BM, BN, WM, WN, DIST,
                  KG, gemm_k_mode(LAYOUT, K), type_name<YT>());
        return hipSuccess;
    }
    static LdsFlag lds_flag[3];  // one per k-mode
    switch (gemm_k_mode(LAYOUT, K)) {
        case kWholeK:
            return launch(gemm_kernel<LAYOUT, BM, BN, WM, WN, DIST, KG, kWholeK, YT>, &lds_flag[0]);
        case kGuardedK:
            return launch(gemm_kernel<LAYOUT, BM, BN, WM, WN, DIST, KG, kGuardedK, YT>,
                          &lds_flag[1]);
        default:
            return launch(gemm_kernel<LAYOUT, BM, BN, WM, WN, DIST, KG, kRaggedK, YT>,
                          &lds_flag[2]);
    }
}

// Tile configuration by problem size, chosen by timing on MI355X: large
// problems use 256 x 256 tiles with 8 waves (all layouts; base-3 4096^3:
// 89.2 -> 78.7 us against 128 x 256 tiles); when those tiles do not fill
// whole rounds of 256 CUs, the columns that do take 256 x 256 tiles and the
// leftover columns smaller tiles (in the same launch when they make one round
// of 128 x 256 tiles, else in a second launch), so no round runs mostly idle. With few tiles and long rows (64 or more k-tiles), two groups of four
// waves split each tile's k-tiles: twice the waves per CU for the same tile.
template <int LAYOUT, typename YT>
hipError_t launch_gemm_cols(const int8_t *xq, const float *scale, const uint8_t *packed,
                            const GammaMap &gamma, int64_t M, int64_t N, int64_t K, YT *y,
                            int64_t ldy, int32_t *acc, hipStream_t s) {
    auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    const int64_t t_wide = tiles(256, 128), t_sq = tiles(128, 128), t_small = tiles(128, 64);
    const int64_t units = row_bytes_of(LAYOUT, K) / GemmCfg<LAYOUT, 128, 64, 2, 2, 2>::LB;
    const int64_t ktiles = (units + 1) / 2;
    const bool long_k = ktiles >= 64;
    // k-tiles from which two groups splitting them pay off on few tiles (see
    // below); rows of K % 16 != 0 bytes load piecewise, take longer per
    // k-tile and gain from 16 on (200 x 2000 x 3000: 2-bit 23.2 -> 19.5 us,
    // base-3 39.7 -> 34.5 us)
    const int64_t split_kt = K % 16 != 0 ? 16 : 32;
#define BL_GEMM_TILE(...)                                                                    \
    return launch_gemm_tile<LAYOUT, __VA_ARGS__>(xq, scale, packed, gamma, M, N, K, y, ldy, acc, \
                                                 s)
    // The narrow tiles run with the same area as one row of four waves, so
    // each code is expanded by one wave only: 64 x 128 in place of 128 x 64
    // (512 x 4096 x 11008 with split k-tiles: 2-bit 40.6 -> 35.5 us, base-3
    // 51.5 -> 39.9 us) and, for 2-bit and 1-bit, 32 x 128 in place of 64 x 64
    // (256 x 4096 x 4096: 14.0 -> 13.5 us).
#define BL_TILE_128x64(...) BL_GEMM_TILE(64, 128, 1, 4, 2 __VA_ARGS__)
#define BL_TILE_64x64(...) BL_GEMM_TILE(32, 128, 1, 4, 2 __VA_ARGS__)
    // 256 x 128 tiles when they make several rounds, or one round that keeps
    // more than half of the 256 CUs busy (measured faster than two rounds of
    // 128 x 128 tiles for the leftover columns of the prefill shape; at
    // exactly half, one round of 128 x 128 tiles is faster), and, except for
    // base-3 (whose weight decode the 256 tokens of a tile share), their last
    // row of tiles is at least three quarters full (384 tokens: 128-row tiles
    // are faster). They run as 128 x 256 tiles of the same area, one row of
    // eight waves of 128 x 32, so that each code is expanded by one wave only
    // (512 x 12288 x 4096: 2-bit 36.9 -> 33.4 us, base-3 44.4 -> 37.3 us).
    const bool rows_fill = LAYOUT == kLayoutBase3 || M % 256 == 0 || M % 256 >= 192;
    if (rows_fill && (t_wide >= 512 || (t_wide > 128 && t_wide <= 256))) {
        if (gemm_dma_fits<LAYOUT, YT>(N, K, ldy))
            return launch_gemm_dma<LAYOUT, 128>(xq, scale, packed, gamma, M, N, K, y, ldy, acc, s);
        BL_GEMM_TILE(128, 256, 1, 8, 2);
    }
    if (long_k) {
        if constexpr (LAYOUT != kLayoutBase3) {
            // at most half a round of 128 x 64 tiles: 64 x 64 tiles, also
            // with split k-tiles, reach twice the CUs (256 x 4096 x 11008:
            // 37.2 -> 25.7 us)
            if (t_small <= 128 && tiles(64, 64) <= 256) BL_TILE_64x64(, 2);
        }
        if (t_small <= 256) BL_TILE_128x64(, 2);
        if (t_sq >= 160) BL_GEMM_TILE(128, 128, 1, 4, 2, 2);
    }
    // base-3, at most half a round of 128 x 64 tiles over split_kt or more
    // k-tiles: two groups split each tile's k-tiles (250 x 1000 x 8200:
    // 97.7 -> 78.5 us, 256 x 4096 x 6144: 31.1 -> 28.7 us; at 26 k-tiles,
    // K = 4096, the split was 1-3% slower)
    if (LAYOUT == kLayoutBase3 && t_small <= 128 && ktiles >= split_kt)
        BL_TILE_128x64(, 2);
    // base-3, most of one round of 128 x 128 tiles: two groups split each
    // tile's k-tiles (768 x 4096 x 4096: 30.4 -> 29.0 us, 640 x 4096 x 4096:
    // 29.9 -> 28.9 us; under 160 tiles the split was slower)
    if (LAYOUT == kLayoutBase3 && t_sq >= 160 && t_sq <= 256)
        BL_GEMM_TILE(128, 128, 1, 4, 2, 2);
    if (t_sq >= 256) BL_GEMM_TILE(128, 128, 1, 4, 2);
    if constexpr (LAYOUT != kLayoutBase3) {
        // up to one and a half rounds of 128 x 64 tiles: 64 x 64 tiles reach
        // more CUs or balance the rounds (256 x 4096 x 4096: 16.1 -> 11.9 us,
        // 512 x 4096 x 4096: 17.6 -> 17.0 us); a base-3 k-tile of 160 codes
        // does not split evenly over 64-row tiles
        // at most one round of them over split_kt or more k-tiles: two groups split
        // each tile's k-tiles (192 x 3000 x 5000: 36.1 -> 29.4 us, 320 x 2048
        // x 8000: 24.7 -> 20.3 us; over more than one round the split was
        // 7-9% slower)
        if (ktiles >= split_kt && tiles(64, 64) <= 256) BL_TILE_64x64(, 2);
        if (t_small <= 384) BL_TILE_64x64();
    }
    BL_TILE_128x64();
#undef BL_TILE_64x64
#undef BL_TILE_128x64
#undef BL_GEMM_TILE
}

// Columns [0, n_main) in 256 x 256 tiles and [n_main, N) in BM2 x 256 tiles,
// one launch.
template <int LAYOUT, int BM2, typename YT>
hipError_t launch_gemm_pair(const int8_t *xq, const float *scale, const uint8_t *packed,
                            const GammaMap &gamma, int64_t M, int64_t N, int64_t K, int64_t n_main,
                            YT *y, int32_t *acc, hipStream_t s) {
    using C1 = GemmCfg<LAYOUT, 256, 256, 1, 8, 2>;
    using C2 = GemmCfg<LAYOUT, BM2, 256, 1, 8, 2>;
    static_assert(C1::SMEM >= C2::SMEM && C1::kThreads == C2::kThreads, "one launch shape");
    const int64_t rb = row_bytes_of(LAYOUT, K);
    const int tm = (int)((M + 255) / 256), tm2 = (int)((M + BM2 - 1) / BM2);
    const int tn1 = (int)((n_main + 255) / 256), tn2 = (int)((N - n_main + 255) / 256);
    GemmArgs<YT> g1{xq, scale, packed, gamma, M, n_main, K, rb, tm, tn1, y, N, acc};
    GemmArgs<YT> g2{xq, scale, packed + n_main * rb, gamma.from_row(n_main), M, N - n_main,
                    K, rb, tm2, tn2, y + n_main, N, acc ? acc + n_main : nullptr};
    g1.band = tile_band(tm, tn1, 256 * K, 256 * rb);
    g2.band = tile_band(tm2, tn2, BM2 * K, 256 * rb);
    const int blocks1 = (tm * tn1 + kXcds - 1) / kXcds * kXcds;
    const int blocks2 = (tm2 * tn2 + kXcds - 1) / kXcds * kXcds;
    auto launch = [&](auto kern, LdsFlag *flag) {
        hipError_t e = allow_dynamic_lds(kern, C1::SMEM, flag);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)(blocks1 + blocks2)), dim3(C1::kThreads), C1::SMEM,
                           s, g1, blocks1, g2);
        return hipGetLastError();
    };
    if (t_plan) {
        plan_note((unsigned)(blocks1 + blocks2), 1, C1::kThreads, C1::SMEM,
                  "gemm_pair_kernel<%d, %d, %s, %d> (%d tiles 256x256 + %d tiles %dx256)", LAYOUT,
                  gemm_k_mode(LAYOUT, K), type_name<YT>(), BM2, tm * tn1, tm2 * tn2, BM2);
        return hipSuccess;
    }
    static LdsFlag lds_flag[3];  // one per k-mode
    switch (gemm_k_mode(LAYOUT, K)) {
        case kWholeK: return launch(gemm_pair_kernel<LAYOUT, kWholeK, YT, BM2>, &lds_flag[0]);
        case kGuardedK: return launch(gemm_pair_kernel<LAYOUT, kGuardedK, YT, BM2>, &lds_flag[1]);
        default: return launch(gemm_pair_kernel<LAYOUT, kRaggedK, YT, BM2>, &lds_flag[2]);
    }
}

template <int LAYOUT, typename YT>
hipError_t launch_gemm_t(const int8_t *xq, const float *scale, const uint8_t *packed,
                         const GammaMap &gamma, int64_t M, int64_t N, int64_t K, YT *y,
                         int32_t *acc, hipStream_t s) {
    constexpr int64_t kCUs = 256;
    const int64_t rb = row_bytes_of(LAYOUT, K);
    {
        const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256;
        if (tm * tn >= kCUs) {
            // columns covered by whole rounds of 256 x 256 tiles
            const int64_t rounds = tm * tn / kCUs;
            int64_t tn_main = rounds * kCUs / tm;
            if (tn_main > tn) tn_main = tn;
            // many row tiles over narrow columns (tm > 256, tm not a multiple
            // of 256, one column of tiles) leave no whole round: no 256 x 256
            // launch, all columns take the smaller tiles
            if (tn_main == 0)
                return launch_gemm_cols<LAYOUT>(xq, scale, packed, gamma, M, N, K, y, N, acc, s);
            const int64_t n_main = tn_main * 256 < N ? tn_main * 256 : N;
            const int64_t n_rest = N - n_main;
            const int64_t t_rest = ((M + 127) / 128) * ((n_rest + 255) / 256);
            if (n_rest > 0 && t_rest >= 128 && t_rest <= kCUs) {
                // 96-row leftover tiles when they still make one round: more
                // CUs share the leftover work (prefill 2048 x 11008 x 4096:
                // 176 tiles of 128 x 256 -> 242 of 96 x 256; at steady clocks
                // with flushed caches base-3 105.0 -> 101.6 us and 111.7 ->
                // 109.4 us on two boxes, 1-bit 91.3 -> 91.3 and 100.7 -> 99.0
                // us, 2-bit within 1% either way)
                const int64_t t_rest96 = ((M + 95) / 96) * ((n_rest + 255) / 256);
                const bool dma = gemm_dma_fits<LAYOUT, YT>(N, K, N);
                if (t_rest96 <= kCUs)
                    return dma ? launch_gemm_dma_pair<LAYOUT, 96>(xq, scale, packed, gamma, M, N,
                                                                  K, n_main, y, acc, s)
                               : launch_gemm_pair<LAYOUT, 96>(xq, scale, packed, gamma, M, N, K,
                                                              n_main, y, acc, s);
                return dma ? launch_gemm_dma_pair<LAYOUT, 128>(xq, scale, packed, gamma, M, N, K,
                                                               n_main, y, acc, s)
                           : launch_gemm_pair<LAYOUT, 128>(xq, scale, packed, gamma, M, N, K,
                                                           n_main, y, acc, s);
            }
            hipError_t e = gemm_dma_fits<LAYOUT, YT>(n_main, K, N)
                               ? launch_gemm_dma<LAYOUT, 256>(xq, scale, packed, gamma, M, n_main,
                                                              K, y, N, acc, s)
                               : launch_gemm_tile<LAYOUT, 256, 256, 1, 8, 2>(
                                     xq, scale, packed, gamma, M, n_main, K, y, N, acc, s);
            if (e != hipSuccess || n_main == N) return e;
            return launch_gemm_cols<LAYOUT>(xq, scale, packed + n_main * rb,
                                            gamma.from_row(n_main), M, N - n_main,
                                            K, y + n_main, N, acc ? acc + n_main : nullptr, s);
        }
    }
    return launch_gemm_cols<LAYOUT>(xq, scale, packed, gamma, M, N, K, y, N, acc, s);
}

}  // namespace

hipError_t launch_forward_gemm(const int8_t *xq, const float *scale, const uint8_t *packed,
                               int layout, const GammaMap &gamma, int64_t M, int64_t N, int64_t K,
                               void *y, int y_dtype, int32_t *acc, hipStream_t stream) {
    if (M > (int64_t)2147483647 || N > (int64_t)2147483647) return hipErrorInvalidValue;
    auto go = [&](auto layout_c) {
        constexpr int L = decltype(layout_c)::value;
        if (y_dtype == kF32)
            return launch_gemm_t<L>(xq, scale, packed, gamma, M, N, K, static_cast<float *>(y),
                                    acc, stream);
        return launch_gemm_t<L>(xq, scale, packed, gamma, M, N, K, static_cast<uint16_t *>(y),
                                acc, stream);
    };
    switch (layout) {
        case kLayout2Bit: return go(std::integral_constant<int, kLayout2Bit>{});
        case kLayoutBase3: return go(std::integral_constant<int, kLayoutBase3>{});
        default: return go(std::integral_constant<int, kLayout1Bit>{});
    }
}

}  // namespace bl
