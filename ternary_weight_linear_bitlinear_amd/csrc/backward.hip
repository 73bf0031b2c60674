// Backward products of a BitLinear layer with the straight-through estimator
// (the backward pass treats rounding as the identity: [QAT-en] "How Gradients
// Flow: Fake Quantization and STE"; [b158] §5.3):
//
//   grad_x[m, k] = gamma * sum_n grad_y[m, n] * c[n, k]   (bf16 x ternary codes)
//   grad_w[n, k] =         sum_m grad_y[m, n] * x[m, k]   (bf16 x bf16)
//
// both accumulated in fp32 on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16).
// One kernel computes C[i, j] = alpha * sum_p A(i, p) * B(p, j) with B stored
// [p][j] (j contiguous) and A stored either [i][p] or [p][i]:
//   grad_x: i = m, j = k, p = n; A = grad_y as stored ([i][p]); B = the codes of
//           the packed weight rows, expanded to bf16 -1 / 0 / +1 on the way into
//           LDS (so the forward's packed matrix is used as is, no transposed copy).
//   grad_w: i = n, j = k, p = m; A = grad_y read as [p][i]; B = x.
//
// Operand tiles are staged through LDS in their natural row-major layout. A
// matrix-core operand needs eight consecutive contraction values per lane;
// where the contraction index runs along LDS rows (B always, A for grad_w) the
// fragments are read with the gfx950 transposing LDS load (ds_read_b64_tr_b16):
// each group of 16 lanes reads a 4 x 16 tile of 16-bit values (lane t of the
// group addresses row t / 4, columns 4 (t % 4)..+3) and lane t receives column
// t of it, i.e. four consecutive rows; two such loads make one operand.
#include "bl_internal.hpp"
#include "device_util.hpp"

namespace bl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

constexpr int kXcds = 8;

// Block tile BI x BJ outputs, contraction slice BP per stage, 8 waves as 2 x 4,
// each wave 128 x 64 outputs as 4 x 2 fragments of 32 x 32.
struct BwdCfg {
    static constexpr int BI = 256, BJ = 256, BP = 64;
    static constexpr int WI = 2, WJ = 4;
    static constexpr int kThreads = 64 * WI * WJ;
    static constexpr int FI = BI / WI / 32, FJ = BJ / WJ / 32;
    static constexpr int KSTEPS = BP / 16;
    // [i][p] tile: rows of BP bf16 (128 B) padded to 144 B; [p][*] tiles: rows of
    // 256 bf16 (512 B) padded to 576 B so the four rows of a transposing load
    // fall in distinct bank groups.
    static constexpr int LD_IP = BP * 2 + 16;
    static constexpr int LD_PX = BI * 2 + 64;
    static constexpr int A_BYTES = BI * LD_IP > BP * LD_PX ? BI * LD_IP : BP * LD_PX;
    static constexpr int B_BYTES = BP * LD_PX;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int SMEM = 2 * STAGE;
    static constexpr int LUT3 = 256 * 8;  // base-3 byte -> five fields (after the stages)
    static_assert(BI == BJ, "one padded [p][*] row length serves A and B");
};

enum { kBDense = 0, kBPacked2 = 1, kBPacked1 = 2, kBPacked3 = 3 };

// Four codes of one 2-bit field (bytes u = c + 1 in 0..2) to four bf16 values
// -1 / 0 / +1 (0xBF80 / 0x0000 / 0x3F80) in two dwords. The byte permute picks
// table bytes by selector: selector (u, u + 4) yields (low byte, high byte).
__device__ __forceinline__ void field_to_bf16(uint32_t f, uint32_t &d0, uint32_t &d1) {
    constexpr uint32_t kLo = 0x00800080u;  // u = 0, 1, 2 -> 0x80, 0x00, 0x80
    constexpr uint32_t kHi = 0x003F00BFu;  // u = 0, 1, 2 -> 0xBF, 0x00, 0x3F
    const uint32_t f4 = f + 0x04040404u;
    const uint32_t s0 = __builtin_amdgcn_perm(f4, f, 0x05010400u);  // u0, u0+4, u1, u1+4
    const uint32_t s1 = __builtin_amdgcn_perm(f4, f, 0x07030602u);  // u2, u2+4, u3, u3+4
    d0 = __builtin_amdgcn_perm(kHi, kLo, s0);
    d1 = __builtin_amdgcn_perm(kHi, kLo, s1);
}

// Base-3 decode table entry for byte v: its five trits t_r = c_r + 1 (first
// code in the least significant trit) as one field per byte, bytes 0..4.
// Bytes 243..255 are not produced by the packing; they read as five zero codes.
__device__ __forceinline__ uint64_t base3_field_entry(uint32_t v) {
    if (v >= 243u) return 0x0101010101ull;
    uint64_t e = 0;
#pragma unroll
    for (int r = 0; r < 5; ++r) {
        e |= (uint64_t)(v % 3u) << (8 * r);
        v /= 3u;
    }
    return e;
}

// Eight bytes of the base-3 layout (words w0, w1, first byte in the low bits)
// as their 40 fields, one per byte, looked up in the table; then the 32 fields
// starting at field `first` (0..4) as eight words of four fields each
// (natural order).
__device__ __forceinline__ void base3_fields(uint32_t w0, uint32_t w1, int first,
                                             const uint64_t *lut, uint32_t (&out)[8]) {
    uint64_t f[5] = {0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t v = ((i < 4 ? w0 : w1) >> (8 * (i % 4))) & 0xFFu;
        const uint64_t e = lut[v];
        constexpr int kSh[8] = {0, 40, 16, 56, 32, 8, 48, 24};  // 8 * (5 i % 8)
        const int w = (5 * i) / 8, sh = kSh[i];
        f[w] |= e << sh;
        if (sh > 24) f[w + 1] |= e >> (64 - sh);
    }
    const int sh = 8 * first;  // 0 .. 32
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint64_t lo = f[w] >> sh;
        const uint64_t hi = sh == 0 ? 0 : f[w + 1] << (64 - sh);
        const uint64_t v = lo | hi;
        out[2 * w] = (uint32_t)v;
        out[2 * w + 1] = (uint32_t)(v >> 32);
    }
}

// The top halves of two fp32 words as one word of two bf16 values.
__device__ __forceinline__ uint32_t top_halves(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Piece `piece` of the exact three-way bf16 split of fp32 values x = hi + mid
// + lo: hi is x with its low 16 bits cleared, mid the same of x - hi, lo =
// x - hi - mid. Each subtraction is exact, and the pieces carry 8 + 8 + 8 of
// x's 24 significant bits, so every piece is a bf16 value (for |x| >= 2^-110;
// below that lo can fall among fp32 subnormals and lose bits under 2^-133).
// All pieces share x's sign, so |hi| + |mid| + |lo| = |x|.
__device__ __forceinline__ uint32_t f32_piece_bits(uint32_t ux, int piece) {
    if (piece == 0) return ux;
    const float x = __uint_as_float(ux);
    const float r = x - __uint_as_float(ux & 0xFFFF0000u);
    const uint32_t ur = __float_as_uint(r);
    if (piece == 1) return ur;
    return __float_as_uint(r - __uint_as_float(ur & 0xFFFF0000u));
}

// F32 = 1 (grad_x): A holds fp32 values; the contraction runs three times over
// p, once per bf16 piece of A (hi, mid, lo), into the same accumulators.
// F32 = 2 (grad_W): A and B hold fp32 values; six passes multiply the piece
// pairs hi.hi, hi.mid, mid.hi, hi.lo, lo.hi and mid.mid. With |mid| < 2^-7 |x|
// and |lo| < 2^-14 |x|, the three pairs left out (mid.lo, lo.mid, lo.lo) add
// up to less than 2^-20 |a b|, so every product is exact to within 2^-20 of
// its magnitude.
constexpr int kPassesF32[3] = {1, 3, 6};
constexpr int kPieceA6[6] = {0, 0, 1, 0, 2, 1}, kPieceB6[6] = {0, 1, 0, 2, 0, 1};

template <bool A_T, int BSRC, int F32 = 0>
__global__ __launch_bounds__(BwdCfg::kThreads) void bwd_gemm_kernel(
    const void *__restrict__ Av, int64_t lda, const void *__restrict__ Bv, int64_t ldb,
    int64_t I, int64_t J, int64_t P, const float *__restrict__ alpha_p, int tiles_i,
    int tiles_j, float *__restrict__ C, int64_t ldc) {
    using G = BwdCfg;
    constexpr bool A_F32 = F32 >= 1, B_F32 = F32 == 2;
    static_assert(F32 != 1 || !A_T, "fp32 A alone: grad_x, A stored [i][p]");
    static_assert(F32 != 2 || (A_T && BSRC == kBDense), "fp32 A and B: grad_W");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint64_t *lut = reinterpret_cast<uint64_t *>(smem + G::SMEM);  // base-3 only

    const int ntiles = tiles_i * tiles_j;
    const int per_xcd = (ntiles + kXcds - 1) / kXcds;
    const int b = blockIdx.x;
    const int t = (b % kXcds) * per_xcd + b / kXcds;
    if (t >= ntiles) return;
    const int64_t i0 = (int64_t)(t / tiles_j) * G::BI;
    const int64_t j0 = (int64_t)(t % tiles_j) * G::BJ;

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    const int wi = wave / G::WJ, wj = wave % G::WJ;

    // ---- global -> register staging, one contraction slice per stage ------
    constexpr int A_CH = G::BI * G::BP / 8 / G::kThreads;  // 16-byte chunks per thread
    constexpr int B_CH = BSRC == kBDense ? G::BP * G::BJ / 8 / G::kThreads : 1;
    constexpr int A_W = A_F32 ? 2 : 1;  // 16-byte loads per chunk of 8 values
    v4i a_reg[A_CH][A_W];
    bool a_ok[A_CH];
    constexpr int B_W = B_F32 ? 2 : 1;
    v4i b_reg[B_CH][B_W];  // dense: 16-byte chunks (two for fp32); packed: one piece
    bool b_ok[B_CH];
    const uint16_t *A16 = static_cast<const uint16_t *>(Av);
    const float *A32 = static_cast<const float *>(Av);
    const uint16_t *B16 = static_cast<const uint16_t *>(Bv);
    const float *B32 = static_cast<const float *>(Bv);
    const uint8_t *B8 = static_cast<const uint8_t *>(Bv);

    // Out-of-range pieces read a valid address and are zeroed when stored
    // to LDS (contiguous dimensions are multiples of 8, so a 16-byte chunk
    // is entirely inside or outside).
    auto load_stage = [&](int64_t p0) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < A_CH; ++c) {
            const int q = tid + c * G::kThreads;
            int64_t off;
            if (!A_T) {  // [i][p]: 8 chunks per tile row
                const int64_t i = i0 + q / (G::BP / 8), p = p0 + 8 * (q % (G::BP / 8));
                a_ok[c] = i < I && p < P;
                off = i * lda + p;
            } else {     // [p][i]: 32 chunks per tile row
                const int64_t p = p0 + q / (G::BI / 8), i = i0 + 8 * (q % (G::BI / 8));
                a_ok[c] = p < P && i < I;
                off = p * lda + i;
            }
            if constexpr (A_F32) {
                const v4i *src = reinterpret_cast<const v4i *>(A32 + (a_ok[c] ? off : 0));
                a_reg[c][0] = src[0];
                a_reg[c][1] = src[1];
            } else {
                a_reg[c][0] = *reinterpret_cast<const v4i *>(A16 + (a_ok[c] ? off : 0));
            }
        }
        if constexpr (BSRC == kBDense) {
#pragma unroll
            for (int c = 0; c < B_CH; ++c) {
                const int q = tid + c * G::kThreads;
                const int64_t p = p0 + q / (G::BJ / 8), j = j0 + 8 * (q % (G::BJ / 8));
                b_ok[c] = p < P && j < J;
                if constexpr (B_F32) {
                    const v4i *src = reinterpret_cast<const v4i *>(B32 + (b_ok[c] ? p * ldb + j : 0));
                    b_reg[c][0] = src[0];
                    b_reg[c][1] = src[1];
                } else {
                    b_reg[c][0] = *reinterpret_cast<const v4i *>(B16 + (b_ok[c] ? p * ldb + j : 0));
                }
            }
        } else if constexpr (BSRC == kBPacked2) {
            // 64 rows x 64 packed bytes: 8 bytes (32 codes) per thread
            const int64_t p = p0 + tid / 8;
            const int64_t byte = j0 / 4 + 8 * (tid % 8);
            b_ok[0] = p < P && byte + 8 <= ldb;
            const uint2 v = *reinterpret_cast<const uint2 *>(B8 + (b_ok[0] ? p * ldb + byte : 0));
            b_reg[0][0] = v4i{(int)v.x, (int)v.y, 0, 0};
        } else if constexpr (BSRC == kBPacked1) {
            // 64 rows x 32 packed bytes: one 32-code word per thread
            const int64_t p = p0 + tid / 8;
            const int64_t byte = j0 / 8 + 4 * (tid % 8);
            b_ok[0] = p < P && byte + 4 <= ldb;
            const uint32_t v = *reinterpret_cast<const uint32_t *>(B8 + (b_ok[0] ? p * ldb + byte : 0));
            b_reg[0][0] = v4i{(int)v, 0, 0, 0};
        } else {
            // base-3: the eight bytes holding codes c0 .. c0 + 31 start at byte
            // b0 = c0 / 5, inside the three aligned dwords from b0 & ~3 (row
            // bytes are a multiple of 16, so each dword is wholly inside or
            // past the row; those past it read as 121 = five zero codes)
            const int64_t p = p0 + tid / 8;
            const int64_t c0 = j0 + 32 * (tid % 8);
            const int64_t b0 = c0 / 5, al = b0 & ~(int64_t)3;
            const bool row_ok = p < P;
            const uint32_t *row = reinterpret_cast<const uint32_t *>(B8 + (row_ok ? p : 0) * ldb);
            uint32_t d[3];
#pragma unroll
            for (int i = 0; i < 3; ++i)
                d[i] = row_ok && al + 4 * i < ldb ? row[al / 4 + i] : 0x79797979u;
            const uint32_t sh = (uint32_t)(b0 - al);
            b_ok[0] = row_ok;
            b_reg[0][0] = v4i{(int)__builtin_amdgcn_alignbyte(d[1], d[0], sh),
                           (int)__builtin_amdgcn_alignbyte(d[2], d[1], sh), (int)(c0 - 5 * b0), 0};
        }
    };

    // pass: which piece (pair) of fp32 operands this stage carries
    auto store_stage = [&](uint8_t *st, int pass) __attribute__((always_inline)) {
        uint8_t *As = st;
        uint8_t *Bs = st + G::A_BYTES;
        const v4i z = {0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < A_CH; ++c) {
            const int q = tid + c * G::kThreads;
            const int off = !A_T ? (q / (G::BP / 8)) * G::LD_IP + 16 * (q % (G::BP / 8))
                                 : (q / (G::BI / 8)) * G::LD_PX + 16 * (q % (G::BI / 8));
            v4i v;
            if constexpr (A_F32) {
                const int pa = B_F32 ? kPieceA6[pass] : pass;
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e] = f32_piece_bits((uint32_t)a_reg[c][e / 4][e % 4], pa);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (int)top_halves(h[2 * e], h[2 * e + 1]);
            } else {
                v = a_reg[c][0];
            }
            *reinterpret_cast<v4i *>(As + off) = a_ok[c] ? v : z;
        }
        if constexpr (BSRC == kBDense) {
#pragma unroll
            for (int c = 0; c < B_CH; ++c) {
                const int q = tid + c * G::kThreads;
                const int off = (q / (G::BJ / 8)) * G::LD_PX + 16 * (q % (G::BJ / 8));
                v4i v;
                if constexpr (B_F32) {
                    const int pb = kPieceB6[pass];
                    uint32_t h[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) h[e] = f32_piece_bits((uint32_t)b_reg[c][e / 4][e % 4], pb);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = (int)top_halves(h[2 * e], h[2 * e + 1]);
                } else {
                    v = b_reg[c][0];
                }
                *reinterpret_cast<v4i *>(Bs + off) = b_ok[c] ? v : z;
            }
        } else if constexpr (BSRC == kBPacked1) {
            // bit t of byte i of the word is code 4 t + i; u = 2 bit (0 or 2)
            // picks -1 or +1. Rows past P multiply zeros of A.
            const uint32_t word = (uint32_t)b_reg[0][0][0];
            uint8_t *dst = Bs + (tid / 8) * G::LD_PX + 64 * (tid % 8);
            uint32_t d[16];
#pragma unroll
            for (int t = 0; t < 8; ++t)
                field_to_bf16(((word >> t) & 0x01010101u) << 1, d[2 * t], d[2 * t + 1]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<uint4 *>(dst + 16 * q) =
                    make_uint4(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]);
        } else if constexpr (BSRC == kBPacked3) {
            uint32_t f[8];
            base3_fields((uint32_t)b_reg[0][0][0], (uint32_t)b_reg[0][0][1], b_reg[0][0][2], lut, f);
            uint8_t *dst = Bs + (tid / 8) * G::LD_PX + 64 * (tid % 8);
            uint32_t d[16];
#pragma unroll
            for (int w = 0; w < 8; ++w) field_to_bf16(f[w], d[2 * w], d[2 * w + 1]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<uint4 *>(dst + 16 * q) =
                    make_uint4(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]);
        } else {
            // word w holds codes 16 w .. 16 w + 15 of the piece; field s of a
            // word holds its codes 4 s .. 4 s + 3 (one per byte)
            const uint32_t words[2] = {b_ok[0] ? (uint32_t)b_reg[0][0][0] : 0x55555555u,
                                       b_ok[0] ? (uint32_t)b_reg[0][0][1] : 0x55555555u};
            uint8_t *dst = Bs + (tid / 8) * G::LD_PX + 64 * (tid % 8);
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                uint32_t d[8];
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    field_to_bf16((words[w] >> (2 * s)) & 0x03030303u, d[2 * s], d[2 * s + 1]);
                *reinterpret_cast<uint4 *>(dst + 32 * w) = make_uint4(d[0], d[1], d[2], d[3]);
                *reinterpret_cast<uint4 *>(dst + 32 * w + 16) = make_uint4(d[4], d[5], d[6], d[7]);
            }
        }
    };

    // ---- fragments ----------------------------------------------------------
    const int g16 = lane / 16, t16 = lane % 16;
    // transposing load of rows r0 + 8 (g16 / 2) + t16 / 4 (+4 for the second
    // half), columns c0 + 16 (g16 % 2) + 4 (t16 % 4), from a [p][*] tile
    auto tr_frag = [&](const uint8_t *tile, int r0, int c0) __attribute__((always_inline)) -> bf16x8 {
        const int row = r0 + 8 * (g16 / 2) + t16 / 4;
        const int col = c0 + 16 * (g16 % 2) + 4 * (t16 % 4);
        const uint8_t *p = tile + row * G::LD_PX + col * 2;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(p));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(p + 4 * G::LD_PX));
        const v8s both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, both);
    };

    v16f acc[G::FI][G::FJ];
#pragma unroll
    for (int i = 0; i < G::FI; ++i)
#pragma unroll
        for (int j = 0; j < G::FJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    auto compute = [&](const uint8_t *st) __attribute__((always_inline)) {
        const uint8_t *As = st;
        const uint8_t *Bs = st + G::A_BYTES;
#pragma unroll
        for (int ks = 0; ks < G::KSTEPS; ++ks) {
            bf16x8 a[G::FI], bb[G::FJ];
#pragma unroll
            for (int i = 0; i < G::FI; ++i) {
                const int ibase = wi * (G::BI / G::WI) + i * 32;
                if constexpr (!A_T) {
                    // lane: row ibase + lane % 32, contraction 16 ks + 8 (lane / 32) .. +8
                    a[i] = *reinterpret_cast<const bf16x8 *>(
                        As + (ibase + lane % 32) * G::LD_IP + (16 * ks + 8 * (lane / 32)) * 2);
                } else {
                    a[i] = tr_frag(As, 16 * ks, ibase);
                }
            }
#pragma unroll
            for (int j = 0; j < G::FJ; ++j) bb[j] = tr_frag(Bs, 16 * ks, wj * (G::BJ / G::WJ) + j * 32);
#pragma unroll
            for (int i = 0; i < G::FI; ++i)
#pragma unroll
                for (int j = 0; j < G::FJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
        }
    };

    if constexpr (BSRC == kBPacked3) {
        if (tid < 256) lut[tid] = base3_field_entry((uint32_t)tid);
        __syncthreads();
    }
    // stage s: contraction slice s % per_pass of pass s / per_pass (fp32
    // operands: one pass per piece or piece pair)
    const int64_t per_pass = (P + G::BP - 1) / G::BP;
    const int64_t nst = per_pass * kPassesF32[F32];
    auto slice_of = [&](int64_t s) { return (F32 ? s % per_pass : s) * G::BP; };
    auto piece_of = [&](int64_t s) { return F32 ? (int)(s / per_pass) : 0; };
    load_stage(0);
    store_stage(smem, 0);
    __syncthreads();
    for (int64_t s = 0; s < nst; ++s) {
        const bool more = s + 1 < nst;
        if (more) load_stage(slice_of(s + 1));
        compute(smem + (s & 1) * G::STAGE);
        if (more) store_stage(smem + ((s + 1) & 1) * G::STAGE, piece_of(s + 1));
        lds_barrier();
    }

    // ---- epilogue: lane holds D[i][j] for j = lane % 32 and
    // i = 8 (r / 4) + 4 (lane / 32) + r % 4, register r
    const float alpha = alpha_p ? alpha_p[0] : 1.0f;
#pragma unroll
    for (int fi = 0; fi < G::FI; ++fi)
#pragma unroll
        for (int fj = 0; fj < G::FJ; ++fj) {
            const int64_t j = j0 + wj * (G::BJ / G::WJ) + fj * 32 + lane % 32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t i =
                    i0 + wi * (G::BI / G::WI) + fi * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
                if (i < I && j < J) C[i * ldc + j] = acc[fi][fj][r] * alpha;
            }
        }
}

template <bool A_T, int BSRC, int F32 = 0>
hipError_t launch_bwd(const void *A, int64_t lda, const void *B, int64_t ldb, int64_t I,
                      int64_t J, int64_t P, const float *alpha, float *C, int64_t ldc,
                      hipStream_t s) {
    using G = BwdCfg;
    const int ti = (int)((I + G::BI - 1) / G::BI), tj = (int)((J + G::BJ - 1) / G::BJ);
    const int64_t blocks = ((int64_t)ti * tj + kXcds - 1) / kXcds * kXcds;
    auto kern = bwd_gemm_kernel<A_T, BSRC, F32>;
    const int smem = G::SMEM + (BSRC == kBPacked3 ? G::LUT3 : 0);
    static LdsFlag lds_raised{0};
    hipError_t e = allow_dynamic_lds(kern, smem, &lds_raised);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(G::kThreads), smem, s, A, lda, B,
                       ldb, I, J, P, alpha, ti, tj, C, ldc);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float *__restrict__ out, int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += stride) out[i] = 0.f;
}

}  // namespace

hipError_t launch_zero_f32(float *out, int64_t count, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    const int64_t want = (count + 255) / 256;
    const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
    hipLaunchKernelGGL(zero_f32_kernel, dim3(blocks), dim3(256), 0, stream, out, count);
    return hipGetLastError();
}

namespace {
template <int F32>
hipError_t backward_input_t(const void *grad_y, const uint8_t *packed, int layout,
                            const float *gamma, int64_t M, int64_t N, int64_t K, float *grad_x,
                            hipStream_t stream) {
    if (layout == kLayout1Bit)
        return launch_bwd<false, kBPacked1, F32>(grad_y, N, packed, row_bytes_1bit(K), M, K, N,
                                                 gamma, grad_x, K, stream);
    if (layout == kLayoutBase3)
        return launch_bwd<false, kBPacked3, F32>(grad_y, N, packed, row_bytes_base3(K), M, K, N,
                                                 gamma, grad_x, K, stream);
    return launch_bwd<false, kBPacked2, F32>(grad_y, N, packed, row_bytes_2bit(K), M, K, N, gamma,
                                             grad_x, K, stream);
}
}  // namespace

hipError_t launch_backward_input(const void *grad_y, bool grad_y_f32, const uint8_t *packed,
                                 int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                                 float *grad_x, hipStream_t stream) {
    return grad_y_f32 ? backward_input_t<1>(grad_y, packed, layout, gamma, M, N, K, grad_x, stream)
                      : backward_input_t<0>(grad_y, packed, layout, gamma, M, N, K, grad_x, stream);
}

hipError_t launch_backward_weight(const void *grad_y, const void *x, bool f32, int64_t M,
                                  int64_t N, int64_t K, float *grad_w, hipStream_t stream) {
    if (f32) return launch_bwd<true, kBDense, 2>(grad_y, N, x, K, N, K, M, nullptr, grad_w, K, stream);
    return launch_bwd<true, kBDense>(grad_y, N, x, K, N, K, M, nullptr, grad_w, K, stream);
}

}  // namespace bl
