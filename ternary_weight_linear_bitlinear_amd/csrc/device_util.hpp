// Device helpers shared by the kernels: element loads, bf16 rounding, wave
// reductions and the ternary code expansion used by the products.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bl_internal.hpp"

namespace bl {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kPer16B = 4;
    __device__ __forceinline__ static float get(const float *p, int64_t i) { return p[i]; }
};
template <> struct Elem<uint16_t> {
    static constexpr int kPer16B = 8;
    __device__ __forceinline__ static float get(const uint16_t *p, int64_t i) {
        return bf16_bits_to_f32(p[i]);
    }
};

// Load 8 consecutive elements starting at p (16-byte aligned for bf16,
// 32-byte aligned for fp32) as floats.
__device__ __forceinline__ void load8(const float *p, float v[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t *p, float v[8]) {
    const uint4 a = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

// One activation code: q = clamp(rint((x / s) * 127), -127, 127), division,
// then the multiply, then round half to even, in the order the pages write it
// ([b158] §3.2 and §5.2). The quotient is formed with Markstein's correction
// step (IBM J. Res. Dev. 34(1), 1990) from y = 1/s, rounded once per token:
// q0 = x y, r = x - s q0 (exact with one fused multiply-add), q = q0 + r y.
// With y correctly rounded this is the correctly rounded x / s unless the
// residual r underflows, which needs |x / s| < 2^-80; such a quotient rounds
// to code 0 either way. (An exhaustive run over every bf16 x against 20000
// scales found differing quotients only below 2^-88, never a differing code.)
//
// Rounding and the clamp cost no instructions of their own. s is the largest
// |x| of the token (or 1e-6 above it), so for finite x the quotient lies
// within one ulp of [-1, 1] and t = q * 127 within [-127.0001, 127.0001]: the
// clamp can never change the rounded value. Adding 1.5 * 2^23 rounds t to an
// integer (half to even, the default rounding of the add) and leaves that
// integer in the low mantissa bits, so the low byte of the sum's bit pattern
// is the two's-complement code. The multiply and the add stay two rounded
// operations (the library is built without floating-point contraction).
__device__ __forceinline__ uint32_t quant_word(float x, float s, float y) {
    const float q0 = x * y;
    const float r = __builtin_fmaf(-q0, s, x);
    const float t = __builtin_fmaf(r, y, q0) * 127.0f;
    return __float_as_uint(t + 12582912.0f);
}
__device__ __forceinline__ int8_t quant1(float x, float s, float y) {
    return (int8_t)(quant_word(x, s, y) & 0xFFu);
}
// Four codes packed little-endian into one word (three byte permutes).
__device__ __forceinline__ uint32_t quant4(float x0, float x1, float x2, float x3, float s,
                                           float y) {
    const uint32_t lo = __builtin_amdgcn_perm(quant_word(x1, s, y), quant_word(x0, s, y),
                                              0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(quant_word(x3, s, y), quant_word(x2, s, y),
                                              0x0c0c0400u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations (so its LDS writes are visible and its LDS reads have returned),
// then s_barrier. Unlike __syncthreads() it does not wait for outstanding
// global loads into registers, so prefetches issued before it stay in flight.
// The memory clobber keeps the compiler from moving memory accesses across it.
// Only for barriers whose purpose is LDS reuse; global memory written before
// it is not made visible to other waves.
// Immediate of s_waitcnt that waits until at most n vector-memory operations
// of this wave are outstanding (n < 64) and leaves the other counters alone
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// A generic pointer into LDS as the LDS-address-space pointer that
// direct-to-LDS loads take.
__device__ __forceinline__ __attribute__((address_space(3))) void *to_lds(void *p) {
    return (__attribute__((address_space(3))) void *)p;
}

__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Epilogue factors of a segmented matrix: the gammas are loaded once per
// workgroup, f_s = gamma_s * scale / 127 (the epilogue's own order of
// operations) is formed per token, and row n picks its segment's factor.
__device__ __forceinline__ void load_gammas(const GammaMap &gm, float (&gs)[kMaxSegments]) {
#pragma unroll
    for (int s = 0; s < kMaxSegments; ++s) gs[s] = s < gm.nseg ? gm.g[s] : 0.f;
}
__device__ __forceinline__ void seg_factors(const GammaMap &gm, const float (&gs)[kMaxSegments],
                                            float scale, float (&f)[kMaxSegments]) {
#pragma unroll
    for (int s = 0; s < kMaxSegments; ++s) f[s] = s < gm.nseg ? gs[s] * scale / 127.0f : 0.f;
}
// gamma of row n itself (for epilogues that scale by gamma * (scale / 127))
__device__ __forceinline__ float seg_gamma(const GammaMap &gm, const float (&gs)[kMaxSegments],
                                           int64_t n) {
    float r = gs[0];
#pragma unroll
    for (int i = 0; i < kMaxSegments - 1; ++i)
        if (i < gm.nseg - 1) r = n >= gm.bound[i] ? gs[i + 1] : r;
    return r;
}
__device__ __forceinline__ float seg_pick(const GammaMap &gm, const float (&f)[kMaxSegments],
                                          int64_t n) {
    float r = f[0];
#pragma unroll
    for (int i = 0; i < kMaxSegments - 1; ++i)
        r = (i < gm.nseg - 1 && n >= gm.bound[i]) ? f[i + 1] : r;
    return r;
}

// Wave-wide (64 lanes) reductions through cross-lane shuffles.
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Expand one 32-bit word of the 2-bit layout (16 codes) into four dwords of
// signed code bytes in natural order: dword j holds codes 4j..4j+3. The field
// u = (word >> 2j) & 0x03030303 is mapped to c = u - 1 by a byte permute whose
// table holds 0xFF, 0x00, 0x01 at selector values 0, 1, 2.
__device__ __forceinline__ void expand_2bit_word(uint32_t w, int out[4]) {
    constexpr uint32_t kTable = 0x000100FFu;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t u = (w >> (2 * j)) & 0x03030303u;
        out[j] = (int)__builtin_amdgcn_perm(0u, kTable, u);
    }
}

// 1-bit layout: bit j of byte i of a 32-code word is code 4j + i (1 = +1).
// Codes 16h .. 16h + 15 of the word (h = 0, 1) as four words of signed bytes:
// (w >> (4h + t)) & 0x01010101 selects byte 0 (-1) or byte 1 (+1) of the
// table 0x000001FF for codes 16h + 4t .. +3.
__device__ __forceinline__ void expand_1bit_half(uint32_t w, int h, int out[4]) {
    constexpr uint32_t kTable = 0x000001FFu;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t b = (w >> (4 * h + t)) & 0x01010101u;
        out[t] = (int)__builtin_amdgcn_perm(0u, kTable, b);
    }
}

// The same fields without the map to signed codes: dword j of out holds the
// stored u = c + 1 (0, 1, 2) of codes 4j..4j+3 of a 2-bit word. A product
// over u then differs from the product over c by the sum of the other
// operand: sum_k u_k x_k = sum_k c_k x_k + sum_k x_k.
__device__ __forceinline__ void fields_2bit_word(uint32_t w, int out[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = (int)((w >> (2 * j)) & 0x03030303u);
}

// 1-bit fields b = (c + 1) / 2 (0 or 1) of codes 16h + 4t .. +3, t = 0..3:
// sum_k c_k x_k = 2 sum_k b_k x_k - sum_k x_k.
__device__ __forceinline__ void fields_1bit_half(uint32_t w, int h, int out[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) out[t] = (int)((w >> (4 * h + t)) & 0x01010101u);
}

// Base-3 decode table: entry v (0..242) holds the five signed codes t_i - 1
// of v = sum t_i 3^i in bytes 0..4 (bytes 5..7 zero); entries 243..255 are
// zero. Built once per workgroup into LDS from this arithmetic definition.
__device__ __forceinline__ uint64_t base3_entry(uint32_t v) {
    if (v >= 243u) return 0;
    uint64_t e = 0;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const uint32_t t = v % 3u;
        v /= 3u;
        e |= (uint64_t)(uint8_t)(int8_t)((int)t - 1) << (8 * i);
    }
    return e;
}

}  // namespace bl
