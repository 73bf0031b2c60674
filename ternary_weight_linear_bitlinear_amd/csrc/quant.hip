// Weight quantisation (absmean / 1-bit mean, code packing) and per-token INT8
// activation quantisation for gfx950.
//
// Sources: [QAT-en] "QAT and BitNet: A Deep Dive into 1-bit and 1.58-bit
// Quantization-Aware Training", sections "The Ternary Weight Recipe" and
// "The BitLinear Recipe"; [b158] "BitNet b1.58深度解析", §3.1 (absmean),
// §3.2 (per-token INT8), §2.3 / §6.3 (storage layouts), §5.2 (reference
// PyTorch quantisers).
//
// All three kernels are bound by HBM traffic: every element is read once
// with 16-byte vector loads and written once with 16-byte stores.
#include "bl_internal.hpp"
#include "device_util.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxParts = 1024;

// ---------------------------------------------------------------------------
// Pass 1 of the mean: each block sums |w| and w over a grid-strided share of
// the matrix in fp64 and writes one (sum|w|, sum w) pair. The grid size is a
// function of the element count only, so the result is deterministic.
template <typename T>
__global__ __launch_bounds__(kThreads) void absmean_partial_kernel(
    const T *__restrict__ w, int64_t count, double2 *__restrict__ parts) {
    constexpr int V = 8;  // elements per 16-byte (bf16) / 32-byte (fp32) load
    const int64_t nvec = count / V;
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t nth = (int64_t)gridDim.x * kThreads;
    double sa = 0.0, ss = 0.0;
    int64_t i = tid;
    for (; i + 3 * nth < nvec; i += 4 * nth) {
        float v[4][V];
#pragma unroll
        for (int u = 0; u < 4; ++u) load8(w + (i + u * nth) * V, v[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int e = 0; e < V; ++e) {
                sa += (double)fabsf(v[u][e]);
                ss += (double)v[u][e];
            }
        }
    }
    for (; i < nvec; i += nth) {
        float v[V];
        load8(w + i * V, v);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            sa += (double)fabsf(v[e]);
            ss += (double)v[e];
        }
    }
    // tail elements (count not a multiple of 8)
    for (int64_t j = nvec * V + tid; j < count; j += nth) {
        const float x = Elem<T>::get(w, j);
        sa += (double)fabsf(x);
        ss += (double)x;
    }
    __shared__ double red[2][kThreads / 64];
    sa = wave_sum(sa);
    ss = wave_sum(ss);
    const int wid = threadIdx.x / 64, lane = threadIdx.x % 64;
    if (lane == 0) { red[0][wid] = sa; red[1][wid] = ss; }
    __syncthreads();
    if (threadIdx.x == 0) {
        double a = 0.0, b = 0.0;
        for (int k = 0; k < kThreads / 64; ++k) { a += red[0][k]; b += red[1][k]; }
        parts[blockIdx.x] = make_double2(a, b);
    }
}

// Every pack block re-derives the two totals from the partials in the same
// fixed order, so all blocks (and every run) see the same gamma.
__device__ __forceinline__ double2 reduce_parts(const double2 *__restrict__ parts, int nparts) {
    __shared__ double red[2][kThreads / 64];
    double a = 0.0, b = 0.0;
    for (int p = threadIdx.x; p < nparts; p += kThreads) {
        const double2 v = parts[p];
        a += v.x;
        b += v.y;
    }
    a = wave_sum(a);
    b = wave_sum(b);
    const int wid = threadIdx.x / 64, lane = threadIdx.x % 64;
    if (lane == 0) { red[0][wid] = a; red[1][wid] = b; }
    __syncthreads();
    double ta = 0.0, tb = 0.0;
    for (int k = 0; k < kThreads / 64; ++k) { ta += red[0][k]; tb += red[1][k]; }
    return make_double2(ta, tb);
}

// Code decision for one weight.
//  Ternary: c = clamp(rint(fl32(w / d)), -1, 1) with d = fl32(gamma + eps).
//  The result is 0 exactly when fl32(|w| / d) <= 0.5, i.e. when the real
//  quotient |w| / d is at most 0.5 + 2^-25: that midpoint between 0.5 and the
//  next float rounds to 0.5 (even significand), anything above rounds up.
//  So c != 0 iff (double)|w| > d * (0.5 + 2^-25); the product of a 24-bit
//  and a 25-bit significand is exact in fp64, and |w| converts exactly, so
//  the comparison takes the same decision as the fp32 division followed by
//  round-half-even, for every input. A nonzero code has the sign of w.
//  Binary: c = +1 if w > alpha (fp32 compare), else -1.
template <int SCHEME>
struct CodeRule {
    double thr;   // ternary threshold
    float alpha;  // binary centre
    __device__ __forceinline__ int u_of(float w) const {  // u = c + 1
        if (SCHEME == kSchemeTernary) {
            const bool nz = (double)fabsf(w) > thr;
            return nz ? (w > 0.f ? 2 : 0) : 1;
        } else {
            return w > alpha ? 2 : 0;
        }
    }
};

template <int SCHEME>
__device__ __forceinline__ CodeRule<SCHEME> make_rule(const double2 *parts, int nparts,
                                                      int64_t count, float eps,
                                                      float *gamma_out) {
    const double2 tot = reduce_parts(parts, nparts);
    const float gamma = (float)(tot.x / (double)count);
    CodeRule<SCHEME> r;
    const float d = gamma + eps;
    r.thr = (double)d * (0.5 + 0x1p-25);
    r.alpha = (float)(tot.y / (double)count);
    if (blockIdx.x == 0 && threadIdx.x == 0) *gamma_out = gamma;
    return r;
}

// Load elements [k0, k0 + n) of row `row` as floats into v; positions past K
// are reported as padding through the returned count of valid elements.
template <typename T, int NE>
__device__ __forceinline__ int load_run(const T *__restrict__ w, int64_t row, int64_t K,
                                        int64_t k0, float v[NE]) {
    const T *p = w + row * K + k0;
    const int64_t left = K - k0;
    const int valid = left <= 0 ? 0 : (left >= NE ? NE : (int)left);
    const bool vec = (K % 8 == 0) && valid == NE;
    if (vec) {
#pragma unroll
        for (int e = 0; e < NE; e += 8) load8(p + e, v + e);
    } else {
#pragma unroll
        for (int e = 0; e < NE; ++e) v[e] = e < valid ? Elem<T>::get(p, e) : 0.f;
    }
    return valid;
}

// Pass 2, 2-bit layout: one thread writes one 16-byte unit = 64 codes, i.e.
// four 16-code words; word q, byte i, bits 2j hold code 16q + 4j + i.
template <typename T, int SCHEME>
__global__ __launch_bounds__(kThreads) void pack_2bit_kernel(
    const T *__restrict__ w, int64_t N, int64_t K, int64_t rb,
    const double2 *__restrict__ parts, int nparts, float eps,
    uint8_t *__restrict__ packed, float *__restrict__ gamma_out) {
    const CodeRule<SCHEME> rule =
        make_rule<SCHEME>(parts, nparts, N * K, eps, gamma_out);
    const int64_t units_per_row = rb / 16;
    const int64_t units = N * units_per_row;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < units;
         u += (int64_t)gridDim.x * kThreads) {
        const int64_t row = u / units_per_row;
        const int64_t k0 = (u % units_per_row) * 64;
        float v[64];
        const int valid = load_run<T, 64>(w, row, K, k0, v);
        uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 64; ++e) {
            const uint32_t code = e < valid ? (uint32_t)rule.u_of(v[e]) : 1u;
            const int q = e / 16, j = (e % 16) / 4, i = e % 4;
            word[q] |= code << (8 * i + 2 * j);
        }
        *reinterpret_cast<uint4 *>(packed + row * rb + (k0 / 4)) =
            make_uint4(word[0], word[1], word[2], word[3]);
    }
}

// Pass 2, base-3 layout: one thread writes one 16-byte unit = 80 codes; byte
// j is t0 + 3 t1 + 9 t2 + 27 t3 + 81 t4 of codes 5j..5j+4 (t = c + 1).
template <typename T, int SCHEME>
__global__ __launch_bounds__(kThreads) void pack_base3_kernel(
    const T *__restrict__ w, int64_t N, int64_t K, int64_t rb,
    const double2 *__restrict__ parts, int nparts, float eps,
    uint8_t *__restrict__ packed, float *__restrict__ gamma_out) {
    const CodeRule<SCHEME> rule =
        make_rule<SCHEME>(parts, nparts, N * K, eps, gamma_out);
    const int64_t units_per_row = rb / 16;
    const int64_t units = N * units_per_row;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < units;
         u += (int64_t)gridDim.x * kThreads) {
        const int64_t row = u / units_per_row;
        const int64_t k0 = (u % units_per_row) * 80;
        float v[80];
        const int valid = load_run<T, 80>(w, row, K, k0, v);
        uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            uint32_t b = 0;
            uint32_t p = 1;
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                const int e = 5 * j + i;
                const uint32_t t = e < valid ? (uint32_t)rule.u_of(v[e]) : 1u;
                b += t * p;
                p *= 3u;
            }
            word[j / 4] |= b << (8 * (j % 4));
        }
        *reinterpret_cast<uint4 *>(packed + row * rb + (k0 / 5)) =
            make_uint4(word[0], word[1], word[2], word[3]);
    }
}

// Pass 2, 1-bit layout (binary codes only; [QAT-en] "What Does BitLinear
// Change?" stores each +-1 weight in one bit): one thread writes 8 bytes = 64
// codes, i.e. two 32-code words; word q, byte i, bit j holds code 32q + 4j + i,
// 1 for +1. Padding bits are 0.
template <typename T>
__global__ __launch_bounds__(kThreads) void pack_1bit_kernel(
    const T *__restrict__ w, int64_t N, int64_t K, int64_t rb,
    const double2 *__restrict__ parts, int nparts, float eps,
    uint8_t *__restrict__ packed, float *__restrict__ gamma_out) {
    const CodeRule<kSchemeBinary> rule =
        make_rule<kSchemeBinary>(parts, nparts, N * K, eps, gamma_out);
    const int64_t halves_per_row = rb / 8;
    const int64_t halves = N * halves_per_row;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < halves;
         u += (int64_t)gridDim.x * kThreads) {
        const int64_t row = u / halves_per_row;
        const int64_t k0 = (u % halves_per_row) * 64;
        float v[64];
        const int valid = load_run<T, 64>(w, row, K, k0, v);
        uint32_t word[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 64; ++e) {
            const uint32_t bit = e < valid && rule.u_of(v[e]) == 2 ? 1u : 0u;
            const int q = e / 32, j = (e % 32) / 4, i = e % 4;
            word[q] |= bit << (8 * i + j);
        }
        *reinterpret_cast<uint2 *>(packed + row * rb + (k0 / 8)) = make_uint2(word[0], word[1]);
    }
}

// ---------------------------------------------------------------------------
// Per-token INT8 quantisation. One block per token row; thread t owns the
// 8-element chunks t, t + 256, ..., kept in registers between the max
// reduction and the quantisation (J chunks per thread; J = 0 re-reads the
// row from cache for rows longer than 8 * 256 * 8 elements). Each code is
// quant_word() (device_util.hpp): x / s (correctly rounded), then * 127, then round
// half to even.
__device__ __forceinline__ float block_max(float v) {
    __shared__ float red[kThreads / 64];
    v = wave_max(v);
    const int wid = threadIdx.x / 64, lane = threadIdx.x % 64;
    if (lane == 0) red[wid] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int k = 1; k < kThreads / 64; ++k) r = fmaxf(r, red[k]);
    return r;
}

// Eight consecutive elements as loaded (one 16-byte piece of bf16, two of
// fp32), widened to fp32 only after every load of the thread is in flight.
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> {
    uint4 a;
    __device__ __forceinline__ void load(const uint16_t *p) { a = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ void widen(float v[8]) const {
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
};
template <> struct Raw8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = *reinterpret_cast<const float4 *>(p);
        b = *reinterpret_cast<const float4 *>(p + 4);
    }
    __device__ __forceinline__ void widen(float v[8]) const {
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};

template <typename T, int J>
__global__ __launch_bounds__(kThreads) void quant_acts_kernel(
    const T *__restrict__ x, int64_t M, int64_t K, int8_t *__restrict__ xq,
    float *__restrict__ scale) {
    const int64_t m = blockIdx.x;
    const T *row = x + m * K;
    int8_t *out = xq + m * K;
    const bool vec = (K % 8 == 0);
    const int64_t nchunk = (K + 7) / 8;
    float amax = 0.f;
    if (J > 0) {
        float v[J > 0 ? J : 1][8];
        if (vec) {
            // every load first (chunks past the row re-read its last chunk and
            // are zeroed below), so the J loads overlap instead of each
            // waiting for the one before
            Raw8<T> raw[J > 0 ? J : 1];
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int64_t c = threadIdx.x + (int64_t)j * kThreads;
                raw[j].load(row + (c < nchunk ? c : nchunk - 1) * 8);
            }
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int64_t c = threadIdx.x + (int64_t)j * kThreads;
                raw[j].widen(v[j]);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[j][e] = c < nchunk ? v[j][e] : 0.f;
            }
        } else {
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int64_t c = threadIdx.x + (int64_t)j * kThreads;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[j][e] = c < nchunk && c * 8 + e < K ? Elem<T>::get(row, c * 8 + e) : 0.f;
            }
        }
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[j][e]));
        const float s = fmaxf(block_max(amax), 1e-6f);
        const float y = 1.0f / s;
        if (threadIdx.x == 0) scale[m] = s;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int64_t c = threadIdx.x + (int64_t)j * kThreads;
            if (c >= nchunk) continue;
            if (vec) {
                const float *w = v[j];
                *reinterpret_cast<uint2 *>(out + c * 8) =
                    make_uint2(quant4(w[0], w[1], w[2], w[3], s, y),
                               quant4(w[4], w[5], w[6], w[7], s, y));
            } else {
                for (int e = 0; e < 8; ++e)
                    if (c * 8 + e < K) out[c * 8 + e] = quant1(v[j][e], s, y);
            }
        }
    } else {
        for (int64_t k = threadIdx.x; k < K; k += kThreads)
            amax = fmaxf(amax, fabsf(Elem<T>::get(row, k)));
        const float s = fmaxf(block_max(amax), 1e-6f);
        const float y = 1.0f / s;
        if (threadIdx.x == 0) scale[m] = s;
        for (int64_t k = threadIdx.x; k < K; k += kThreads)
            out[k] = quant1(Elem<T>::get(row, k), s, y);
    }
}

template <typename T>
hipError_t quant_acts_t(const T *x, int64_t M, int64_t K, int8_t *xq, float *scale,
                        hipStream_t s) {
    const int64_t nchunk = (K + 7) / 8;
    const int64_t J = (nchunk + kThreads - 1) / kThreads;
    dim3 grid((unsigned)M), block(kThreads);
#define BL_QA(JJ) hipLaunchKernelGGL((quant_acts_kernel<T, JJ>), grid, block, 0, s, x, M, K, xq, scale)
    switch (J) {
        case 1: BL_QA(1); break;
        case 2: BL_QA(2); break;
        case 3: BL_QA(3); break;
        case 4: BL_QA(4); break;
        case 5: BL_QA(5); break;
        case 6: BL_QA(6); break;
        case 7: BL_QA(7); break;
        case 8: BL_QA(8); break;
        default: BL_QA(0); break;
    }
#undef BL_QA
    return hipGetLastError();
}

template <typename T>
hipError_t pack_t(const T *w, int64_t N, int64_t K, int scheme, int layout, float eps,
                  uint8_t *packed, float *gamma, double *ws, hipStream_t s) {
    const int64_t count = N * K;
    const int nparts = absmean_parts(count);
    double2 *parts = reinterpret_cast<double2 *>(ws);
    hipLaunchKernelGGL((absmean_partial_kernel<T>), dim3(nparts), dim3(kThreads), 0, s, w,
                       count, parts);
    const int64_t rb = row_bytes_of(layout, K);
    // one thread per 16-byte unit (8 bytes in the 1-bit layout)
    const int64_t units = N * (rb / (layout == kLayout1Bit ? 8 : 16));
    int64_t blocks = (units + kThreads - 1) / kThreads;
    if (blocks > 65536) blocks = 65536;
    dim3 grid((unsigned)blocks), block(kThreads);
    if (layout == kLayout1Bit) {  // binary codes only (the API checks the scheme)
        hipLaunchKernelGGL((pack_1bit_kernel<T>), grid, block, 0, s, w, N, K, rb, parts, nparts,
                           eps, packed, gamma);
    } else if (layout == kLayout2Bit) {
        if (scheme == kSchemeTernary)
            hipLaunchKernelGGL((pack_2bit_kernel<T, kSchemeTernary>), grid, block, 0, s, w, N, K,
                               rb, parts, nparts, eps, packed, gamma);
        else
            hipLaunchKernelGGL((pack_2bit_kernel<T, kSchemeBinary>), grid, block, 0, s, w, N, K,
                               rb, parts, nparts, eps, packed, gamma);
    } else {
        if (scheme == kSchemeTernary)
            hipLaunchKernelGGL((pack_base3_kernel<T, kSchemeTernary>), grid, block, 0, s, w, N,
                               K, rb, parts, nparts, eps, packed, gamma);
        else
            hipLaunchKernelGGL((pack_base3_kernel<T, kSchemeBinary>), grid, block, 0, s, w, N,
                               K, rb, parts, nparts, eps, packed, gamma);
    }
    return hipGetLastError();
}

}  // namespace

// Scratch of the allocation-free pack (bitlinear_pack_weights_noalloc): the
// mean's per-block partial sums, at most kMaxParts pairs of doubles (16 KiB),
// in a file-scope device array that every GPU the library runs on holds until
// the process ends. Host code never passes the array's name to a kernel (on
// the host it is only a stand-in for the symbol): each device's address is
// looked up once, with that device current, and kept here.
static __device__ __align__(256) double2 scratch[kMaxParts];
static std::atomic<double2 *> g_scratch_addr[64];

hipError_t pack_scratch(double **ptr, size_t *bytes) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    double2 *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void *addr = nullptr;
        e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (addr == nullptr) return hipErrorInvalidSymbol;
        p = static_cast<double2 *>(addr);
        g_scratch_addr[dev].store(p, std::memory_order_release);  // same value if two race
    }
    *ptr = reinterpret_cast<double *>(p);
    *bytes = sizeof(scratch);
    return hipSuccess;
}

size_t pack_scratch_capacity() { return sizeof(scratch); }

int absmean_parts(int64_t count) {
    const int64_t per = (int64_t)kThreads * 8 * 4;  // one unrolled sweep per block
    const int64_t p = (count + per - 1) / per;
    return (int)(p < 1 ? 1 : (p > kMaxParts ? kMaxParts : p));
}

size_t pack_workspace_bytes(int64_t count) {
    return (size_t)absmean_parts(count) * sizeof(double2);
}

hipError_t launch_pack(const void *W, int dtype, int64_t N, int64_t K, int scheme, int layout,
                       float eps, uint8_t *packed, float *gamma, double *workspace,
                       hipStream_t stream) {
    if (dtype == kF32)
        return pack_t(static_cast<const float *>(W), N, K, scheme, layout, eps, packed, gamma,
                      workspace, stream);
    return pack_t(static_cast<const uint16_t *>(W), N, K, scheme, layout, eps, packed, gamma,
                  workspace, stream);
}

hipError_t launch_quant_acts(const void *x, int dtype, int64_t M, int64_t K, int8_t *xq,
                             float *scale, hipStream_t stream) {
    if (dtype == kF32)
        return quant_acts_t(static_cast<const float *>(x), M, K, xq, scale, stream);
    return quant_acts_t(static_cast<const uint16_t *>(x), M, K, xq, scale, stream);
}

}  // namespace bl
