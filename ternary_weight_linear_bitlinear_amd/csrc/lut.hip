// Decode GEMV for the base-3 layout by lookup tables instead of expanding the
// weights. [b158] "BitNet b1.58深度解析" §2.3 and §6.3 note that five
// ternary weights per byte must be unpacked by table lookup or bit operations;
// the study notes page (medicago.top, "BitNet（1.58‑bit）体系", Q5) lists
// table-lookup implementations of weights and activations among the CPU
// kernels' advantages. This kernel puts the tables on the activation side and
// exists to compare that scheme with the in-register decode on MI355X.
//
// One byte v holds five trits t0..t4 (t = c + 1, v = t0 + 3 t1 + 9 t2 + 27 t3
// + 81 t4), so its contribution sum_i c_i x_i splits exactly into a part from
// (t0, t1) = v mod 9 and a part from (t2, t3, t4) = v / 9. For every group of
// five activations the workgroup tabulates both parts (9 + 27 int16 sums) in
// LDS; a weight byte then costs two table reads and an add. v / 9 is
// (v * 57) >> 9, exact for every byte value.
//
// A workgroup owns 16 weight rows, 16 threads per row, each thread taking
// every 16th 16-byte unit of its row. K is processed in chunks of 1024 groups
// (5120 codes, 72 KiB of tables). The chunk's activations are loaded before
// the weights (memory counters complete in issue order), so the tables are
// built while the weight loads are in flight. Partial sums of a row are added
// across its 16 threads with cross-lane shuffles; the sums are exact INT32.
#include "bl_internal.hpp"
#include "device_util.hpp"

namespace bl {
namespace {

constexpr int kLutRows = 16;
constexpr int kLutThreads = 256;            // 16 threads per row
constexpr int kLutGroups = 1024;            // groups of five codes per K chunk
constexpr int kLutEntries = 36;             // 9 + 27 partial sums per group
constexpr int kLutUnits = kLutGroups / 16;  // 16-byte units of a row per chunk
constexpr int kLutUnitsPerThread = kLutUnits / 16;
constexpr int kLutGroupsPerThread = kLutGroups / kLutThreads;
// (+16 bytes: a byte value outside 0..242, which packing never writes, reads at
// most two entries past the last group's tables and stays inside the block)
constexpr size_t kLutSmem = (size_t)kLutGroups * kLutEntries * sizeof(int16_t) + 16;

template <typename YT>
__global__ __launch_bounds__(kLutThreads) void lut_gemv_kernel(
    const int8_t *__restrict__ xq, const float *__restrict__ scale,
    const uint8_t *__restrict__ packed, const GammaMap gm, int64_t N, int64_t K, int64_t rb,
    YT *__restrict__ y, int32_t *__restrict__ acc_out) {
    extern __shared__ __attribute__((aligned(16))) int16_t tab[];
    const int tid = threadIdx.x;
    const int row = tid / 16, part = tid % 16;
    const int64_t n = (int64_t)blockIdx.x * kLutRows + row;
    const bool row_ok = n < N;
    const uint8_t *wrow = packed + (row_ok ? n : 0) * rb;
    const int64_t units = rb / 16;
    float gs[kMaxSegments];
    load_gammas(gm, gs);

    int32_t acc = 0;
    for (int64_t u0 = 0; u0 < units; u0 += kLutUnits) {
        const int64_t g0 = u0 * 16;  // first group of the chunk
        // 1. the five activations of each group this thread tabulates; codes
        //    past K read a valid address and are zeroed when used
        int32_t xr[kLutGroupsPerThread][5];
        bool xk[kLutGroupsPerThread][5];
#pragma unroll
        for (int j = 0; j < kLutGroupsPerThread; ++j)
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                const int64_t k = 5 * (g0 + tid + kLutThreads * j) + i;
                xk[j][i] = k < K;
                xr[j][i] = xq[xk[j][i] ? k : 0];
            }
        // 2. this thread's weight units of the chunk
        uint4 wv[kLutUnitsPerThread];
        bool wok[kLutUnitsPerThread];
#pragma unroll
        for (int i = 0; i < kLutUnitsPerThread; ++i) {
            const int64_t u = u0 + part + 16 * i;
            wok[i] = row_ok && u < units;
            wv[i] = *reinterpret_cast<const uint4 *>(wok[i] ? wrow + u * 16 : packed);
        }
        // 3. tables: entry lo = t0 + 3 t1 holds (t0-1) x0 + (t1-1) x1; entry
        //    9 + hi, hi = t2 + 3 t3 + 9 t4, holds (t2-1) x2 + (t3-1) x3 + (t4-1) x4
        lds_barrier();  // the previous chunk's lookups are done
#pragma unroll
        for (int j = 0; j < kLutGroupsPerThread; ++j) {
            int x[5];
#pragma unroll
            for (int i = 0; i < 5; ++i) x[i] = xk[j][i] ? xr[j][i] : 0;
            int16_t e[kLutEntries];
#pragma unroll
            for (int t1 = 0; t1 < 3; ++t1)
#pragma unroll
                for (int t0 = 0; t0 < 3; ++t0)
                    e[t0 + 3 * t1] = (int16_t)((t0 - 1) * x[0] + (t1 - 1) * x[1]);
#pragma unroll
            for (int t4 = 0; t4 < 3; ++t4)
#pragma unroll
                for (int t3 = 0; t3 < 3; ++t3)
#pragma unroll
                    for (int t2 = 0; t2 < 3; ++t2)
                        e[9 + t2 + 3 * t3 + 9 * t4] =
                            (int16_t)((t2 - 1) * x[2] + (t3 - 1) * x[3] + (t4 - 1) * x[4]);
            // 72 bytes per group: nine 8-byte stores
            uint2 *dst = reinterpret_cast<uint2 *>(tab + (tid + kLutThreads * j) * kLutEntries);
#pragma unroll
            for (int q = 0; q < kLutEntries / 4; ++q) {
                const uint32_t a = (uint16_t)e[4 * q] | ((uint32_t)(uint16_t)e[4 * q + 1] << 16);
                const uint32_t b = (uint16_t)e[4 * q + 2] | ((uint32_t)(uint16_t)e[4 * q + 3] << 16);
                dst[q] = make_uint2(a, b);
            }
        }
        lds_barrier();
        // 4. two table reads per weight byte
#pragma unroll
        for (int i = 0; i < kLutUnitsPerThread; ++i) {
            if (!wok[i]) continue;
            const uint32_t w[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
            const int gl = (part + 16 * i) * 16;  // chunk-local group of byte 0
#pragma unroll
            for (int b = 0; b < 16; ++b) {
                const uint32_t v = (w[b / 4] >> (8 * (b % 4))) & 0xFFu;
                const uint32_t hi = (v * 57u) >> 9;
                const uint32_t lo = v - 9u * hi;
                const int16_t *t = tab + (gl + b) * kLutEntries;
                acc += (int32_t)t[lo] + (int32_t)t[9 + hi];
            }
        }
    }

    // the 16 threads of a row are 16 consecutive lanes
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (part != 0 || !row_ok) return;
    // one matrix: one factor; stacked segments pick the row's own (a
    // wave-uniform branch, so the common case skips the selection)
    float f;
    if (gm.nseg == 1) {
        f = gs[0] * scale[0] / 127.0f;
    } else {
        float fs[kMaxSegments];
        seg_factors(gm, gs, scale[0], fs);
        f = seg_pick(gm, fs, n);
    }
    const float v = (float)acc * f;
    if constexpr (sizeof(YT) == 4)
        y[n] = v;
    else
        y[n] = (YT)f32_to_bf16_rne(v);
    if (acc_out) acc_out[n] = acc;
}

template <typename YT>
hipError_t launch_lut_t(const int8_t *xq, const float *scale, const uint8_t *packed,
                        const GammaMap &gamma, int64_t N, int64_t K, YT *y, int32_t *acc,
                        hipStream_t s) {
    auto kern = lut_gemv_kernel<YT>;
    static LdsFlag lds_raised{0};
    hipError_t e = allow_dynamic_lds(kern, kLutSmem, &lds_raised);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)((N + kLutRows - 1) / kLutRows)), dim3(kLutThreads),
                       kLutSmem, s, xq, scale, packed, gamma, N, K, row_bytes_base3(K), y, acc);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_lut(const int8_t *xq, const float *scale, const uint8_t *packed,
                              const GammaMap &gamma, int64_t N, int64_t K, void *y, int y_dtype,
                              int32_t *acc, hipStream_t stream) {
    if (y_dtype == kF32)
        return launch_lut_t(xq, scale, packed, gamma, N, K, static_cast<float *>(y), acc, stream);
    return launch_lut_t(xq, scale, packed, gamma, N, K, static_cast<uint16_t *>(y), acc, stream);
}

}  // namespace bl
