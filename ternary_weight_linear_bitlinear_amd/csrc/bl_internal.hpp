// Internal declarations shared by the library's translation units (the
// kernels and the C ABI). Nothing here is part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <stddef.h>
#include <stdint.h>
#include <string>

namespace bl {

// Dry runs of the product dispatch (bitlinear_forward_plan). While a sink is
// installed on the calling thread, the product launchers append one line per
// launch they would make -- the kernel instantiation as the profiler names it,
// the grid, the block and the dynamic LDS bytes -- and launch nothing.
struct PlanSink {
    std::string text;
    int launches = 0;
};
inline thread_local PlanSink *t_plan = nullptr;

// Appends "<kernel> grid=GXxGY block=B lds=S" to the installed sink.
inline void plan_note(unsigned gx, unsigned gy, unsigned block, size_t lds, const char *fmt, ...) {
    char name[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(name, sizeof name, fmt, ap);
    va_end(ap);
    char line[640];
    snprintf(line, sizeof line, "%s grid=%ux%u block=%u lds=%zu\n", name, gx, gy, block, lds);
    t_plan->text += line;
    t_plan->launches += 1;
}

// Type names as the profiler prints kernel template arguments.
template <typename T> constexpr const char *type_name();
template <> constexpr const char *type_name<float>() { return "float"; }
template <> constexpr const char *type_name<uint16_t>() { return "unsigned short"; }

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kLayout2Bit = 0;
constexpr int kLayoutBase3 = 1;
constexpr int kLayout1Bit = 2;  // binary codes only
constexpr int kSchemeTernary = 0;
constexpr int kSchemeBinary = 1;
constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// Tokens per launch-row of the weight-streaming (decode) kernel; larger
// batches run as several such chunks in one launch (see skinny_handles).
constexpr int64_t kSkinnyMaxM = 16;

// Kernels using more than 64 KiB of dynamic LDS (gfx950 has 160 KiB per CU)
// must raise their limit, to what the kernel's static LDS leaves free (asking
// for all 160 KiB fails when the kernel also has static arrays), once per
// kernel and device. `done` is owned by the caller, one per kernel, with one
// bit per device (devices past 63 set the attribute on every call). Setting
// the attribute twice is harmless, so two threads racing here only repeat
// the call. A request above the free space is refused here instead of
// failing at launch.
constexpr size_t kLdsBytesPerCu = 160 * 1024;
using LdsFlag = std::atomic<uint64_t>;
template <typename F>
hipError_t allow_dynamic_lds(F *kernel, size_t bytes, LdsFlag *done) {
    if (bytes <= 65536) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t{1} << dev : 0;
    if (bit != 0 && (done->load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
    constexpr size_t kLdsBytes = kLdsBytesPerCu;
    hipFuncAttributes attr{};
    e = hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(kernel));
    if (e != hipSuccess) return e;
    if (attr.sharedSizeBytes + bytes > kLdsBytes) return hipErrorInvalidValue;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(kLdsBytes - attr.sharedSizeBytes));
    if (e == hipSuccess && bit != 0) done->fetch_or(bit, std::memory_order_release);
    return e;
}

// Compute units of the current device, queried once per device; 0 if the
// query fails (callers then size grids without it).
inline int device_cu_count() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0 &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) {
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Weight scales of a packed matrix whose rows form up to kMaxSegments
// consecutive segments, each quantised on its own (Q, K and V stacked into one
// matrix, for instance). Row n belongs to segment s = the number of bounds
// <= n; a plain matrix is one segment.
constexpr int kMaxSegments = 8;
struct GammaMap {
    const float *g;                     // device array, one gamma per segment
    int64_t bound[kMaxSegments - 1];    // first row of segments 1 .. nseg - 1
    int nseg;
    static GammaMap single(const float *gamma) {
        GammaMap m{};
        m.g = gamma;
        m.nseg = 1;
        return m;
    }
    // the same matrix seen from row `off` on (launches over a column range)
    GammaMap from_row(int64_t off) const {
        GammaMap m = *this;
        for (int i = 0; i < nseg - 1; ++i) m.bound[i] -= off;
        return m;
    }
};

inline int64_t row_bytes_2bit(int64_t K) { return ((K + 3) / 4 + 15) / 16 * 16; }
inline int64_t row_bytes_base3(int64_t K) { return ((K + 4) / 5 + 15) / 16 * 16; }
inline int64_t row_bytes_1bit(int64_t K) { return ((K + 7) / 8 + 15) / 16 * 16; }
inline int64_t row_bytes_of(int layout, int64_t K) {
    return layout == kLayout2Bit    ? row_bytes_2bit(K)
           : layout == kLayoutBase3 ? row_bytes_base3(K)
                                    : row_bytes_1bit(K);
}

// ---- weight quantisation (quant.hip) -------------------------------------
// Number of partial sums the mean reduction writes for `count` elements.
int absmean_parts(int64_t count);
// Bytes of workspace: one (sum|w|, sum w) pair of doubles per part.
size_t pack_workspace_bytes(int64_t count);
hipError_t launch_pack(const void *W, int dtype, int64_t N, int64_t K, int scheme,
                       int layout, float eps, uint8_t *packed, float *gamma,
                       double *workspace, hipStream_t stream);
hipError_t launch_quant_acts(const void *x, int dtype, int64_t M, int64_t K,
                             int8_t *xq, float *scale, hipStream_t stream);
// Device address and size of the library's own pack scratch on the current
// device (looked up on the first call per device).
hipError_t pack_scratch(double **ptr, size_t *bytes);
size_t pack_scratch_capacity();  // bytes of that scratch (host-only, no device needed)

// ---- products (skinny.hip, gemm.hip) -------------------------------------
// Whether the weight-streaming kernel (in 16-token chunks) or the tiled GEMM
// takes an M x N x K product in `layout`.
bool skinny_handles(int64_t M, int64_t N, int64_t K, int layout);
hipError_t launch_forward_skinny(const int8_t *xq, const float *scale,
                                 const uint8_t *packed, int layout,
                                 const GammaMap &gamma, int64_t M, int64_t N,
                                 int64_t K, void *y, int y_dtype, int32_t *acc,
                                 hipStream_t stream);
// Fused per-token quantisation + product for M <= fused_decode_max_m().
int64_t fused_decode_max_m();
hipError_t launch_linear_decode(const void *x, int x_dtype, const uint8_t *packed, int layout,
                                const GammaMap &gamma, int64_t M, int64_t N, int64_t K, void *y,
                                int y_dtype, int32_t *acc, hipStream_t stream);
hipError_t launch_forward_gemm(const int8_t *xq, const float *scale,
                               const uint8_t *packed, int layout,
                               const GammaMap &gamma, int64_t M, int64_t N,
                               int64_t K, void *y, int y_dtype, int32_t *acc,
                               hipStream_t stream);


// One token against base-3 codes by activation-side lookup tables (lut.hip).
hipError_t launch_forward_lut(const int8_t *xq, const float *scale, const uint8_t *packed,
                              const GammaMap &gamma, int64_t N, int64_t K, void *y, int y_dtype,
                              int32_t *acc, hipStream_t stream);

// ---- backward products (backward.hip) ------------------------------------
// grad_x [M, K] fp32 = gamma * grad_y [M, N] (bf16, or fp32 when grad_y_f32) x codes of
// packed [N, row_bytes] in `layout` (2-bit, base-3 or 1-bit).
hipError_t launch_backward_input(const void *grad_y, bool grad_y_f32, const uint8_t *packed,
                                 int layout, const float *gamma, int64_t M, int64_t N, int64_t K,
                                 float *grad_x, hipStream_t stream);
// grad_w [N, K] fp32 = grad_y^T ([M, N]) x x ([M, K]), both bf16, or both fp32 when f32.
hipError_t launch_backward_weight(const void *grad_y, const void *x, bool f32, int64_t M,
                                  int64_t N, int64_t K, float *grad_w, hipStream_t stream);
// out[0 : count) = 0 (a kernel, so it can be captured in a graph).
hipError_t launch_zero_f32(float *out, int64_t count, hipStream_t stream);

}  // namespace bl
