// Measurement probes for the benchmark (not part of the BitLinear library):
// the ceilings the hot path's kernels are compared with on the machine at
// hand, beside the datasheet peaks.
//   - a plain streaming read of a buffer (16-byte loads, nothing written but
//     one word per block in a branch that never runs for real data), for the
//     HBM ceiling at the decode layer's size and at a size far past the caches;
//   - an empty kernel, for the launch cadence of a captured graph;
//   - a loop of independent v_mfma_i32_32x32x32_i8 on register operands, for
//     the dense INT8 matrix-core rate at the clock the chip holds under load.
// C entry points take device pointers and a hipStream_t as void*; each
// returns 0, or the HIP error code of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

namespace {

// U loads of 16 bytes per thread in flight before any is consumed; the grid
// strides over the buffer. `tag` is never matched by the xor of real data in
// practice; the store only keeps the loads alive.
template <int U>
__global__ __launch_bounds__(256) void read_kernel(const uint4 *__restrict__ p, int64_t n16,
                                                   uint32_t tag, uint32_t *__restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t x = 0;
    for (int64_t base = (int64_t)blockIdx.x * 256 + threadIdx.x; base < n16;
         base += stride * U) {
        uint4 v[U];
        if (base + (U - 1) * stride < n16) {  // every load in range: no guards
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = p[base + u * stride];
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = base + u * stride;
                v[u] = i < n16 ? p[i] : make_uint4(0u, 0u, 0u, 0u);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (x == tag) out[blockIdx.x] = x;
}

__global__ void empty_kernel() {}

// Each wave keeps CH independent accumulator chains; every iteration issues
// one v_mfma_i32_32x32x32_i8 per chain (2 * 32 * 32 * 32 = 65536 ops each).
template <int CH>
__global__ __launch_bounds__(256) void mfma_i8_kernel(int iters, int seed,
                                                      int32_t *__restrict__ out) {
    const v4i a = {seed, seed + 1, seed + 2, (int)threadIdx.x};
    const v4i b = {seed ^ 5, seed ^ 7, seed ^ 9, (int)blockIdx.x};
    v16i acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[c][e] = c + e;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[c][e];
    if (s == 0x7fffffff) out[blockIdx.x] = s;
}

}  // namespace

extern "C" {

// Streaming read of `bytes` (a multiple of 16) at p; `blocks` blocks of 256
// threads, `unroll` in {1, 2, 4, 8} loads in flight per thread. out needs
// `blocks` words (written only on a tag match).
int probe_read(const void *p, int64_t bytes, int blocks, int unroll, uint32_t *out,
               void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint4 *q = static_cast<const uint4 *>(p);
    const int64_t n16 = bytes / 16;
    const uint32_t tag = 0x9E3779B9u;
    switch (unroll) {
        case 1: hipLaunchKernelGGL(read_kernel<1>, dim3(blocks), dim3(256), 0, s, q, n16, tag, out); break;
        case 2: hipLaunchKernelGGL(read_kernel<2>, dim3(blocks), dim3(256), 0, s, q, n16, tag, out); break;
        case 4: hipLaunchKernelGGL(read_kernel<4>, dim3(blocks), dim3(256), 0, s, q, n16, tag, out); break;
        default: hipLaunchKernelGGL(read_kernel<8>, dim3(blocks), dim3(256), 0, s, q, n16, tag, out); break;
    }
    return (int)hipGetLastError();
}

int probe_empty(void *stream) {
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
    return (int)hipGetLastError();
}

// blocks x 4 waves, each `iters` iterations of 8 independent chains. Returns
// the launch status; the caller times it (ops = blocks * 4 * iters * 8 * 65536).
int probe_mfma_i8(int blocks, int iters, int32_t *out, void *stream) {
    hipLaunchKernelGGL(mfma_i8_kernel<8>, dim3(blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), iters, 3, out);
    return (int)hipGetLastError();
}

}  // extern "C"
