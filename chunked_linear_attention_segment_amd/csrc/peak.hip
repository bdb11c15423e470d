// peak.hip -- in-run ceilings of the two units the Memory Caching path is bound by: the bf16
// matrix cores (the gated prefill read) and HBM (the decode read of the cached states).
//
// These kernels are measurement aids for the benchmark, not part of the Memory Caching
// operations: they do no Memory Caching arithmetic, and libmc does not link them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mc_peak.h"

typedef __bf16 pk_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float pk_f32x16_t __attribute__((ext_vector_type(16)));

namespace {

constexpr int kChains = 4;  // independent accumulators per wave: hides the MFMA dependency latency

// Back-to-back v_mfma_f32_32x32x16_bf16 from registers: no memory traffic inside the loop.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* out) {
    const int lane = threadIdx.x & 63;
    // small operands (|a*b| ~ 1e-6) keep the accumulators finite over any loop length
    pk_bf16x8_t a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(1e-3f * (float)((lane + j) & 7));
        b[j] = (__bf16)(1e-3f * (float)((lane * 3 + j) & 7));
    }
    pk_f32x16_t acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int c = 0; c < kChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Streaming read: workgroup g reads the contiguous 16-byte words [g*per, (g+1)*per) with
// non-temporal loads, four per thread in flight, and folds them with xor; one word per wave is
// written so the loads cannot be dropped.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ src,
                                                          size_t n16, size_t per,
                                                          uint32_t* __restrict__ out) {
    const size_t b0 = (size_t)blockIdx.x * per;
    const size_t b1 = b0 + per < n16 ? b0 + per : n16;
    uint32_t acc = 0;
    for (size_t i = b0 + threadIdx.x; i < b1; i += 4 * 256) {
        u32x4_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            v[u] = i + u * 256 < b1 ? __builtin_nontemporal_load(src + i + u * 256)
                                    : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if ((threadIdx.x & 63) == 0) out[((size_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6] = acc;
}

// Plain copy of n16 16-byte words: the kernel of known traffic (n16*16 bytes read, the same
// written) that HBM byte counters are scaled by.
__global__ __launch_bounds__(256) void copy16_kernel(const uint4* __restrict__ src,
                                                     uint4* __restrict__ dst, size_t n16) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

}  // namespace

extern "C" {

int mcpeak_mfma_out_floats(int n_blocks) { return n_blocks * 256; }

double mcpeak_mfma_flops(int n_blocks, int iters) {
    // per wave and iteration: 4 * kChains MFMAs of 32x32x16 multiply-adds
    return (double)n_blocks * 4.0 * iters * 4.0 * kChains * (2.0 * 32 * 32 * 16);
}

int mcpeak_mfma(int n_blocks, int iters, float* out, void* stream) {
    if (n_blocks <= 0 || iters <= 0 || !out) return 1;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(n_blocks), dim3(256), 0, (hipStream_t)stream, iters,
                       out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int mcpeak_stream_out_words(int n_blocks) { return n_blocks * 4; }

int mcpeak_stream_read(const void* src, size_t bytes, int n_blocks, uint32_t* out, void* stream) {
    if (!src || !out || n_blocks <= 0 || (bytes & 15) || ((uintptr_t)src & 15)) return 1;
    const size_t n16 = bytes / 16;
    const size_t per = (n16 + n_blocks - 1) / n_blocks;
    hipLaunchKernelGGL(stream_read_kernel, dim3(n_blocks), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4_t*)src, n16, per, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int mcpeak_copy(const void* src, void* dst, size_t bytes, int n_blocks, void* stream) {
    if (!src || !dst || n_blocks <= 0 || (bytes & 15) || ((uintptr_t)src & 15) ||
        ((uintptr_t)dst & 15))
        return 1;
    hipLaunchKernelGGL(copy16_kernel, dim3(n_blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint4*)src, (uint4*)dst, bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
