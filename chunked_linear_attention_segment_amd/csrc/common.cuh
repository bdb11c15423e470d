// common.cuh -- device helpers shared by the HIP kernels of libmc (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mc {

typedef uint16_t bf16_t;  // bf16 storage (the upper 16 bits of an IEEE fp32)

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

// Load element i of a tensor stored as fp32 (T = float) or bf16 (T = bf16_t) as fp32.
template <typename T> __device__ __forceinline__ float ld(const T* p, size_t i);
template <> __device__ __forceinline__ float ld<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld<bf16_t>(const bf16_t* p, size_t i) {
    return bf16_to_f32(p[i]);
}

template <typename T> __device__ __forceinline__ void st(T* p, size_t i, float v);
template <> __device__ __forceinline__ void st<float>(float* p, size_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void st<bf16_t>(bf16_t* p, size_t i, float v) {
    p[i] = f32_to_bf16(v);
}

// The feature map phi applied to queries and keys: identity, or elu(z) + 1
// (z + 1 for z > 0, e^z otherwise) -- linear attention's kernel feature map.
__device__ __forceinline__ float feature(float z, int phi) {
    return phi == 0 ? z : (z > 0.f ? z + 1.f : __expf(z));
}

__device__ __forceinline__ float warp_sum(float v, int width) {
    for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, width);
    return v;
}

__device__ __forceinline__ float warp_max(float v, int width) {
    for (int o = width / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, width));
    return v;
}

}  // namespace mc
