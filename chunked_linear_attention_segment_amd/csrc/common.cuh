// common.cuh -- device helpers shared by the HIP kernels of libmc (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mc {

typedef uint16_t bf16_t;  // bf16 storage (the upper 16 bits of an IEEE fp32)

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __bf16 hw_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float hw_f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 in one 32-bit word (lo in bits 0..15), round to nearest even: the
// gfx950 conversion instruction (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const hw_f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, hw_bf16x2_t));
}

// fp32 -> bf16, round to nearest even.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return (bf16_t)(pack_bf16x2(f, 0.f) & 0xffffu); }

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

// Load 8 consecutive elements starting at element i (16-byte aligned for bf16, 32-byte for
// fp32) as fp32.
template <typename T> __device__ __forceinline__ void ld8(const T* p, size_t i, float* o);
template <> __device__ __forceinline__ void ld8<float>(const float* p, size_t i, float* o) {
    const float4 a = *reinterpret_cast<const float4*>(p + i);
    const float4 b = *reinterpret_cast<const float4*>(p + i + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
template <> __device__ __forceinline__ void ld8<bf16_t>(const bf16_t* p, size_t i, float* o) {
    const uint4 v = *reinterpret_cast<const uint4*>(p + i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        o[2 * e] = __uint_as_float(w[e] << 16);
        o[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}

// Eight consecutive values v[e] * scale stored at p[i..i+8) (16 bytes for bf16, 32 for fp32;
// i a multiple of 8 from an aligned base).
template <typename T> __device__ __forceinline__ void st8(T* p, size_t i, const float* v, float scale);
template <> __device__ __forceinline__ void st8<float>(float* p, size_t i, const float* v, float scale) {
    *reinterpret_cast<float4*>(p + i) = make_float4(v[0] * scale, v[1] * scale, v[2] * scale, v[3] * scale);
    *reinterpret_cast<float4*>(p + i + 4) = make_float4(v[4] * scale, v[5] * scale, v[6] * scale, v[7] * scale);
}
template <> __device__ __forceinline__ void st8<bf16_t>(bf16_t* p, size_t i, const float* v, float scale) {
    *reinterpret_cast<uint4*>(p + i) =
        make_uint4(pack_bf16x2(v[0] * scale, v[1] * scale), pack_bf16x2(v[2] * scale, v[3] * scale),
                   pack_bf16x2(v[4] * scale, v[5] * scale), pack_bf16x2(v[6] * scale, v[7] * scale));
}

// The feature map phi applied to queries and keys: identity, or elu(z) + 1
// (z + 1 for z > 0, e^z otherwise) -- linear attention's kernel feature map.
__device__ __forceinline__ float feature(float z, int phi) {
    return phi == 0 ? z : (z > 0.f ? z + 1.f : __expf(z));
}

// Segment boundaries (SegArg, mc_internal.h): first token and length of segment s, and the
// segment of token t (the largest s with off[s] <= t); n = 0 is the constant length C.
template <typename SA>
__device__ __forceinline__ int seg_first(const SA& sg, int s, int C) {
    return sg.n ? sg.off[s] : s * C;
}
template <typename SA>
__device__ __forceinline__ int seg_length(const SA& sg, int s, int C, int L) {
    return sg.n ? sg.off[s + 1] - sg.off[s] : min(C, L - s * C);
}
template <typename SA>
__device__ __forceinline__ int seg_of(const SA& sg, int t, int C) {
    if (!sg.n) return t / C;
    int lo = 0, hi = sg.n;  // off[lo] <= t < off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sg.off[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
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
