// decode.hip -- one MC decode step: online update, gate over the cached segments, read of
// every cached state (HBM-bound streaming) and the emission at a segment boundary.
//
// Memory Caching paper §3 (Eq. 4b) and §3.1 (Eq. 9-10) applied to one new token per
// sequence: the online memory takes the token first, the gate is a softmax over
// <u, MeanPooling> of every cached segment and of the online segment (its prefix mean),
// and y = gamma_on M_on phi(q) + sum_i gamma_i M^(i) phi(q).  When the online segment then
// holds C tokens its state and mean become cache slot n and the online memory restarts.
//
// Three launches on the caller's stream:
//   decode_update_gate  per (b,h): M_on += v phi(k)^T, online read, logits, softmax;
//                       emission of M_on into the cache
//   decode_stream       per (split, b,h): gamma-weighted read of a slice of cached states
//   decode_combine      per (b,h): y = online term + split partials; x-sum update and the
//                       emission of the segment mean (after every head has read the old sum)
#include "common.cuh"
#include "mc_internal.h"

namespace mc {

// Block-wide reductions over 256 threads (4 waves of 64).
__device__ __forceinline__ float block_max256(float v, float* red) {
    v = warp_max(v, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_sum256(float v, float* red) {
    v = warp_sum(v, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

template <typename T, typename TC, int DK, int DV>
__global__ __launch_bounds__(256) void decode_update_gate_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ u, const T* __restrict__ x, float* __restrict__ M_on,
    const float* __restrict__ xsum, int count, TC* __restrict__ M_cache,
    const float* __restrict__ P_cache, int n, int n_cap, int emit, int DG, int H, int xh,
    int phi, float* __restrict__ gamma, float* __restrict__ y_on) {
    constexpr int TPR = 256 / DV;
    constexpr int CPT = DK / TPR;
    __shared__ float sk[DK], sq[DK], sv[DV], sp[256];
    __shared__ float red[4];
    const size_t bh = blockIdx.x;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const size_t bx = (size_t)b * xh + (xh == 1 ? 0 : h);
    const int tid = threadIdx.x;
    for (int r = tid; r < DK; r += 256) {
        sk[r] = feature(ld(k, bh * DK + r), phi);
        sq[r] = feature(ld(q, bh * DK + r), phi);
    }
    for (int c = tid; c < DV; c += 256) sv[c] = ld(v, bh * DV + c);
    // prefix mean of the online segment including the new token
    const float inv = 1.f / (float)(count + 1);
    for (int e = tid; e < DG; e += 256) sp[e] = (xsum[bx * DG + e] + ld(x, bx * DG + e)) * inv;
    __syncthreads();

    // online memory update and read (row c, columns r0..r0+CPT-1 of this thread)
    const int c = tid / TPR, r0 = (tid % TPR) * CPT;
    float* mrow = M_on + (bh * DV + c) * DK + r0;
    float acc = 0.f;
    float mloc[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        mloc[i] = mrow[i] + sv[c] * sk[r0 + i];
        acc += mloc[i] * sq[r0 + i];
    }
    acc = warp_sum(acc, TPR);
    if (emit) {
        TC* dst = M_cache + ((bh * n_cap + n) * DV + c) * (size_t)DK + r0;
#pragma unroll
        for (int i = 0; i < CPT; ++i) { st(dst, i, mloc[i]); mrow[i] = 0.f; }
    } else {
#pragma unroll
        for (int i = 0; i < CPT; ++i) mrow[i] = mloc[i];
    }

    // logits: a_i = <u, P_i> for the n cached segments, a_on = <u, prefix mean>
    const T* ub = u + bh * DG;
    float a_on = 0.f;
    for (int e = 0; e < DG; ++e) a_on += ld(ub, e) * sp[e];
    float lmax = a_on;
    for (int i = tid; i < n; i += 256) {
        const float* Pi = P_cache + (bx * n_cap + i) * DG;
        float a = 0.f;
        for (int e = 0; e < DG; ++e) a += ld(ub, e) * Pi[e];
        gamma[bh * (n_cap + 1) + i] = a;
        lmax = fmaxf(lmax, a);
    }
    const float mx = block_max256(lmax, red);
    float lsum = (tid == 0) ? __expf(a_on - mx) : 0.f;
    for (int i = tid; i < n; i += 256) lsum += __expf(gamma[bh * (n_cap + 1) + i] - mx);
    const float z = block_sum256(lsum, red);
    const float inv_z = 1.f / z;
    for (int i = tid; i < n; i += 256) {
        float* g = gamma + bh * (n_cap + 1) + i;
        *g = __expf(*g - mx) * inv_z;
    }
    if (tid % TPR == 0) y_on[bh * DV + c] = __expf(a_on - mx) * inv_z * acc;
}

// Streams cached states [sp*per, min(n, (sp+1)*per)) of one (b,h).  Row c of a state is
// read as DK/8 chunks of 8 elements; thread tid always takes chunk (tid % CPR) of rows
// tid/CPR + pass*RPP, so its slice of phi(q) stays in registers.
template <typename T, typename TC, int DK, int DV>
__global__ __launch_bounds__(256) void decode_stream_kernel(const T* __restrict__ q,
                                                            const TC* __restrict__ M_cache,
                                                            const float* __restrict__ gamma,
                                                            int n, int n_cap, int per, int phi,
                                                            float* __restrict__ partial,
                                                            int splits) {
    constexpr int CPR = DK / 8;        // chunks per row
    constexpr int RPP = 256 / CPR;     // rows per pass
    constexpr int PASSES = DV / RPP;
    const int sp = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int kc = (tid % CPR) * 8;
    const int r0 = tid / CPR;
    float qv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = feature(ld(q, bh * DK + kc + e), phi);
    float acc[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) acc[p] = 0.f;
    const int i0 = sp * per, i1 = min(n, i0 + per);
    const float* g = gamma + bh * (n_cap + 1);
    for (int i = i0; i < i1; ++i) {
        const TC* Si = M_cache + (bh * n_cap + i) * (size_t)(DV * DK);
        const float gi = g[i];
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const TC* row = Si + (size_t)(r0 + p * RPP) * DK + kc;
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d += ld(row, e) * qv[e];
            acc[p] += gi * d;
        }
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const float r = warp_sum(acc[p], CPR);
        if (tid % CPR == 0) partial[(bh * splits + sp) * DV + r0 + p * RPP] = r;
    }
}

template <typename T>
__global__ void decode_combine_kernel(const float* __restrict__ y_on,
                                      const float* __restrict__ partial, int splits, int DV,
                                      const T* __restrict__ x, float* __restrict__ xsum,
                                      float* __restrict__ P_cache, int n, int n_cap, int emit,
                                      int C, int DG, int H, int xh, T* __restrict__ y) {
    const size_t bh = blockIdx.x;
    const int b = (int)(bh / H), h = (int)(bh % H);
    for (int c = threadIdx.x; c < DV; c += blockDim.x) {
        float acc = y_on[bh * DV + c];
        for (int sp = 0; sp < splits; ++sp) acc += partial[(bh * splits + sp) * DV + c];
        st(y, bh * DV + c, acc);
    }
    // x-sum of the online segment (shared by the heads when xh == 1: head 0 owns it)
    if (xh == 1 ? h == 0 : true) {
        const size_t bx = (size_t)b * xh + (xh == 1 ? 0 : h);
        for (int e = threadIdx.x; e < DG; e += blockDim.x) {
            const float s = xsum[bx * DG + e] + ld(x, bx * DG + e);
            if (emit) {
                P_cache[(bx * n_cap + n) * DG + e] = s / (float)C;
                xsum[bx * DG + e] = 0.f;
            } else {
                xsum[bx * DG + e] = s;
            }
        }
    }
}

template <typename T, typename TC, int DK, int DV>
static int launch_decode_t(const mc_dims& d, const void* q, const void* k, const void* v,
                           const void* u, const void* x, float* M_on, float* xsum, int count,
                           void* M_cache, float* P_cache, int n, int n_cap, int emit, void* y,
                           void* ws, hipStream_t st) {
    const DecodeWorkspace w = decode_workspace(d, n_cap, n);
    float* gamma = (float*)ws;
    float* partial = (float*)((char*)ws + w.gamma);
    float* y_on = (float*)((char*)ws + w.gamma + w.partial);
    const int BH = d.B * d.H;
    hipLaunchKernelGGL((decode_update_gate_kernel<T, TC, DK, DV>), dim3(BH), dim3(256), 0, st,
                       (const T*)q, (const T*)k, (const T*)v, (const T*)u, (const T*)x, M_on,
                       xsum, count, (TC*)M_cache, P_cache, n, n_cap, emit, d.d_g, d.H,
                       d.x_heads, d.phi, gamma, y_on);
    const int splits = w.splits;
    const int per = (n_cap + splits - 1) / splits;
    hipLaunchKernelGGL((decode_stream_kernel<T, TC, DK, DV>), dim3(splits, BH), dim3(256), 0, st,
                       (const T*)q, (const TC*)M_cache, gamma, n, n_cap, per, d.phi, partial,
                       splits);
    hipLaunchKernelGGL(decode_combine_kernel<T>, dim3(BH), dim3(128), 0, st, y_on, partial,
                       splits, d.d_v, (const T*)x, xsum, P_cache, n, n_cap, emit, d.seg_len,
                       d.d_g, d.H, d.x_heads, (T*)y);
    return (int)hipGetLastError();
}

int launch_decode_step(const mc_dims& d, const void* q, const void* k, const void* v,
                       const void* u, const void* x, float* M_on, float* xsum_on,
                       int count_on, void* M_cache, float* P_cache, int n_cached, int n_cap,
                       int emit, void* y, void* ws, void* stream) {
    hipStream_t st = (hipStream_t)stream;
#define MC_DEC(DK, DV)                                                                      \
    if (d.d_k == DK && d.d_v == DV)                                                         \
        return d.dtype == MC_BF16                                                           \
                   ? launch_decode_t<bf16_t, bf16_t, DK, DV>(d, q, k, v, u, x, M_on,        \
                                                             xsum_on, count_on, M_cache,    \
                                                             P_cache, n_cached, n_cap,      \
                                                             emit, y, ws, st)               \
                   : launch_decode_t<float, float, DK, DV>(d, q, k, v, u, x, M_on, xsum_on, \
                                                           count_on, M_cache, P_cache,      \
                                                           n_cached, n_cap, emit, y, ws,    \
                                                           st);
    MC_DEC(128, 128)
    MC_DEC(128, 64)
    MC_DEC(64, 128)
    MC_DEC(64, 64)
#undef MC_DEC
    return (int)hipErrorInvalidValue;
}

}  // namespace mc
