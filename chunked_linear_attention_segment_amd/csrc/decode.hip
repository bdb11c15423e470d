// decode.hip -- one MC decode step: online update, gate over the cached segments, read of
// every cached state (HBM-bound streaming) and the emission at a segment boundary.
//
// Memory Caching paper §3 (Eq. 4b) and §3.1 (Eq. 9-10) applied to one new token per
// sequence: the online memory takes the token first, the gate is a softmax over
// <u, MeanPooling> of every cached segment and of the online segment (its prefix mean),
// and y = gamma_on M_on phi(q) + sum_i gamma_i M^(i) phi(q).  When the online segment then
// holds C tokens its state and mean become cache slot n and the online memory restarts.
// Without u every logit is 0 and the read is the plain mean of the n + 1 memories: memory
// caching applied after pre-training (the paper's appendix on the MC variants), which
// decodes with an average of the cached memories and no learned weights.
//
// Two launches on the caller's stream:
//   decode_read     1 + R workgroups per (b,h).  Workgroup 0 updates the online memory with
//                   the token, reads it and forms the online logit from the prefix mean; at a
//                   segment boundary it moves the state into cache slot n.  Workgroup r >= 1
//                   takes a contiguous run of cached states: their logits <u, P_i>, a softmax
//                   local to the run (its max m_r and sum l_r of exp(a_i - m_r)) and the
//                   weighted read sum_i exp(a_i - m_r) M^(i) phi(q) of the run.
//   decode_combine  per (b,h): merges the partial softmaxes of the runs into y (the softmax
//                   over all logits, regrouped); x-sum update and the emission of the segment
//                   mean (after every head has read the old sum)
//
// The cached states are read once, with 16-byte non-temporal loads, so the step streams
// the cache at HBM rate; everything else is small.
#include <mutex>

#include "common.cuh"
#include "mc_internal.h"

namespace mc {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDecodeThreads = 256;

// Block-wide sum over 256 threads (4 waves of 64).
__device__ __forceinline__ float block_sum256(float v, float* red) {
    v = warp_sum(v, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// <16-byte chunk of a cached state row, matching slice of phi(q)>
template <typename TC> __device__ __forceinline__ float chunk_dot(u32x4_t c, const float* qv);
template <> __device__ __forceinline__ float chunk_dot<bf16_t>(u32x4_t c, const float* qv) {
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        d += __uint_as_float(c[e] << 16) * qv[2 * e];
        d += __uint_as_float(c[e] & 0xffff0000u) * qv[2 * e + 1];
    }
    return d;
}
template <> __device__ __forceinline__ float chunk_dot<float>(u32x4_t c, const float* qv) {
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) d += __uint_as_float(c[e]) * qv[e];
    return d;
}

// Four consecutive fp32 values of the online state stored at cache precision.
template <typename TC> __device__ __forceinline__ void store4(TC* p, const float* m);
template <> __device__ __forceinline__ void store4<float>(float* p, const float* m) {
    *reinterpret_cast<float4*>(p) = make_float4(m[0], m[1], m[2], m[3]);
}
template <> __device__ __forceinline__ void store4<bf16_t>(bf16_t* p, const float* m) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]));
}

struct DecodeArgs {
    const void *q, *k, *v, *u, *x;
    float* M_on;
    const float* xsum;
    void* M_cache;
    const float* P_cache;
    float* partial;  // [B*H, 1 + runs, DV]
    float* ml;       // [B*H, 1 + runs, 2]: (m, l) of each partial softmax
    int count, n, n_cap, per, runs, emit, DG, H, xh, phi;
};

// Workgroup 0 of (b,h): M_on += v phi(k)^T, read with phi(q), online logit; emission.
// Thread t covers 4-column chunks (t % CPR) of rows t / CPR + p * RPP.
template <typename T, typename TC, int DK, int DV>
__device__ __forceinline__ void decode_online(const DecodeArgs& a, size_t bh) {
    constexpr int CPR = DK / 4;
    constexpr int RPP = kDecodeThreads / CPR;
    constexpr int PASSES = DV / RPP;
    __shared__ float sk[DK], sq[DK], sv[DV], red[4];
    const int tid = threadIdx.x;
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);
    const size_t bx = (size_t)b * a.xh + (a.xh == 1 ? 0 : h);
    for (int r = tid; r < DK; r += kDecodeThreads) {
        sk[r] = feature(ld((const T*)a.k, bh * DK + r), a.phi);
        sq[r] = feature(ld((const T*)a.q, bh * DK + r), a.phi);
    }
    for (int c = tid; c < DV; c += kDecodeThreads) sv[c] = ld((const T*)a.v, bh * DV + c);
    // online logit: <u, prefix mean of the online segment including the new token>
    float au = 0.f;
    if (tid < a.DG && a.u)  // without u every logit is 0: the uniform (post-training) read
        au = ld((const T*)a.u, bh * a.DG + tid) *
             (a.xsum[bx * a.DG + tid] + ld((const T*)a.x, bx * a.DG + tid));
    const float a_on = block_sum256(au, red) / (float)(a.count + 1);  // syncs sk, sq, sv too

    const int kc = (tid % CPR) * 4, r0 = tid / CPR;
    float acc[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int c = r0 + p * RPP;
        float* mrow = a.M_on + (bh * DV + c) * DK + kc;
        const float4 m4 = *reinterpret_cast<const float4*>(mrow);
        float m[4] = {m4.x, m4.y, m4.z, m4.w};
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            m[e] += sv[c] * sk[kc + e];
            d += m[e] * sq[kc + e];
        }
        acc[p] = d;
        if (a.emit) {
            TC* dst = (TC*)a.M_cache + ((bh * a.n_cap + a.n) * DV + c) * (size_t)DK + kc;
            store4<TC>(dst, m);
            *reinterpret_cast<float4*>(mrow) = make_float4(0.f, 0.f, 0.f, 0.f);
        } else {
            *reinterpret_cast<float4*>(mrow) = make_float4(m[0], m[1], m[2], m[3]);
        }
    }
    const size_t slot = bh * (size_t)(1 + a.runs);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const float r = warp_sum(acc[p], CPR);
        if (tid % CPR == 0) a.partial[slot * DV + r0 + p * RPP] = r;
    }
    if (tid == 0) {
        a.ml[slot * 2] = a_on;
        a.ml[slot * 2 + 1] = 1.f;
    }
}

// Workgroup r >= 1 of (b,h): cached states [(r-1)*per, min(n, r*per)).  Thread t always takes
// the 16-byte chunk t + 256 p of a state (column chunk t % CPR of row t / CPR + p * RPP), so
// its slice of phi(q) stays in registers; SPI states are loaded per iteration.
template <typename T, typename TC, int DK, int DV>
__device__ __forceinline__ void decode_run(const DecodeArgs& a, size_t bh, int r) {
    constexpr int E = 16 / (int)sizeof(TC);   // elements per 16-byte chunk
    constexpr int CPR = DK / E;               // chunks per row
    constexpr int RPP = kDecodeThreads / CPR; // rows per pass
    constexpr int PASSES = DV / RPP;          // chunks per thread and state
    constexpr int SCH = DV * DK / E;          // chunks per state
    constexpr int SPI = PASSES >= 16 ? 1 : 16 / PASSES;
    __shared__ float su[256], sa[kDecodeRun];
    const int tid = threadIdx.x;
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);
    const size_t bx = (size_t)b * a.xh + (a.xh == 1 ? 0 : h);
    const int i0 = (r - 1) * a.per, cnt = min(a.n, i0 + a.per) - i0;  // >= 1 by the grid

    for (int e = tid; e < a.DG; e += kDecodeThreads)
        su[e] = a.u ? ld((const T*)a.u, bh * a.DG + e) : 0.f;
    const int kc = (tid % CPR) * E;
    float qv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) qv[e] = feature(ld((const T*)a.q, bh * DK + kc + e), a.phi);
    __syncthreads();
    // logits of the run: 16 lanes per cached segment
    {
        const int g = tid >> 4, l = tid & 15;
        for (int j = g; j < cnt; j += kDecodeThreads / 16) {
            const float* Pi = a.P_cache + (bx * a.n_cap + i0 + j) * a.DG;
            float s = 0.f;
            if (a.u)
                for (int e = l; e < a.DG; e += 16) s += su[e] * Pi[e];
            s = warp_sum(s, 16);
            if (l == 0) sa[j] = s;
        }
    }
    __syncthreads();
    float m = -INFINITY;
    for (int j = 0; j < cnt; ++j) m = fmaxf(m, sa[j]);

    float acc[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) acc[p] = 0.f;
    const u32x4_t* base =
        reinterpret_cast<const u32x4_t*>((const TC*)a.M_cache +
                                         (bh * a.n_cap + i0) * (size_t)(DV * DK)) + tid;
    int j = 0;
    for (; j + SPI <= cnt; j += SPI) {
        u32x4_t c[SPI][PASSES];
#pragma unroll
        for (int s = 0; s < SPI; ++s)
#pragma unroll
            for (int p = 0; p < PASSES; ++p)
                c[s][p] = __builtin_nontemporal_load(base + (size_t)(j + s) * SCH + p * 256);
#pragma unroll
        for (int s = 0; s < SPI; ++s) {
            const float w = __expf(sa[j + s] - m);
#pragma unroll
            for (int p = 0; p < PASSES; ++p) acc[p] += w * chunk_dot<TC>(c[s][p], qv);
        }
    }
    for (; j < cnt; ++j) {
        u32x4_t c[PASSES];
#pragma unroll
        for (int p = 0; p < PASSES; ++p)
            c[p] = __builtin_nontemporal_load(base + (size_t)j * SCH + p * 256);
        const float w = __expf(sa[j] - m);
#pragma unroll
        for (int p = 0; p < PASSES; ++p) acc[p] += w * chunk_dot<TC>(c[p], qv);
    }
    const size_t slot = bh * (size_t)(1 + a.runs) + r;
    const int r0 = tid / CPR;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const float s = warp_sum(acc[p], CPR);
        if (tid % CPR == 0) a.partial[slot * DV + r0 + p * RPP] = s;
    }
    if (tid == 0) {
        float l = 0.f;
        for (int jj = 0; jj < cnt; ++jj) l += __expf(sa[jj] - m);
        a.ml[slot * 2] = m;
        a.ml[slot * 2 + 1] = l;
    }
}

// One-dimensional grid: block id = bh * (1 + runs) + r.
template <typename T, typename TC, int DK, int DV>
__global__ __launch_bounds__(kDecodeThreads) void decode_read_kernel(DecodeArgs a) {
    const size_t bh = blockIdx.x / (1 + a.runs);
    const int r = (int)(blockIdx.x % (1 + a.runs));
    if (r == 0)
        decode_online<T, TC, DK, DV>(a, bh);
    else
        decode_run<T, TC, DK, DV>(a, bh, r);
}

// y = sum_r e^{m_r - m} Y_r / sum_r e^{m_r - m} l_r with m = max_r m_r: the softmax over all
// n + 1 logits, summed run by run.
template <typename T>
__global__ void decode_combine_kernel(const float* __restrict__ partial,
                                      const float* __restrict__ ml, int slots, int DV,
                                      const T* __restrict__ x, float* __restrict__ xsum,
                                      float* __restrict__ P_cache, int n, int n_cap, int emit,
                                      int C, int DG, int H, int xh, T* __restrict__ y) {
    const size_t bh = blockIdx.x;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const float* mlb = ml + bh * slots * 2;
    float m = -INFINITY;
    for (int s = 0; s < slots; ++s) m = fmaxf(m, mlb[2 * s]);
    float z = 0.f;
    for (int s = 0; s < slots; ++s) z += __expf(mlb[2 * s] - m) * mlb[2 * s + 1];
    const float inv_z = 1.f / z;
    for (int c = threadIdx.x; c < DV; c += blockDim.x) {
        float acc = 0.f;
        for (int s = 0; s < slots; ++s)
            acc += __expf(mlb[2 * s] - m) * partial[(bh * slots + s) * DV + c];
        st(y, bh * DV + c, acc * inv_z);
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
                           void* ws, int ws_cap, hipStream_t st) {
    const DecodeWorkspace w = decode_workspace(d, ws_cap, n);
    DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.u = u; a.x = x;
    a.M_on = M_on; a.xsum = xsum; a.M_cache = M_cache; a.P_cache = P_cache;
    a.partial = (float*)ws;
    a.ml = (float*)((char*)ws + w.partial);
    a.count = count; a.n = n; a.n_cap = n_cap; a.emit = emit;
    a.per = kDecodeRun;
    a.runs = (n + a.per - 1) / a.per;
    a.DG = d.d_g; a.H = d.H; a.xh = d.x_heads; a.phi = d.phi;
    const size_t BH = (size_t)d.B * d.H;
    const size_t blocks = BH * (size_t)(1 + a.runs);
    if (blocks > 0x7fffffffu || a.runs + 1 > w.slots) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_read_kernel<T, TC, DK, DV>), dim3((unsigned)blocks),
                       dim3(kDecodeThreads), 0, st, a);
    hipLaunchKernelGGL(decode_combine_kernel<T>, dim3((unsigned)BH), dim3(128), 0, st,
                       a.partial, a.ml, 1 + a.runs, d.d_v, (const T*)x, xsum, P_cache, n, n_cap,
                       emit, d.seg_len, d.d_g, d.H, d.x_heads, (T*)y);
    return (int)hipGetLastError();
}

int launch_decode_step(const mc_dims& d, const void* q, const void* k, const void* v,
                       const void* u, const void* x, float* M_on, float* xsum_on,
                       int count_on, void* M_cache, float* P_cache, int n_cached, int n_cap,
                       int emit, void* y, void* ws, int ws_cap, void* stream) {
    hipStream_t st = (hipStream_t)stream;
#define MC_DEC(DK, DV)                                                                      \
    if (d.d_k == DK && d.d_v == DV)                                                         \
        return d.dtype == MC_BF16                                                           \
                   ? launch_decode_t<bf16_t, bf16_t, DK, DV>(d, q, k, v, u, x, M_on,        \
                                                             xsum_on, count_on, M_cache,    \
                                                             P_cache, n_cached, n_cap,      \
                                                             emit, y, ws, ws_cap, st)       \
                   : launch_decode_t<float, float, DK, DV>(d, q, k, v, u, x, M_on, xsum_on, \
                                                           count_on, M_cache, P_cache,      \
                                                           n_cached, n_cap, emit, y, ws,    \
                                                           ws_cap, st);
    MC_DEC(128, 128)
    MC_DEC(128, 64)
    MC_DEC(64, 128)
    MC_DEC(64, 64)
#undef MC_DEC
    return (int)hipErrorInvalidValue;
}

// The decode step's scratch (the partial softmaxes of the runs) for callers that cannot
// allocate: one fixed buffer per GPU, shared by every call on that GPU.  Host code never
// uses the array's name as an address: the device address is taken once per device, with
// that device current, and kept in noalloc_dev.
static __device__ __align__(256) unsigned char scratch[MC_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex noalloc_mu;
void* noalloc_dev[kMaxDevices];
}  // namespace

int noalloc_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(noalloc_mu);
    if (!noalloc_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        if (!p) return (int)hipErrorInvalidSymbol;
        noalloc_dev[dev] = p;
    }
    *out = noalloc_dev[dev];
    return 0;
}

}  // namespace mc
