// backward.hip -- gradients of the GRM prefill with respect to Q, K, V, U and X.
//
// Memory Caching paper: the segment memories of §3 (Eq. 4b), the softmax context gate of §3.1
// (Eq. 10) and the gated read (Eq. 9), differentiated token by token.  With o_i = M^(i) phi(q_t)
// for the cached segments i < s, o_s = M_t^(s) phi(q_t) for the online one, gamma the gate
// and y_t = sum_i gamma_i o_i:
//   dgamma_i = <dy_t, o_i>,  da_i = gamma_i (dgamma_i - D_t),  D_t = sum_i gamma_i dgamma_i
//   du_t = sum_{i<s} da_i P_i + da_s ptilde_t,  dP_i = sum_t da_t^(i) u_t,  dptilde_t = da_s u_t
//   dphi(q_t) = sum_{i<s} gamma_i M^(i)^T dy_t + gamma_s M_t^(s)^T dy_t
//   dM^(i) = sum_{t after segment i} gamma_t^(i) dy_t phi(q_t)^T
//   for r in segment i:  E_r = dM^(i) + sum_{t >= r in segment i} gamma_t^(s) dy_t phi(q_t)^T,
//                        dv_r = E_r phi(k_r),  dphi(k_r) = E_r^T v_r
//   dx_r = dP_i / |S_i| + sum_{t >= r in segment i} da_t^(s) u_t / (j_t + 1)
//   dq = dphi(q) phi'(q), dk = dphi(k) phi'(k), phi'(z) = min(phi(z), 1) for elu + 1.
//
// The launches, in order (one stream), for the generic path (fp32, or widths the MFMA
// backward does not take; the bf16 d_k = d_v = 128 path replaces the first four lines with
// the kernels of backward_mfma.hip):
//   aon, xps            online logits and segment-causal prefix sums of X (forward helpers)
//   scan_online x2      O_on[t] = M_t^(s) phi(q_t), and Ot[t] = M_t^(s)T dy_t (the same scan
//                       with q := dy, k := v, v := phi(k))
//   bwd_cached_kernel   per token: the softmax statistics, dgamma_i for every segment read,
//                       D_t, and the cached part of dphi(q_t)
//   bwd_gate_kernel     per token: da_i (written over dgamma), du_t, and dq = (cached part +
//                       gamma_s Ot[t]) phi'(q)
//   bwd_dm_kernel       per cached segment i: dM^(i)
//   bwd_online_kernel   per segment, tokens in reverse: E_r and E_r^T, dv_r and dk_r
//   bwd_dxw_kernel, bwd_dp_kernel, bwd_dxf_kernel
//                       the x gradients: per-token prefix-mean terms, partial dP_i over token
//                       ranges, then dP_i / |S_i| plus the reverse cumulative sums
// Every kernel accumulates in fp32 registers; all gradients are written in fp32.
#include "common.cuh"
#include "mc_internal.h"

namespace mc {

namespace {

constexpr int BTT = 32;  // tokens per tile

__device__ __forceinline__ float dfeature_from(float f, int phi) {
    return phi ? fminf(f, 1.f) : 1.f;  // elu + 1: 1 where phi(z) = z + 1 > 1, e^z = phi(z) else
}

// Softmax statistics, dgamma for every segment a token reads, D_t, and the cached part of
// dphi(q).  8 threads per token: thread p owns value columns c = p + 8m and key columns
// r = p + 8m; states are read from global memory (shared by the tile's tokens through L1/L2).
template <typename T, typename TS, int DK, int DV>
__global__ __launch_bounds__(256) void bwd_cached_kernel(
    const T* __restrict__ Q, const T* __restrict__ U, const float* __restrict__ aon,
    const TS* __restrict__ S, const float* __restrict__ P, const float* __restrict__ O_on,
    const T* __restrict__ dY, int L, int C, int NS, int DG, int H, int xh, int phi,
    float* __restrict__ dG, float* __restrict__ lse_o, float* __restrict__ D_o,
    float* __restrict__ gs_o, float* __restrict__ dQ) {
    constexpr int CPV = DV / 8, CPK = DK / 8;
    __shared__ float sq[BTT][DK];
    __shared__ float sdy[BTT][DV];
    const int tile0 = blockIdx.x * BTT;
    const size_t bh = blockIdx.y;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const size_t bx = (size_t)b * xh + (xh == 1 ? 0 : h);
    const int tid = threadIdx.x, tt = tid / 8, p = tid % 8;
    const int t = tile0 + tt;
    const bool valid = t < L;
    const int tc = valid ? t : L - 1;
    const int s = tc / C;
    const int s_hi = (min(L, tile0 + BTT) - 1) / C;

    for (int e = tid; e < BTT * DK; e += 256) {
        const int tk = min(tile0 + e / DK, L - 1);
        sq[e / DK][e % DK] = feature(ld(Q, (bh * L + tk) * DK + e % DK), phi);
    }
    for (int e = tid; e < BTT * DV; e += 256) {
        const int tk = min(tile0 + e / DV, L - 1);
        sdy[e / DV][e % DV] = ld(dY, (bh * L + tk) * DV + e % DV);
    }
    __syncthreads();

    const int gch = DG / 8;
    const size_t urow = (bh * L + tc) * DG;
    const float a_on = aon[bh * L + tc];
    // pass 1: max and sum of the softmax over the segments 0..s
    float mx = a_on, l = 1.f;
    for (int i = 0; i < s_hi; ++i) {
        const float* Pi = P + (bx * NS + i) * DG;
        float a = 0.f;
        for (int e = p * gch; e < (p + 1) * gch; ++e) a += ld(U, urow + e) * Pi[e];
        a = warp_sum(a, 8);
        if (i < s) {
            const float mn = fmaxf(mx, a);
            l = l * __expf(mx - mn) + __expf(a - mn);
            mx = mn;
        }
    }
    const float lse = mx + __logf(l);
    // pass 2: dgamma_i = <dy, M^(i) phi(q)> and gamma_i M^(i)^T dy for every cached segment
    float dq[CPK];
#pragma unroll
    for (int m = 0; m < CPK; ++m) dq[m] = 0.f;
    float D = 0.f;
    for (int i = 0; i < s_hi; ++i) {
        const float* Pi = P + (bx * NS + i) * DG;
        float a = 0.f;
        for (int e = p * gch; e < (p + 1) * gch; ++e) a += ld(U, urow + e) * Pi[e];
        a = warp_sum(a, 8);
        if (i >= s) continue;  // uniform over the 8 threads of a token
        const float g = __expf(a - lse);
        const TS* Si = S + (bh * NS + i) * (size_t)(DV * DK);
        float part = 0.f;
#pragma unroll
        for (int m = 0; m < CPV; ++m) {
            const int c = p + 8 * m;
            float dot = 0.f;
#pragma unroll 4
            for (int r = 0; r < DK; r += 8) {  // 16-byte (bf16) / 32-byte (fp32) row slices
                float v[8];
                ld8(Si, (size_t)c * DK + r, v);
#pragma unroll
                for (int e = 0; e < 8; ++e) dot += v[e] * sq[tt][r + e];
            }
            part += sdy[tt][c] * dot;
        }
        const float dgi = warp_sum(part, 8);
        D += g * dgi;
        if (valid && p == 0) dG[(bh * L + t) * NS + i] = dgi;
#pragma unroll
        for (int m = 0; m < CPK; ++m) {
            const int r = p + 8 * m;
            float acc = 0.f;
#pragma unroll 8
            for (int c = 0; c < DV; ++c) acc += ld(Si, (size_t)c * DK + r) * sdy[tt][c];
            dq[m] += g * acc;
        }
    }
    // the online segment: dgamma_s = <dy, O_on[t]>
    float part = 0.f;
#pragma unroll
    for (int m = 0; m < CPV; ++m) part += sdy[tt][p + 8 * m] * O_on[(bh * L + tc) * DV + p + 8 * m];
    const float dgs = warp_sum(part, 8);
    const float gsv = __expf(a_on - lse);
    D += gsv * dgs;
    if (!valid) return;
    if (p == 0) {
        dG[(bh * L + t) * NS + s] = dgs;
        lse_o[bh * L + t] = lse;
        D_o[bh * L + t] = D;
        gs_o[bh * L + t] = gsv;
    }
#pragma unroll
    for (int m = 0; m < CPK; ++m) dQ[(bh * L + t) * DK + p + 8 * m] = dq[m];
}

// Softmax backward per token: da_i = gamma_i (dgamma_i - D) written over dgamma, du_t, and the
// final dq.  8 threads per token; thread p owns gate columns [p DG/8, (p+1) DG/8).
template <typename T, int DK>
__global__ __launch_bounds__(256) void bwd_gate_kernel(
    const T* __restrict__ Q, const T* __restrict__ U, const float* __restrict__ P,
    const float* __restrict__ xps, const float* __restrict__ lse_i,
    const float* __restrict__ D_i, const float* __restrict__ gs_i, const float* __restrict__ Ot,
    int L, int C, int NS, int DG, int H, int xh, int phi, float* __restrict__ dG,
    float* __restrict__ dU, float* __restrict__ dQ) {
    constexpr int CPK = DK / 8;
    const int tile0 = blockIdx.x * BTT;
    const size_t bh = blockIdx.y;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const size_t bx = (size_t)b * xh + (xh == 1 ? 0 : h);
    const int tid = threadIdx.x, tt = tid / 8, p = tid % 8;
    const int t = tile0 + tt;
    const bool valid = t < L;
    const int tc = valid ? t : L - 1;
    const int s = tc / C, j = tc - s * C;
    const int s_hi = (min(L, tile0 + BTT) - 1) / C;
    const int gch = DG / 8;
    const size_t urow = (bh * L + tc) * DG;
    const size_t grow = (bh * L + tc) * NS;
    const float lse = lse_i[bh * L + tc], D = D_i[bh * L + tc];

    float du[32];  // DG <= 256, so gch <= 32
#pragma unroll
    for (int k = 0; k < 32; ++k) du[k] = 0.f;
    for (int i = 0; i < s_hi; ++i) {
        const float* Pi = P + (bx * NS + i) * DG;
        float a = 0.f;
        for (int e = p * gch; e < (p + 1) * gch; ++e) a += ld(U, urow + e) * Pi[e];
        a = warp_sum(a, 8);
        if (i >= s) continue;
        const float da = __expf(a - lse) * (dG[grow + i] - D);
        if (valid && p == 0) dG[grow + i] = da;
#pragma unroll
        for (int k = 0; k < 32; ++k)
            if (k < gch) du[k] += da * Pi[p * gch + k];
    }
    if (!valid) return;
    const float das = gs_i[bh * L + t] * (dG[grow + s] - D);
    if (p == 0) dG[grow + s] = das;
    const float* xr = xps + (bx * L + t) * DG;
    const float inv = 1.f / (float)(j + 1);
#pragma unroll
    for (int k = 0; k < 32; ++k)
        if (k < gch) dU[urow + p * gch + k] = du[k] + das * xr[p * gch + k] * inv;
    const float gsv = gs_i[bh * L + t];
#pragma unroll
    for (int m = 0; m < CPK; ++m) {
        const int r = p + 8 * m;
        const size_t o = (bh * L + t) * DK + r;
        const float f = feature(ld(Q, o), phi);
        dQ[o] = (dQ[o] + gsv * Ot[o]) * dfeature_from(f, phi);
    }
}

// dM^(i) = sum over the tokens after segment i of gamma_t^(i) dy_t phi(q_t)^T, one workgroup
// per (segment i, b*H+h); thread `tid` owns row c = tid / TPR and CPT columns of it.
template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void bwd_dm_kernel(
    const T* __restrict__ Q, const T* __restrict__ U, const float* __restrict__ P,
    const float* __restrict__ lse_i, const T* __restrict__ dY, int L, int C, int NS, int DG,
    int H, int xh, int phi, float* __restrict__ dM) {
    constexpr int TPR = 256 / DV, CPT = DK / TPR;
    __shared__ float sq[BTT][DK];
    __shared__ float sdy[BTT][DV];
    __shared__ float sg[BTT];
    const int i = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const size_t bx = (size_t)b * xh + (xh == 1 ? 0 : h);
    const int tid = threadIdx.x, c = tid / TPR, r0 = (tid % TPR) * CPT;
    const float* Pi = P + (bx * NS + i) * DG;
    float m[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) m[k] = 0.f;
    for (int t0 = (i + 1) * C; t0 < L; t0 += BTT) {
        const int n = min(BTT, L - t0);
        __syncthreads();
        for (int e = tid; e < n * DK; e += 256)
            sq[e / DK][e % DK] = feature(ld(Q, (bh * L + t0) * DK + e), phi);
        for (int e = tid; e < n * DV; e += 256) sdy[e / DV][e % DV] = ld(dY, (bh * L + t0) * DV + e);
        {  // gamma_t^(i) = exp(<u_t, P_i> - lse_t), 8 threads per token
            const int tt = tid / 8, p = tid % 8, gch = DG / 8;
            const int tk = t0 + min(tt, n - 1);
            float a = 0.f;
            for (int e = p * gch; e < (p + 1) * gch; ++e) a += ld(U, (bh * L + tk) * DG + e) * Pi[e];
            a = warp_sum(a, 8);
            if (p == 0) sg[tt] = tt < n ? __expf(a - lse_i[bh * L + tk]) : 0.f;
        }
        __syncthreads();
        for (int jj = 0; jj < n; ++jj) {
            const float w = sg[jj] * sdy[jj][c];
#pragma unroll
            for (int k = 0; k < CPT; ++k) m[k] += w * sq[jj][r0 + k];
        }
    }
    float* out = dM + (bh * NS + i) * (size_t)(DV * DK) + (size_t)c * DK + r0;
#pragma unroll
    for (int k = 0; k < CPT; ++k) out[k] = m[k];
}

// Per segment, tokens in reverse: E = dM^(i) + sum_{t >= r} gamma_t^(s) dy_t phi(q_t)^T kept
// twice -- E (row c per thread group, for dv_r = E phi(k_r)) and E^T (row r per thread group,
// for dphi(k_r) = E^T v_r) -- so both reads reduce only within a thread group.
template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void bwd_online_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dY, const float* __restrict__ gs_i, const float* __restrict__ dM,
    int L, int C, int NS, int phi, float* __restrict__ dK, float* __restrict__ dV) {
    constexpr int TA = 256 / DV, CA = DK / TA;  // E:   row c = tid / TA, columns ra..ra+CA
    constexpr int TB = 256 / DK, CB = DV / TB;  // E^T: row r = tid / TB, columns cb..cb+CB
    __shared__ float sq[BTT][DK];
    __shared__ float sk[BTT][DK];
    __shared__ float sv[BTT][DV];
    __shared__ float sdy[BTT][DV];
    __shared__ float sgs[BTT];
    const int s = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int c = tid / TA, ra = (tid % TA) * CA;
    const int r = tid / TB, cb = (tid % TB) * CB;
    const int t0 = s * C, len = min(C, L - t0);
    const float* dMi = dM + (bh * NS + s) * (size_t)(DV * DK);
    float ea[CA], eb[CB];
#pragma unroll
    for (int k = 0; k < CA; ++k) ea[k] = dMi[(size_t)c * DK + ra + k];
#pragma unroll
    for (int k = 0; k < CB; ++k) eb[k] = dMi[(size_t)(cb + k) * DK + r];
    const int ntile = (len + BTT - 1) / BTT;
    for (int tile = ntile - 1; tile >= 0; --tile) {
        const int j0 = t0 + tile * BTT;
        const int n = min(BTT, t0 + len - j0);
        __syncthreads();
        for (int e = tid; e < n * DK; e += 256) {
            sq[e / DK][e % DK] = feature(ld(Q, (bh * L + j0) * DK + e), phi);
            sk[e / DK][e % DK] = feature(ld(K, (bh * L + j0) * DK + e), phi);
        }
        for (int e = tid; e < n * DV; e += 256) {
            sv[e / DV][e % DV] = ld(V, (bh * L + j0) * DV + e);
            sdy[e / DV][e % DV] = ld(dY, (bh * L + j0) * DV + e);
        }
        if (tid < n) sgs[tid] = gs_i[bh * L + j0 + tid];
        __syncthreads();
        for (int jj = n - 1; jj >= 0; --jj) {
            const float g = sgs[jj];
            const float wa = g * sdy[jj][c];
            float pa = 0.f;
#pragma unroll
            for (int k = 0; k < CA; ++k) {
                ea[k] += wa * sq[jj][ra + k];
                pa += ea[k] * sk[jj][ra + k];
            }
            const float wb = g * sq[jj][r];
            float pb = 0.f;
#pragma unroll
            for (int k = 0; k < CB; ++k) {
                eb[k] += wb * sdy[jj][cb + k];
                pb += eb[k] * sv[jj][cb + k];
            }
            pa = warp_sum(pa, TA);
            pb = warp_sum(pb, TB);
            const size_t tok = bh * L + j0 + jj;
            if (tid % TA == 0) dV[tok * DV + c] = pa;
            if (tid % TB == 0) dK[tok * DK + r] = pb * dfeature_from(sk[jj][r], phi);
        }
    }
}

// dx in three steps (x head bx; with one shared x head its sums run over every head):
//   bwd_dxw_kernel    w_t = sum_h da_t^(s) u_t / (j_t + 1), the prefix-mean term of token t
//                     (da_t^(s) read from dA [B,H,L,NS], or from [B,H,L] with diag set)
//   bwd_dp_kernel     partial dP_i = sum_h sum_t da_t^(i) u_t over one token range (3-D grid:
//                     segment, x head, token range; token lanes reduced through LDS)
//   bwd_dxf_kernel    dP_i from the partials; dx_r = dP_i / |S_i| + sum_{t >= r in S_i} w_t
template <typename T>
__global__ __launch_bounds__(256) void bwd_dxw_kernel(const T* __restrict__ U,
                                                      const float* __restrict__ dA, int diag,
                                                      int L, int C, int NS, int DG, int H,
                                                      int xh, float* __restrict__ w) {
    const int t0 = blockIdx.x * 64;
    const size_t bx = blockIdx.y;
    const int b = (int)(bx / xh), hx = (int)(bx % xh);
    const int h0 = xh == 1 ? 0 : hx, h1 = xh == 1 ? H : hx + 1;
    if (DG % 8 == 0) {  // 8 consecutive columns per thread and step
        const int g8 = DG / 8;
        for (int idx = threadIdx.x; idx < 64 * g8; idx += 256) {
            const int t = t0 + idx / g8, e = (idx % g8) * 8;
            if (t >= L) break;
            const int s = t / C, j = t - s * C;
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int h = h0; h < h1; ++h) {
                const size_t bh = (size_t)b * H + h;
                const float a = dA[diag ? bh * L + t : (bh * L + t) * NS + s];
                float u[8];
                ld8(U, (bh * L + t) * DG + e, u);
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k] += a * u[k];
            }
            const float inv = 1.f / (float)(j + 1);
            float* o = w + (bx * L + t) * DG + e;
            *reinterpret_cast<float4*>(o) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
            *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
        }
        return;
    }
    for (int idx = threadIdx.x; idx < 64 * DG; idx += 256) {
        const int t = t0 + idx / DG, e = idx % DG;
        if (t >= L) break;
        const int s = t / C, j = t - s * C;
        float acc = 0.f;
        for (int h = h0; h < h1; ++h) {
            const size_t bh = (size_t)b * H + h;
            acc += dA[diag ? bh * L + t : (bh * L + t) * NS + s] * ld(U, (bh * L + t) * DG + e);
        }
        w[(bx * L + t) * DG + e] = acc / (float)(j + 1);
    }
}

template <typename T>
__global__ __launch_bounds__(256) void bwd_dp_kernel(const T* __restrict__ U,
                                                     const float* __restrict__ dA, int L, int C,
                                                     int NS, int DG, int H, int xh, int RL,
                                                     float* __restrict__ part) {
    __shared__ float red[256];
    const int i = blockIdx.x;
    const size_t bx = blockIdx.y;
    const int rg = blockIdx.z;
    const int b = (int)(bx / xh), hx = (int)(bx % xh);
    const int h0 = xh == 1 ? 0 : hx, h1 = xh == 1 ? H : hx + 1;
    const int TL = 256 / DG;  // token lanes (DG <= 256)
    const int tid = threadIdx.x, e = tid % DG, tl = tid / DG;
    const int lo = max(rg * RL, (i + 1) * C), hi = min(L, (rg + 1) * RL);
    float acc = 0.f;
    if (tl < TL)
        for (int h = h0; h < h1; ++h) {
            const size_t bh = (size_t)b * H + h;
            for (int t = lo + tl; t < hi; t += TL)
                acc += dA[(bh * L + t) * NS + i] * ld(U, (bh * L + t) * DG + e);
        }
    red[tid] = acc;
    __syncthreads();
    if (tid < DG) {
        float v = 0.f;
        for (int k = 0; k < TL; ++k) v += red[k * DG + tid];
        part[(((size_t)rg * NS + i) * gridDim.y + bx) * DG + tid] = v;
    }
}

__global__ __launch_bounds__(256) void bwd_dxf_kernel(const float* __restrict__ part,
                                                      const float* __restrict__ w, int L, int C,
                                                      int NS, int DG, int NR,
                                                      float* __restrict__ dX) {
    const int i = blockIdx.x;
    const size_t bx = blockIdx.y;
    const int e = threadIdx.x;
    if (e >= DG) return;  // no barriers below
    float dp = 0.f;
    for (int rg = 0; rg < NR; ++rg) dp += part[(((size_t)rg * NS + i) * gridDim.y + bx) * DG + e];
    const int t0 = i * C, len = min(C, L - t0);
    const float base = dp / (float)len;
    float tail = 0.f;
    for (int jj = len - 1; jj >= 0; --jj) {
        const size_t o = (bx * L + t0 + jj) * DG + e;
        tail += w[o];
        dX[o] = base + tail;
    }
}

__global__ void feature_kernel_bf16(const bf16_t* __restrict__ K, size_t n, int phi,
                                    bf16_t* __restrict__ out) {
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n;
         e += (size_t)gridDim.x * blockDim.x)
        out[e] = f32_to_bf16(feature(bf16_to_f32(K[e]), phi));
}
__global__ void feature_kernel_f32(const float* __restrict__ K, size_t n, int phi,
                                   float* __restrict__ out) {
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n;
         e += (size_t)gridDim.x * blockDim.x)
        out[e] = feature(K[e], phi);
}

template <typename T, typename TS, int DK, int DV>
int launch_bwd_t(const mc_dims& d, const BwdBuffers& w, const void* Q, const void* K,
                 const void* V, const void* U, const void* S, const float* P, const void* dY,
                 float* dQ, float* dK, float* dV, float* dU, float* dX, bool fast,
                 hipStream_t st) {
    const int NS = (d.L + d.seg_len - 1) / d.seg_len;
    const dim3 tiles((d.L + BTT - 1) / BTT, d.B * d.H);
    if (!fast) {  // dgamma, the gate backward and dM on the fp32 vector units
        hipLaunchKernelGGL((bwd_cached_kernel<T, TS, DK, DV>), tiles, dim3(256), 0, st,
                           (const T*)Q, (const T*)U, w.aon, (const TS*)S, P, w.on, (const T*)dY,
                           d.L, d.seg_len, NS, d.d_g, d.H, d.x_heads, d.phi, w.dG, w.lse, w.D,
                           w.gs, dQ);
        hipLaunchKernelGGL((bwd_gate_kernel<T, DK>), tiles, dim3(256), 0, st, (const T*)Q,
                           (const T*)U, P, w.xps, w.lse, w.D, w.gs, w.ot, d.L, d.seg_len, NS,
                           d.d_g, d.H, d.x_heads, d.phi, w.dG, dU, dQ);
        hipLaunchKernelGGL((bwd_dm_kernel<T, DK, DV>), dim3(NS, d.B * d.H), dim3(256), 0, st,
                           (const T*)Q, (const T*)U, P, w.lse, (const T*)dY, d.L, d.seg_len, NS,
                           d.d_g, d.H, d.x_heads, d.phi, w.dM);
    }
    if (fast) {
        const int rc = launch_bwd_online_mfma(d, w, Q, K, V, dY, dK, dV, st);
        if (rc) return rc;
    } else {
        hipLaunchKernelGGL((bwd_online_kernel<T, DK, DV>), dim3(NS, d.B * d.H), dim3(256), 0, st,
                           (const T*)Q, (const T*)K, (const T*)V, (const T*)dY, w.gs, w.dM,
                           d.L, d.seg_len, NS, d.phi, dK, dV);
    }
    // x gradients; the prefix sums of X are no longer needed, so w_t goes in their place
    const int bxn = d.B * d.x_heads;
    hipLaunchKernelGGL((bwd_dxw_kernel<T>), dim3((d.L + 63) / 64, bxn), dim3(256), 0, st,
                       (const T*)U, w.dG, fast ? 1 : 0, d.L, d.seg_len, NS, d.d_g, d.H, d.x_heads, w.xps);
    // dP_i: partial sums over token ranges, or (MFMA path) per head from the dM walk
    const int RL = bwd_dp_range(d.L);
    int NR = (d.L + RL - 1) / RL;
    if (fast)
        NR = d.x_heads == 1 ? d.H : 1;
    else
        hipLaunchKernelGGL((bwd_dp_kernel<T>), dim3(NS, bxn, NR), dim3(256), 0, st, (const T*)U,
                           w.dG, d.L, d.seg_len, NS, d.d_g, d.H, d.x_heads, RL, w.dpp);
    hipLaunchKernelGGL(bwd_dxf_kernel, dim3(NS, bxn), dim3(256), 0, st, w.dpp, w.xps, d.L,
                       d.seg_len, NS, d.d_g, NR, dX);
    return (int)hipGetLastError();
}

}  // namespace

int launch_grm_backward(const mc_dims& d, const BwdBuffers& w, const void* Q, const void* K,
                        const void* V, const void* U, const void* X, const float* M,
                        const uint16_t* M_lo, const float* P, const void* dY, float* dQ,
                        float* dK, float* dV, float* dU, float* dX, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    const bool fast = bwd_fast(d);
    int rc = launch_xps(d, X, w.xps, w.xtail, stream);
    if (rc) return rc;
    // phi(K) in the input dtype: the values of the transposed online read
    BwdBuffers wb = w;
    if (d.phi) {
        const size_t n = (size_t)d.B * d.H * d.L * d.d_k;
        const int blocks = (int)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
        if (d.dtype == MC_BF16)
            hipLaunchKernelGGL(feature_kernel_bf16, dim3(blocks), dim3(256), 0, st,
                               (const bf16_t*)K, n, d.phi, (bf16_t*)w.khat);
        else
            hipLaunchKernelGGL(feature_kernel_f32, dim3(blocks), dim3(256), 0, st,
                               (const float*)K, n, d.phi, (float*)w.khat);
    } else {
        wb.khat = nullptr;
    }
    if (fast) {
        // the forward's gate pass (softmax numerators per read tile), the online read's
        // product with dy (dgamma of the online segment, into on as [B,H,L]), then dgamma,
        // dphi(q), the gate backward and dM on MFMA
        rc = launch_gate_w(d, U, w.xps, P, w.pf, w.W, w.won, w.inv_l, stream);
        if (!rc) rc = launch_scan_mfma_dgs(d, Q, K, V, dY, w.on, stream);
        if (!rc) rc = launch_bwd_fast(d, wb, Q, K, V, U, M, M_lo, P, dY, dQ, dU, stream);
        if (rc) return rc;
    } else {
        rc = launch_aon(d, X, U, w.aon, stream);
        if (!rc) rc = launch_scan_online(d, Q, K, V, w.on, stream);
        if (rc) return rc;
        // Ot[t] = M_t^(s)T dy_t: the online scan with q := dy, k := v, v := phi(k)
        mc_dims dt = d;
        dt.d_k = d.d_v;
        dt.d_v = d.d_k;
        dt.phi = MC_PHI_IDENTITY;
        rc = launch_scan_online(dt, dY, V, wb.khat ? wb.khat : K, w.ot, stream);
        if (rc) return rc;
    }
#define MC_BW(DK, DV)                                                                        \
    if (d.d_k == DK && d.d_v == DV)                                                          \
        return d.dtype == MC_BF16                                                            \
                   ? launch_bwd_t<bf16_t, bf16_t, DK, DV>(d, w, Q, K, V, U, M_lo, P, dY, dQ, \
                                                          dK, dV, dU, dX, fast, st)          \
                   : launch_bwd_t<float, float, DK, DV>(d, w, Q, K, V, U, M, P, dY, dQ, dK,  \
                                                        dV, dU, dX, fast, st);
    MC_BW(128, 128)
    MC_BW(128, 64)
    MC_BW(64, 128)
    MC_BW(64, 64)
#undef MC_BW
    return (int)hipErrorInvalidValue;
}

}  // namespace mc
