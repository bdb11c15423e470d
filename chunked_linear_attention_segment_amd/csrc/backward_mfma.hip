// backward_mfma.hip -- the bf16, d_k = d_v = 128 backward of the GRM prefill on MFMA.
//
// The same gradients as backward.hip (Memory Caching paper, Eq. 4b / 9 / 10 differentiated
// token by token), organised around the dense contractions:
//   dphi(q_t) = sum_{i<s} gamma_i M^(i)^T dy_t + gamma_s M_t^(s)^T dy_t is the gated read of
//     Eq. 9 with the roles swapped -- queries dy, keys v, values phi(k), states M^(i)^T, the
//     same gate -- so it runs on the forward read kernel (grm_read_kernel) with transposed
//     bf16 states (transpose_states_kernel) and the forward gate pass's softmax numerators.
//   dgamma_t^(i) = <dy_t, M^(i) phi(q_t)>: bwd_dgamma_kernel, per 256-token tile, streams the
//     states through LDS and contracts each with the tile's phi(q) on MFMA, then reduces the
//     products against dy in registers.
//   dM^(i) = sum_t gamma_t^(i) dy_t phi(q_t)^T: bwd_dm_mfma_kernel, per cached segment, walks
//     the later tokens in chunks of 64 (the scan's state-update contraction with phi(q) in
//     place of phi(k) and gamma dy in place of v).
//   bwd_gate_fast_kernel: the softmax backward from the gate numerators W, 1/l and the online
//     weight (gamma_i = W_i / l), dgamma of the online segment, du_t and dq.
#include "common.cuh"
#include "mc_internal.h"

namespace mc {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// phi applied to 8 bf16 values (4 words)
__device__ __forceinline__ u32x4_t phi8(u32x4_t v, int phi) {
    if (!phi) return v;
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(feature(bf_lo(v[e]), 1), feature(bf_hi(v[e]), 1));
    return o;
}

// M [BH*NS][DV][DK] fp32 -> MT [BH*NS][DK][DV] bf16, 32 x 32 tiles through LDS.
__global__ __launch_bounds__(256) void transpose_states_kernel(const float* __restrict__ M,
                                                               int DV, int DK,
                                                               bf16_t* __restrict__ MT) {
    __shared__ float tile[32][33];
    const size_t st = blockIdx.x;
    const int r0 = blockIdx.y * 32, c0 = blockIdx.z * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    const float* src = M + st * (size_t)DV * DK;
    bf16_t* dst = MT + st * (size_t)DV * DK;
    for (int y = ty; y < 32; y += 8) tile[y][tx] = src[(size_t)(c0 + y) * DK + r0 + tx];
    __syncthreads();
    for (int y = ty; y < 32; y += 8) dst[(size_t)(r0 + y) * DV + c0 + tx] = f32_to_bf16(tile[tx][y]);
}

constexpr int DT = 256;     // tokens per dgamma workgroup: 4 waves x 2 blocks of 32
constexpr int SROW = 136;   // LDS row stride (bf16) of a staged state: 16 bytes of padding

// dgamma_t^(i) for i < s_t, d_k = d_v = 128.  Wave w owns tokens t0 + 64w .. + 63 (two blocks
// of 32); per state: O^(i) = M^(i) phi(q) as 4 (rows) x 2 (token blocks) accumulator tiles,
// then dgamma = sum_c dy[c] O[c][t] (16 rows per lane, the two half-waves combined).  States are
// double-buffered in LDS, loaded one ahead through registers.
__global__ __launch_bounds__(256, 1) void bwd_dgamma_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ dY, const bf16_t* __restrict__ M_lo,
    int L, int C, int NS, int phi, float* __restrict__ dG) {
    __shared__ __attribute__((aligned(16))) bf16_t ms[2][128][SROW];
    const int ntile = gridDim.x;
    const int tile = ntile - 1 - blockIdx.x;  // the tiles that read the most states first
    const size_t bh = blockIdx.y;
    const int t0 = tile * DT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, half = lane >> 5;
    const int s_hi = (min(L, t0 + DT) - 1) / C;
    if (s_hi == 0) return;  // uniform: no token of the tile reads a cached state

    u32x4_t qb[2][8];
    float dyv[2][4][16];
    int tok[2], stok[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int t = t0 + wave * 64 + tb * 32 + l32;
        const bool ok = t < L;
        tok[tb] = t;
        stok[tb] = ok ? t / C : 0;
        const bf16_t* qr = Q + (bh * L + (ok ? t : 0)) * 128 + half * 8;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (ok) v = phi8(*reinterpret_cast<const u32x4_t*>(qr + ks * 16), phi);
            qb[tb][ks] = v;
        }
        const bf16_t* dr = dY + (bh * L + (ok ? t : 0)) * 128;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2_t w = {0u, 0u};
                if (ok) w = *reinterpret_cast<const u32x2_t*>(dr + cb * 32 + 8 * g + 4 * half);
                dyv[tb][cb][4 * g + 0] = bf_lo(w[0]);
                dyv[tb][cb][4 * g + 1] = bf_hi(w[0]);
                dyv[tb][cb][4 * g + 2] = bf_lo(w[1]);
                dyv[tb][cb][4 * g + 3] = bf_hi(w[1]);
            }
    }

    const bf16_t* Sb = M_lo + bh * (size_t)NS * 128 * 128;
    u32x4_t pre[8];  // one state: 128 rows x 16 chunks of 16 bytes, 8 chunks per thread
    auto load_state = [&](int i) {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(Sb + (size_t)i * 128 * 128);
#pragma unroll
        for (int it = 0; it < 8; ++it) pre[it] = src[tid + 256 * it];
    };
    auto store_state = [&](int buf) {
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int idx = tid + 256 * it;
            *reinterpret_cast<u32x4_t*>(&ms[buf][idx >> 4][(idx & 15) * 8]) = pre[it];
        }
    };
    load_state(0);
    store_state(0);
    __syncthreads();
    const f32x16_t zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                           0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < s_hi; ++i) {
        const int buf = i & 1;
        if (i + 1 < s_hi) load_state(i + 1);
        f32x16_t acc[4][2];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const u32x4_t a =
                    *reinterpret_cast<const u32x4_t*>(&ms[buf][cb * 32 + l32][ks * 16 + half * 8]);
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
                    acc[cb][tb] = mfma32(a, qb[tb][ks], ks == 0 ? zero : acc[cb][tb]);
            }
        }
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            float part = 0.f;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) part += dyv[tb][cb][r] * acc[cb][tb][r];
            part += __shfl_xor(part, 32);
            if (half == 0 && tok[tb] < L && i < stok[tb])
                dG[(bh * L + tok[tb]) * NS + i] = part;
        }
        if (i + 1 < s_hi) store_state(buf ^ 1);
        __syncthreads();
    }
}

constexpr int CHK = 64;    // tokens per chunk of the dM walk
constexpr int TPAD = 72;   // row stride (bf16) of the token-indexed LDS tiles

// dM^(i) (stored [c][r] like the states) for d_k = d_v = 128: M^T-style accumulation
// dM^T[r][c] += sum_t phi(q_t)[r] (gamma_t^(i) dy_t[c]); wave w owns value columns
// c in [32w, 32w+32) and keeps the four 32-row blocks of r in its accumulators.  phi(q)^T and
// (gamma dy)^T are staged in LDS with token pairs packed in 32-bit words (the token index is
// the contraction index).  gamma_t^(i) = W_t^(i) / l_t from the forward gate pass.
__global__ __launch_bounds__(256, 1) void bwd_dm_mfma_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ dY, const uint16_t* __restrict__ Wg,
    const float* __restrict__ inv_l, int L, int C, int NS, int phi, float* __restrict__ dM) {
    __shared__ __attribute__((aligned(16))) bf16_t qt[128][TPAD];  // phi(q)^T [r][t]
    __shared__ __attribute__((aligned(16))) bf16_t gt[128][TPAD];  // (gamma dy)^T [c][t]
    __shared__ float sg[CHK];
    const int i = blockIdx.x;  // low i (the most tokens) is dispatched first
    const size_t bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, half = lane >> 5;
    const int T = (L + kGateTile - 1) / kGateTile;
    f32x16_t mt[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt[db][r] = 0.f;
    for (int j0 = (i + 1) * C; j0 < L; j0 += CHK) {
        const int n = min(CHK, L - j0);
        if (tid < CHK) {
            const int t = j0 + tid;
            float g = 0.f;
            if (tid < n)
                g = bf16_to_f32(Wg[((bh * T + t / kGateTile) * NS + i) * kGateTile + t % kGateTile]) *
                    inv_l[bh * L + t];
            sg[tid] = g;
        }
        __syncthreads();
        // stage phi(q)^T and (gamma dy)^T, token pairs packed in 32-bit words
        for (int it = tid; it < (CHK / 2) * 16; it += 256) {
            const int p = it % (CHK / 2), dc = (it / (CHK / 2)) * 8;
            const int r0 = 2 * p, r1 = 2 * p + 1;
            u32x4_t a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
            u32x4_t ya = {0u, 0u, 0u, 0u}, yb = {0u, 0u, 0u, 0u};
            if (r0 < n) {
                a = phi8(*reinterpret_cast<const u32x4_t*>(Q + (bh * L + j0 + r0) * 128 + dc), phi);
                ya = *reinterpret_cast<const u32x4_t*>(dY + (bh * L + j0 + r0) * 128 + dc);
            }
            if (r1 < n) {
                b = phi8(*reinterpret_cast<const u32x4_t*>(Q + (bh * L + j0 + r1) * 128 + dc), phi);
                yb = *reinterpret_cast<const u32x4_t*>(dY + (bh * L + j0 + r1) * 128 + dc);
            }
            const float g0 = sg[r0], g1 = sg[r1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                *reinterpret_cast<uint32_t*>(&qt[dc + 2 * e][r0]) = (a[e] & 0xffffu) | (b[e] << 16);
                *reinterpret_cast<uint32_t*>(&qt[dc + 2 * e + 1][r0]) = (a[e] >> 16) | (b[e] & 0xffff0000u);
                *reinterpret_cast<uint32_t*>(&gt[dc + 2 * e][r0]) =
                    pack_bf16x2(g0 * bf_lo(ya[e]), g1 * bf_lo(yb[e]));
                *reinterpret_cast<uint32_t*>(&gt[dc + 2 * e + 1][r0]) =
                    pack_bf16x2(g0 * bf_hi(ya[e]), g1 * bf_hi(yb[e]));
            }
        }
        __syncthreads();
        const int cv = wave * 32 + l32;
        u32x4_t gb[CHK / 16];
#pragma unroll
        for (int ks = 0; ks < CHK / 16; ++ks)
            gb[ks] = *reinterpret_cast<const u32x4_t*>(&gt[cv][ks * 16 + half * 8]);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int r = db * 32 + l32;
#pragma unroll
            for (int ks = 0; ks < CHK / 16; ++ks) {
                const u32x4_t qa = *reinterpret_cast<const u32x4_t*>(&qt[r][ks * 16 + half * 8]);
                mt[db] = mfma32(qa, gb[ks], mt[db]);
            }
        }
        __syncthreads();
    }
    // dM[c][r]: lane holds c = 32 wave + l32 and r = 32 db + 8g + 4 half + e
    const int cv = wave * 32 + l32;
    float* out = dM + ((bh * NS + i) * 128 + cv) * (size_t)128;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4*>(out + db * 32 + 8 * g + 4 * half) =
                make_float4(mt[db][4 * g], mt[db][4 * g + 1], mt[db][4 * g + 2], mt[db][4 * g + 3]);
}

// The softmax backward from the forward gate pass: gamma_i = W_t^(i) / l_t (i < s),
// gamma_s = won_t / l_t; dgamma of the online segment <dy_t, O_on[t]>; D_t; da_i written over
// dgamma; du_t; the online weight for the segment walk; dq = dphi(q) phi'(q) with dphi(q) the
// bf16 output of the swapped read.  8 threads per token.
template <int DK>
__global__ __launch_bounds__(256) void bwd_gate_fast_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ U, const float* __restrict__ P,
    const float* __restrict__ xps, const uint16_t* __restrict__ Wg,
    const float* __restrict__ won, const float* __restrict__ inv_l,
    const float* __restrict__ O_on, const bf16_t* __restrict__ dY,
    const bf16_t* __restrict__ dqh, int L, int C, int NS, int DG, int DV, int H, int xh,
    int phi, float* __restrict__ dG, float* __restrict__ gs_o, float* __restrict__ dU,
    float* __restrict__ dQ) {
    constexpr int CPK = DK / 8;
    const int tile0 = blockIdx.x * 32;
    const size_t bh = blockIdx.y;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const size_t bx = (size_t)b * xh + (xh == 1 ? 0 : h);
    const int tid = threadIdx.x, tt = tid / 8, p = tid % 8;
    const int t = tile0 + tt;
    const bool valid = t < L;
    const int tc = valid ? t : L - 1;
    const int s = tc / C, j = tc - s * C;
    const int T = (L + kGateTile - 1) / kGateTile;
    const uint16_t* wrow = Wg + ((bh * T + tc / kGateTile) * NS) * kGateTile + tc % kGateTile;
    const size_t grow = (bh * L + tc) * NS;
    const float il = inv_l[bh * L + tc];
    // dgamma of the online segment and D = sum_i gamma_i dgamma_i (segments dealt over p)
    float part = 0.f;
    for (int c = p; c < DV; c += 8) part += bf16_to_f32(dY[(bh * L + tc) * DV + c]) * O_on[(bh * L + tc) * DV + c];
    const float dgs = warp_sum(part, 8);
    const float gsv = won[bh * L + tc] * il;
    float dpart = 0.f;
    for (int i = p; i < s; i += 8) dpart += bf16_to_f32(wrow[(size_t)i * kGateTile]) * il * dG[grow + i];
    const float D = warp_sum(dpart, 8) + gsv * dgs;
    if (!valid) return;  // no shuffles below
    const int gch = DG / 8;
    float du[32];  // DG <= 256
#pragma unroll
    for (int k = 0; k < 32; ++k) du[k] = 0.f;
    for (int i = 0; i < s; ++i) {
        const float da = bf16_to_f32(wrow[(size_t)i * kGateTile]) * il * (dG[grow + i] - D);
        const float* Pi = P + (bx * NS + i) * DG + p * gch;
#pragma unroll
        for (int k = 0; k < 32; ++k)
            if (k < gch) du[k] += da * Pi[k];
        if ((i & 7) == p) dG[grow + i] = da;
    }
    const float das = gsv * (dgs - D);
    if (p == 0) {
        dG[grow + s] = das;
        gs_o[bh * L + t] = gsv;
    }
    const float* xr = xps + (bx * L + t) * DG + p * gch;
    const float inv = 1.f / (float)(j + 1);
    const size_t urow = (bh * L + t) * DG + p * gch;
#pragma unroll
    for (int k = 0; k < 32; ++k)
        if (k < gch) dU[urow + k] = du[k] + das * xr[k] * inv;
#pragma unroll
    for (int m = 0; m < CPK; ++m) {
        const size_t o = (bh * L + t) * DK + p + 8 * m;
        const float f = feature(bf16_to_f32(Q[o]), phi);
        dQ[o] = bf16_to_f32(dqh[o]) * (phi ? fminf(f, 1.f) : 1.f);
    }
}

}  // namespace

int launch_bwd_fast(const mc_dims& d, const BwdBuffers& w, const void* Q, const void* K,
                    const void* V, const void* U, const float* M, const uint16_t* M_lo,
                    const float* P, const void* dY, float* dQ, float* dU, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    const int NS = (d.L + d.seg_len - 1) / d.seg_len;
    const int BH = d.B * d.H;
    // transposed bf16 states for the swapped read
    hipLaunchKernelGGL(transpose_states_kernel, dim3(BH * NS, d.d_k / 32, d.d_v / 32), dim3(256),
                       0, st, M, d.d_v, d.d_k, (bf16_t*)w.mt);
    // dphi(q) = the gated read with queries dy, keys v, values phi(k), states M^T
    mc_dims ds = d;
    ds.d_k = d.d_v;
    ds.d_v = d.d_k;
    ds.phi = MC_PHI_IDENTITY;
    GateWeights gw;
    gw.W = w.W;
    gw.won = w.won;
    gw.inv_l = w.inv_l;
    int rc = launch_read_mfma(ds, false, 0, dY, V, w.khat ? w.khat : K, U, w.xps,
                              (const uint16_t*)w.mt, P, nullptr, nullptr, gw, w.dqh, stream);
    if (rc) return rc;
    hipLaunchKernelGGL(bwd_dgamma_kernel, dim3((d.L + DT - 1) / DT, BH), dim3(256), 0, st,
                       (const bf16_t*)Q, (const bf16_t*)dY, (const bf16_t*)M_lo, d.L, d.seg_len,
                       NS, d.phi, w.dG);
    hipLaunchKernelGGL((bwd_gate_fast_kernel<128>), dim3((d.L + 31) / 32, BH), dim3(256), 0, st,
                       (const bf16_t*)Q, (const bf16_t*)U, P, w.xps, w.W, w.won, w.inv_l, w.on,
                       (const bf16_t*)dY, (const bf16_t*)w.dqh, d.L, d.seg_len, NS, d.d_g, d.d_v,
                       d.H, d.x_heads, d.phi, w.dG, w.gs, dU, dQ);
    hipLaunchKernelGGL(bwd_dm_mfma_kernel, dim3(NS, BH), dim3(256), 0, st, (const bf16_t*)Q,
                       (const bf16_t*)dY, w.W, w.inv_l, d.L, d.seg_len, NS, d.phi, w.dM);
    return (int)hipGetLastError();
}

}  // namespace mc
