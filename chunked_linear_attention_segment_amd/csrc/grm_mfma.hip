// grm_mfma.hip -- the Gated Residual Memory read on bf16 MFMA (gfx950), fused with the gate.
//
// Memory Caching paper §3.1, Eq. (9)-(10): for token t of segment s
//     y_t = gamma^(s) M_t^(s) phi(q_t) + sum_{i<s} gamma^(i) M^(i) phi(q_t),
//     gamma_t = softmax( <u_t, P_0>, ..., <u_t, P_{s-1}>, <u_t, prefix mean of X> ).
// The online term M_t^(s) phi(q_t) arrives as O_on from the scan.  The same kernel serves
// Sparse Selective Caching (gitcode explainer §3.4) when SSC = true: a token then weighs
// only the segments listed for it in idx, the softmax runs over those plus the online one.
//
// Layout of the computation (transposed, so the per-token gate is a per-lane scalar):
//   Y^T[c, t] = sum_i w_t^(i) * (M^(i) Qhat^T)[c, t]
// One workgroup = 256 consecutive tokens of one (b, h), 8 waves.  Wave (cw, tw) owns output
// rows c in [cw*DV/2, (cw+1)*DV/2) and tokens [64 tw, 64 tw + 64).  Per cached state i:
//   A = M^(i) (d_v x d_k bf16, staged once in LDS for all waves, XOR-swizzled 16-B chunks),
//   B = phi(q)^T (kept in registers for the whole kernel),
//   the 32x32x16 MFMA partial product is scaled by the token's weight w_t^(i) and added to
//   the fp32 accumulator.
// The gate runs on MFMA too, in blocks of 32 states: logits^T = P_block (hi + lo bf16 split
// of the fp32 means) x U^T, then an online softmax per token (running max m_t and sum l_t;
// the accumulator is rescaled by exp(m_old - m_new) at each block).  The online term enters
// as the initial accumulator with weight exp(a_on - m) = 1 at m = a_on.
#include "common.cuh"
#include "mc_internal.h"

namespace mc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16_t mfma32x32x16(const u32x4_t& a, const u32x4_t& b,
                                                 const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

constexpr int GT = 256;   // tokens per workgroup
constexpr int GSB = 32;   // states per gate block
constexpr int GTHREADS = 512;

template <int DK, int DV, bool SSC>
struct GrmSmem {
    static constexpr int DGP = 256;  // padded gate width held in LDS
    bf16_t state[2][DV * DK];
    bf16_t p_hi[GSB * DGP];
    bf16_t p_lo[GSB * DGP];
    float w[GSB][GT];
    float scale[GT];
    float m0[GT];
    float inv_l[GT];
    uint32_t any_sel;
};

// Map the flat block index to (b*H+h, tile).  Blocks are dealt round-robin to the 8 XCDs;
// when B*H is a multiple of 8 each XCD takes whole heads (its L2 then holds that head's
// cached states), and inside a head the tiles with the most cached states go first.
__device__ __forceinline__ void grm_tile_of_block(int bid, int BH, int T, int& bh, int& tile) {
    if (BH % 8 == 0) {
        const int xcd = bid % 8, local = bid / 8;
        bh = xcd + 8 * (local / T);
        tile = T - 1 - local % T;
    } else {
        bh = bid / T;
        tile = T - 1 - bid % T;
    }
}

template <int DK, int DV, bool SSC>
__global__ __launch_bounds__(GTHREADS, 1) void grm_mfma_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ U, const float* __restrict__ xcum,
    const bf16_t* __restrict__ S, const float* __restrict__ P, const float* __restrict__ O_on,
    const int32_t* __restrict__ idx, int top_k, int BH, int H, int L, int C, int NS, int DG,
    int xh, int phi, bf16_t* __restrict__ Y) {
    constexpr int CPR = DK / 8;        // 16-byte chunks per state row
    constexpr int KS = DK / 16;        // MFMA k-steps over d_k
    constexpr int CB = DV / 64;        // 32-row blocks per wave (a wave owns DV/2 rows)
    constexpr int STAGE = DV * DK / 8 / GTHREADS;  // 16-byte chunks each thread stages
    static_assert(STAGE >= 1, "state too small for the staging layout");
    typedef GrmSmem<DK, DV, SSC> Smem;
    __shared__ __attribute__((aligned(16))) char smem_raw[sizeof(Smem)];
    Smem& sm = *reinterpret_cast<Smem*>(smem_raw);

    const int T = (L + GT - 1) / GT;
    int bh, tile;
    grm_tile_of_block(blockIdx.x, BH, T, bh, tile);
    const int b = bh / H, h = bh % H;
    const size_t bx = (size_t)b * xh + (xh == 1 ? 0 : h);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi32 = lane >> 5;
    const int cw = wave >> 2, tw = wave & 3;
    const int tile0 = tile * GT;
    const int last = min(L, tile0 + GT) - 1;
    const int s_hi = last / C;  // states 0..s_hi-1 are read by some token of the tile

    // ---- online logit a_on[t] = <u_t, prefix mean of X> (two threads per token) ----
    {
        const int tau = tid >> 1, half = tid & 1;
        const int t = min(tile0 + tau, L - 1);
        const float inv = 1.f / (float)(t % C + 1);
        const bf16_t* ur = U + ((size_t)bh * L + t) * DG;
        const float* xr = xcum + (bx * L + t) * DG;
        float a = 0.f;
        for (int e = half; e < DG; e += 2) a += bf16_to_f32(ur[e]) * (xr[e] * inv);
        a += __shfl_xor(a, 1, 64);
        if (half == 0) sm.m0[tau] = a;
    }

    // ---- B operand: phi(q)^T fragments of this wave's 64 tokens, kept in registers ----
    u32x4_t qf[2][KS];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int t = min(tile0 + tw * 64 + tb * 32 + l32, L - 1);
        const bf16_t* qr = Q + ((size_t)bh * L + t) * DK + hi32 * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4_t v = *reinterpret_cast<const u32x4_t*>(qr + ks * 16);
            if (phi) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x0 = __uint_as_float(v[e] << 16);
                    const float x1 = __uint_as_float(v[e] & 0xffff0000u);
                    v[e] = pack_bf16x2(feature(x0, 1), feature(x1, 1));
                }
            }
            qf[tb][ks] = v;
        }
    }

    // ---- accumulator = O_on (the online term, weight 1 relative to m = a_on) ----
    f32x16_t acc[CB][2];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int t = min(tile0 + tw * 64 + tb * 32 + l32, L - 1);
            const float* orow = O_on + ((size_t)bh * L + t) * DV + cw * (DV / 2) + cb * 32 + hi32 * 4;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 v = *reinterpret_cast<const float4*>(orow + g * 8);
                acc[cb][tb][4 * g + 0] = v.x;
                acc[cb][tb][4 * g + 1] = v.y;
                acc[cb][tb][4 * g + 2] = v.z;
                acc[cb][tb][4 * g + 3] = v.w;
            }
        }

    // ---- gate state: wave `wave` owns the softmax of tokens [32 wave, 32 wave + 32) ----
    const int gt = wave * 32 + l32;  // tile-local token of this lane in the gate phase
    const int gtok = min(tile0 + gt, L - 1);
    const int gs = gtok / C;
    const bool gvalid = (tile0 + gt) < L;
    const int32_t* gsel = SSC ? idx + ((size_t)bh * L + gtok) * top_k : nullptr;
    __syncthreads();
    float m_tok = sm.m0[gt], l_tok = 1.f;

    // ---- staging of cached state i into LDS buffer `buf` (XOR swizzle of 16-B chunks) ----
    const bf16_t* Sbh = S + (size_t)bh * NS * DV * DK;
    u32x4_t stg[STAGE];
    auto stage_load = [&](int i) {
        const bf16_t* src = Sbh + (size_t)i * DV * DK;
#pragma unroll
        for (int m = 0; m < STAGE; ++m) {
            const int q = tid + GTHREADS * m;
            stg[m] = *reinterpret_cast<const u32x4_t*>(src + (size_t)q * 8);
        }
    };
    auto stage_store = [&](int buf) {
#pragma unroll
        for (int m = 0; m < STAGE; ++m) {
            const int q = tid + GTHREADS * m;
            const int c = q / CPR, kc = q % CPR;
            *reinterpret_cast<u32x4_t*>(&sm.state[buf][c * DK + ((kc ^ (c % CPR)) * 8)]) = stg[m];
        }
    };

    if (s_hi > 0) {
        stage_load(0);
        stage_store(0);
    }
    const int nblk = (s_hi + GSB - 1) / GSB;
    const int gch = (DG + 7) / 8;  // 8-element chunks of the gate width
    for (int blk = 0; blk < nblk; ++blk) {
        const int i0 = blk * GSB;
        // -- stage the means of states [i0, i0+32) as bf16 hi/lo pairs --
        for (int e = tid; e < GSB * Smem::DGP / 2; e += GTHREADS) {
            const int r = e / (Smem::DGP / 2), k2 = (e % (Smem::DGP / 2)) * 2;
            float p0 = 0.f, p1 = 0.f;
            if (i0 + r < s_hi && k2 < DG) {
                const float* pr = P + (bx * NS + i0 + r) * DG + k2;
                p0 = pr[0];
                p1 = pr[1];
            }
            const bf16_t h0 = f32_to_bf16(p0), h1 = f32_to_bf16(p1);
            const bf16_t l0 = f32_to_bf16(p0 - bf16_to_f32(h0)), l1 = f32_to_bf16(p1 - bf16_to_f32(h1));
            *reinterpret_cast<uint32_t*>(&sm.p_hi[r * Smem::DGP + k2]) = (uint32_t)h0 | ((uint32_t)h1 << 16);
            *reinterpret_cast<uint32_t*>(&sm.p_lo[r * Smem::DGP + k2]) = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
        if (SSC && tid == 0) sm.any_sel = 0u;
        __syncthreads();
        // -- gate logits for this wave's 32 tokens x 32 states (MFMA, hi + lo) --
        f32x16_t lg;
#pragma unroll
        for (int r = 0; r < 16; ++r) lg[r] = 0.f;
        const bf16_t* ur = U + ((size_t)bh * L + gtok) * DG;
        for (int kc = 0; kc < (gch + 1) / 2; ++kc) {
            const int e = kc * 16 + hi32 * 8;
            u32x4_t bu = {0u, 0u, 0u, 0u};
            if (e < DG) bu = *reinterpret_cast<const u32x4_t*>(ur + e);
            const u32x4_t ah = *reinterpret_cast<const u32x4_t*>(&sm.p_hi[l32 * Smem::DGP + e]);
            const u32x4_t al = *reinterpret_cast<const u32x4_t*>(&sm.p_lo[l32 * Smem::DGP + e]);
            lg = mfma32x32x16(ah, bu, lg);
            lg = mfma32x32x16(al, bu, lg);
        }
        // -- online softmax update for the lane's token --
        uint32_t bits = 0u;
        if (SSC) {
            for (int c = 0; c < top_k; ++c) {
                const int sc_i = gsel[c];
                const int d = sc_i - i0;
                if (sc_i >= 0 && d >= 0 && d < GSB) bits |= 1u << d;
            }
        }
        float bm = -INFINITY;
        bool ok[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r / 4) + 4 * hi32 + (r % 4);
            ok[r] = gvalid && (i0 + row) < gs && (!SSC || ((bits >> row) & 1u));
            if (ok[r]) bm = fmaxf(bm, lg[r]);
        }
        bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
        const float m_new = fmaxf(m_tok, bm);
        const float sc = __expf(m_tok - m_new);
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r / 4) + 4 * hi32 + (r % 4);
            const float wv = ok[r] ? __expf(lg[r] - m_new) : 0.f;
            ps += wv;
            sm.w[row][gt] = wv;
        }
        ps += __shfl_xor(ps, 32, 64);
        l_tok = l_tok * sc + ps;
        m_tok = m_new;
        if (hi32 == 0) sm.scale[gt] = sc;
        if (SSC) {
            // union over the workgroup of the states any token selected in this block
            uint32_t any = bits;
            for (int o = 1; o < 64; o <<= 1) any |= __shfl_xor(any, o, 64);
            if (lane == 0 && any) atomicOr(&sm.any_sel, any);
        }
        __syncthreads();
        // -- rescale the accumulator to the new running max --
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const float s = sm.scale[tw * 64 + tb * 32 + l32];
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) acc[cb][tb] *= s;
        }
        const uint32_t any_sel = SSC ? sm.any_sel : 0xffffffffu;
        // -- the 32 states of this block --
        const int i_end = min(s_hi, i0 + GSB);
        for (int i = i0; i < i_end; ++i) {
            const int buf = i & 1;
            if (i + 1 < s_hi) stage_load(i + 1);
            if (!SSC || ((any_sel >> (i - i0)) & 1u)) {
                f32x16_t pp[CB][2];
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) pp[cb][tb][r] = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        const int c = cw * (DV / 2) + cb * 32 + l32;
                        const int kc = 2 * ks + hi32;
                        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
                            &sm.state[buf][c * DK + ((kc ^ (c % CPR)) * 8)]);
#pragma unroll
                        for (int tb = 0; tb < 2; ++tb) pp[cb][tb] = mfma32x32x16(a, qf[tb][ks], pp[cb][tb]);
                    }
                }
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    const float wv = sm.w[i - i0][tw * 64 + tb * 32 + l32];
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) acc[cb][tb] += wv * pp[cb][tb];
                }
            }
            if (i + 1 < s_hi) stage_store(buf ^ 1);
            __syncthreads();
        }
    }
    if (hi32 == 0) sm.inv_l[gt] = 1.f / l_tok;
    __syncthreads();

    // ---- y = acc / l, stored as bf16 (4 consecutive rows c per register group) ----
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int t = tile0 + tw * 64 + tb * 32 + l32;
        if (t >= L) continue;
        const float il = sm.inv_l[tw * 64 + tb * 32 + l32];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            bf16_t* yr = Y + ((size_t)bh * L + t) * DV + cw * (DV / 2) + cb * 32 + hi32 * 4;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 v;
                v.x = pack_bf16x2(acc[cb][tb][4 * g + 0] * il, acc[cb][tb][4 * g + 1] * il);
                v.y = pack_bf16x2(acc[cb][tb][4 * g + 2] * il, acc[cb][tb][4 * g + 3] * il);
                *reinterpret_cast<uint2*>(yr + g * 8) = v;
            }
        }
    }
}

template <int DK, int DV, bool SSC>
static int launch_grm_mfma_t(const mc_dims& d, int top_k, const void* Q, const void* U,
                             const float* xcum, const uint16_t* M_lo, const float* P,
                             const float* O_on, const int32_t* idx, void* Y, hipStream_t st) {
    const int NS = (d.L + d.seg_len - 1) / d.seg_len;
    const int T = (d.L + GT - 1) / GT;
    const int BH = d.B * d.H;
    hipLaunchKernelGGL((grm_mfma_kernel<DK, DV, SSC>), dim3(BH * T), dim3(GTHREADS), 0, st,
                       (const bf16_t*)Q, (const bf16_t*)U, xcum, (const bf16_t*)M_lo, P, O_on,
                       idx, top_k, BH, d.H, d.L, d.seg_len, NS, d.d_g, d.x_heads, d.phi,
                       (bf16_t*)Y);
    return (int)hipGetLastError();
}

// bf16 GRM / SSC read on MFMA.  Returns -1 when the sizes are not covered (caller falls
// back to the generic kernel), else the HIP status of the launch.
int launch_read_mfma(const mc_dims& d, bool ssc, int top_k, const void* Q, const void* U,
                     const float* xcum, const uint16_t* M_lo, const float* P,
                     const float* O_on, const int32_t* idx, void* Y, void* stream) {
    if (d.dtype != MC_BF16) return -1;
    hipStream_t st = (hipStream_t)stream;
#define MC_MF(DK, DV)                                                                        \
    if (d.d_k == DK && d.d_v == DV)                                                          \
        return ssc ? launch_grm_mfma_t<DK, DV, true>(d, top_k, Q, U, xcum, M_lo, P, O_on,    \
                                                     idx, Y, st)                             \
                   : launch_grm_mfma_t<DK, DV, false>(d, top_k, Q, U, xcum, M_lo, P, O_on,   \
                                                      idx, Y, st);
    MC_MF(128, 128)
    MC_MF(128, 64)
    MC_MF(64, 128)
    MC_MF(64, 64)
#undef MC_MF
    return -1;
}

}  // namespace mc
