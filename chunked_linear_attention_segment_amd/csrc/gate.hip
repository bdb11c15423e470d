// gate.hip -- the Gated Residual Memory gate as its own pass, ahead of the gated read.
//
// Memory Caching paper §3.1, Eq. (10): for token t of segment s
//     a_t^(i) = <u_t, P_i>                      (i < s: the completed segments' means)
//     a_t^(s) = <u_t, prefix mean of X over t's segment up to t>   (the online segment)
//     gamma_t = softmax(a_t^(0..s)).
// With SSC selections (the Sparse Selective Caching read, gitcode explainer §3.4) only the
// token's selected segments and the online one enter the softmax: the others get weight 0.
// Segment boundaries are the constant length C or the offsets table (by value).
// For every read tile of RT consecutive tokens of one (b, h) this pass writes the softmax
// numerators against the token's own max logit m_t = max_i a_t^(i):
//     W[b,h,tile][i][t] = bf16(exp(a_t^(i) - m_t))  for the rows i < s_hi of the tile
//                         (s_hi = the segment of the tile's last token; 0 where i >= s),
//     won[b,h,t]   = exp(a_t^(s) - m_t),
//     inv_l[b,h,t] = 1 / (won + sum_{i<s} exp(a_t^(i) - m_t)),
// so the read multiplies state i by W, the online read by won, and the sum by inv_l.
//
// One workgroup = half a read tile (128 tokens) of G heads of one sequence, 4 waves of 32
// tokens.  The logits run on bf16
// MFMA with each mean split into a bf16 high part and a bf16 remainder (about 16 mantissa
// bits; laid out as MFMA fragments once, by pfrag_kernel, for every workgroup to share through
// the caches), u_t exact in bf16, fp32 accumulation.  Up to 128 states the logits stay in
// registers: m_t is taken over them, then the numerators are written, transposed through LDS
// into 16-byte stores of whole rows.  With more states pass 1 takes m_t over every logit and
// pass 2 forms them again for the numerators.
#include <type_traits>

#include "common.cuh"
#include "mc_internal.h"

namespace mc {
namespace {

typedef __bf16 gbf16x8_t __attribute__((ext_vector_type(8)));
typedef float gf32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t gu32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ gf32x16_t mfma_gate(const gu32x4_t& a, const gu32x4_t& b,
                                               const gf32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(gbf16x8_t, a),
                                                   __builtin_bit_cast(gbf16x8_t, b), c, 0, 0, 0);
}

// The means as MFMA A fragments, once for every workgroup: for 32-state block g, k-step kc and
// part (0: bf16 high, 1: bf16 remainder P - high), lane (l32, hi32) holds the 8 values of state
// 32 g + l32, gate columns 16 kc + 8 hi32 .. + 8, as 16 contiguous bytes.  States past NS are 0.
__global__ void pfrag_kernel(const float* __restrict__ P, int NS, int DG,
                             uint4* __restrict__ Pf) {
    const int NB = (NS + 31) / 32, KC = DG / 16;
    const size_t bx = blockIdx.y;
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;  // (g, kc, lane)
    if (idx >= NB * KC * 64) return;
    const int lane = idx % 64, kc = (idx / 64) % KC, g = idx / (64 * KC);
    const int row = 32 * g + (lane & 31), c0 = kc * 16 + (lane >> 5) * 8;
    uint32_t hw[4] = {0u, 0u, 0u, 0u}, lw[4] = {0u, 0u, 0u, 0u};
    if (row < NS) {
        const float* pr = P + (bx * NS + row) * DG + c0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float a = pr[2 * q], b = pr[2 * q + 1];
            hw[q] = pack_bf16x2(a, b);
            lw[q] = pack_bf16x2(a - __uint_as_float(hw[q] << 16),
                                b - __uint_as_float(hw[q] & 0xffff0000u));
        }
    }
    uint4* o = Pf + ((bx * NB + g) * KC + kc) * 2 * 64 + lane;
    o[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    o[64] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
}

constexpr int GT = 256;           // tokens per read tile (the rows of W cover one tile)
constexpr int GW = 128;           // tokens per workgroup: half a read tile, 32 per wave
constexpr int GDG_MAX = 128;      // widest gate (U fragments held in registers)
constexpr int GPF_STATES = 128;   // means staged in LDS (more are read from the caches)

template <bool SSC>
__global__ __launch_bounds__(256, 2) void gate_w_kernel(
    const bf16_t* __restrict__ U, const float* __restrict__ xps, const uint4* __restrict__ Pf,
    int H, int L, int C, int NS, int DG, int xh, int G, const int32_t* __restrict__ idx,
    int top_k, bf16_t* __restrict__ W, float* __restrict__ won_out,
    float* __restrict__ inv_l_out, const SegArg sg) {
    // the means' fragments of the first GPF_STATES states, staged once for the G heads
    __shared__ __attribute__((aligned(16))) uint4 pfl[GPF_STATES / 32 * (GDG_MAX / 16) * 2 * 64];
    // numerators of one 32-state block, [state][token], before the 16-byte stores
    __shared__ __attribute__((aligned(16))) bf16_t wt[32][GW];
    const int T = (L + GT - 1) / GT;
    const int half = blockIdx.x & 1, tile = blockIdx.x >> 1;
    const int bh0 = blockIdx.y * G;        // G consecutive heads of one sequence (shared X)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi32 = lane >> 5;
    const int h0 = tile * GT + half * GW;  // first token of this workgroup
    if (h0 >= L) return;                   // (the whole workgroup: no barrier is skipped)
    const int last = min(L, tile * GT + GT) - 1;
    const int s_hi = seg_of(sg, last, C);  // rows of W the read of this tile uses
    const size_t bx = (size_t)(bh0 / H) * xh + (xh == 1 ? 0 : bh0 % H);
    const int KC = DG / 16;
    const uint4* Pfb = Pf + bx * ((NS + 31) / 32) * KC * 2 * 64;
    const bool lds_pf = s_hi <= GPF_STATES;
    if (lds_pf) {
        const int n = (s_hi + 31) / 32 * KC * 2 * 64;
        for (int i = tid; i < n; i += 256) pfl[i] = Pfb[i];
    }
    __syncthreads();

    const int tl = 32 * wave + l32;        // token within the workgroup
    const bool val = h0 + tl < L;
    const int tok = min(h0 + tl, L - 1);
    const int seg = seg_of(sg, tok, C);
    // the token's prefix sum of X (its lane half's 8 of every 16 columns), shared by the heads
    float4 xv[GDG_MAX / 16][2];
    {
        const float* xr = xps + (bx * L + tok) * DG + hi32 * 8;
#pragma unroll
        for (int kc = 0; kc < GDG_MAX / 16; ++kc)
            if (kc < KC) {
                xv[kc][0] = *reinterpret_cast<const float4*>(xr + kc * 16);
                xv[kc][1] = *reinterpret_cast<const float4*>(xr + kc * 16 + 4);
            }
    }
    // u_t of head g as the B operand of the logits (token = column, k = 16 kc + 8 hi32 + e)
    gu32x4_t ub[GDG_MAX / 16];
    auto load_u = [&](int g, gu32x4_t (&dst)[GDG_MAX / 16]) {
#pragma unroll
        for (int kc = 0; kc < GDG_MAX / 16; ++kc)
            if (kc < KC)
                dst[kc] = *reinterpret_cast<const gu32x4_t*>(
                    U + ((size_t)(bh0 + g) * L + tok) * DG + kc * 16 + hi32 * 8);
    };
    for (int g = 0; g < G; ++g) {
        const int bh = bh0 + g;
        bf16_t* Wt = W + ((size_t)bh * T + tile) * NS * GT + half * GW;
        load_u(g, ub);
        // the online logit <u_t, xps_t> / (j + 1); the lane halves are summed
        float dot = 0.f;
#pragma unroll
        for (int kc = 0; kc < GDG_MAX / 16; ++kc) {
            if (kc < KC) {
                const float4 x0 = xv[kc][0], x1 = xv[kc][1];
                const gu32x4_t u = ub[kc];
                dot += __uint_as_float(u[0] << 16) * x0.x + __uint_as_float(u[0] & 0xffff0000u) * x0.y;
                dot += __uint_as_float(u[1] << 16) * x0.z + __uint_as_float(u[1] & 0xffff0000u) * x0.w;
                dot += __uint_as_float(u[2] << 16) * x1.x + __uint_as_float(u[2] & 0xffff0000u) * x1.y;
                dot += __uint_as_float(u[3] << 16) * x1.z + __uint_as_float(u[3] & 0xffff0000u) * x1.w;
            }
        }
        dot += __shfl_xor(dot, 32, 64);
        const float a_on = dot / (float)(tok - seg_first(sg, seg, C) + 1);
        // logits^T of states i0 .. i0+31 (rows; A = the means' high and remainder fragments)
        // x the wave's 32 tokens.  Accumulator element r is state i0 + 8 (r / 4) + 4 hi32 +
        // r % 4; a state counts for token t when it is a completed segment before t's, others
        // get -inf.  Where the fragments come from is a compile-time argument: with both
        // sources in one loop the compiler waits for every load and store in flight (the next
        // head's u, the numerators' stores) before each MFMA.
        auto logits = [&](int i0, auto from_lds) {
            constexpr bool FL = decltype(from_lds)::value;
            // the high and remainder parts accumulate separately (two independent MFMA
            // chains), and each k-step's fragments are read one step ahead
            gf32x16_t lg, lr;
#pragma unroll
            for (int r = 0; r < 16; ++r) lg[r] = lr[r] = 0.f;
            const size_t f0 = (size_t)(i0 / 32) * KC * 2 * 64 + lane;
            auto frag = [&](int kc, gu32x4_t& h, gu32x4_t& r) {
                if constexpr (FL) {
                    h = __builtin_bit_cast(gu32x4_t, pfl[f0 + kc * 128]);
                    r = __builtin_bit_cast(gu32x4_t, pfl[f0 + kc * 128 + 64]);
                } else {
                    h = __builtin_bit_cast(gu32x4_t, Pfb[f0 + kc * 128]);
                    r = __builtin_bit_cast(gu32x4_t, Pfb[f0 + kc * 128 + 64]);
                }
            };
            gu32x4_t fh[2], fr[2];
            frag(0, fh[0], fr[0]);
#pragma unroll
            for (int kc = 0; kc < GDG_MAX / 16; ++kc) {
                if (kc >= KC) break;
                if (kc + 1 < KC) frag(kc + 1, fh[(kc + 1) & 1], fr[(kc + 1) & 1]);
                lg = mfma_gate(fh[kc & 1], ub[kc], lg);
                lr = mfma_gate(fr[kc & 1], ub[kc], lr);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) lg[r] += lr[r];
            const int lim = seg - i0 - 4 * hi32;
            // SSC: only the token's selected segments (its idx row) keep their logits
            uint32_t sel = 0xffffffffu;
            if constexpr (SSC) {
                sel = 0u;
                const int32_t* row = idx + ((size_t)bh * L + tok) * top_k;
                for (int c = 0; c < top_k; ++c) {
                    const int dd = row[c] - i0;
                    if (row[c] >= 0 && dd >= 0 && dd < 32) sel |= 1u << dd;
                }
                sel >>= 4 * hi32;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = 8 * (r / 4) + (r % 4);
                if (!(rr < lim && ((sel >> rr) & 1u))) lg[r] = -INFINITY;
            }
            return lg;
        };
        auto passes = [&](auto from_lds) {
        // pass 1: m_t over every logit
        float m = a_on;
        for (int i0 = 0; i0 < s_hi; i0 += 32) {
            const gf32x16_t lg = logits(i0, from_lds);
            float bm = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) bm = fmaxf(bm, lg[r]);
            m = fmaxf(m, fmaxf(bm, __shfl_xor(bm, 32, 64)));
        }
        // pass 2: numerators of rows < s_hi (0 for tokens past L) through LDS to 16-byte
        // stores of whole rows
        float l = 0.f;
        for (int i0 = 0; i0 < s_hi; i0 += 32) {
            const gf32x16_t lg = logits(i0, from_lds);
            float ps = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float wv = val ? __expf(lg[r] - m) : 0.f;
                ps += wv;
                wt[8 * (r / 4) + 4 * hi32 + (r % 4)][tl] = f32_to_bf16(wv);
            }
            l += ps + __shfl_xor(ps, 32, 64);
            __syncthreads();
            const int rows = min(32, s_hi - i0);
#pragma unroll
            for (int q = 0; q < 32 * GW / 8 / 256; ++q) {
                const int c = q * 256 + tid, row = c / (GW / 8), col = (c % (GW / 8)) * 8;
                if (row < rows)
                    *reinterpret_cast<uint4*>(Wt + (size_t)(i0 + row) * GT + col) =
                        *reinterpret_cast<const uint4*>(&wt[row][col]);
            }
            __syncthreads();
        }
        if (val && !hi32) {
            const float wo = __expf(a_on - m);
            won_out[(size_t)bh * L + tok] = wo;
            inv_l_out[(size_t)bh * L + tok] = 1.f / (l + wo);
        }
        };
        // up to GPF_STATES states (the means staged in LDS): one pass, the logits kept in
        // registers between the max and the numerators
        auto one_pass = [&]() {
            gf32x16_t lgs[GPF_STATES / 32];
            float m = a_on;
#pragma unroll
            for (int b = 0; b < GPF_STATES / 32; ++b) {
                if (b * 32 >= s_hi) break;
                lgs[b] = logits(b * 32, std::true_type{});
                float bm = -INFINITY;
#pragma unroll
                for (int r = 0; r < 16; ++r) bm = fmaxf(bm, lgs[b][r]);
                m = fmaxf(m, fmaxf(bm, __shfl_xor(bm, 32, 64)));
            }
            float l = 0.f;
#pragma unroll
            for (int b = 0; b < GPF_STATES / 32; ++b) {
                if (b * 32 >= s_hi) break;
                float ps = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float wv = val ? __expf(lgs[b][r] - m) : 0.f;
                    ps += wv;
                    wt[8 * (r / 4) + 4 * hi32 + (r % 4)][tl] = f32_to_bf16(wv);
                }
                l += ps + __shfl_xor(ps, 32, 64);
                __syncthreads();
                const int rows = min(32, s_hi - b * 32);
#pragma unroll
                for (int q = 0; q < 32 * GW / 8 / 256; ++q) {
                    const int c = q * 256 + tid, row = c / (GW / 8), col = (c % (GW / 8)) * 8;
                    if (row < rows)
                        *reinterpret_cast<uint4*>(Wt + (size_t)(b * 32 + row) * GT + col) =
                            *reinterpret_cast<const uint4*>(&wt[row][col]);
                }
                __syncthreads();
            }
            if (val && !hi32) {
                const float wo = __expf(a_on - m);
                won_out[(size_t)bh * L + tok] = wo;
                inv_l_out[(size_t)bh * L + tok] = 1.f / (l + wo);
            }
        };
        if (lds_pf)
            one_pass();
        else
            passes(std::false_type{});
    }
}

}  // namespace

static const SegArg kConstSegG{};  // constant segment length

size_t gate_pfrag_bytes(const mc_dims& d, int n_seg) {
    const int NS = n_seg ? n_seg : (d.L + d.seg_len - 1) / d.seg_len;
    return (size_t)d.B * d.x_heads * ((NS + 31) / 32) * (d.d_g / 16) * 2 * 64 * 16;
}

int launch_gate_w(const mc_dims& d, const void* U, const float* xps, const float* P,
                  void* pfrag, uint16_t* W, float* won, float* inv_l, void* stream,
                  const int32_t* idx, int top_k, const SegArg* sgp) {
    const SegArg& sg = sgp ? *sgp : kConstSegG;
    const int NS = sg.n ? sg.n : (d.L + d.seg_len - 1) / d.seg_len;
    const int T = (d.L + GT - 1) / GT;
    const int nf = ((NS + 31) / 32) * (d.d_g / 16) * 64;
    hipLaunchKernelGGL(pfrag_kernel, dim3((nf + 255) / 256, d.B * d.x_heads), dim3(256), 0,
                       (hipStream_t)stream, P, NS, d.d_g, (uint4*)pfrag);
    // heads sharing one X (x_heads = 1) are taken G at a time, so a workgroup loads the prefix
    // sums of X once for G heads -- fewer heads per workgroup when that leaves too few
    // workgroups to keep every CU's memory requests in flight (a workgroup walks its heads in
    // turn)
    int G = d.x_heads == 1 ? (d.H % 8 == 0 ? 8 : (d.H % 4 == 0 ? 4 : (d.H % 2 == 0 ? 2 : 1))) : 1;
    while (G > 1 && (size_t)T * 2 * (d.B * d.H / G) < 1024) G /= 2;
    if (idx)
        hipLaunchKernelGGL(gate_w_kernel<true>, dim3(T * 2, d.B * d.H / G), dim3(256), 0,
                           (hipStream_t)stream, (const bf16_t*)U, xps, (const uint4*)pfrag, d.H,
                           d.L, d.seg_len, NS, d.d_g, d.x_heads, G, idx, top_k, (bf16_t*)W, won,
                           inv_l, sg);
    else
        hipLaunchKernelGGL(gate_w_kernel<false>, dim3(T * 2, d.B * d.H / G), dim3(256), 0,
                           (hipStream_t)stream, (const bf16_t*)U, xps, (const uint4*)pfrag, d.H,
                           d.L, d.seg_len, NS, d.d_g, d.x_heads, G, nullptr, 0, (bf16_t*)W, won,
                           inv_l, sg);
    return (int)hipGetLastError();
}

}  // namespace mc
