// readout.hip -- the MC read path: context gate, Gated Residual Memory read and the
// Sparse Selective Caching read (generic fp32-accumulating VALU kernels, any supported d).
//
// Memory Caching paper §3.1, Eq. (9)-(10):
//   a_t^(i) = <u_t, MeanPooling(S^(i))> for the cached segments i < s,
//   a_t^(s) = <u_t, prefix mean of X over t's segment up to t>  (the online segment),
//   gamma_t = softmax_i a_t^(i),
//   y_t     = gamma^(s) M_t^(s) phi(q_t) + sum_{i<s} gamma^(i) M^(i) phi(q_t).
// Sparse Selective Caching (gitcode explainer §3.4): the same read over the Top-k cached
// segments by router score a_t^(i), plus the online memory, with the softmax over those.
#include <algorithm>

#include "common.cuh"
#include "mc_internal.h"

namespace mc {

// Online gate logit of every token: a_on[b,h,t] = <u_t, prefix mean of X over t's segment>
// (Memory Caching paper §3.1, Eq. 10 with the causal prefix mean for the online segment).
// One workgroup per (segment, b, group of 4 heads): the segment's X is walked in chunks of
// 64 tokens; the inclusive prefix sums of a chunk are formed in LDS (thread e scans column
// e, carrying the sums of the earlier chunks); then each dot product <u_t, xcum_t> is taken
// by 16 lanes, each over 8-element slices of the gate width (16-byte loads of U).
template <typename T>
__global__ __launch_bounds__(256) void aon_kernel(const T* __restrict__ X,
                                                  const T* __restrict__ U, int L, int C,
                                                  int DG, int H, int xh,
                                                  float* __restrict__ a_on, const SegArg sg) {
    __shared__ float xs[64][260];
    __shared__ float carry[256];
    const int s = blockIdx.x, b = blockIdx.y, h0 = blockIdx.z * 4;
    const int t0 = seg_first(sg, s, C), len = seg_length(sg, s, C, L);
    const int tid = threadIdx.x;
    const int q = tid & 15, slot = tid >> 4;  // 16 lanes per dot product, 16 dots at a time
    const int nh = min(4, H - h0);
    // with per-head X each head of the group needs its own prefix sums
    const int npass = (xh == 1) ? 1 : nh;
    for (int pass = 0; pass < npass; ++pass) {
        const int hx = (xh == 1) ? 0 : h0 + pass;
        const T* Xb = X + ((size_t)b * xh + hx) * L * DG;
        for (int e = tid; e < DG; e += 256) carry[e] = 0.f;
        for (int j0 = 0; j0 < len; j0 += 64) {
            const int n = min(64, len - j0);
            __syncthreads();
            // four rows' loads in flight per thread (clamped to the chunk), then their stores
            const int nitem = n * (DG / 8);
            for (int b0 = 0; b0 < nitem; b0 += 4 * 256) {
                float v[4][8];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int e8 = min(b0 + u * 256 + tid, nitem - 1);
                    ld8(Xb, (size_t)(t0 + j0 + e8 / (DG / 8)) * DG + (e8 % (DG / 8)) * 8, v[u]);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int e8 = b0 + u * 256 + tid;
                    if (e8 < nitem) {
                        const int r = e8 / (DG / 8), e = (e8 % (DG / 8)) * 8;
#pragma unroll
                        for (int k = 0; k < 8; ++k) xs[r][e + k] = v[u][k];
                    }
                }
            }
            __syncthreads();
            for (int e = tid; e < DG; e += 256) {
                float acc = carry[e];
                for (int r = 0; r < n; ++r) {
                    acc += xs[r][e];
                    xs[r][e] = acc;
                }
                carry[e] = acc;
            }
            __syncthreads();
            const int nhp = (xh == 1) ? nh : 1;  // heads served by this pass
            // 16 dot products per slot at most, their U loads issued four at a time
            constexpr int NIT = 16, NB = 4;
            for (int k0 = 0; k0 < NIT; k0 += NB) {
            float uv[NB][8];
#pragma unroll
            for (int kq = 0; kq < NB; ++kq) {  // loads clamped to valid rows, used only if ok
                const int k = k0 + kq;
                const int item = slot + 16 * k;
                const int hh = min((xh == 1) ? item / 64 : pass, nh - 1), tt = min(item % 64, n - 1);
                ld8(U + (((size_t)b * H + h0 + hh) * L + t0 + j0 + tt) * DG,
                    (size_t)min(q * 8, DG - 8), uv[kq]);
            }
#pragma unroll
            for (int kq = 0; kq < NB; ++kq) {
                const int k = k0 + kq;
                const int item = slot + 16 * k;
                const int hh = (xh == 1) ? item / 64 : pass, tt = item % 64;
                float a = 0.f;
                if (q * 8 < DG && tt < n) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) a += uv[kq][e] * xs[tt][q * 8 + e];
                }
                // widths beyond 128: the remaining 8-element slices of this lane
                for (int e0 = q * 8 + 128; e0 < DG && item < nhp * 64 && tt < n; e0 += 128) {
                    float u2[8];
                    ld8(U + (((size_t)b * H + h0 + hh) * L + t0 + j0 + tt) * DG, (size_t)e0, u2);
#pragma unroll
                    for (int e = 0; e < 8; ++e) a += u2[e] * xs[tt][e0 + e];
                }
                a = warp_sum(a, 16);
                if (q == 0 && item < nhp * 64 && tt < n)
                    a_on[((size_t)b * H + h0 + hh) * L + t0 + j0 + tt] = a / (float)(j0 + tt + 1);
            }
            }
        }
        __syncthreads();
    }
}

static int launch_aon_sg(const mc_dims& d, const void* X, const void* U, float* a_on,
                         const SegArg& sg, hipStream_t st) {
    const int NS = sg.n ? sg.n : (d.L + d.seg_len - 1) / d.seg_len;
    dim3 grid(NS, d.B, (d.H + 3) / 4);
    if (d.dtype == MC_BF16)
        hipLaunchKernelGGL(aon_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)X,
                           (const bf16_t*)U, d.L, d.seg_len, d.d_g, d.H, d.x_heads, a_on, sg);
    else
        hipLaunchKernelGGL(aon_kernel<float>, grid, dim3(256), 0, st, (const float*)X,
                           (const float*)U, d.L, d.seg_len, d.d_g, d.H, d.x_heads, a_on, sg);
    return (int)hipGetLastError();
}

static const SegArg kConstSegR{};  // constant segment length

int launch_aon(const mc_dims& d, const void* X, const void* U, float* a_on, void* stream) {
    return launch_aon_sg(d, X, U, a_on, kConstSegR, (hipStream_t)stream);
}

// Segment-causal prefix sums of X in fp32: xps[b, xh, t, e] = sum of X[b, xh, r, e] over r from
// the first token of t's segment to t (the numerator of the online segment's prefix mean,
// Memory Caching paper §3.1, Eq. 10).  The sequence is cut into chunks of XCH tokens, one
// workgroup per (chunk, b*xh) and one thread per column, which scans its column of the chunk
// in registers and restarts at every segment start.  Three launches:
//   TAIL = true   tails[chunk, e]: the chunk's sum over its rows in the segment of its last
//                 row (the whole chunk unless a segment starts inside it)
//   group sums    of XSC consecutive tails (xps_group_kernel)
//   TAIL = false  the carry of the chunk's first segment (the tails of the earlier chunks that
//                 segment spans, whole groups by their group sums) plus the in-chunk scan,
//                 written to xps
constexpr int XCH = 64;
constexpr int XSC = 16;  // chunks per group of the second level of chunk sums

template <typename T, bool TAIL>
__global__ __launch_bounds__(256) void xps_kernel(const T* __restrict__ X, int L, int C, int DG,
                                                  float* __restrict__ tails,
                                                  float* __restrict__ xps, const SegArg sg) {
    const int c = blockIdx.x, nch = gridDim.x;
    const size_t bx = blockIdx.y;
    const int e = threadIdx.x;
    if (e >= DG) return;  // no barriers below
    const int c0 = c * XCH, c1 = min(L, c0 + XCH);
    const T* Xb = X + bx * (size_t)L * DG;
    // every row's load issued before the first sum (rows past the end read the last row and
    // are not summed): a load under a branch would be waited for row by row
    float v[XCH];
#pragma unroll
    for (int r = 0; r < XCH; ++r) v[r] = ld<T>(Xb, (size_t)min(c0 + r, c1 - 1) * DG + e);
    float run = 0.f;
    int si = seg_of(sg, c0, C);           // segment of the chunk's first row
    const int ss = seg_first(sg, si, C);  // and its start
    if (!TAIL) {
        // the sums of the segment's earlier chunks cs .. c-1 (chunk cs holds its start): whole
        // groups of XSC chunks by their group sums, the chunks before and after one by one
        const float* stails = tails + (size_t)gridDim.y * nch * DG;
        const int nsc = (nch + XSC - 1) / XSC;
        const int cs = ss / XCH;
        const int A = min(c, (cs + XSC - 1) / XSC * XSC), B = max(A, c / XSC * XSC);
        // rows lo .. hi-1 of a [row][DG] table added in order, eight loads in flight at a time
        auto add_rows = [&](const float* tab, int lo, int hi) {
            for (int i0 = lo; i0 < hi; i0 += 8) {
                float t[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) t[u] = tab[(size_t)min(i0 + u, hi - 1) * DG + e];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (i0 + u < hi) run += t[u];
            }
        };
        add_rows(tails + bx * nch * DG, cs, A);
        add_rows(stails + bx * nsc * DG, A / XSC, B / XSC);
        add_rows(tails + bx * nch * DG, B, c);
    }
    int nb = seg_first(sg, si + 1, C);  // the next segment start
    float* out = xps + (bx * L + c0) * DG + e;
    // the running sums first (in place of the rows), the stores after: stores among the sums
    // would make every row's load be waited for with all stores before it
#pragma unroll
    for (int r = 0; r < XCH; ++r) {
        const int t = c0 + r;
        if (t < c1) {
            if (t == nb) {
                run = 0.f;
                ++si;
                nb = seg_first(sg, si + 1, C);
            }
            run += v[r];
            v[r] = run;
        }
    }
    if (!TAIL) {
#pragma unroll
        for (int r = 0; r < XCH; ++r)
            if (c0 + r < c1) out[(size_t)r * DG] = v[r];
    }
    if (TAIL) tails[(bx * nch + c) * DG + e] = run;
}

// Group sums of the chunk sums: group g of (b, x head) = chunks g XSC .. g XSC + XSC - 1.  Only
// groups that lie inside one segment are read (there the chunk sums are whole-chunk sums).
__global__ __launch_bounds__(256) void xps_group_kernel(const float* __restrict__ tails,
                                                        int nch, int DG,
                                                        float* __restrict__ stails) {
    const int g = blockIdx.x, nsc = gridDim.x;
    const size_t bx = blockIdx.y;
    const int e = threadIdx.x;
    if (e >= DG) return;
    float t[XSC];  // every load issued before the first sum
#pragma unroll
    for (int i = 0; i < XSC; ++i) t[i] = tails[(bx * nch + min(g * XSC + i, nch - 1)) * DG + e];
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < XSC; ++i)
        if (g * XSC + i < nch) a += t[i];
    stails[(bx * nsc + g) * DG + e] = a;
}

// Online logits from the prefix sums: a_on[t] = <u_t, xps_t> / (j_t + 1), 8 threads per token.
template <typename T>
__global__ __launch_bounds__(256) void aon_xps_kernel(const T* __restrict__ U,
                                                      const float* __restrict__ xps, int L,
                                                      int C, int DG, int H, int xh,
                                                      float* __restrict__ a_on, const SegArg sg) {
    const size_t bh = blockIdx.y;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const size_t bx = (size_t)b * xh + (xh == 1 ? 0 : h);
    const int t = blockIdx.x * 32 + threadIdx.x / 8, p = threadIdx.x % 8;
    const bool valid = t < L;
    const int tc = valid ? t : L - 1;
    const int j = tc - seg_first(sg, seg_of(sg, tc, C), C);
    // thread p takes the 8-element slices p, p + 8, ... of the gate width (16-byte loads of U,
    // 32-byte loads of the prefix sums)
    float a = 0.f;
    for (int e = 8 * p; e < DG; e += 64) {
        float u[8], x[8];
        ld8(U + (bh * L + tc) * DG, (size_t)e, u);
        ld8(xps + (bx * L + tc) * DG, (size_t)e, x);
#pragma unroll
        for (int k = 0; k < 8; ++k) a += u[k] * x[k];
    }
    a = warp_sum(a, 8);
    if (valid && p == 0) a_on[bh * L + t] = a / (float)(j + 1);
}

// chunk sums, then their group sums
size_t xps_tail_floats(const mc_dims& d) {
    const size_t nch = (d.L + XCH - 1) / XCH;
    return (size_t)d.B * d.x_heads * (nch + (nch + XSC - 1) / XSC) * d.d_g;
}

static int launch_xps_sg(const mc_dims& d, const void* X, float* xps, float* tails,
                         const SegArg& sg, hipStream_t st) {
    if (d.d_g > 256) return (int)hipErrorInvalidValue;
    const int nch = (d.L + XCH - 1) / XCH;
    const dim3 grid(nch, d.B * d.x_heads);
    const dim3 block((d.d_g + 63) / 64 * 64);
    float* stails = tails + (size_t)d.B * d.x_heads * nch * d.d_g;
    if (d.dtype == MC_BF16)
        hipLaunchKernelGGL((xps_kernel<bf16_t, true>), grid, block, 0, st, (const bf16_t*)X, d.L,
                           d.seg_len, d.d_g, tails, xps, sg);
    else
        hipLaunchKernelGGL((xps_kernel<float, true>), grid, block, 0, st, (const float*)X, d.L,
                           d.seg_len, d.d_g, tails, xps, sg);
    // the group sums are read only for a segment longer than (XSC - 1) XCH tokens
    int longest = sg.n ? 0 : d.seg_len;
    for (int i = 0; i < sg.n; ++i) longest = std::max(longest, sg.off[i + 1] - sg.off[i]);
    if (longest > (XSC - 1) * XCH)
        hipLaunchKernelGGL(xps_group_kernel, dim3((nch + XSC - 1) / XSC, d.B * d.x_heads), block,
                           0, st, tails, nch, d.d_g, stails);
    if (d.dtype == MC_BF16)
        hipLaunchKernelGGL((xps_kernel<bf16_t, false>), grid, block, 0, st, (const bf16_t*)X, d.L,
                           d.seg_len, d.d_g, tails, xps, sg);
    else
        hipLaunchKernelGGL((xps_kernel<float, false>), grid, block, 0, st, (const float*)X, d.L,
                           d.seg_len, d.d_g, tails, xps, sg);
    return (int)hipGetLastError();
}

int launch_xps(const mc_dims& d, const void* X, float* xps, float* tails, void* stream) {
    return launch_xps_sg(d, X, xps, tails, kConstSegR, (hipStream_t)stream);
}

// Generic read kernel.  A workgroup covers TT = 32 consecutive tokens of one (b, h); the 8
// threads of a token share its gate (online softmax over the segments it reads) and each
// owns DV/8 consecutive output columns c = p DV/8 + m (vector loads of the online read and
// vector stores of y).  State i is read straight from global memory
// (TS = fp32 states for fp32 inputs, the bf16 copy for bf16 inputs).  SSC = true restricts
// each token to the segments listed in idx.
template <typename T, typename TS, int DK, int DV, bool SSC>
__global__ __launch_bounds__(256) void readout_valu_kernel(
    const T* __restrict__ Q, const T* __restrict__ U, const float* __restrict__ aon,
    const TS* __restrict__ S, const float* __restrict__ P, const float* __restrict__ O_on,
    const int32_t* __restrict__ idx, int top_k, int L, int C, int NS, int DG, int H, int xh,
    int phi, T* __restrict__ Y, float* __restrict__ gamma, const SegArg sg) {
    constexpr int TT = 32;
    constexpr int CPT = DV / 8;
    __shared__ float sq[TT][DK];

    const int tile0 = blockIdx.x * TT;
    const size_t bh = blockIdx.y;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const size_t bx = (size_t)b * xh + (xh == 1 ? 0 : h);
    const int tid = threadIdx.x;
    const int tt = tid / 8, p = tid % 8;
    const int t = tile0 + tt;
    const bool valid = t < L;
    const int tc = valid ? t : L - 1;  // clamped token for address formation
    const int s = seg_of(sg, tc, C);
    const int last = min(L, tile0 + TT) - 1;
    const int s_hi = seg_of(sg, last, C);  // largest segment index in this tile

    for (int e = tid; e < TT * DK; e += 256) {
        const int r = e % DK, tk = min(tile0 + e / DK, L - 1);
        sq[e / DK][r] = feature(ld(Q, (bh * L + tk) * DK + r), phi);
    }
    __syncthreads();

    // this thread's slice of u_t for the gate dots
    const int gch = DG / 8;
    const size_t urow = (bh * L + tc) * DG;
    const float a_on = aon[bh * L + tc];
    int sel[16];
    if (SSC) {
        for (int c = 0; c < 16; ++c) sel[c] = (c < top_k) ? idx[(bh * L + tc) * top_k + c] : -1;
    }

    float acc[CPT];
    float mx = a_on, l = 1.f;
    const size_t orow = (bh * L + tc) * DV + (size_t)p * CPT;
#pragma unroll
    for (int m = 0; m < CPT; m += 4) {
        const float4 o = *reinterpret_cast<const float4*>(O_on + orow + m);
        acc[m] = o.x;
        acc[m + 1] = o.y;
        acc[m + 2] = o.z;
        acc[m + 3] = o.w;
    }

    for (int i = 0; i < s_hi; ++i) {
        bool use = valid && i < s;
        if (SSC && use) {
            bool found = false;
            for (int c = 0; c < top_k && c < 16; ++c) found |= (sel[c] == i);
            use = found;
        }
        if (SSC && !__syncthreads_or(use)) continue;
        float a = 0.f;
        const float* Pi = P + (bx * NS + i) * DG;
        for (int e = p * gch; e < (p + 1) * gch; ++e) a += ld(U, urow + e) * Pi[e];
        a = warp_sum(a, 8);
        if (!use) continue;
        const float mn = fmaxf(mx, a);
        const float sc = __expf(mx - mn);
        const float w = __expf(a - mn);
        l = l * sc + w;
        mx = mn;
        const TS* Si = S + (bh * NS + i) * (size_t)(DV * DK);
#pragma unroll
        for (int m = 0; m < CPT; ++m) {
            const TS* row = Si + (size_t)(p * CPT + m) * DK;
            float dot = 0.f;
#pragma unroll 4
            for (int r = 0; r < DK; r += 8) {  // 16-byte (bf16) / 32-byte (fp32) row slices
                float v[8];
                ld8(row, (size_t)r, v);
#pragma unroll
                for (int e = 0; e < 8; ++e) dot += v[e] * sq[tt][r + e];
            }
            acc[m] = acc[m] * sc + w * dot;
        }
    }
    if (!valid) return;
    const float inv_l = 1.f / l;
#pragma unroll
    for (int m = 0; m < CPT; m += 8) st8(Y, (bh * L + t) * DV + (size_t)p * CPT + m, &acc[m], inv_l);

    if (gamma) {
        float* gr = gamma + (bh * L + t) * (size_t)NS;
        for (int i = p; i < NS; i += 8) {
            float g = 0.f;
            if (i == s) {
                g = __expf(a_on - mx) * inv_l;
            } else if (i < s) {
                bool use = true;
                if (SSC) {
                    use = false;
                    for (int c = 0; c < top_k && c < 16; ++c) use |= (sel[c] == i);
                }
                if (use) {
                    float a = 0.f;
                    const float* Pi = P + (bx * NS + i) * DG;
                    for (int e = 0; e < DG; ++e) a += ld(U, urow + e) * Pi[e];
                    g = __expf(a - mx) * inv_l;
                }
            }
            gr[i] = g;
        }
    }
}

template <typename T, typename TS, int DK, int DV, bool SSC>
static int launch_readout_t(const mc_dims& d, int top_k, const void* Q, const void* U,
                            const float* aon, const void* S, const float* P,
                            const float* O_on, const int32_t* idx, void* Y, float* gamma,
                            hipStream_t st, const SegArg& sg = kConstSegR) {
    const int NS = sg.n ? sg.n : (d.L + d.seg_len - 1) / d.seg_len;
    dim3 grid((d.L + 31) / 32, d.B * d.H);
    hipLaunchKernelGGL((readout_valu_kernel<T, TS, DK, DV, SSC>), grid, dim3(256), 0, st,
                       (const T*)Q, (const T*)U, aon, (const TS*)S, P, O_on, idx, top_k, d.L,
                       d.seg_len, NS, d.d_g, d.H, d.x_heads, d.phi, (T*)Y, gamma, sg);
    return (int)hipGetLastError();
}

template <bool SSC>
static int launch_readout(const mc_dims& d, int top_k, const void* Q, const void* U,
                          const float* aon, const float* M, const uint16_t* M_lo,
                          const float* P, const float* O_on, const int32_t* idx, void* Y,
                          float* gamma, hipStream_t st, const SegArg& sg = kConstSegR) {
#define MC_RD(DK, DV)                                                                      \
    if (d.d_k == DK && d.d_v == DV)                                                        \
        return d.dtype == MC_BF16                                                          \
                   ? launch_readout_t<bf16_t, bf16_t, DK, DV, SSC>(d, top_k, Q, U, aon,   \
                                                                   M_lo, P, O_on, idx, Y,  \
                                                                   gamma, st, sg)          \
                   : launch_readout_t<float, float, DK, DV, SSC>(d, top_k, Q, U, aon, M,  \
                                                                 P, O_on, idx, Y, gamma,   \
                                                                 st, sg);
    MC_RD(128, 128)
    MC_RD(128, 64)
    MC_RD(64, 128)
    MC_RD(64, 64)
#undef MC_RD
    return (int)hipErrorInvalidValue;
}

// gamma_t^(i) written out on request (a diagnostic output of the bf16 path, whose fused
// kernel never materialises the weights): one thread per token, fp32, straight from
// the definition.
template <typename T>
__global__ void gamma_kernel(const T* __restrict__ U, const float* __restrict__ aon,
                             const float* __restrict__ P, int L, int C, int NS, int DG, int H,
                             int xh, float* __restrict__ gamma, const SegArg sg) {
    const int t = blockIdx.x * 64 + threadIdx.x;
    const size_t bh = blockIdx.y;
    if (t >= L) return;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const size_t bx = (size_t)b * xh + (xh == 1 ? 0 : h);
    const int s = seg_of(sg, t, C);
    const T* u = U + (bh * L + t) * DG;
    const float a_on = aon[bh * L + t];
    auto logit = [&](int i) {
        const float* Pi = P + (bx * NS + i) * DG;
        float a = 0.f;
        for (int e = 0; e < DG; ++e) a += ld(u, e) * Pi[e];
        return a;
    };
    float mx = a_on;
    for (int i = 0; i < s; ++i) mx = fmaxf(mx, logit(i));
    float z = __expf(a_on - mx);
    for (int i = 0; i < s; ++i) z += __expf(logit(i) - mx);
    float* gr = gamma + (bh * L + t) * (size_t)NS;
    for (int i = 0; i < NS; ++i)
        gr[i] = i < s ? __expf(logit(i) - mx) / z : (i == s ? __expf(a_on - mx) / z : 0.f);
}

// Arbitrary boundaries: online logits, then the generic read with the online term O_on of
// mc_scan_prefill_segs.
int launch_grm_readout_segs(const mc_dims& d, const SegArg& sg, const void* Q, const void* U,
                            const void* X, const float* M, const uint16_t* M_lo, const float* P,
                            const float* O_on, float* aon, float* xps, float* xtail, void* Y,
                            float* gamma, void* stream, const SegGate& gate, const void* K,
                            const void* V, const PieceOnline* pon) {
    hipStream_t st = (hipStream_t)stream;
    int rc;
    auto logits = [&]() {  // the online logits token by token from the prefix sums
        const dim3 grid((d.L + 31) / 32, d.B * d.H);
        if (d.dtype == MC_BF16)
            hipLaunchKernelGGL(aon_xps_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)U,
                               xps, d.L, d.seg_len, d.d_g, d.H, d.x_heads, aon, sg);
        else
            hipLaunchKernelGGL(aon_xps_kernel<float>, grid, dim3(256), 0, st, (const float*)U,
                               xps, d.L, d.seg_len, d.d_g, d.H, d.x_heads, aon, sg);
        return (int)hipGetLastError();
    };
    if (xps) {  // prefix sums of X per segment
        rc = launch_xps_sg(d, X, xps, xtail, sg, st);
        if (rc) return rc;
        // bf16 widths 64/128: the MFMA read with the segment table (the online term from
        // O_on; its gate as its own pass when the workspace holds that pass's buffers, else
        // in-kernel, online logits included), then gamma on request
        GateWeights gw;
        if (gate.W && read_mfma_covers(d) && d.d_k == 128 && d.d_v == 128) {
            rc = launch_gate_w(d, U, xps, P, gate.pf, gate.W, gate.won, gate.inv_l, stream,
                               nullptr, 0, &sg);
            if (rc) return rc;
            gw.W = gate.W;
            gw.won = gate.won;
            gw.inv_l = gate.inv_l;
        }
        // (without O_on: the online term formed in the read over pieces, pon)
        rc = launch_read_mfma(d, false, 0, Q, K, V, U, xps, M_lo, P, O_on, nullptr, gw, Y, stream,
                              &sg, O_on ? nullptr : pon);
        if (rc >= 0) {
            if (rc || !gamma) return rc;
            if ((rc = logits())) return rc;
            hipLaunchKernelGGL(gamma_kernel<bf16_t>, dim3((d.L + 63) / 64, d.B * d.H), dim3(64),
                               0, st, (const bf16_t*)U, aon, P, d.L, d.seg_len, sg.n, d.d_g,
                               d.H, d.x_heads, gamma, sg);
            return (int)hipGetLastError();
        }
        if (!O_on) return (int)hipErrorInvalidValue;  // the generic read takes O_on
        rc = logits();  // not covered: the generic read below
    } else {
        rc = launch_aon_sg(d, X, U, aon, sg, st);
    }
    if (rc) return rc;
#define MC_RD(DK, DV)                                                                      \
    if (d.d_k == DK && d.d_v == DV)                                                        \
        return d.dtype == MC_BF16                                                          \
                   ? launch_readout_t<bf16_t, bf16_t, DK, DV, false>(d, 0, Q, U, aon, M_lo, \
                                                                     P, O_on, nullptr, Y,  \
                                                                     gamma, st, sg)        \
                   : launch_readout_t<float, float, DK, DV, false>(d, 0, Q, U, aon, M, P,  \
                                                                   O_on, nullptr, Y,       \
                                                                   gamma, st, sg);
    MC_RD(128, 128)
    MC_RD(128, 64)
    MC_RD(64, 128)
    MC_RD(64, 64)
#undef MC_RD
    return (int)hipErrorInvalidValue;
}

int launch_grm_readout(const mc_dims& d, const void* Q, const void* K, const void* V,
                       const void* U, const float* aon, const float* xps, const float* M,
                       const uint16_t* M_lo, const float* P, const float* O_on,
                       const GateWeights& gw, void* Y, float* gamma, void* stream) {
    if (!read_mfma_covers(d))
        return launch_readout<false>(d, 0, Q, U, aon, M, M_lo, P, O_on, nullptr, Y, gamma,
                                     (hipStream_t)stream);
    int rc = launch_read_mfma(d, false, 0, Q, K, V, U, xps, M_lo, P, O_on, nullptr, gw, Y,
                              stream);
    if (rc || !gamma) return rc;
    const int NS = (d.L + d.seg_len - 1) / d.seg_len;
    hipLaunchKernelGGL(gamma_kernel<bf16_t>, dim3((d.L + 63) / 64, d.B * d.H), dim3(64), 0,
                       (hipStream_t)stream, (const bf16_t*)U, aon, P, d.L, d.seg_len, NS,
                       d.d_g, d.H, d.x_heads, gamma, kConstSegR);
    return (int)hipGetLastError();
}

// Arbitrary boundaries without the routed read: the generic read restricted to the selections
// of idx, with the online term O_on of mc_scan_prefill_segs and the online logits aon.
int launch_ssc_readout_segs(const mc_dims& d, const SegArg& sg, int top_k, const void* Q,
                            const void* U, const float* aon, const float* M,
                            const uint16_t* M_lo, const float* P, const float* O_on,
                            const int32_t* idx, void* Y, void* stream) {
    return launch_readout<true>(d, top_k, Q, U, aon, M, M_lo, P, O_on, idx, Y, nullptr,
                                (hipStream_t)stream, sg);
}

int launch_aon_segs(const mc_dims& d, const SegArg& sg, const void* X, const void* U,
                    float* a_on, void* stream, float* xps, float* tails) {
    hipStream_t st = (hipStream_t)stream;
    if (!xps) return launch_aon_sg(d, X, U, a_on, sg, st);
    // through the prefix sums: the work per token does not depend on its segment's length
    int rc = launch_xps_sg(d, X, xps, tails, sg, st);
    if (rc) return rc;
    const dim3 grid((d.L + 31) / 32, d.B * d.H);
    if (d.dtype == MC_BF16)
        hipLaunchKernelGGL(aon_xps_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)U, xps,
                           d.L, d.seg_len, d.d_g, d.H, d.x_heads, a_on, sg);
    else
        hipLaunchKernelGGL(aon_xps_kernel<float>, grid, dim3(256), 0, st, (const float*)U, xps,
                           d.L, d.seg_len, d.d_g, d.H, d.x_heads, a_on, sg);
    return (int)hipGetLastError();
}

int launch_ssc_readout(const mc_dims& d, int top_k, const void* Q, const void* K,
                       const void* V, const void* U, const float* aon, const float* xps,
                       const float* M,
                       const uint16_t* M_lo, const float* P, const float* O_on,
                       const int32_t* idx, void* Y, void* stream) {
    if (read_mfma_ssc_covers(d, O_on != nullptr))
        return launch_read_mfma(d, true, top_k, Q, K, V, U, xps, M_lo, P, O_on, idx,
                                GateWeights{}, Y, stream);
    return launch_readout<true>(d, top_k, Q, U, aon, M, M_lo, P, O_on, idx, Y, nullptr,
                                (hipStream_t)stream);
}

// ---------------------------------------------------------------------------------------
// SSC selection.  The Top-k decision is taken on fp64 router scores formed exactly as the
// definition reads: the segment mean of X summed in token order and divided by the segment
// length, then <u_t, mean> accumulated over the gate width in order, every product and sum
// rounded separately (no fused multiply-add).  Ties go to the lower segment index.

// Segment means in fp64, stored gate column major: P64T[bx][e][s] for s < NSP (NS rounded up
// to SEL_W; the padding rows are 0), so that the means of a run of segments at one gate column
// are contiguous.
template <typename T>
__global__ void seg_mean64_kernel(const T* __restrict__ X, int L, int C, int NS, int NSP, int DG,
                                  double* __restrict__ P64T, const SegArg sg) {
    const int s = blockIdx.x;
    const size_t bx = blockIdx.y;
    const int t0 = s < NS ? seg_first(sg, s, C) : 0;
    const int len = s < NS ? seg_length(sg, s, C, L) : 0;
    for (int e = threadIdx.x; e < DG; e += blockDim.x) {
        double acc = 0.0;
        // sixteen rows' loads in flight, then their sums in token order
        for (int j0 = 0; j0 < len; j0 += 16) {
            double v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                v[u] = (double)ld(X, (bx * L + t0 + min(j0 + u, len - 1)) * DG + e);
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (j0 + u < len) acc = __dadd_rn(acc, v[u]);
        }
        P64T[(bx * DG + e) * NSP + s] = len > 0 ? __ddiv_rn(acc, (double)len) : 0.0;
    }
}

// u p and acc + m, each rounded to fp64 on its own: the header
// functions __dmul_rn / __dadd_rn are plain * and +, which the compiler may contract into
// one fused multiply-add, so contraction is switched off here explicitly
__device__ __forceinline__ double dmul_sep(double u, double p) {
#pragma clang fp contract(off)
    return u * p;
}
__device__ __forceinline__ double dadd_sep(double acc, double m) {
#pragma clang fp contract(off)
    return acc + m;
}

// SEL_T tokens of one (b, h) per workgroup of 4 waves.  The router score of token t and
// segment i is <u_t, mean_i> summed over the gate width e = 0, 1, ... in order, every product
// and every sum rounded separately (the oracle's order).  Lane l of every wave owns tokens
// 2 l, 2 l + 1, 128 + 2 l and 129 + 2 l of the tile; the waves split the candidate segments in
// runs of SEL_W (wave w takes segments c0 + SEL_W w .. + SEL_W - 1 of chunk c0), so a wave's
// means are the same for all its lanes and come through scalar loads, SEL_EB gate columns per
// batch (a scalar load can only be waited for together with all others in flight, so each
// wait should cover as much arithmetic as possible).  The tile's u values (exact in fp64) are
// staged in LDS a slab of SEL_E gate columns at a time and shared by the waves.  Every lane
// keeps, per token, a top-k list of its wave's candidates, presented in segment order, a
// candidate entering only if strictly larger, so the lower index wins ties.  The lists of
// waves 1..3 are then merged into wave 0's under the same order (larger score, then lower
// index first), and wave 0 writes the indices in ascending order, -1 padded.
constexpr int SEL_T = 256;  // tokens per workgroup (4 per lane)
constexpr int SEL_W = 8;    // segments per wave per chunk
constexpr int SEL_E = 16;   // gate columns per LDS slab
constexpr int SEL_EB = 4;   // gate columns per batch of scalar loads
static_assert(SEL_T == kSscTile, "the selection's tiles are the routed read's");

template <int KMAX>
__device__ __forceinline__ void sel_insert(double (&best)[KMAX], int (&bi)[KMAX], int top_k,
                                           double a, int i) {
    // first slot that is empty or holds an entry that (a, i) precedes
    int pos = top_k;
#pragma unroll
    for (int c = KMAX - 1; c >= 0; --c)
        if (c < top_k && (bi[c] < 0 || a > best[c] || (a == best[c] && i < bi[c]))) pos = c;
    if (pos >= top_k) return;
#pragma unroll
    for (int c = KMAX - 1; c > 0; --c)
        if (c < top_k && c > pos) { best[c] = best[c - 1]; bi[c] = bi[c - 1]; }
#pragma unroll
    for (int c = 0; c < KMAX; ++c)
        if (c == pos) { best[c] = a; bi[c] = i; }
}

// The same for a list that only ever receives candidates in ascending index order, whose empty
// slots hold -inf: (a, i) then precedes an entry exactly when a is strictly larger.  The list
// stays sorted, so the slots the candidate passes form a prefix of the comparisons from the end.
template <int KMAX>
__device__ __forceinline__ void sel_insert_asc(double (&best)[KMAX], int (&bi)[KMAX], int top_k,
                                               double a, int i) {
    bool gt[KMAX];
#pragma unroll
    for (int c = 0; c < KMAX; ++c) gt[c] = c < top_k && a > best[c];
#pragma unroll
    for (int c = KMAX - 1; c >= 0; --c) {
        if (!gt[c]) continue;
        const bool from_prev = c > 0 && gt[c - 1];
        best[c] = from_prev ? best[c > 0 ? c - 1 : 0] : a;
        bi[c] = from_prev ? bi[c > 0 ? c - 1 : 0] : i;
    }
}

template <typename T>
__device__ __forceinline__ void ld8_f64(const T* p, double (&v)[8]);
template <>
__device__ __forceinline__ void ld8_f64<bf16_t>(const bf16_t* p, double (&v)[8]) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = (double)__uint_as_float(q[j] << 16);
        v[2 * j + 1] = (double)__uint_as_float(q[j] & 0xffff0000u);
    }
}
template <>
__device__ __forceinline__ void ld8_f64<float>(const float* p, double (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// local token of lane l's a-th token
__device__ __forceinline__ int sel_tok(int lane, int a) { return 128 * (a >> 1) + 2 * lane + (a & 1); }

// the routing tail's per-state counters: at most this many segments
constexpr int SEL_NS_MAX = 4096;

template <int KMAX, int TPL>
constexpr int sel_lds_doubles() {
    // TPL = 4 (one pass over the tile): the u slab, or, after it, the lists being merged and
    // the final lists (SEL_T x KMAX scores and indices) and the per-state counters.
    // TPL = 1 (four passes of 64 tokens): the u slab (also the merge area of a pass), then
    // the final lists, which live across the passes, then the counters.
    return TPL == 4 ? (SEL_E * SEL_T > SEL_T * KMAX * 3 / 2 + (SEL_NS_MAX + 2) / 2
                           ? SEL_E * SEL_T
                           : SEL_T * KMAX * 3 / 2 + (SEL_NS_MAX + 2) / 2)
                    : SEL_E * SEL_T + SEL_T * KMAX * 3 / 2 + (SEL_NS_MAX + 2) / 2;
}

// Selection outputs beyond idx, for the routed read (all null: idx only).  Per token: the
// normalised online weight.  Per read tile of SEL_T tokens (tile = t / SEL_T, T tiles per
// head): the tile's (token, selected segment) pairs sorted by segment, as tile-local token
// numbers ptok and normalised weights pw (SEL_T * top_k slots), and the start of each
// segment's run poff[i] (NS + 1 entries, the last = the number of pairs).
struct SelRoute {
    const float* aon;  // [B, H, L] the online logits <u_t, prefix mean of X over t's segment>
    float* won;        // [B, H, L]
    int32_t* ptok;     // [B*H, T, SEL_T * top_k]
    float* pw;         // [B*H, T, SEL_T * top_k]
    int32_t* poff;     // [B*H, T, NS + 1]
    int NS;
};

// TPL tokens per lane: 4 (lists of up to 8 entries), or 1 with the tile taken in four passes
// of 64 tokens (lists of 16, which for four tokens would not stay in registers).
template <typename T, int KMAX, int TPL>
__device__ __forceinline__ void ssc_select_body(const T* __restrict__ U,
                                                const double* __restrict__ P64T, int L, int C,
                                                int NSP, int DG, int H, int xh, int top_k,
                                                int32_t* __restrict__ idx, const SelRoute& rt,
                                                const SegArg& sg) {
    static_assert(TPL == 4 || TPL == 1, "tokens per lane");
    constexpr int NPT = 64 * TPL;     // tokens per pass
    constexpr int NP = SEL_T / NPT;   // passes
    __shared__ __attribute__((aligned(16))) double lds[sel_lds_doubles<KMAX, TPL>()];
    double (*us)[SEL_T] = reinterpret_cast<double (*)[SEL_T]>(lds);
    // merge area of a pass ([pass-local token][KMAX]) and the final lists ([token][KMAX])
    double* mb = lds;
    int* mi = reinterpret_cast<int*>(mb + NPT * KMAX);
    double* fb = TPL == 4 ? lds : lds + SEL_E * SEL_T;
    int* fi = reinterpret_cast<int*>(fb + SEL_T * KMAX);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t bh = blockIdx.y;
    const int tile = gridDim.x - 1 - blockIdx.x;  // the latest tokens (most candidates) first
    const int t0 = tile * SEL_T;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const size_t bx = (size_t)b * xh + (xh == 1 ? 0 : h);
    const int ntok = min(SEL_T, L - t0);
    const T* Ut = U + (bh * L + t0) * DG;
    const double* Pb = P64T + bx * DG * NSP;
    // which run of a chunk a wave takes rotates from workgroup to workgroup, so that the
    // SIMDs share the work of chunks whose later runs hold no candidates
    const int run = (wave + blockIdx.x + blockIdx.y) & 3;
    // tile token of lane's a-th token in pass ps, and its place in the merge area
    auto tok_of = [&](int ps, int a) { return TPL == 4 ? sel_tok(lane, a) : NPT * ps + lane; };
    auto loc_of = [&](int a) { return TPL == 4 ? sel_tok(lane, a) : lane; };
    for (int ps = 0; ps < NP; ++ps) {
        const int pt0 = NPT * ps;  // first tile token of the pass
        const int pn = min(NPT, ntok - pt0);
        if (pn <= 0) break;
        const int smax = seg_of(sg, t0 + pt0 + pn - 1, C);  // segments 0..smax-1 are candidates
        int s_of[TPL];
#pragma unroll
        for (int a = 0; a < TPL; ++a)
            s_of[a] = tok_of(ps, a) < ntok ? seg_of(sg, t0 + tok_of(ps, a), C) : 0;
        double best[TPL][KMAX];
        int bi[TPL][KMAX];
#pragma unroll
        for (int a = 0; a < TPL; ++a)
#pragma unroll
            for (int c = 0; c < KMAX; ++c) { best[a][c] = -INFINITY; bi[a][c] = -1; }
        for (int c0 = 0; c0 < smax; c0 += 4 * SEL_W) {
            const int sw = c0 + SEL_W * run;  // this wave's first segment
            const bool act = sw < smax;
            double acc[TPL][SEL_W];
#pragma unroll
            for (int a = 0; a < TPL; ++a)
#pragma unroll
                for (int j = 0; j < SEL_W; ++j) acc[a][j] = 0.0;
            for (int e0 = 0; e0 < DG; e0 += SEL_E) {
                const int ek = min(SEL_E, DG - e0);  // a multiple of 8 (gate widths are)
                __syncthreads();                     // the previous slab is consumed
                for (int p = tid; p < (ek / 8) * NPT; p += 256) {
                    const int tok = pt0 + p % NPT, e = 8 * (p / NPT);
                    double v[8];
                    if (tok < ntok)
                        ld8_f64(Ut + (size_t)tok * DG + e0 + e, v);
                    else
#pragma unroll
                        for (int j = 0; j < 8; ++j) v[j] = 0.0;
#pragma unroll
                    for (int j = 0; j < 8; ++j) us[e + j][tok] = v[j];
                }
                __syncthreads();
                if (act) {
                    for (int e = 0; e < ek; e += SEL_EB) {
                        const double* pr = Pb + (size_t)(e0 + e) * NSP + sw;
                        double pv[SEL_EB][SEL_W];
#pragma unroll
                        for (int q = 0; q < SEL_EB; ++q)
#pragma unroll
                            for (int j = 0; j < SEL_W; ++j) pv[q][j] = pr[(size_t)q * NSP + j];
#pragma unroll
                        for (int q = 0; q < SEL_EB; ++q) {
                            double uu[TPL];
                            if constexpr (TPL == 4) {
                                const double2 u0 =
                                    *reinterpret_cast<const double2*>(&us[e + q][2 * lane]);
                                const double2 u1 =
                                    *reinterpret_cast<const double2*>(&us[e + q][128 + 2 * lane]);
                                uu[0] = u0.x;
                                uu[1] = u0.y;
                                uu[2 % TPL] = u1.x;
                                uu[3 % TPL] = u1.y;
                            } else {
                                uu[0] = us[e + q][pt0 + lane];
                            }
#pragma unroll
                            for (int a = 0; a < TPL; ++a) {
                                double m[SEL_W];
#pragma unroll
                                for (int j = 0; j < SEL_W; ++j) m[j] = dmul_sep(uu[a], pv[q][j]);
#pragma unroll
                                for (int j = 0; j < SEL_W; ++j)
                                    acc[a][j] = dadd_sep(acc[a][j], m[j]);
                            }
                        }
                    }
                }
            }
            if (act) {
#pragma unroll
                for (int a = 0; a < TPL; ++a)
#pragma unroll
                    for (int j = 0; j < SEL_W; ++j)
                        if (sw + j < s_of[a])
                            sel_insert_asc<KMAX>(best[a], bi[a], top_k, acc[a][j], sw + j);
            }
        }
        // waves 1..3 hand their lists to wave 0 through LDS, one wave at a time
        for (int w = 1; w < 4; ++w) {
            __syncthreads();
            if (wave == w) {
#pragma unroll
                for (int a = 0; a < TPL; ++a)
#pragma unroll
                    for (int c = 0; c < KMAX; ++c) {
                        mb[loc_of(a) * KMAX + c] = best[a][c];
                        mi[loc_of(a) * KMAX + c] = bi[a][c];
                    }
            }
            __syncthreads();
            if (wave == 0) {
#pragma unroll
                for (int a = 0; a < TPL; ++a)
#pragma unroll
                    for (int c = 0; c < KMAX; ++c) {
                        const int i = mi[loc_of(a) * KMAX + c];
                        if (c < top_k && i >= 0)
                            sel_insert<KMAX>(best[a], bi[a], top_k, mb[loc_of(a) * KMAX + c], i);
                    }
            }
        }
        // wave 0's lists go to the final lists
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int a = 0; a < TPL; ++a)
#pragma unroll
                for (int c = 0; c < KMAX; ++c) {
                    fb[tok_of(ps, a) * KMAX + c] = best[a][c];
                    fi[tok_of(ps, a) * KMAX + c] = bi[a][c];
                }
        }
    }
    // from here on thread t takes the tile's token t
    __syncthreads();
    const int t = tid;
    const bool tv = t < ntok;
    // the token's selection in ascending index order (-1 padded) with the scores alongside
    int oi[KMAX];
    double oa[KMAX];
    {
        int li[KMAX];
        double la[KMAX];
#pragma unroll
        for (int c = 0; c < KMAX; ++c) {
            li[c] = tv && c < top_k ? fi[t * KMAX + c] : -1;
            la[c] = tv && c < top_k ? fb[t * KMAX + c] : 0.0;
        }
        int prev = -1;
#pragma unroll
        for (int c = 0; c < KMAX; ++c) {
            int nxt = -1;
            double an = 0.0;
#pragma unroll
            for (int e = 0; e < KMAX; ++e)
                if (li[e] > prev && (nxt < 0 || li[e] < nxt)) { nxt = li[e]; an = la[e]; }
            oi[c] = nxt;
            oa[c] = an;
            if (nxt >= 0) prev = nxt;
        }
    }
    if (tv) {
        int32_t* out = idx + (bh * L + t0 + t) * top_k;
#pragma unroll
        for (int c = 0; c < KMAX; ++c)
            if (c < top_k) out[c] = oi[c];
    }
    if (!rt.ptok) return;
    // softmax over the selected segments' logits (the exact scores) and the online logit;
    // weights normalised
    float w[KMAX], won = 0.f;
    if (tv) {
        const int tg = t0 + t;
        const double a_on = (double)rt.aon[bh * L + tg];
        double m = a_on;
#pragma unroll
        for (int c = 0; c < KMAX; ++c)
            if (oi[c] >= 0) m = fmax(m, oa[c]);
        won = __expf((float)(a_on - m));
        float l = won;
#pragma unroll
        for (int c = 0; c < KMAX; ++c) {
            w[c] = oi[c] >= 0 ? __expf((float)(oa[c] - m)) : 0.f;
            l += w[c];
        }
        const float inv = 1.f / l;
        won *= inv;
#pragma unroll
        for (int c = 0; c < KMAX; ++c) w[c] *= inv;
        rt.won[bh * L + tg] = won;
    }
    // counting sort of the tile's (token, segment) pairs by segment
    const int NS = rt.NS;
    int* cnt = fi + SEL_T * KMAX;  // NS + 1 counters after the final lists
    for (int i = tid; i <= NS; i += 256) cnt[i] = 0;
    __syncthreads();
    int slot[KMAX];
#pragma unroll
    for (int c = 0; c < KMAX; ++c) slot[c] = oi[c] >= 0 ? atomicAdd(&cnt[oi[c]], 1) : 0;
    __syncthreads();
    if (wave == 0) {  // exclusive prefix sums, 64 segments at a time
        int carry = 0;
        for (int base = 0; base < NS; base += 64) {
            const int v = base + lane < NS ? cnt[base + lane] : 0;
            int x = v;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(x, o, 64);
                if (lane >= o) x += y;
            }
            if (base + lane < NS) cnt[base + lane] = carry + x - v;
            carry += __shfl(x, 63, 64);
        }
        if (lane == 0) cnt[NS] = carry;
    }
    __syncthreads();
    const size_t tb = bh * gridDim.x + tile;
    int32_t* ptok = rt.ptok + tb * SEL_T * top_k;
    float* pw = rt.pw + tb * SEL_T * top_k;
#pragma unroll
    for (int c = 0; c < KMAX; ++c)
        if (oi[c] >= 0) {
            const int p = cnt[oi[c]] + slot[c];
            ptok[p] = t;
            pw[p] = w[c];
        }
    for (int i = tid; i <= NS; i += 256) rt.poff[tb * (NS + 1) + i] = cnt[i];
}

template <typename T, int KMAX>
__global__ __launch_bounds__(256) void ssc_select_kernel(const T* __restrict__ U,
                                                         const double* __restrict__ P64T, int L,
                                                         int C, int NSP, int DG, int H, int xh,
                                                         int top_k, int32_t* __restrict__ idx,
                                                         const SelRoute rt, const SegArg sg) {
    ssc_select_body<T, KMAX, 4>(U, P64T, L, C, NSP, DG, H, xh, top_k, idx, rt, sg);
}

// lists of up to 16 entries: one token per lane, the tile in four passes
template <typename T>
__global__ __launch_bounds__(256) void ssc_select_wide_kernel(
    const T* __restrict__ U, const double* __restrict__ P64T, int L, int C, int NSP, int DG,
    int H, int xh, int top_k, int32_t* __restrict__ idx, const SelRoute rt, const SegArg sg) {
    ssc_select_body<T, 16, 1>(U, P64T, L, C, NSP, DG, H, xh, top_k, idx, rt, sg);
}

template <typename T, int KMAX>
static void launch_select_t(const mc_dims& d, int top_k, const T* U, const double* P64T, int NSP,
                            int32_t* idx, const SelRoute& rt, const SegArg& sg, hipStream_t st) {
    dim3 g((d.L + SEL_T - 1) / SEL_T, d.B * d.H);
    if constexpr (KMAX == 16)
        hipLaunchKernelGGL((ssc_select_wide_kernel<T>), g, dim3(256), 0, st, U, P64T, d.L,
                           d.seg_len, NSP, d.d_g, d.H, d.x_heads, top_k, idx, rt, sg);
    else
        hipLaunchKernelGGL((ssc_select_kernel<T, KMAX>), g, dim3(256), 0, st, U, P64T, d.L,
                           d.seg_len, NSP, d.d_g, d.H, d.x_heads, top_k, idx, rt, sg);
}

template <typename T>
static void launch_select_k(const mc_dims& d, int top_k, const T* U, const double* P64T, int NSP,
                            int32_t* idx, const SelRoute& rt, const SegArg& sg, hipStream_t st) {
    if (top_k <= 4)
        launch_select_t<T, 4>(d, top_k, U, P64T, NSP, idx, rt, sg, st);
    else if (top_k <= 8)
        launch_select_t<T, 8>(d, top_k, U, P64T, NSP, idx, rt, sg, st);
    else
        launch_select_t<T, 16>(d, top_k, U, P64T, NSP, idx, rt, sg, st);
}

size_t ssc_means_bytes(const mc_dims& d, int n_seg) {
    const int NS = n_seg ? n_seg : (d.L + d.seg_len - 1) / d.seg_len;
    const int NSP = (NS + SEL_W - 1) / SEL_W * SEL_W;
    return sizeof(double) * (size_t)d.B * d.x_heads * d.d_g * NSP;
}

int launch_ssc_select(const mc_dims& d, int top_k, const void* U, const void* X,
                      double* P64T, int32_t* idx, void* stream, const SscRoute* route,
                      const SegArg* sgp) {
    hipStream_t st = (hipStream_t)stream;
    const SegArg& sg = sgp ? *sgp : kConstSegR;
    const int NS = sg.n ? sg.n : (d.L + d.seg_len - 1) / d.seg_len;
    const int NSP = (NS + SEL_W - 1) / SEL_W * SEL_W;
    SelRoute rt{};
    if (route) {
        if (NS > SEL_NS_MAX || top_k > 16) return (int)hipErrorInvalidValue;
        rt.aon = route->aon;
        rt.won = route->won;
        rt.ptok = route->ptok;
        rt.pw = route->pw;
        rt.poff = route->poff;
        rt.NS = NS;
    }
    dim3 g1(NSP, d.B * d.x_heads);
    const int threads = d.d_g < 256 ? ((d.d_g + 63) / 64) * 64 : 256;
    if (d.dtype == MC_BF16) {
        hipLaunchKernelGGL(seg_mean64_kernel<bf16_t>, g1, dim3(threads), 0, st,
                           (const bf16_t*)X, d.L, d.seg_len, NS, NSP, d.d_g, P64T, sg);
        launch_select_k<bf16_t>(d, top_k, (const bf16_t*)U, P64T, NSP, idx, rt, sg, st);
    } else {
        hipLaunchKernelGGL(seg_mean64_kernel<float>, g1, dim3(threads), 0, st, (const float*)X,
                           d.L, d.seg_len, NS, NSP, d.d_g, P64T, sg);
        launch_select_k<float>(d, top_k, (const float*)U, P64T, NSP, idx, rt, sg, st);
    }
    return (int)hipGetLastError();
}

}  // namespace mc
