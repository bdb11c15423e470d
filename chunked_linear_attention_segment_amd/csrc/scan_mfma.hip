// scan_mfma.hip -- the MC write path on bf16 MFMA (gfx950): per-segment chunked scan.
//
// Memory Caching paper §3, Eq. (4b): inside segment s the memory starts from zero and runs
// M_t = M_{t-1} + v_t phi(k_t)^T; its state after the segment's last token is cached, and
// token t reads the memory after its own update (§3.1, Eq. 6/8): O_on[t] = M_t^(s) phi(q_t).
//
// One workgroup per (segment, b*H+h); the segment is walked in chunks of CH = 64 tokens.
// ON = false emits only the segment states (the read path then forms the online term itself).
// With M_prev the state before the chunk, for every token t of the chunk
//     O_on[t] = M_prev phi(q_t) + sum_{r <= t in chunk} (phi(q_t) . phi(k_r)) v_r
//     M      += sum_{r in chunk} v_r phi(k_r)^T
// all on 32x32x16 bf16 MFMA with fp32 accumulation.  Wave w (DV/32 waves) owns value rows
// cv in [32w, 32w+32): it keeps the fp32 state M^T[d][cv] of those rows in its accumulator
// registers for the whole segment, and its bf16 copy doubles as the A operand of the
// M_prev phi(q) term -- the accumulator's row order is reproduced in the k order of the
// phi(q) operand, so no shuffle is needed.  phi(k) and v are staged transposed in LDS (the
// token index is the contraction index of the state update); the causal score block
// S^T[r][t] = phi(k_r) . phi(q_t) goes through LDS as bf16.
//
// SW = true: the SWLA memory of window 2 (the paper's sliding-window linear attention,
// Eq. 28): M_t = alpha_t M_{t-1} + beta_t v_{t-1} phi(k_{t-1})^T + lam_t v_t phi(k_t)^T, the
// previous token taken only inside the segment.  Unrolled, the weight of v_r phi(k_r)^T in
// M_t (r <= t, same segment) is
//     c[t][r] = lam_t                                       (r = t)
//     c[t][r] = (alpha_{r+1} lam_r + beta_{r+1}) * alpha_{r+2} ... alpha_t   (r < t).
// The register state between chunks is Z = alpha_{j0} M_{j0-1} + beta_{j0} v_{j0-1} k_{j0-1}^T
// (the memory at the chunk's first token minus that token's own write), so inside the chunk
//     M_t = (alpha_{j0+1} ... alpha_t) Z + sum_{j0 <= r <= t} c[t][r] v_r phi(k_r)^T.
// Per chunk the weights c[t][r] are formed in LDS as running products down each column
// (exact for any alpha, zeros included); the online read scales the Z term per token and the
// scores by c[t][r], and the state update scales Z and weights each key with its final
// coefficient: c[e][r] at the segment's end e, else that of Z at the next chunk's first
// token, alpha_{e+1} c[e][r] (+ beta_{e+1} for r = e).
#include "common.cuh"
#include "mc_internal.h"

namespace mc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16_t scan_mfma(const u32x4_t& a, const u32x4_t& b,
                                              const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pk2(float lo, float hi) { return pack_bf16x2(lo, hi); }

// phi applied to 4 bf16 values held in two 32-bit words.
__device__ __forceinline__ u32x2_t phi4(u32x2_t v, int phi) {
    if (!phi) return v;
    u32x2_t o;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const float x0 = __uint_as_float(v[e] << 16);
        const float x1 = __uint_as_float(v[e] & 0xffff0000u);
        o[e] = pk2(feature(x0, 1), feature(x1, 1));
    }
    return o;
}

// One 16-byte direct global->LDS load per lane: the 16 bytes at base + voff land at LDS
// address lds_base + 16 * lane (lds_base wave-uniform).  The kernel waits for these loads
// itself (s_waitcnt vmcnt) before the barrier that publishes a tile.
__device__ __forceinline__ void scan_dma16(const void* base, uint32_t voff, uint32_t lds_base) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_base), "v"(voff), "s"(base)
                 : "memory", "m0");
#pragma clang diagnostic pop
}

constexpr int CH = 64;    // tokens per chunk
constexpr int TPAD = 72;  // row stride (elements) of the token-indexed LDS tiles

// (held to 256 registers, two waves per SIMD, so one workgroup's memory waits are covered by
// another's work)
template <int DK, int DV, bool ON, bool SW>
__global__ __launch_bounds__(DV * 2, 2) void scan_mfma_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    int L, int C, int NS, int phi, float* __restrict__ M, bf16_t* __restrict__ M_lo,
    float* __restrict__ O_on, SwlaGates gt, const SegArg sg, const float* __restrict__ M0,
    const bf16_t* __restrict__ dY, float* __restrict__ dgs) {
    constexpr int NT = DV * 2;      // threads: one wave per 32 value rows
    constexpr int DB = DK / 32;     // 32-row blocks of d
    constexpr int KSD = DK / 16;    // k-steps over d
    constexpr int GW = SW ? CH : 1; // SWLA tables (1-element placeholders otherwise)
    // phi(k)^T [d][r], v^T [cv][r] and the masked scores [t][r]; without SWLA the chunk's k,
    // v and q rows arrive in the same places first (see below)
    constexpr int KBE = DK * TPAD > CH * DK ? DK * TPAD : CH * DK;
    constexpr int VBE = DV * TPAD > CH * DV ? DV * TPAD : CH * DV;
    constexpr int QBE = !ON ? 8 : (CH * TPAD > CH * DK ? CH * TPAD : CH * DK);
    __shared__ __attribute__((aligned(16))) bf16_t kbuf[KBE];
    __shared__ __attribute__((aligned(16))) bf16_t vbuf[VBE];
    __shared__ __attribute__((aligned(16))) bf16_t qbuf[QBE];
    bf16_t(*kt)[TPAD] = reinterpret_cast<bf16_t(*)[TPAD]>(kbuf);
    bf16_t(*vt)[TPAD] = reinterpret_cast<bf16_t(*)[TPAD]>(vbuf);
    bf16_t(*sc)[TPAD] = reinterpret_cast<bf16_t(*)[TPAD]>(qbuf);
    __shared__ float cf[GW][GW + 1];  // SWLA weights c[t][r] of the chunk
    __shared__ float dz[GW];          // SWLA decay of Z at chunk token t: alpha_{j0+1..j0+t}
    __shared__ float ga[GW + 1], gb[GW + 1], gl[GW];  // the chunk's gates (+ next token's)
    // with dgs: each wave's share of <dy_t, O_on[t]> per chunk token (chunk parity buffers)
    __shared__ float red[ON ? 2 : 1][ON ? DV / 32 : 1][ON ? CH : 1];
    // the chunk's dy rows as loaded (the backward's <dy, O_on>; not SWLA)
    __shared__ __attribute__((aligned(16))) bf16_t yn[ON && !SW ? CH * DV : 8];
    bf16_t* const kn = kbuf;  // the chunk's k, v, q rows as loaded
    bf16_t* const vn = vbuf;
    bf16_t* const qn = qbuf;

    const int s = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int t0 = seg_first(sg, s, C);
    const int len = seg_length(sg, s, C, L);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, half = lane >> 5;

    f32x16_t mt[DB];  // M^T[d][cv] for this wave's 32 value rows, fp32
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt[db][r] = 0.f;
    u32x4_t ma[KSD];  // bf16 copy of M_prev in A-operand form (k-step k = rows 16k..16k+15)
    if (M0) {  // the memory before the segment's first token (a piece of a longer segment)
        const float* m0 = M0 + ((blockIdx.y * (size_t)NS + blockIdx.x) * DV + wave * 32 + (threadIdx.x & 31)) * DK;
        const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 v = *reinterpret_cast<const float4*>(m0 + db * 32 + 8 * g + 4 * hf);
                mt[db][4 * g] = v.x;
                mt[db][4 * g + 1] = v.y;
                mt[db][4 * g + 2] = v.z;
                mt[db][4 * g + 3] = v.w;
            }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                ma[2 * db + hh] = u32x4_t{pk2(mt[db][8 * hh + 0], mt[db][8 * hh + 1]),
                                          pk2(mt[db][8 * hh + 2], mt[db][8 * hh + 3]),
                                          pk2(mt[db][8 * hh + 4], mt[db][8 * hh + 5]),
                                          pk2(mt[db][8 * hh + 6], mt[db][8 * hh + 7])};
    }

    const bf16_t* Qs = Q + (bh * L + t0) * DK;
    const bf16_t* Ks = K + (bh * L + t0) * DK;
    const bf16_t* Vs = V + (bh * L + t0) * DV;

    const size_t gbase = bh * L + t0;
    // dgs of the chunk at jp from the waves' shares (read after the barrier that ends it)
    auto flush_dgs = [&](int jp) {
        if constexpr (ON) {
            int tf = tid;  // (re-formed per call, not held across the chunk loop)
            asm volatile("" : "+v"(tf));
            if (tf < min(CH, len - jp)) {
                float a = 0.f;
#pragma unroll
                for (int w = 0; w < DV / 32; ++w) a += red[(jp / CH) & 1][w][tf];
                dgs[gbase + jp + tf] = a;
            }
        }
    };
    {
        // The chunk's rows of k, v and q (and dy) arrive in LDS as whole rows by direct
        // global->LDS loads; row r's 16-byte chunk c sits at c ^ (r % chunks per row), and rows
        // past the chunk are loaded clamped to its last row (their products are masked).  The
        // fragments and the items of the transposed tiles are read into registers; after a
        // barrier phi(k)^T and the masked scores are written over the k and q rows, after
        // another v^T over the v rows.  That keeps the workgroup small enough for two per CU, so
        // one's loads are covered by the other's products.  The next chunk's rows load once the transposed
        // tiles have been consumed.
        auto tile_at = [&](const bf16_t* tile, int D, int r, int e) -> const bf16_t* {
            const int cpr = D / 8;
            return tile + r * D + ((((e >> 3) ^ (r % cpr)) << 3) | (e & 7));
        };
        // a tile's LDS byte address (the low 32 bits of its generic address), wave-uniform
        auto lds_base = [](const bf16_t* tile) -> uint32_t {
            return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)tile);
        };
        auto dma_tile = [&](const bf16_t* src, int D, uint32_t tile_base, int jn, int nn) {
            const int cpr = D / 8;
            int lo = lane;  // (formed per call, not held across the chunk loop)
            asm volatile("" : "+v"(lo));
#pragma unroll
            for (int m = 0; m < CH * (D / 8) / NT; ++m) {
                const int p = (m * (NT / 64) + wave) * 64 + lo;  // destination chunk
                const int r = p / cpr, c = (p % cpr) ^ (r % cpr);
                const uint32_t voff = (uint32_t)(((jn + min(r, nn - 1)) * D + c * 8) * 2);
                scan_dma16(src, voff, __builtin_amdgcn_readfirstlane(
                    tile_base + (uint32_t)((m * (NT / 64) + wave) * 64 * 16)));
            }
        };
        auto dma_kvq = [&](int jn, int nn) {
            dma_tile(Ks, DK, lds_base(kn), jn, nn);
            dma_tile(Vs, DV, lds_base(vn), jn, nn);
            if constexpr (ON) dma_tile(Qs, DK, lds_base(qn), jn, nn);
        };
        auto dma_y = [&](int jn, int nn) {
            if constexpr (ON && !SW) {
                if (dgs) dma_tile(dY + gbase * DV, DV, lds_base(yn), jn, nn);
            }
        };
        // SWLA: the gates of a chunk's tokens (slot CH: the token after the chunk; zero past the
        // segment), loaded into registers a chunk ahead and stored to LDS at the chunk's start
        float pga = 0.f, pgb = 0.f, pgl = 0.f;
        auto load_gates = [&](int jn) {
            if constexpr (SW) {
                const int nc = min(CH, len - jn);
                const bool in = tid <= CH && jn + tid < len && tid <= nc;
                pga = in ? gt.alpha[gbase + jn + tid] : 0.f;
                pgb = in ? gt.beta[gbase + jn + tid] : 0.f;
                pgl = in && tid < nc ? gt.lam[gbase + jn + tid] : 0.f;
            }
        };
        constexpr int NIK = (CH / 2) * (DK / 8) / NT, NIV = (CH / 2) * (DV / 8) / NT;
        static_assert(NIK * NT == (CH / 2) * (DK / 8) && NIV * NT == (CH / 2) * (DV / 8),
                      "staging items per thread");
        constexpr int SBW = (3 + NT / 64 - 1) / (NT / 64);  // score blocks per wave
        if (len > 0) {
            dma_kvq(0, min(CH, len));
            dma_y(0, min(CH, len));
            load_gates(0);
        }
        for (int j0 = 0; j0 < len; j0 += CH) {
            const int n = min(CH, len - j0);
            const bool more = j0 + CH < len;
            const int nn = more ? min(CH, len - j0 - CH) : 0;
            // this chunk's rows have landed for this lane; after the barrier for every lane
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (dgs && j0 > 0) flush_dgs(j0 - CH);
            const bool last = j0 + n == len;  // the segment ends in this chunk
            if constexpr (SW) {
                if (tid <= CH) {
                    ga[tid] = pga;
                    gb[tid] = pgb;
                    if (tid < CH) gl[tid] = pgl;
                }
                __syncthreads();
                if (tid < CH) {  // column r: c[r][r] = lam_r, then a running product down t
                    const int r = tid;
                    float c = gl[r];
                    cf[r][r] = c;
                    if (r + 1 < CH) {
                        c = ga[r + 1] * gl[r] + gb[r + 1];
                        cf[r + 1][r] = c;
#pragma unroll 8
                        for (int t = r + 2; t < CH; ++t) {
                            c *= ga[t];
                            cf[t][r] = c;
                        }
                    }
                } else if (tid == CH) {
                    float p = 1.f;
                    dz[0] = p;
#pragma unroll 8
                    for (int t = 1; t < CH; ++t) {
                        p *= ga[t];
                        dz[t] = p;
                    }
                }
                __syncthreads();
            }
            // SWLA: final weight of each key of the chunk in the state carried out of it, and
            // the factor on the incoming state
            float zs = 1.f;
            if constexpr (SW) zs = last ? dz[n - 1] : ga[CH] * dz[CH - 1];
            auto key_weight = [&](int r) -> float {
                if (r >= n) return 0.f;
                return last ? cf[n - 1][r] : ga[CH] * cf[CH - 1][r] + (r == CH - 1 ? gb[CH] : 0.f);
            };
            // the lane indices as the compiler cannot see them: the LDS addresses below are
            // formed per chunk, not held in registers across the chunk loop
            int ln = l32, hf = half, td = tid;
            asm volatile("" : "+v"(ln), "+v"(hf), "+v"(td));
            // ---- phi(q) B-fragments (k order of the accumulator rows), O^T = M_prev phi(q)^T ----
            u32x4_t qb[2][KSD];
            f32x16_t ot[2];
            if (ON) {
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    const int tl = tb * 32 + ln;
                    const bool ok = tl < n;
#pragma unroll
                    for (int ks = 0; ks < KSD; ++ks) {
                        u32x2_t lo = {0u, 0u}, hi = {0u, 0u};
                        if (ok) {
                            lo = phi4(*reinterpret_cast<const u32x2_t*>(tile_at(qn, DK, tl, ks * 16 + hf * 4)), phi);
                            hi = phi4(*reinterpret_cast<const u32x2_t*>(tile_at(qn, DK, tl, ks * 16 + 8 + hf * 4)), phi);
                        }
                        qb[tb][ks] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
                    }
                }
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) ot[tb][r] = 0.f;
                if (j0 > 0 || M0) {  // the A operand is the bf16 copy of M_prev, packed here
#pragma unroll
                    for (int ks = 0; ks < KSD; ++ks) {
                        const int db = ks / 2, hh = ks % 2;
                        const u32x4_t mk = {pk2(mt[db][8 * hh + 0], mt[db][8 * hh + 1]),
                                            pk2(mt[db][8 * hh + 2], mt[db][8 * hh + 3]),
                                            pk2(mt[db][8 * hh + 4], mt[db][8 * hh + 5]),
                                            pk2(mt[db][8 * hh + 6], mt[db][8 * hh + 7])};
#pragma unroll
                        for (int tb = 0; tb < 2; ++tb) ot[tb] = scan_mfma(mk, qb[tb][ks], ot[tb]);
                    }
                    if constexpr (SW) {  // the state decays by alpha_{j0+1} .. alpha_t before t reads it
#pragma unroll
                        for (int tb = 0; tb < 2; ++tb) ot[tb] *= dz[tb * 32 + ln];
                    }
                }
            }
            // ---- the wave's causal score blocks S^T[r][t] = phi(k_r).phi(q_t), r <= t: blocks
            //      (rb,tb) = (0,0), (0,1), (1,1); block (1,0) is all masked and never read ----
            f32x16_t sacc[SBW];
#pragma unroll
            for (int q = 0; q < SBW; ++q) {
                const int blk = wave + q * (NT / 64);
                if (!ON || blk >= 3) continue;
                const int rb = blk == 2 ? 1 : 0, tb = blk == 0 ? 0 : 1;
                const int rl = rb * 32 + ln;
                const bool ok = rl < n;
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[q][r] = 0.f;
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) {
                    u32x2_t lo = {0u, 0u}, hi = {0u, 0u};
                    if (ok) {
                        lo = phi4(*reinterpret_cast<const u32x2_t*>(tile_at(kn, DK, rl, ks * 16 + hf * 4)), phi);
                        hi = phi4(*reinterpret_cast<const u32x2_t*>(tile_at(kn, DK, rl, ks * 16 + 8 + hf * 4)), phi);
                    }
                    sacc[q] = scan_mfma(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, tb ? qb[1][ks] : qb[0][ks],
                                        sacc[q]);
                }
            }
            // the items of the transposed tiles: token pair (2p, 2p + 1), columns dc .. dc + 7
            u32x4_t ki[NIK][2];
#pragma unroll
            for (int m = 0; m < NIK; ++m) {
                const int it = td + m * NT, p = it % (CH / 2), dc = (it / (CH / 2)) * 8;
                const u32x4_t z = {0u, 0u, 0u, 0u};
                ki[m][0] = 2 * p < n ? *reinterpret_cast<const u32x4_t*>(tile_at(kn, DK, 2 * p, dc)) : z;
                ki[m][1] = 2 * p + 1 < n ? *reinterpret_cast<const u32x4_t*>(tile_at(kn, DK, 2 * p + 1, dc)) : z;
            }
            __syncthreads();  // the k and q rows have been read: phi(k)^T and the scores go there
            // ---- phi(k)^T and v^T (token pairs packed in 32-bit words), the masked scores ----
#pragma unroll
            for (int m = 0; m < NIK; ++m) {
                const int it = tid + m * NT, p = it % (CH / 2), dc = (it / (CH / 2)) * 8;
                const int r0 = 2 * p, r1 = 2 * p + 1;
                const u32x4_t a = ki[m][0], b = ki[m][1];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float a0 = __uint_as_float(a[e] << 16), a1 = __uint_as_float(a[e] & 0xffff0000u);
                    float b0 = __uint_as_float(b[e] << 16), b1 = __uint_as_float(b[e] & 0xffff0000u);
                    if (phi) {
                        a0 = r0 < n ? feature(a0, 1) : 0.f;
                        a1 = r0 < n ? feature(a1, 1) : 0.f;
                        b0 = r1 < n ? feature(b0, 1) : 0.f;
                        b1 = r1 < n ? feature(b1, 1) : 0.f;
                    }
                    if constexpr (SW) {
                        const float w0 = key_weight(r0), w1 = key_weight(r1);
                        a0 *= w0;
                        a1 *= w0;
                        b0 *= w1;
                        b1 *= w1;
                    }
                    *reinterpret_cast<uint32_t*>(&kt[dc + 2 * e][r0]) = pk2(a0, b0);
                    *reinterpret_cast<uint32_t*>(&kt[dc + 2 * e + 1][r0]) = pk2(a1, b1);
                }
            }
#pragma unroll
            for (int q = 0; q < SBW; ++q) {
                const int blk = wave + q * (NT / 64);
                if (!ON || blk >= 3) continue;
                const int rb = blk == 2 ? 1 : 0, tb = blk == 0 ? 0 : 1;
                const int t = tb * 32 + l32;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int r = rb * 32 + 8 * g + 4 * half;
                    float v0 = (r + 0 <= t) ? sacc[q][4 * g + 0] : 0.f;
                    float v1 = (r + 1 <= t) ? sacc[q][4 * g + 1] : 0.f;
                    float v2 = (r + 2 <= t) ? sacc[q][4 * g + 2] : 0.f;
                    float v3 = (r + 3 <= t) ? sacc[q][4 * g + 3] : 0.f;
                    if constexpr (SW) {
                        v0 = (r + 0 <= t) ? v0 * cf[t][r + 0] : 0.f;
                        v1 = (r + 1 <= t) ? v1 * cf[t][r + 1] : 0.f;
                        v2 = (r + 2 <= t) ? v2 * cf[t][r + 2] : 0.f;
                        v3 = (r + 3 <= t) ? v3 * cf[t][r + 3] : 0.f;
                    }
                    *reinterpret_cast<u32x2_t*>(&sc[t][r]) = u32x2_t{pk2(v0, v1), pk2(v2, v3)};
                }
            }
            // the v items, then v^T over the v rows once every wave has read its items
            u32x4_t vi[NIV][2];
#pragma unroll
            for (int m = 0; m < NIV; ++m) {
                const int it = td + m * NT, p = it % (CH / 2), dc = (it / (CH / 2)) * 8;
                const u32x4_t z = {0u, 0u, 0u, 0u};
                vi[m][0] = 2 * p < n ? *reinterpret_cast<const u32x4_t*>(tile_at(vn, DV, 2 * p, dc)) : z;
                vi[m][1] = 2 * p + 1 < n ? *reinterpret_cast<const u32x4_t*>(tile_at(vn, DV, 2 * p + 1, dc)) : z;
            }
            __syncthreads();
#pragma unroll
            for (int m = 0; m < NIV; ++m) {
                const int it = tid + m * NT, p = it % (CH / 2), dc = (it / (CH / 2)) * 8;
                const int r0 = 2 * p;
                const u32x4_t a = vi[m][0], b = vi[m][1];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    *reinterpret_cast<uint32_t*>(&vt[dc + 2 * e][r0]) = (a[e] & 0xffffu) | (b[e] << 16);
                    *reinterpret_cast<uint32_t*>(&vt[dc + 2 * e + 1][r0]) =
                        (a[e] >> 16) | (b[e] & 0xffff0000u);
                }
            }
            __syncthreads();
            // ---- O^T += v^T S^T (intra-chunk term) and M^T += phi(k)^T v (state update) ----
            const int cv = wave * 32 + l32;
            u32x4_t va[CH / 16];
#pragma unroll
            for (int ks = 0; ks < CH / 16; ++ks)
                va[ks] = *reinterpret_cast<const u32x4_t*>(&vt[cv][ks * 16 + half * 8]);
#pragma unroll
            for (int tb = 0; tb < 2 && ON; ++tb) {
                const int t = tb * 32 + l32;
#pragma unroll
                for (int ks = 0; ks < (tb + 1) * 2; ++ks) {
                    const u32x4_t sb = *reinterpret_cast<const u32x4_t*>(&sc[t][ks * 16 + half * 8]);
                    ot[tb] = scan_mfma(va[ks], sb, ot[tb]);
                }
            }
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d = db * 32 + l32;
                if constexpr (SW) mt[db] *= zs;
#pragma unroll
                for (int ks = 0; ks < CH / 16; ++ks) {
                    const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(&kt[d][ks * 16 + half * 8]);
                    mt[db] = scan_mfma(ka, va[ks], mt[db]);
                }
            }
            // ---- online read out: O_on[t][cv] (4 consecutive cv per register group), or its
            // product with dy_t summed over the wave's value rows ----
#pragma unroll
            for (int tb = 0; tb < 2 && ON; ++tb) {
                const int tl = tb * 32 + l32;
                if (!SW && dgs) {  // (the backward's pass: never with SWLA gates)
                    float part = 0.f;
                    if (tl < n) {
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const u32x2_t y = *reinterpret_cast<const u32x2_t*>(
                                tile_at(yn, DV, tb * 32 + ln, wave * 32 + 8 * g + hf * 4));
                            part += ot[tb][4 * g] * __uint_as_float(y[0] << 16) +
                                    ot[tb][4 * g + 1] * __uint_as_float(y[0] & 0xffff0000u) +
                                    ot[tb][4 * g + 2] * __uint_as_float(y[1] << 16) +
                                    ot[tb][4 * g + 3] * __uint_as_float(y[1] & 0xffff0000u);
                        }
                    }
                    part += __shfl_xor(part, 32);
                    if (half == 0) red[(j0 / CH) & 1][wave][tl] = part;
                } else if (tl < n) {
                    float* orow = O_on + (bh * L + t0 + j0 + tl) * DV + wave * 32 + half * 4;
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *reinterpret_cast<float4*>(orow + 8 * g) =
                            make_float4(ot[tb][4 * g], ot[tb][4 * g + 1], ot[tb][4 * g + 2],
                                        ot[tb][4 * g + 3]);
                }
            }
            __syncthreads();  // the transposed tiles, the scores and dy have been read
            if (more) {
                dma_kvq(j0 + CH, nn);
                dma_y(j0 + CH, nn);
                load_gates(j0 + CH);
            }
        }
    }
    if (dgs && len > 0) flush_dgs(((len - 1) / CH) * CH);
    // ---- emit the segment state: M[cv][d] (fp32 and bf16), 4 consecutive d per group ----
    if (!M) return;  // online read only
    int te = tid;  // (the thread index re-formed here, not held across the chunk loop)
    asm volatile("" : "+v"(te));
    const int cv = (te >> 6) * 32 + (te & 31), he = (te & 63) >> 5;
    const size_t mo = ((bh * NS + s) * DV + cv) * (size_t)DK;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = db * 32 + 8 * g + 4 * he;
            *reinterpret_cast<float4*>(M + mo + d) =
                make_float4(mt[db][4 * g], mt[db][4 * g + 1], mt[db][4 * g + 2], mt[db][4 * g + 3]);
            if (M_lo)  // (optional: the pieces of a split segment keep only fp32)
                *reinterpret_cast<u32x2_t*>(M_lo + mo + d) =
                    u32x2_t{pk2(mt[db][4 * g], mt[db][4 * g + 1]), pk2(mt[db][4 * g + 2], mt[db][4 * g + 3])};
        }
}

static const SegArg kConstSegM{};  // constant segment length

template <int DK, int DV>
static int launch_scan_mfma_t(const mc_dims& d, const void* Q, const void* K, const void* V,
                              float* M, uint16_t* M_lo, float* O_on, const SwlaGates& gt,
                              hipStream_t st, const SegArg& sg = kConstSegM,
                              const float* M0 = nullptr, const void* dY = nullptr,
                              float* dgs = nullptr) {
    const int NS = sg.n ? sg.n : (d.L + d.seg_len - 1) / d.seg_len;
#define MC_SCAN(ON, SW)                                                                        \
    hipLaunchKernelGGL((scan_mfma_kernel<DK, DV, ON, SW>), dim3(NS, d.B * d.H), dim3(DV * 2),   \
                       0, st, (const bf16_t*)Q, (const bf16_t*)K, (const bf16_t*)V, d.L,        \
                       d.seg_len, NS, d.phi, M, (bf16_t*)M_lo, O_on, gt, sg, M0,           \
                       (const bf16_t*)dY, dgs)
    if (gt.alpha) {  // SWLA: the read takes the online term from O_on, so it is always written
        if (!O_on) return (int)hipErrorInvalidValue;
        MC_SCAN(true, true);
    } else if (O_on || dgs) {
        MC_SCAN(true, false);
    } else {
        MC_SCAN(false, false);
    }
#undef MC_SCAN
    return (int)hipGetLastError();
}

// Any segment boundaries (the offsets passed by value), bf16: states, their bf16 copy and the
// optional online read; -1 when the sizes are not covered.
int launch_scan_mfma_segs(const mc_dims& d, const SegArg& sg, const void* Q, const void* K,
                          const void* V, float* M, uint16_t* M_lo, float* O_on, void* stream,
                          const float* M0) {
    if (d.dtype != MC_BF16) return -1;  // (M_lo may be NULL: pieces of a split segment)
    hipStream_t st = (hipStream_t)stream;
    const SwlaGates none{};
#define MC_SD(DK, DV)                                                                          \
    if (d.d_k == DK && d.d_v == DV)                                                            \
        return launch_scan_mfma_t<DK, DV>(d, Q, K, V, M, M_lo, O_on, none, st, sg, M0);
    MC_SD(128, 128)
    MC_SD(128, 64)
    MC_SD(64, 128)
    MC_SD(64, 64)
#undef MC_SD
    return -1;
}

// The online read alone (no state output) on the MFMA scan; -1 when the sizes are not covered.
int launch_scan_mfma_online(const mc_dims& d, const void* Q, const void* K, const void* V,
                            float* O_on, void* stream) {
    if (d.dtype != MC_BF16 || !O_on) return -1;
    hipStream_t st = (hipStream_t)stream;
    const SwlaGates none{};
#define MC_SD(DK, DV)                                                                          \
    if (d.d_k == DK && d.d_v == DV)                                                            \
        return launch_scan_mfma_t<DK, DV>(d, Q, K, V, nullptr, nullptr, O_on, none, st);
    MC_SD(128, 128)
    MC_SD(128, 64)
    MC_SD(64, 128)
    MC_SD(64, 64)
#undef MC_SD
    return -1;
}

// The online read's product with dy per token, dgs[t] = <dy_t, O_on[t]> ([B,H,L]), in place
// of O_on; -1 when the sizes are not covered.
int launch_scan_mfma_dgs(const mc_dims& d, const void* Q, const void* K, const void* V,
                         const void* dY, float* dgs, void* stream) {
    if (d.dtype != MC_BF16 || !dgs) return -1;
    hipStream_t st = (hipStream_t)stream;
    const SwlaGates none{};
#define MC_SD(DK, DV)                                                                          \
    if (d.d_k == DK && d.d_v == DV)                                                            \
        return launch_scan_mfma_t<DK, DV>(d, Q, K, V, nullptr, nullptr, nullptr, none, st,     \
                                          kConstSegM, nullptr, dY, dgs);
    MC_SD(128, 128)
    MC_SD(128, 64)
    MC_SD(64, 128)
    MC_SD(64, 64)
#undef MC_SD
    return -1;
}

// bf16 scan on MFMA (constant segments, or the offsets sg); -1 when the sizes are not
// covered (the caller uses the generic kernel).
int launch_scan_mfma(const mc_dims& d, const void* Q, const void* K, const void* V, float* M,
                     uint16_t* M_lo, float* O_on, const SwlaGates& gt, void* stream,
                     const SegArg* sg) {
    if (d.dtype != MC_BF16 || !M_lo) return -1;
    hipStream_t st = (hipStream_t)stream;
    const SegArg& seg = sg ? *sg : kConstSegM;
#define MC_SD(DK, DV)                                                                          \
    if (d.d_k == DK && d.d_v == DV)                                                            \
        return launch_scan_mfma_t<DK, DV>(d, Q, K, V, M, M_lo, O_on, gt, st, seg);
    MC_SD(128, 128)
    MC_SD(128, 64)
    MC_SD(64, 128)
    MC_SD(64, 64)
#undef MC_SD
    return -1;
}

}  // namespace mc
