// grm_mfma.hip -- the Gated Residual Memory read on bf16 MFMA (gfx950), fused with the gate.
//
// Memory Caching paper §3.1, Eq. (9)-(10): for token t of segment s
//     y_t = gamma^(s) M_t^(s) phi(q_t) + sum_{i<s} gamma^(i) M^(i) phi(q_t),
//     gamma_t = softmax( <u_t, P_0>, ..., <u_t, P_{s-1}>, a_on[t] ),
// a_on[t] = <u_t, prefix mean of X over t's segment> (the online segment's logit).  The
// online term M_t^(s) phi(q_t) is read from O_on when the scan wrote it, else (FON = true)
// formed in the kernel from K and V.  With SSC = true the kernel is
// the Sparse Selective Caching read (gitcode explainer §3.4): a token weighs only the
// segments listed for it in idx, and its softmax runs over those and the online segment.
//
// Layout (transposed, so a token's gate weight is a per-lane scalar):
//     Y^T[c, t] = sum_i w_t^(i) (M^(i) Qhat^T)[c, t]
// A workgroup is 256 consecutive tokens of one (b, h) and 8 waves (two per SIMD); wave
// (cw, tw) owns value rows [cw*DV/2, (cw+1)*DV/2) and tokens [64 tw, 64 tw + 64).  Per
// cached state i:
//   A = M^(i) (d_v x d_k bf16): staged once in LDS for the workgroup by direct global->LDS
//       loads that stream state i+1 in while state i is read (two buffers); each load
//       instruction copies whole rows (coalesced), and 16-byte chunks are XOR-swizzled per
//       row so the fragment reads are bank-conflict free;
//   B = phi(q)^T: kept in registers for the whole kernel;
//   the 32x32x16 MFMA partial product is scaled by the token weights and added to the fp32
//   accumulator.
// The gate runs on MFMA in blocks of 32 states: wave w forms logits^T = P_block U^T for
// tokens [32 w, 32 w + 32) (the fp32 means split into bf16 hi + lo parts, so the
// logits keep ~16 mantissa bits), then an online softmax per token (running max m_t and sum
// l_t; the accumulator is rescaled by exp(m_old - m_new) per block).  The weights of block
// b+1 are formed while block b is still being read (two LDS weight buffers), so the gate
// costs no extra workgroup barrier.  The online term enters as the initial accumulator with
// weight exp(a_on - m) = 1 at m = a_on.
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


constexpr int GT = 256;       // tokens per workgroup
constexpr int GSB = 32;       // states per gate block
constexpr int GTHREADS = 512; // 8 waves

// One 16-byte direct global->LDS load per lane: the 16 bytes at base + voff land at LDS
// address lds_base + 16*lane (lds_base wave-uniform).  Issued as inline assembly so that
// the compiler does not serialise LDS reads of the other buffer behind it; the kernel waits
// for these loads itself (s_waitcnt vmcnt) before the barrier that publishes a buffer.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t lds_base) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_base), "v"(voff), "s"(base)
                 : "memory", "m0");
#pragma clang diagnostic pop
}

template <int DK, int DV>
struct GrmSmem {
    bf16_t state[2][DV * DK];
    float w[2][GSB][GT];   // gate weights of the current / next block
    float scale[2][GT];    // exp(m_old - m_new) applied when a block starts
    float inv_l[GT];
    uint32_t any_sel[2];   // SSC: states of the block some token of the tile selected
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

template <int DK, int DV, bool SSC, bool FON, int PHI>
__global__ __launch_bounds__(GTHREADS, 1) void grm_mfma_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ U, const float* __restrict__ aon,
    const bf16_t* __restrict__ S, const float* __restrict__ P, const float* __restrict__ O_on,
    const int32_t* __restrict__ idx, int top_k, int BH, int H, int L, int C, int NS, int DG,
    int xh, bf16_t* __restrict__ Y) {
    constexpr int KS = DK / 16;        // MFMA k-steps over d_k
    constexpr int CB = DV / 64;        // 32-row blocks per wave (a wave owns DV/2 rows)
    constexpr int TB = 2;              // 32-token blocks per wave
    constexpr int CPR = DK / 8;        // 16-byte chunks per state row
    constexpr int STAGE = DV * DK / 8 / GTHREADS;  // direct loads per lane per state
    static_assert(STAGE >= 1 && DV * DK / 8 % GTHREADS == 0, "staging layout");
    typedef GrmSmem<DK, DV> Smem;
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
    const int nblk = (s_hi + GSB - 1) / GSB;

    // ---- direct global -> LDS staging of state i into buffer `buf`: load m of wave w
    //      fills LDS chunks [(m*waves + w)*64, +64) -- whole rows, so each load instruction
    //      reads contiguous memory; chunk (c, kc) is stored at kc ^ (c % CPR) of row c.  The
    //      per-lane byte offsets inside a state are fixed. ----
    const bf16_t* Sbh = S + (size_t)bh * NS * DV * DK;
    uint32_t soff[STAGE];
#pragma unroll
    for (int m = 0; m < STAGE; ++m) {
        const int p = (m * (GTHREADS / 64) + wave) * 64 + lane;
        const int c = p / CPR, kc = (p % CPR) ^ (c % CPR);
        soff[m] = (uint32_t)((c * DK + kc * 8) * 2);
    }
    // A-fragment reads: row c = (its 32-row block) + l32 and chunk 2 ks + hi32 sit at byte
    // 16 * ((2 ks + hi32) ^ (l32 % CPR)) of the row (CPR divides 32).  `swz` is made opaque
    // once per loop iteration (asm below) so the compiler recomputes these offsets with one
    // xor per fragment instead of keeping all of them live in registers across the loop.
    uint32_t swz = (uint32_t)(l32 % CPR);
    auto stage = [&](int i, int buf) {
        const bf16_t* src = Sbh + (size_t)i * DV * DK;
#pragma unroll
        for (int m = 0; m < STAGE; ++m) {
            const int p0 = (m * (GTHREADS / 64) + wave) * 64;
            const uint32_t base = (uint32_t)(uintptr_t)&sm.state[buf][p0 * 8];
            lds_dma16(src, soff[m], __builtin_amdgcn_readfirstlane(base));
        }
    };

    // ---- gate state: wave w owns the softmax of tokens [32 w, 32 w + 32); both lane
    //      halves hold the same running max / sum ----
    constexpr int GB = 1;  // 32-token gate blocks per wave
    int gtl[GB], gtok[GB], gseg[GB];
    bool gval[GB];
    float m_tok[GB], l_tok[GB];
#pragma unroll
    for (int g = 0; g < GB; ++g) {
        gtl[g] = wave * 32 + l32;
        gval[g] = (tile0 + gtl[g]) < L;
        gtok[g] = min(tile0 + gtl[g], L - 1);
        gseg[g] = gtok[g] / C;
        m_tok[g] = aon[(size_t)bh * L + gtok[g]];
        l_tok[g] = 1.f;
    }

    // logits of block nb for the lane's tokens, softmax update, weights into buffer nb & 1
    auto gate = [&](int nb) {
        const int i0 = nb * GSB, wb = nb & 1;
        f32x16_t lg[GB];
#pragma unroll
        for (int g = 0; g < GB; ++g)
#pragma unroll
            for (int r = 0; r < 16; ++r) lg[g][r] = 0.f;
        // one 16-wide k-step: P rows split into bf16 hi + lo (the logits keep ~16 mantissa
        // bits), times the U fragment of the lane's token
        auto kstep = [&](const float4& p0, const float4& p1, const u32x4_t (&bu)[GB]) {
            const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
            u32x4_t ah, al;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t hh = pack_bf16x2(pv[2 * q], pv[2 * q + 1]);
                ah[q] = hh;
                al[q] = pack_bf16x2(pv[2 * q] - __uint_as_float(hh << 16),
                                    pv[2 * q + 1] - __uint_as_float(hh & 0xffff0000u));
            }
#pragma unroll
            for (int g = 0; g < GB; ++g) {
                lg[g] = mfma32x32x16(ah, bu[g], lg[g]);
                lg[g] = mfma32x32x16(al, bu[g], lg[g]);
            }
        };
        const bool prow_ok = (i0 + l32) < s_hi;
        const float* pr = P + (bx * NS + (prow_ok ? i0 + l32 : 0)) * DG + hi32 * 8;
        for (int kc = 0; kc < DG / 16; ++kc) {
            const int e = kc * 16;
            float4 p0 = make_float4(0.f, 0.f, 0.f, 0.f), p1 = p0;
            if (prow_ok) {
                p0 = *reinterpret_cast<const float4*>(pr + e);
                p1 = *reinterpret_cast<const float4*>(pr + e + 4);
            }
            u32x4_t bu[GB];
#pragma unroll
            for (int g = 0; g < GB; ++g)
                bu[g] = *reinterpret_cast<const u32x4_t*>(
                    U + ((size_t)bh * L + gtok[g]) * DG + e + hi32 * 8);
            kstep(p0, p1, bu);
        }
        uint32_t wave_any = 0u;
#pragma unroll
        for (int g = 0; g < GB; ++g) {
            uint32_t bits = 0xffffffffu;
            if (SSC) {
                bits = 0u;
                const int32_t* sel = idx + ((size_t)bh * L + gtok[g]) * top_k;
                for (int c = 0; c < top_k; ++c) {
                    const int d = sel[c] - i0;
                    if (sel[c] >= 0 && d >= 0 && d < GSB) bits |= 1u << d;
                }
            }
            // accumulator row 8*(r/4) + 4*hi32 + r%4 is state i0 + that row: the per-r part is
            // an immediate compared against one per-lane limit
            const int lim = gval[g] ? gseg[g] - i0 - 4 * hi32 : 0;
            const uint32_t bsh = bits >> (4 * hi32);
            float bm = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = 8 * (r / 4) + (r % 4);
                const bool ok = rr < lim && ((bsh >> rr) & 1u);
                lg[g][r] = ok ? lg[g][r] : -INFINITY;
                bm = fmaxf(bm, lg[g][r]);
            }
            bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
            const float m_new = fmaxf(m_tok[g], bm);
            const float sc = __expf(m_tok[g] - m_new);
            float ps = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 8 * (r / 4) + 4 * hi32 + (r % 4);
                const float wv = __expf(lg[g][r] - m_new);  // exp(-inf) = 0 for masked rows
                ps += wv;
                sm.w[wb][row][gtl[g]] = wv;
            }
            ps += __shfl_xor(ps, 32, 64);
            l_tok[g] = l_tok[g] * sc + ps;
            m_tok[g] = m_new;
            if (hi32 == 0) sm.scale[wb][gtl[g]] = sc;
            if (SSC) wave_any |= bits;
        }
        if (SSC) {
            for (int o = 1; o < 64; o <<= 1) wave_any |= __shfl_xor(wave_any, o, 64);
            if (lane == 0 && wave_any) atomicOr(&sm.any_sel[wb], wave_any);
        }
    };


    // ---- B operand: phi(q)^T fragments of this wave's 64 tokens, kept in registers ----
    u32x4_t qf[TB][KS];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const int t = min(tile0 + tw * 64 + tb * 32 + l32, L - 1);
        const bf16_t* qr = Q + ((size_t)bh * L + t) * DK + hi32 * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4_t v = *reinterpret_cast<const u32x4_t*>(qr + ks * 16);
            if (PHI) {
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

    // ---- accumulator = the online term M_t^(s) phi(q_t), weight 1 relative to m = a_on ----
    f32x16_t acc[CB][TB];
    if (FON) {
        // Formed here from K and V, as the masked linear attention of each token over the
        // keys of its own segment up to itself (the same sum as the scan's recurrence):
        // chunks of 64 keys from the segment start of the tile's first token to its last
        // token; scores S^T[r][t] = phi(k_r).phi(q_t) on MFMA with the phi(q) fragments
        // already in registers, masked to segment(t) start <= r <= t, rounded to bf16 and
        // multiplied by v^T.  The score accumulator's row order is reproduced in the k
        // order of the v^T operand, so the scores need no reshuffle.  LDS: phi(k) rows in
        // the first state buffer, v^T in the weight buffers (both free before the loop).
        constexpr int VTP = 72;  // row stride (elements) of the v^T tile
        static_assert(2 * DV * VTP * 2 <= (int)sizeof(float) * 2 * GSB * GT, "v^T tile size");
        static_assert(64 * DK <= DV * DK, "key tile size");
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[cb][tb][r] = 0.f;
        const int k_lo = (tile0 / C) * C;
        const int nkc = (last - k_lo) / 64 + 1;
        const int wt0 = tile0 + tw * 64;
        const int wt_last = min(wt0 + 63, L - 1);
        const int wseg0 = (min(wt0, L - 1) / C) * C;
        const bf16_t* Kbh = K + (size_t)bh * L * DK;
        const bf16_t* Vbh = V + (size_t)bh * L * DV;
        // k rows of chunk kc -> state buffer kc & 1 (direct loads of whole rows, chunks
        // XOR-swizzled as the states are; rows past the last token read token `last`, their
        // scores are masked)
        constexpr int KLD = 64 * DK / 8 / GTHREADS;  // direct loads per lane per key chunk
        auto stage_k = [&](int kc) {
            const int k0 = k_lo + kc * 64;
#pragma unroll
            for (int m = 0; m < KLD; ++m) {
                const int p0 = (m * (GTHREADS / 64) + wave) * 64;
                const int p = p0 + lane;
                const int r = p / CPR, c8 = (p % CPR) ^ (r % CPR);
                const int key = min(k0 + r, last);
                const uint32_t base = (uint32_t)(uintptr_t)&sm.state[kc & 1][p0 * 8];
                lds_dma16(Kbh, (uint32_t)(((size_t)key * DK + c8 * 8) * 2),
                          __builtin_amdgcn_readfirstlane(base));
            }
        };
        // v rows of chunk kc: one token pair x 8 columns per lane, transposed into v^T
        const int vp = tid % 32, vdc = (tid / 32) * 8;
        const bool vlane = vdc < DV;
        u32x4_t va0 = {0u, 0u, 0u, 0u}, va1 = va0;
        auto load_v = [&](int kc) {
            const int k0 = k_lo + kc * 64;
            va0 = u32x4_t{0u, 0u, 0u, 0u};
            va1 = va0;
            if (vlane && k0 + 2 * vp <= last)
                va0 = *reinterpret_cast<const u32x4_t*>(Vbh + (size_t)(k0 + 2 * vp) * DV + vdc);
            if (vlane && k0 + 2 * vp + 1 <= last)
                va1 = *reinterpret_cast<const u32x4_t*>(Vbh + (size_t)(k0 + 2 * vp + 1) * DV + vdc);
        };
        auto store_v = [&](int kc) {
            bf16_t* vt = reinterpret_cast<bf16_t*>(&sm.w[0][0][0]) + (kc & 1) * DV * VTP;
            if (!vlane) return;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                *reinterpret_cast<uint32_t*>(&vt[(vdc + 2 * e) * VTP + 2 * vp]) =
                    (va0[e] & 0xffffu) | (va1[e] << 16);
                *reinterpret_cast<uint32_t*>(&vt[(vdc + 2 * e + 1) * VTP + 2 * vp]) =
                    (va0[e] >> 16) | (va1[e] & 0xffff0000u);
            }
        };
        stage_k(0);
        load_v(0);
        store_v(0);
        for (int kc = 0; kc < nkc; ++kc) {
            const int k0 = k_lo + kc * 64;
            asm volatile("" : "+v"(swz));
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (kc + 1 < nkc) {
                stage_k(kc + 1);
                load_v(kc + 1);
            }
            const bf16_t* ks_lds = sm.state[kc & 1];
            const bf16_t* vt_lds = reinterpret_cast<const bf16_t*>(&sm.w[0][0][0]) + (kc & 1) * DV * VTP;
            if (!(k0 > wt_last || k0 + 63 < wseg0)) {  // some key of this chunk is read
            // every (key, token) pair of the chunk is read when all keys precede the wave's
            // first token and none precedes the segment start of its last token
            const bool full = (k0 + 63 <= wt0) && (k0 >= (wt_last / C) * C);
            // one 32-token block at a time keeps the score registers to 2 x 16
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const int t = wt0 + tb * 32 + l32;
                if (k0 > wt0 + tb * 32 + 31) continue;  // keys all after this token block
                f32x16_t sc[2];
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sc[rb][r] = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) {
                        u32x4_t ka = *reinterpret_cast<const u32x4_t*>(
                            &ks_lds[(rb * 32 + l32) * DK + (((2 * ks + hi32) ^ swz) * 8)]);
                        if (PHI) {  // the key tile holds raw k; phi is applied per fragment
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                ka[e] = pack_bf16x2(feature(__uint_as_float(ka[e] << 16), 1),
                                                    feature(__uint_as_float(ka[e] & 0xffff0000u), 1));
                        }
                        sc[rb] = mfma32x32x16(ka, qf[tb][ks], sc[rb]);
                    }
                const int tseg = (t / C) * C;
                u32x4_t sb[4];
                if (!full) {  // mask to segment(t) start <= r <= t
                    // key r = k0 + 4*hi32 + (an immediate per accumulator element)
                    const int hi_lim = t - k0 - 4 * hi32, lo_lim = tseg - k0 - 4 * hi32;
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int rr = rb * 32 + 8 * (i / 4) + (i % 4);
                            if (rr > hi_lim || rr < lo_lim) sc[rb][i] = 0.f;
                        }
                }
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        sb[2 * rb + q] = u32x4_t{pack_bf16x2(sc[rb][8 * q + 0], sc[rb][8 * q + 1]),
                                                 pack_bf16x2(sc[rb][8 * q + 2], sc[rb][8 * q + 3]),
                                                 pack_bf16x2(sc[rb][8 * q + 4], sc[rb][8 * q + 5]),
                                                 pack_bf16x2(sc[rb][8 * q + 6], sc[rb][8 * q + 7])};
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const int c = cw * (DV / 2) + cb * 32 + l32;
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        const uint2 lo = *reinterpret_cast<const uint2*>(&vt_lds[c * VTP + 16 * kk + 4 * hi32]);
                        const uint2 hi = *reinterpret_cast<const uint2*>(&vt_lds[c * VTP + 16 * kk + 8 + 4 * hi32]);
                        const u32x4_t va = {lo.x, lo.y, hi.x, hi.y};
                        acc[cb][tb] = mfma32x32x16(va, sb[kk], acc[cb][tb]);
                    }
                }
            }
            }
            if (kc + 1 < nkc) store_v(kc + 1);  // its buffer was last read in chunk kc-1
        }
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
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
    }

    if (SSC && tid < 2) sm.any_sel[tid] = 0u;
    __syncthreads();
    if (s_hi > 0) stage(0, 0);
    if (nblk > 0) gate(0);

    // ---- the cached states, one workgroup barrier per state ----
    for (int i = 0; i < s_hi; ++i) {
        const int buf = i & 1, j = i % GSB, wb = (i / GSB) & 1;
        asm volatile("" : "+v"(swz));
        // state i has landed for this lane; after the barrier for every lane, every wave is
        // done with state i-1 and the weights of this block are published
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (i + 1 < s_hi) stage(i + 1, buf ^ 1);
        if (SSC && j == 0 && tid == 0) sm.any_sel[wb ^ 1] = 0u;
        if (j == 0) {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const float s = sm.scale[wb][tw * 64 + tb * 32 + l32];
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) acc[cb][tb] *= s;
            }
        }
        if (!SSC || ((sm.any_sel[wb] >> j) & 1u)) {
            float w[TB];
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) w[tb] = sm.w[wb][j][tw * 64 + tb * 32 + l32];
            const bf16_t* st = sm.state[buf];
            f32x16_t pp[CB][TB];
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) pp[cb][tb][r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
                        &st[(cw * (DV / 2) + cb * 32 + l32) * DK + (((2 * ks + hi32) ^ swz) * 8)]);
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb) pp[cb][tb] = mfma32x32x16(a, qf[tb][ks], pp[cb][tb]);
                }
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) acc[cb][tb] += w[tb] * pp[cb][tb];
        }
        // the next block's weights, while the other waves still read this block's
        if (j == GSB - 1 && i + 1 < s_hi) gate(i / GSB + 1);
    }
#pragma unroll
    for (int g = 0; g < GB; ++g)
        if (hi32 == 0) sm.inv_l[gtl[g]] = 1.f / l_tok[g];
    __syncthreads();

    // ---- y = acc / l, stored as bf16 (4 consecutive rows c per register group) ----
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
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

template <int DK, int DV, bool SSC, bool FON, int PHI>
static void launch_grm_mfma_k(const mc_dims& d, int top_k, const void* Q, const void* K,
                              const void* V, const void* U, const float* aon,
                              const uint16_t* M_lo, const float* P, const float* O_on,
                              const int32_t* idx, void* Y, hipStream_t st) {
    const int NS = (d.L + d.seg_len - 1) / d.seg_len;
    const int T = (d.L + GT - 1) / GT;
    const int BH = d.B * d.H;
    hipLaunchKernelGGL((grm_mfma_kernel<DK, DV, SSC, FON, PHI>), dim3(BH * T), dim3(GTHREADS), 0,
                       st, (const bf16_t*)Q, (const bf16_t*)K, (const bf16_t*)V,
                       (const bf16_t*)U, aon, (const bf16_t*)M_lo, P, O_on, idx, top_k, BH, d.H,
                       d.L, d.seg_len, NS, d.d_g, d.x_heads, (bf16_t*)Y);
}

template <int DK, int DV, bool SSC>
static int launch_grm_mfma_t(const mc_dims& d, int top_k, const void* Q, const void* K,
                             const void* V, const void* U, const float* aon,
                             const uint16_t* M_lo, const float* P, const float* O_on,
                             const int32_t* idx, void* Y, hipStream_t st) {
    // the online term is formed in the kernel (from K and V) when the scan did not write it;
    // the feature map is a template argument so the key fragments' loop has no branches
    if (O_on)
        d.phi ? launch_grm_mfma_k<DK, DV, SSC, false, 1>(d, top_k, Q, K, V, U, aon, M_lo, P,
                                                         O_on, idx, Y, st)
              : launch_grm_mfma_k<DK, DV, SSC, false, 0>(d, top_k, Q, K, V, U, aon, M_lo, P,
                                                         O_on, idx, Y, st);
    else
        d.phi ? launch_grm_mfma_k<DK, DV, SSC, true, 1>(d, top_k, Q, K, V, U, aon, M_lo, P,
                                                        O_on, idx, Y, st)
              : launch_grm_mfma_k<DK, DV, SSC, true, 0>(d, top_k, Q, K, V, U, aon, M_lo, P,
                                                        O_on, idx, Y, st);
    return (int)hipGetLastError();
}

// bf16 GRM / SSC read on MFMA.  Returns -1 when the sizes are not covered (the caller
// falls back to the generic kernel), else the HIP status of the launch.
bool read_mfma_covers(const mc_dims& d) {
    return d.dtype == MC_BF16 && d.d_g % 16 == 0 && (d.d_k == 64 || d.d_k == 128) &&
           (d.d_v == 64 || d.d_v == 128);
}

int launch_read_mfma(const mc_dims& d, bool ssc, int top_k, const void* Q, const void* K,
                     const void* V, const void* U, const float* aon, const uint16_t* M_lo,
                     const float* P, const float* O_on, const int32_t* idx, void* Y,
                     void* stream) {
    if (!read_mfma_covers(d)) return -1;
    hipStream_t st = (hipStream_t)stream;
#define MC_MF(DK, DV)                                                                        \
    if (d.d_k == DK && d.d_v == DV)                                                          \
        return ssc ? launch_grm_mfma_t<DK, DV, true>(d, top_k, Q, K, V, U, aon, M_lo, P,     \
                                                     O_on, idx, Y, st)                       \
                   : launch_grm_mfma_t<DK, DV, false>(d, top_k, Q, K, V, U, aon, M_lo, P,    \
                                                      O_on, idx, Y, st);
    MC_MF(128, 128)
    MC_MF(128, 64)
    MC_MF(64, 128)
    MC_MF(64, 64)
#undef MC_MF
    return -1;
}

}  // namespace mc
