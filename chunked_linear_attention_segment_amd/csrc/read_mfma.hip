// read_mfma.hip -- the Gated Residual Memory read on bf16 MFMA (gfx950), fused with the gate
// and the online term.
//
// Memory Caching paper §3.1, Eq. (9)-(10): for token t of segment s
//     y_t = gamma^(s) M_t^(s) phi(q_t) + sum_{i<s} gamma^(i) M^(i) phi(q_t),
//     gamma_t = softmax( <u_t, P_0>, ..., <u_t, P_{s-1}>, a_on[t] ),
// a_on[t] = <u_t, prefix mean of X over t's segment> (the online segment's logit), formed here
// from xps, the segment-causal prefix sums of X.  With
// SSC = true it is the Sparse Selective Caching read (gitcode explainer §3.4): a token weighs
// only the segments listed for it in idx, and its softmax runs over those and the online
// segment.  The online term M_t^(s) phi(q_t) is formed here from K and V (FON = true) as the
// masked linear attention of t over the keys of its segment up to itself, or read from O_on.
//
// One workgroup = 256 consecutive tokens of one (b, h), 4 waves, one wave per SIMD (so a wave
// has 512 registers: the fp32 accumulators live in the accumulation registers).  Wave w owns
// the 32-token blocks w and 7 - w of the tile (pairing a short and a long causal prefix, so
// the online term costs every SIMD the same) and every value row.  Layout (transposed, so a
// token's weight is a per-lane scalar):
//     Y^T[c, t] = sum_i M^(i) [c, :] (w_t^(i) phi(q_t))
// Phases:
//   1. gate: the means P are staged in LDS; the logits <u_t, P_i> run on MFMA (P split into
//      bf16 hi + lo parts, so a logit keeps ~16 mantissa bits).  One pass over 32-state blocks
//      keeps a running max m_t (starting from the online logit), writes the softmax numerators
//      of each block against the max known at that block (bf16, LDS) and sums l_t with
//      rescaling; the read later scales block b by exp(m_b - m_t).  Tiles with more states
//      than LDS holds weights for take the max over every logit first instead;
//   2. online term: chunks of 64 keys; scores phi(k).phi(q) on MFMA, masked to the token's
//      segment and causal, scaled by the online weight exp(a_on - m_t), times v;
//   3. cached states: state i (d_v x d_k bf16) is streamed into LDS by direct global->LDS
//      loads two states ahead of the read (three buffers); per k-step the B operand is
//      bf16(w_t^(i) phi(q_t)) from fp32 copies of phi(q) held in registers, so the MFMA
//      accumulates the weighted sum directly.  The loop body is written in issue order
//      (the file is compiled without the machine schedulers): A fragments are read from LDS
//      two k-steps ahead, and every MFMA is followed by the three VALU ops that build a
//      quarter of a B fragment of the next k-step, which the matrix unit hides;
//   4. y = acc / l_t in bf16 (with the gate pass: staged through LDS into whole-row stores).
#include <atomic>
#include <climits>
#include <type_traits>

#include "common.cuh"
#include "mc_internal.h"

namespace mc {
namespace {

typedef __bf16 rbf16x8_t __attribute__((ext_vector_type(8)));
typedef float rf32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t ru32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ rf32x16_t mfma_bf16(const ru32x4_t& a, const ru32x4_t& b,
                                               const rf32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(rbf16x8_t, a),
                                                   __builtin_bit_cast(rbf16x8_t, b), c, 0, 0, 0);
}

constexpr int RT = 256;        // tokens per workgroup
constexpr int RTHREADS = 256;  // 4 waves
constexpr int NBUF = 3;        // state buffers: the load of state i+2 overlaps the read of state i
constexpr int PM_FLOATS = 16384;  // LDS capacity for staged means (64 KB)
constexpr int DG_MAX = 128;    // widest gate the kernel takes (U fragments held in registers)

// One 16-byte direct global->LDS load per lane: the 16 bytes at base + voff land at LDS
// address lds_base + 16*lane (lds_base wave-uniform).  Inline assembly so the compiler does
// not serialise LDS reads of the other buffer behind it; the kernel waits for these loads
// itself (s_waitcnt vmcnt) before the barrier that publishes a buffer.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_base) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_base), "v"(voff), "s"(base)
                 : "memory", "m0");
#pragma clang diagnostic pop
}

__device__ __forceinline__ void wait_all_and_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// states whose weights LDS holds at once (SSC keeps its selection bits beside them)
template <bool SSC> struct WCap { static constexpr int v = SSC ? 96 : 128; };

// SSC: one bit per state of the super-block that some token of the tile selected (GRM reads
// every state and keeps no bits, which leaves LDS for three state buffers)
template <bool SSC, int W> struct SelBits { uint32_t any_sel[W / 32]; };
template <int W> struct SelBits<false, W> {};

template <int DK, int DV, bool SSC>
struct ReadSmem : SelBits<SSC, WCap<SSC>::v> {
    static constexpr int WMAX = WCap<SSC>::v;
    // region A: the staged means (gate), then key / value^T chunks (online term), then the two
    // state buffers
    union {
        float pm[PM_FLOATS];
        struct {
            bf16_t k[2][64 * DK];
            bf16_t vt[2][DV * 64];
        } kv;
        bf16_t state[NBUF][DV * DK];
    } a;
    bf16_t w[WMAX][RT];           // softmax numerators of a super-block of states, [state][token]
};

// Map the flat block index to (b*H+h, tile).  Blocks are dealt round-robin to the 8 XCDs;
// when B*H is a multiple of 8 each XCD takes whole heads (its L2 then holds that head's
// cached states), and inside a head the tiles with the most cached states go first.
__device__ __forceinline__ void tile_of_block(int bid, int BH, int T, int& bh, int& tile) {
    if (BH % 8 == 0) {
        const int xcd = bid % 8, local = bid / 8;
        bh = xcd + 8 * (local / T);
        tile = T - 1 - local % T;
    } else {
        bh = bid / T;
        tile = T - 1 - bid % T;
    }
}

// One 256-token tile: flat block index bid (see tile_of_block), LDS at smem_raw.
template <int DK, int DV, bool SSC, bool FON, int PHI, bool PRE, bool PCS>
__device__ __forceinline__ void grm_read_tile(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ U, const float* __restrict__ xps, const bf16_t* __restrict__ S,
    const float* __restrict__ P, const float* __restrict__ O_on,
    const int32_t* __restrict__ idx, const bf16_t* __restrict__ Wg,
    const float* __restrict__ won_g, const float* __restrict__ inv_l_g, int top_k, int BH,
    int H, int L, int C, int NS, int DG, int xh, bf16_t* __restrict__ Y, const SegArg& sg,
    const PieceOnline& pon, char* smem_raw, int bid) {
    static_assert(!(PRE && SSC), "precomputed weights are a GRM mode");
    static_assert(!PCS || (FON && sizeof(PieceOnline) > 0), "pieces: the online term formed here");
    static_assert(RT == kGateTile, "the gate pass writes weights per read tile");
    constexpr int KS = DK / 16;  // MFMA k-steps over d_k
    constexpr int CB = DV / 32;  // 32-row blocks of the value dimension
    constexpr int TB = 2;        // 32-token blocks per wave
    constexpr int CPR = DK / 8;  // 16-byte chunks per state / key row
    constexpr int STAGE = DV * DK / 8 / RTHREADS;  // direct loads per lane per state
    static_assert(STAGE >= 1 && (DV * DK / 8) % RTHREADS == 0, "state staging layout");
    typedef ReadSmem<DK, DV, SSC> Smem;
    constexpr int WMAX = Smem::WMAX;
    static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget");
    Smem& sm = *reinterpret_cast<Smem*>(smem_raw);

    const int T = (L + RT - 1) / RT;
    int bh, tile;
    tile_of_block(bid, BH, T, bh, tile);
    // the thread index re-formed per tile, so that values derived from it are not held in
    // registers across the tiles of a persistent workgroup
    int tid_o = threadIdx.x;
    asm volatile("" : "+v"(tid_o));
    const int tid = tid_o, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi32 = lane >> 5;
    const int tile0 = tile * RT;
    const int last = min(L, tile0 + RT) - 1;
    const int s_hi = seg_of(sg, last, C);  // states 0..s_hi-1 are read by some token of the tile
    const size_t bx = (size_t)(bh / H) * xh + (xh == 1 ? 0 : bh % H);
    const float* Pbx = P + bx * NS * DG;

    // the lane's two tokens (one per 32-token block of the wave)
    int tl[TB], tok[TB], seg[TB];
    bool val[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const int blk = tb == 0 ? wave : 7 - wave;
        tl[tb] = 32 * blk + l32;
        val[tb] = tile0 + tl[tb] < L;
        tok[tb] = min(tile0 + tl[tb], L - 1);
        seg[tb] = seg_of(sg, tok[tb], C);
    }

    // =============================== 1. gate =================================================
    // super-blocks of SBS states: the means of one super-block fit the staging area
    const int SBS = min(WMAX, (PM_FLOATS / DG) & ~31);
    const int CPRP = DG / 4;                       // 16-byte chunks per mean row
    const int G = min(16, CPRP & -CPRP);           // XOR group: largest power of 2 dividing CPRP
    ru32x4_t ub[TB][DG_MAX / 16];  // U fragments (B operand of the logits), token = column
    auto load_u = [&]() {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int kc = 0; kc < DG_MAX / 16; ++kc)
                if (kc < DG / 16)
                    ub[tb][kc] = *reinterpret_cast<const ru32x4_t*>(
                        U + ((size_t)bh * L + tok[tb]) * DG + kc * 16 + hi32 * 8);
    };
    if constexpr (!PRE) load_u();
    // online logit a_on = <u_t, xps_t> / (j + 1): the lane half hi32 holds the u values
    // 16 kc + 8 hi32 .. + 8 of its U fragments; the halves are summed
    float m[TB], l[TB], won[TB], a_on[TB];
    if constexpr (!PRE) {
    float4 xv[TB][DG_MAX / 16][2];  // every load issued before the first product
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const float* xr = xps + (bx * L + tok[tb]) * DG + hi32 * 8;
#pragma unroll
        for (int kc = 0; kc < DG_MAX / 16; ++kc)
            if (kc < DG / 16) {
                xv[tb][kc][0] = *reinterpret_cast<const float4*>(xr + kc * 16);
                xv[tb][kc][1] = *reinterpret_cast<const float4*>(xr + kc * 16 + 4);
            }
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        float dot = 0.f;
#pragma unroll
        for (int kc = 0; kc < DG_MAX / 16; ++kc) {
            if (kc < DG / 16) {
                const float4 x0 = xv[tb][kc][0], x1 = xv[tb][kc][1];
                const ru32x4_t u = ub[tb][kc];
                dot += __uint_as_float(u[0] << 16) * x0.x + __uint_as_float(u[0] & 0xffff0000u) * x0.y;
                dot += __uint_as_float(u[1] << 16) * x0.z + __uint_as_float(u[1] & 0xffff0000u) * x0.w;
                dot += __uint_as_float(u[2] << 16) * x1.x + __uint_as_float(u[2] & 0xffff0000u) * x1.y;
                dot += __uint_as_float(u[3] << 16) * x1.z + __uint_as_float(u[3] & 0xffff0000u) * x1.w;
            }
        }
        dot += __shfl_xor(dot, 32, 64);
        a_on[tb] = dot / (float)(tok[tb] - seg_first(sg, seg[tb], C) + 1);
        m[tb] = a_on[tb];
        l[tb] = 0.f;
    }
    }

    // P rows [i0, i0 + n) -> sm.a.pm: row r at r * DG floats, its 16-byte chunk c stored at
    // c ^ (r % G) so the logits' row-per-lane reads spread over the banks
    auto stage_means = [&](int i0, int n) {
        const int total = n * CPRP;
        for (int p0 = wave * 64; p0 < total; p0 += RTHREADS) {
            const int p = p0 + lane;
            const int r = p / CPRP, pos = p % CPRP;
            const int c = pos ^ (r & (G - 1));
            const uint32_t base = (uint32_t)(uintptr_t)&sm.a.pm[p0 * 4];
            if (p < total)
                dma16(Pbx, (uint32_t)(((size_t)(i0 + r) * DG + c * 4) * 4),
                      __builtin_amdgcn_readfirstlane(base));
        }
    };
    // logits^T of 32 states (rows) x the lane's tokens (columns): rows from the staging area
    // (row0 = the block's first row there) or, when from_lds is false, from P directly.  The
    // source is a compile-time argument: with both in one loop the compiler would wait for every
    // load in flight before each MFMA.
    auto logits = [&](int i0, int row0, auto from_lds_c, rf32x16_t (&lg)[TB]) {
        constexpr bool from_lds = decltype(from_lds_c)::value;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int r = 0; r < 16; ++r) lg[tb][r] = 0.f;
        const int prow = min(i0 + l32, max(s_hi - 1, 0));
        const int sw = l32 & (G - 1);
#pragma unroll
        for (int kc = 0; kc < DG_MAX / 16; ++kc) {
            if (kc >= DG / 16) break;
            float pv[8];
            const int c0 = kc * 4 + hi32 * 2;
            if constexpr (from_lds) {
                const float* pr = &sm.a.pm[(row0 + l32) * DG];
                const float4 a0 = *reinterpret_cast<const float4*>(pr + ((c0 ^ sw) * 4));
                const float4 a1 = *reinterpret_cast<const float4*>(pr + (((c0 + 1) ^ sw) * 4));
                pv[0] = a0.x; pv[1] = a0.y; pv[2] = a0.z; pv[3] = a0.w;
                pv[4] = a1.x; pv[5] = a1.y; pv[6] = a1.z; pv[7] = a1.w;
            } else {
                const float* pr = Pbx + (size_t)prow * DG + c0 * 4;
                const float4 a0 = *reinterpret_cast<const float4*>(pr);
                const float4 a1 = *reinterpret_cast<const float4*>(pr + 4);
                pv[0] = a0.x; pv[1] = a0.y; pv[2] = a0.z; pv[3] = a0.w;
                pv[4] = a1.x; pv[5] = a1.y; pv[6] = a1.z; pv[7] = a1.w;
            }
            ru32x4_t ah, al;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t hh = pack_bf16x2(pv[2 * q], pv[2 * q + 1]);
                ah[q] = hh;
                al[q] = pack_bf16x2(pv[2 * q] - __uint_as_float(hh << 16),
                                    pv[2 * q + 1] - __uint_as_float(hh & 0xffff0000u));
            }
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                lg[tb] = mfma_bf16(ah, ub[tb][kc], lg[tb]);
                lg[tb] = mfma_bf16(al, ub[tb][kc], lg[tb]);
            }
        }
        // accumulator row 8*(r/4) + 4*hi32 + r%4 is state i0 + that row; a state counts for
        // token t when it is a completed segment before t's (and, for SSC, selected for t)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            uint32_t bits = 0xffffffffu;
            if (SSC) {
                bits = 0u;
                const int32_t* sel = idx + ((size_t)bh * L + tok[tb]) * top_k;
                for (int c = 0; c < top_k; ++c) {
                    const int d = sel[c] - i0;
                    if (sel[c] >= 0 && d >= 0 && d < 32) bits |= 1u << d;
                }
            }
            const int lim = val[tb] ? seg[tb] - i0 - 4 * hi32 : 0;
            const uint32_t bsh = bits >> (4 * hi32);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = 8 * (r / 4) + (r % 4);
                if (!(rr < lim && ((bsh >> rr) & 1u))) lg[tb][r] = -INFINITY;
            }
        }
    };
    // Numerators of a super-block -> sm.w (bf16), sums into l, SSC selection bits.  With
    // `running` the max is taken on the way (one logits pass): block bi's numerators are
    // exp(a - mb[bi]) with mb[bi] the max over the online logit and blocks 0..bi, and l is
    // rescaled whenever the max grows; the state loop multiplies block bi's weights by
    // exp(mb[bi] - m) once m is final.  Without it m is already final (mb[bi] = m).
    constexpr int NBLK = WMAX / 32;
    float mb[NBLK][TB];
#pragma unroll
    for (int b = 0; b < NBLK; ++b)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) mb[b][tb] = 0.f;
    auto weights = [&](int sb0, auto from_lds, bool running) {
        const int n = min(SBS, s_hi - sb0);
#pragma unroll
        for (int bi = 0; bi < NBLK; ++bi) {
            const int b0 = bi * 32;
            if (b0 >= n) break;
            rf32x16_t lg[TB];
            logits(sb0 + b0, b0, from_lds, lg);
            if (running) {
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    float bm = -INFINITY;
#pragma unroll
                    for (int r = 0; r < 16; ++r) bm = fmaxf(bm, lg[tb][r]);
                    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
                    const float mn = fmaxf(m[tb], bm);
                    l[tb] *= __expf(m[tb] - mn);
                    m[tb] = mn;
                }
            }
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) mb[bi][tb] = m[tb];
            uint32_t any = 0u;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                float ps = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 8 * (r / 4) + 4 * hi32 + (r % 4);
                    const float wv = __expf(lg[tb][r] - m[tb]);  // 0 for masked states
                    ps += wv;
                    if (b0 + row < WMAX) sm.w[b0 + row][tl[tb]] = f32_to_bf16(wv);
                    if (SSC && wv > 0.f) any |= 1u << row;
                }
                l[tb] += ps + __shfl_xor(ps, 32, 64);  // the other lane half holds the other rows
            }
            if constexpr (SSC) {
                for (int o = 1; o < 64; o <<= 1) any |= __shfl_xor(any, o, 64);
                if (lane == 0 && any) atomicOr(&sm.any_sel[b0 / 32], any);
            }
        }
    };

    // PRE: the numerators of a super-block of rows, written by the gate pass, -> sm.w by direct
    // loads (row i of the tile: RT bf16, token order)
    const bf16_t* Wt = Wg + ((size_t)bh * T + tile) * NS * RT;
    auto stage_w = [&](int i0, int n) {
        const int total = n * (RT / 8);
        for (int p0 = wave * 64; p0 < total; p0 += RTHREADS) {
            const uint32_t base = (uint32_t)(uintptr_t)&sm.w[0][p0 * 8];
            if (p0 + lane < total)
                dma16(Wt, (uint32_t)(((size_t)i0 * RT + (p0 + lane) * 8) * 2),
                      __builtin_amdgcn_readfirstlane(base));
        }
    };

    if constexpr (SSC) {
        if (tid < WMAX / 32) sm.any_sel[tid] = 0u;
    }
    if constexpr (PRE) {
        // the gate ran as its own pass: its numerators land in sm.w while the online term
        // runs; per token the online weight and 1/l (kept in l)
        if (s_hi > 0) stage_w(0, min(s_hi, SBS));
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            won[tb] = won_g[(size_t)bh * L + tok[tb]];
            l[tb] = inv_l_g[(size_t)bh * L + tok[tb]];
        }
    } else {
    if (s_hi > SBS) {
        // more states than one super-block: pass 1 takes m_t over every logit first, so the
        // numerators of every super-block are final when written
        for (int sb0 = 0; sb0 < s_hi; sb0 += SBS) {
            const int n = min(SBS, s_hi - sb0);
            if (sb0 > 0) __syncthreads();  // the previous super-block's means are consumed
            stage_means(sb0, n);
            wait_all_and_barrier();
            for (int b0 = 0; b0 < n; b0 += 32) {
                rf32x16_t lg[TB];
                logits(sb0 + b0, b0, std::true_type{}, lg);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    float bm = -INFINITY;
#pragma unroll
                    for (int r = 0; r < 16; ++r) bm = fmaxf(bm, lg[tb][r]);
                    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
                    m[tb] = fmaxf(m[tb], bm);
                }
            }
        }
        __syncthreads();
        stage_means(0, SBS);
        wait_all_and_barrier();
        weights(0, std::true_type{}, false);
    } else if (s_hi > 0) {
        stage_means(0, s_hi);
        wait_all_and_barrier();
        weights(0, std::true_type{}, true);
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) won[tb] = __expf(a_on[tb] - m[tb]);
    }

    __syncthreads();  // the staged means are consumed (region A is free)

    // =============================== 2. online term ==========================================
    rf32x16_t acc[CB][TB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[cb][tb][r] = 0.f;
    uint32_t swz = (uint32_t)(l32 % CPR);  // XOR of a row's 16-byte chunks (row % CPR = l32 % CPR)
    // phi(q) of the lane's tokens in fp32 (scaled by each state's weight in the state loop):
    // k = 16 ks + 8 hi32 + e, the B operand's k order
    float qf[TB][KS][8];
    if (FON) {
        // phi(q) of the lane's tokens as bf16 B fragments: k = 16 ks + 8 hi32 + e
        ru32x4_t qb[TB][KS];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const bf16_t* qr = Q + ((size_t)bh * L + tok[tb]) * DK + hi32 * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                ru32x4_t v = *reinterpret_cast<const ru32x4_t*>(qr + ks * 16);
                if (PHI) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = pack_bf16x2(feature(__uint_as_float(v[e] << 16), 1),
                                           feature(__uint_as_float(v[e] & 0xffff0000u), 1));
                }
                qb[tb][ks] = v;
            }
        }
        // the first key of token t's online walk: its segment's start, or with pieces the start
        // of its piece (the memory of the segment's earlier pieces is added below from M0)
        auto base_of = [&](int t) {
            if constexpr (PCS) {
                const int f = sg.off[seg_of(sg, t, C)];
                return f + (t - f) / pon.PL * pon.PL;
            } else {
                return (t / C) * C;
            }
        };
        const int k_lo = base_of(tile0);
        const int nkc = (last - k_lo) / 64 + 1;
        const bf16_t* Kbh = K + (size_t)bh * L * DK;
        const bf16_t* Vbh = V + (size_t)bh * L * DV;
        int tfirst[TB], tlast[TB], tseg0[TB], tsegl[TB], tbase[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            tfirst[tb] = tile0 + (tl[tb] - l32);          // the 32-token block's first token
            tlast[tb] = min(tfirst[tb] + 31, L - 1);
            tseg0[tb] = base_of(min(tfirst[tb], L - 1));  // walk start of its first token
            tsegl[tb] = base_of(tlast[tb]);               // and of its last
            tbase[tb] = base_of(tok[tb]);                 // and of the lane's token
        }
        // keys of chunk kc -> k[kc & 1]: whole rows per load instruction, chunks XOR-swizzled by
        // row; keys past the last token read token `last` (their scores are masked)
        constexpr int KLD = 64 * DK / 8 / RTHREADS;
        auto stage_k = [&](int kc) {
            const int k0 = k_lo + kc * 64;
#pragma unroll
            for (int mm = 0; mm < KLD; ++mm) {
                const int p0 = (mm * 4 + wave) * 64;
                const int p = p0 + lane;
                const int r = p / CPR, c8 = (p % CPR) ^ (r % CPR);
                const int key = min(k0 + r, last);
                const uint32_t base = (uint32_t)(uintptr_t)&sm.a.kv.k[kc & 1][p0 * 8];
                dma16(Kbh, (uint32_t)(((size_t)key * DK + c8 * 8) * 2),
                      __builtin_amdgcn_readfirstlane(base));
            }
        };
        // values of chunk kc, transposed into vt[kc & 1] = v^T [DV][64 keys]: lane holds keys
        // 2 vp, 2 vp + 1 and DV/8 value columns from vdc.  A row's keys are stored in the MFMA's
        // k order, so that an A fragment is one 16-byte read: 16-byte chunk 2 kk + h of a row
        // holds keys 16 kk + 4 h + (0..3) and 16 kk + 8 + 4 h + (0..3).  A row is 128 bytes
        // (half the banks), so chunks are XOR-swizzled by (row / 2) % 8: the reads of 16
        // consecutive rows then cover every bank once
        constexpr int VCOLS = DV / 8;
        const int vp = tid % 32, vdc = (tid / 32) * VCOLS;
        ru32x4_t va[2][VCOLS / 8];
        auto load_v = [&](int kc) {
            const int k0 = k_lo + kc * 64;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int key = k0 + 2 * vp + e;
#pragma unroll
                for (int g = 0; g < VCOLS / 8; ++g)
                    va[e][g] = key <= last ? *reinterpret_cast<const ru32x4_t*>(
                                                 Vbh + (size_t)key * DV + vdc + g * 8)
                                           : ru32x4_t{0u, 0u, 0u, 0u};
            }
        };
        auto store_v = [&](int kc) {
            bf16_t* vt = sm.a.kv.vt[kc & 1];
#pragma unroll
            for (int g = 0; g < VCOLS / 8; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c0 = vdc + g * 8 + 2 * e;  // value columns c0, c0 + 1 (c0 even)
                    // keys 2 vp, 2 vp + 1: group vp / 8, chunk half h, position in the chunk
                    const int r = vp % 8, h = (r >> 1) & 1, pos = 2 * (r & 1) + 4 * (r >> 2);
                    const int pc = (((vp / 8) * 2 + h) ^ ((c0 >> 1) & 7)) * 8 + pos;
                    *reinterpret_cast<uint32_t*>(&vt[c0 * 64 + pc]) =
                        (va[0][g][e] & 0xffffu) | (va[1][g][e] << 16);
                    *reinterpret_cast<uint32_t*>(&vt[(c0 + 1) * 64 + pc]) =
                        (va[0][g][e] >> 16) | (va[1][g][e] & 0xffff0000u);
                }
        };
        stage_k(0);
        load_v(0);
        store_v(0);
        for (int kc = 0; kc < nkc; ++kc) {
            const int k0 = k_lo + kc * 64;
            asm volatile("" : "+v"(swz));
            wait_all_and_barrier();
            if (kc + 1 < nkc) {
                stage_k(kc + 1);
                load_v(kc + 1);
            }
            if constexpr (PHI != 0) {
                // phi(k) in place over the chunk's key tile, once per element (the fragments
                // are read once per token block); the barrier waits on LDS only, so the next
                // chunk's loads stay in flight
                bf16_t* kw = sm.a.kv.k[kc & 1];
#pragma unroll
                for (int mm = 0; mm < 64 * DK / 8 / RTHREADS; ++mm) {
                    ru32x4_t* pk = reinterpret_cast<ru32x4_t*>(kw + (mm * RTHREADS + tid) * 8);
                    ru32x4_t v = *pk;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = pack_bf16x2(feature(__uint_as_float(v[e] << 16), 1),
                                           feature(__uint_as_float(v[e] & 0xffff0000u), 1));
                    *pk = v;
                }
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            }
            const bf16_t* kt = sm.a.kv.k[kc & 1];
            const bf16_t* vt = sm.a.kv.vt[kc & 1];
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                // keys all after the block's tokens, or all before its earliest segment start
                if (k0 > tlast[tb] || k0 + 63 < tseg0[tb]) continue;
                const bool full = (k0 + 63 <= tfirst[tb]) && (k0 >= tsegl[tb]);
                // scores S^T = phi(K) phi(Q)^T; K fragments read two k-steps ahead
                auto kfrag = [&](int ks, int rb) {  // (the key tile holds phi(k))
                    return *reinterpret_cast<const ru32x4_t*>(
                        &kt[(rb * 32 + l32) * DK + (((2 * ks + hi32) ^ swz) * 8)]);
                };
                rf32x16_t sc[2];
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sc[rb][r] = 0.f;
                ru32x4_t kf[3][2];
                kf[0][0] = kfrag(0, 0);
                kf[0][1] = kfrag(0, 1);
                kf[1][0] = kfrag(1, 0);
                kf[1][1] = kfrag(1, 1);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (ks + 2 < KS) {
                        kf[(ks + 2) % 3][0] = kfrag(ks + 2, 0);
                        kf[(ks + 2) % 3][1] = kfrag(ks + 2, 1);
                    }
                    sc[0] = mfma_bf16(kf[ks % 3][0], qb[tb][ks], sc[0]);
                    sc[1] = mfma_bf16(kf[ks % 3][1], qb[tb][ks], sc[1]);
                }
                // mask to segment(t) start <= key <= t; key = k0 + 4*hi32 + (an immediate)
                const int t = tok[tb];
                if (!full) {
                    const int hi_lim = t - k0 - 4 * hi32, lo_lim = tbase[tb] - k0 - 4 * hi32;
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int rr = rb * 32 + 8 * (i / 4) + (i % 4);
                            if (rr > hi_lim || rr < lo_lim) sc[rb][i] = 0.f;
                        }
                }
                // scores x the online weight, in bf16: the accumulator's row order is the k
                // order the v^T reads below use, so no reshuffle is needed
                ru32x4_t sb[4];
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const float wo = won[tb];
                        sb[2 * rb + q] = ru32x4_t{
                            pack_bf16x2(sc[rb][8 * q + 0] * wo, sc[rb][8 * q + 1] * wo),
                            pack_bf16x2(sc[rb][8 * q + 2] * wo, sc[rb][8 * q + 3] * wo),
                            pack_bf16x2(sc[rb][8 * q + 4] * wo, sc[rb][8 * q + 5] * wo),
                            pack_bf16x2(sc[rb][8 * q + 6] * wo, sc[rb][8 * q + 7] * wo)};
                    }
                // acc += v^T S^T: consecutive MFMAs go to different value blocks (independent
                // accumulators), v^T fragments read three MFMAs ahead.  Fragment n = (k-step kk,
                // value block cb) is chunk 2 kk + hi32 of its row
                constexpr int NV = CB * 4;
                auto vfrag = [&](int n) {
                    const int c = (n % CB) * 32 + l32, kk = n / CB;
                    return *reinterpret_cast<const ru32x4_t*>(
                        &vt[c * 64 + (((2 * kk + hi32) ^ ((c >> 1) & 7)) * 8)]);
                };
                ru32x4_t vf[4];
                vf[0] = vfrag(0);
                vf[1] = vfrag(1);
                vf[2] = vfrag(2);
#pragma unroll
                for (int n = 0; n < NV; ++n) {
                    if (n + 3 < NV) vf[(n + 3) % 4] = vfrag(n + 3);
                    acc[n % CB][tb] = mfma_bf16(vf[n % 4], sb[n / CB], acc[n % CB][tb]);
                }
            }
            if (kc + 1 < nkc) store_v(kc + 1);  // its buffer was last read in chunk kc - 1
        }
        if constexpr (PCS) {
            // the memory of the earlier pieces of the token's segment, M0 of its piece (bf16
            // [d_v][d_k], none for a segment's first piece), with the online weight:
            // acc += M0 bf16(won phi(q)).  The wave takes the distinct pieces of its tokens in
            // ascending order, a token's weight zero outside its own piece.
            int pc[TB];
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const int f = sg.off[seg[tb]];
                const int j = (tok[tb] - f) / pon.PL;
                pc[tb] = (val[tb] && j > 0) ? pon.pfirst[seg[tb]] + j : INT_MAX;
            }
            int cur = -1;
            for (;;) {
                int nx = INT_MAX;
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
                    if (pc[tb] > cur) nx = min(nx, pc[tb]);
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) nx = min(nx, __shfl_xor(nx, o, 64));
                if (nx == INT_MAX) break;
                cur = nx;
                ru32x4_t qw[TB][KS];
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const float w = pc[tb] == cur ? won[tb] : 0.f;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            qw[tb][ks][e] =
                                pack_bf16x2(__uint_as_float(qb[tb][ks][e] << 16) * w,
                                            __uint_as_float(qb[tb][ks][e] & 0xffff0000u) * w);
                }
                const bf16_t* m0 = reinterpret_cast<const bf16_t*>(pon.M0) +
                                   ((size_t)bh * pon.NP + cur) * (size_t)(DV * DK) + l32 * DK +
                                   hi32 * 8;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const ru32x4_t a =
                            *reinterpret_cast<const ru32x4_t*>(m0 + cb * 32 * DK + ks * 16);
#pragma unroll
                        for (int tb = 0; tb < TB; ++tb)
                            acc[cb][tb] = mfma_bf16(a, qw[tb][ks], acc[cb][tb]);
                    }
            }
        }
        if (PHI == 0) {  // the raw q fragments are phi(q): widen them instead of reloading q
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        qf[tb][ks][2 * e] = __uint_as_float(qb[tb][ks][e] << 16);
                        qf[tb][ks][2 * e + 1] = __uint_as_float(qb[tb][ks][e] & 0xffff0000u);
                    }
        }
    } else if constexpr (PRE) {
        // (the kernels that form the gate themselves add the online term in the epilogue:
        // seeding the accumulators here would take them out of the accumulation registers)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const float* orow = O_on + ((size_t)bh * L + tok[tb]) * DV + cb * 32 + hi32 * 4;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 v = *reinterpret_cast<const float4*>(orow + g * 8);
                    acc[cb][tb][4 * g + 0] = v.x * won[tb];
                    acc[cb][tb][4 * g + 1] = v.y * won[tb];
                    acc[cb][tb][4 * g + 2] = v.z * won[tb];
                    acc[cb][tb][4 * g + 3] = v.w * won[tb];
                }
            }
    }
    if (!(FON && PHI == 0)) {  // else widened from the online term's fragments
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const bf16_t* qr = Q + ((size_t)bh * L + tok[tb]) * DK + hi32 * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                float v[8];
                ld8<bf16_t>(qr, ks * 16, v);
#pragma unroll
                for (int e = 0; e < 8; ++e) qf[tb][ks][e] = PHI ? feature(v[e], 1) : v[e];
            }
        }
    }
    wait_all_and_barrier();  // region A is free for the states

    // =============================== 3. cached states ========================================
    // state i -> state[buf]: load m of wave w fills chunks [(m*4 + w)*64, +64) -- whole rows, so
    // each load instruction reads contiguous memory; chunk (c, kc) sits at kc ^ (c % CPR)
    const bf16_t* Sbh = S + (size_t)bh * NS * DV * DK;
    uint32_t soff[STAGE];
#pragma unroll
    for (int mm = 0; mm < STAGE; ++mm) {
        const int p = (mm * 4 + wave) * 64 + lane;
        const int c = p / CPR, kc = (p % CPR) ^ (c % CPR);
        soff[mm] = (uint32_t)((c * DK + kc * 8) * 2);
    }
    auto stage = [&](int i, int buf) {
        const bf16_t* src = Sbh + (size_t)i * DV * DK;
#pragma unroll
        for (int mm = 0; mm < STAGE; ++mm) {
            const int p0 = (mm * 4 + wave) * 64;
            const uint32_t base = (uint32_t)(uintptr_t)&sm.a.state[buf][p0 * 8];
            dma16(src, soff[mm], __builtin_amdgcn_readfirstlane(base));
        }
    };
    if (s_hi > 0) stage(0, 0);
    if (s_hi > 1) stage(1, 1);
    float cf[TB];  // exp(mb[block] - m) of the block being read
    for (int i = 0, buf = 0; i < s_hi; ++i, buf = (buf == NBUF - 1 ? 0 : buf + 1)) {
        const int il = i % SBS;
        asm volatile("" : "+v"(swz));
        // state i has landed for this lane (the loads of state i+1, issued later, may still be
        // in flight); after the barrier for every lane, and every wave is done with state i-1
        if (i + 1 < s_hi)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(STAGE) : "memory");
        else
            wait_all_and_barrier();
        if (i + 2 < s_hi) stage(i + 2, buf == 0 ? NBUF - 1 : buf - 1);
        if (il == 0 && i > 0) {  // next super-block of weights (means read from P directly)
            if constexpr (PRE) {
                __syncthreads();
                stage_w(i, min(SBS, s_hi - i));
                wait_all_and_barrier();
            } else {
                if constexpr (SSC) {
                    if (tid < WMAX / 32) sm.any_sel[tid] = 0u;
                }
                load_u();
                __syncthreads();
                weights(i, std::false_type{}, false);
                __syncthreads();
            }
        }
        if (!PRE && (il & 31) == 0) {  // entering block il / 32 of the super-block: its correction
            const int bi = il >> 5;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                float mbi = mb[0][tb];
#pragma unroll
                for (int b = 1; b < NBLK; ++b) mbi = bi == b ? mb[b][tb] : mbi;
                cf[tb] = __expf(mbi - m[tb]);
            }
        }
        if constexpr (SSC) {
            if (!((sm.any_sel[il / 32] >> (il % 32)) & 1u)) continue;
        }
        float w[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
            w[tb] = PRE ? bf16_to_f32(sm.w[il][tl[tb]]) : bf16_to_f32(sm.w[il][tl[tb]]) * cf[tb];
        const bf16_t* st = sm.a.state[buf];
        // software pipeline in issue order: A fragments two k-steps ahead (three register
        // sets); each MFMA of k-step ks is followed by the three VALU ops that build a quarter
        // of one B fragment of k-step ks + 1 (two products and their bf16 pack)
        ru32x4_t af[3][CB], bq[2][TB];
        auto load_a = [&](int ks) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
                af[ks % 3][cb] = *reinterpret_cast<const ru32x4_t*>(
                    &st[(cb * 32 + l32) * DK + (((2 * ks + hi32) ^ swz) * 8)]);
        };
        auto b_piece = [&](int ks, int tb, int e) {
            bq[ks & 1][tb][e] = pack_bf16x2(qf[tb][ks][2 * e] * w[tb], qf[tb][ks][2 * e + 1] * w[tb]);
        };
        load_a(0);
        if (KS > 1) load_a(1);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int e = 0; e < 4; ++e) b_piece(0, tb, e);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            // the next k-step's B operand is TB * 4 pieces, spread evenly over the MFMAs
            constexpr int NM = CB * TB, PPM = (TB * 4) / NM;
            static_assert(PPM >= 1 && PPM * NM == TB * 4, "B pieces per MFMA");
#pragma unroll
            for (int n = 0; n < NM; ++n) {
                const int cb = n / TB, tb = n % TB;
                acc[cb][tb] = mfma_bf16(af[ks % 3][cb], bq[ks & 1][tb], acc[cb][tb]);
                if (ks + 1 < KS) {
#pragma unroll
                    for (int pc = n * PPM; pc < (n + 1) * PPM; ++pc) b_piece(ks + 1, pc / 4, pc % 4);
                }
                if (n == 1 && ks + 2 < KS) load_a(ks + 2);
            }
        }
    }

    // =============================== 4. y = acc / l =========================================
    if constexpr (PRE) {
        // staged through region A (free once every wave is past its last state) so that the
        // stores write whole rows: token row r of the tile at r * DV, its 16-byte chunk c at
        // c ^ (r % NCH), which keeps the lanes' writes (32 rows, one chunk) on distinct banks.
        // (The kernels that form the gate themselves hold more registers here and store
        // directly.)
        constexpr int NCH = DV / 8;  // 16-byte chunks per row of y
        static_assert(RT * DV * sizeof(bf16_t) <= sizeof(sm.a), "y tile fits region A");
        bf16_t* ys = reinterpret_cast<bf16_t*>(&sm.a);
        __syncthreads();
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int r = tl[tb];
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint2 v;
                    v.x = pack_bf16x2(acc[cb][tb][4 * g + 0] * l[tb], acc[cb][tb][4 * g + 1] * l[tb]);
                    v.y = pack_bf16x2(acc[cb][tb][4 * g + 2] * l[tb], acc[cb][tb][4 * g + 3] * l[tb]);
                    const int c = (cb * 4 + g) ^ (r % NCH);
                    *reinterpret_cast<uint2*>(&ys[r * DV + c * 8 + hi32 * 4]) = v;
                }
        }
        __syncthreads();
        const int nrow = last - tile0 + 1;  // rows of the tile inside the sequence
#pragma unroll
        for (int it = 0; it < RT * NCH / RTHREADS; ++it) {
            const int idx = it * RTHREADS + tid, r = idx / NCH, c = idx % NCH;
            if (r < nrow)
                *reinterpret_cast<uint4*>(Y + ((size_t)bh * L + tile0 + r) * DV + c * 8) =
                    *reinterpret_cast<const uint4*>(&ys[r * DV + ((c ^ (r % NCH)) * 8)]);
        }
    } else {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            if (!val[tb]) continue;
            const float il = 1.f / (l[tb] + won[tb]);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                bf16_t* yr = Y + ((size_t)bh * L + tok[tb]) * DV + cb * 32 + hi32 * 4;
                // the online term read from O_on (when the kernel did not form it) joins here
                float4 o[4];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    o[g] = make_float4(0.f, 0.f, 0.f, 0.f);
                    if constexpr (!FON)
                        o[g] = *reinterpret_cast<const float4*>(
                            O_on + ((size_t)bh * L + tok[tb]) * DV + cb * 32 + hi32 * 4 + g * 8);
                }
                const float wo = FON ? 0.f : won[tb];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint2 v;
                    v.x = pack_bf16x2((acc[cb][tb][4 * g + 0] + wo * o[g].x) * il,
                                      (acc[cb][tb][4 * g + 1] + wo * o[g].y) * il);
                    v.y = pack_bf16x2((acc[cb][tb][4 * g + 2] + wo * o[g].z) * il,
                                      (acc[cb][tb][4 * g + 3] + wo * o[g].w) * il);
                    *reinterpret_cast<uint2*>(yr + g * 8) = v;
                }
            }
        }
    }
}

// The kernel: one tile per workgroup, or (the precomputed-gate read, with a grid of one
// workgroup per CU) a share of the tiles per workgroup, taken in turn.  Nothing is shared
// between tiles but the LDS, which the barrier after each tile hands back.
template <int DK, int DV, bool SSC, bool FON, int PHI, bool PRE, bool PCS>
__global__ __launch_bounds__(RTHREADS, 1) void grm_read_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ U, const float* __restrict__ xps, const bf16_t* __restrict__ S,
    const float* __restrict__ P, const float* __restrict__ O_on,
    const int32_t* __restrict__ idx, const bf16_t* __restrict__ Wg,
    const float* __restrict__ won_g, const float* __restrict__ inv_l_g, int top_k, int BH,
    int H, int L, int C, int NS, int DG, int xh, bf16_t* __restrict__ Y, const SegArg sg,
    const PieceOnline pon) {
    __shared__ __attribute__((aligned(16))) char smem_raw[sizeof(ReadSmem<DK, DV, SSC>)];
    if constexpr (PRE) {
        const int nblk = BH * ((L + RT - 1) / RT);
        // block indices dealt in stripes of the grid, every other stripe in reverse, so that
        // each workgroup gets an even share of the heavy (early) and light (late) tiles; with
        // a grid of whole XCD rounds a workgroup's tiles are all of its own XCD
        const int G = gridDim.x, g = blockIdx.x;
        const int R = G % 8 == 0 ? 8 : 1, W = G / R, x = g % R, w = g / R;
        for (int k = 0;; ++k) {
            const int bid = (k * W + ((k & 1) ? W - 1 - w : w)) * R + x;
            if (bid >= nblk) break;
            grm_read_tile<DK, DV, SSC, FON, PHI, PRE, PCS>(Q, K, V, U, xps, S, P, O_on, idx, Wg,
                                                           won_g, inv_l_g, top_k, BH, H, L, C,
                                                           NS, DG, xh, Y, sg, pon, smem_raw, bid);
            __syncthreads();
        }
    } else {
        grm_read_tile<DK, DV, SSC, FON, PHI, PRE, PCS>(Q, K, V, U, xps, S, P, O_on, idx, Wg,
                                                       won_g, inv_l_g, top_k, BH, H, L, C, NS,
                                                       DG, xh, Y, sg, pon, smem_raw, blockIdx.x);
    }
}

// Compute units of the current device (0 when the query fails), looked up once per device.
int cu_count() {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cached[kMaxDev];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

template <int DK, int DV, bool SSC, bool FON, int PHI, bool PRE, bool PCS>
void launch_k(const mc_dims& d, int top_k, const void* Q, const void* K, const void* V,
              const void* U, const float* xps, const uint16_t* M_lo, const float* P,
              const float* O_on, const int32_t* idx, const GateWeights& gw, void* Y,
              hipStream_t st, const SegArg& sg, const PieceOnline& pon) {
    const int NS = sg.n ? sg.n : (d.L + d.seg_len - 1) / d.seg_len;
    const int T = (d.L + RT - 1) / RT;
    const int BH = d.B * d.H;
    // the precomputed-gate read runs one workgroup per CU (a workgroup fills a CU's LDS), each
    // walking its share of the tiles: no dispatch between tiles, and a CU's tiles stay in order
    int grid = BH * T;
    if constexpr (PRE) {
        const int ncu = cu_count();
        if (ncu > 0 && grid > ncu) grid = ncu;
    }
    hipLaunchKernelGGL((grm_read_kernel<DK, DV, SSC, FON, PHI, PRE, PCS>), dim3(grid),
                       dim3(RTHREADS), 0, st, (const bf16_t*)Q, (const bf16_t*)K,
                       (const bf16_t*)V, (const bf16_t*)U, xps, (const bf16_t*)M_lo, P, O_on,
                       idx, (const bf16_t*)gw.W, gw.won, gw.inv_l, top_k, BH, d.H, d.L,
                       d.seg_len, NS, d.d_g, d.x_heads, (bf16_t*)Y, sg, pon);
}

template <int DK, int DV, bool SSC, bool PRE>
int launch_t(const mc_dims& d, int top_k, const void* Q, const void* K, const void* V,
             const void* U, const float* xps, const uint16_t* M_lo, const float* P,
             const float* O_on, const int32_t* idx, const GateWeights& gw, void* Y,
             hipStream_t st, const SegArg& sg, const PieceOnline* pon = nullptr) {
    // the online term is formed in the kernel (from K and V) when the scan did not write it;
    // the feature map is a template argument so the key fragments' loop has no branches
#define MC_K(FON, PHI)                                                                         \
    launch_k<DK, DV, SSC, FON, PHI, PRE, false>(d, top_k, Q, K, V, U, xps, M_lo, P, O_on, idx, \
                                                gw, Y, st, sg, PieceOnline{})
    if (pon) {  // segment offsets, the online term formed here over pieces
        if constexpr (PRE && !SSC) {
            if (d.phi)
                launch_k<DK, DV, false, true, 1, true, true>(d, 0, Q, K, V, U, xps, M_lo, P,
                                                             nullptr, idx, gw, Y, st, sg, *pon);
            else
                launch_k<DK, DV, false, true, 0, true, true>(d, 0, Q, K, V, U, xps, M_lo, P,
                                                             nullptr, idx, gw, Y, st, sg, *pon);
            return (int)hipGetLastError();
        } else {
            return -1;
        }
    }
    if (O_on) {
        // the SSC kernels that form the gate themselves and take the online term given run out
        // of registers at d_v = 128 (they would spill); their callers take another read
        if constexpr (SSC && DV == 128)
            return -1;
        else
            d.phi ? MC_K(false, 1) : MC_K(false, 0);
    } else {
        d.phi ? MC_K(true, 1) : MC_K(true, 0);
    }
#undef MC_K
    return (int)hipGetLastError();
}

}  // namespace

// bf16 inputs with d_k, d_v in {64, 128} and a gate of at most DG_MAX (a multiple of 16)
bool read_mfma_covers(const mc_dims& d) {
    return d.dtype == MC_BF16 && d.d_g % 16 == 0 && d.d_g <= DG_MAX &&
           (d.d_k == 64 || d.d_k == 128) && (d.d_v == 64 || d.d_v == 128);
}

// the SSC read with the gate formed in the kernel: not for d_v = 128 with the online term
// given (see launch_t)
bool read_mfma_ssc_covers(const mc_dims& d, bool online_given) {
    return read_mfma_covers(d) && !(online_given && d.d_v == 128);
}

static const SegArg kConstSegRd{};  // constant segment length

int launch_read_mfma(const mc_dims& d, bool ssc, int top_k, const void* Q, const void* K,
                     const void* V, const void* U, const float* xps, const uint16_t* M_lo,
                     const float* P, const float* O_on, const int32_t* idx,
                     const GateWeights& gw, void* Y, void* stream, const SegArg* sgp,
                     const PieceOnline* pon) {
    if (!read_mfma_covers(d)) return -1;
    // segment offsets: GRM with the online read given, or formed here over pieces after the
    // gate pass (the gate pass takes the offsets too)
    if (sgp && sgp->n && (ssc || (!O_on && !(pon && gw.W)))) return -1;
    if (pon && !(sgp && sgp->n)) return -1;
    const SegArg& sg = sgp ? *sgp : kConstSegRd;
    hipStream_t st = (hipStream_t)stream;
    if (gw.W) {  // the gate ran as its own pass (d_k = d_v = 128 GRM)
        if (ssc || d.d_k != 128 || d.d_v != 128) return -1;
        return launch_t<128, 128, false, true>(d, 0, Q, K, V, U, xps, M_lo, P, O_on, idx, gw, Y,
                                               st, sg, O_on ? nullptr : pon);
    }
#define MC_RD(DK, DV)                                                                          \
    if (d.d_k == DK && d.d_v == DV)                                                            \
        return ssc ? launch_t<DK, DV, true, false>(d, top_k, Q, K, V, U, xps, M_lo, P, O_on,    \
                                                   idx, gw, Y, st, sg)                         \
                   : launch_t<DK, DV, false, false>(d, top_k, Q, K, V, U, xps, M_lo, P, O_on,  \
                                                    idx, gw, Y, st, sg);
    MC_RD(128, 128)
    MC_RD(128, 64)
    MC_RD(64, 128)
    MC_RD(64, 64)
#undef MC_RD
    return -1;
}

}  // namespace mc
