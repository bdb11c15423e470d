// dgamma_mfma.hip -- dgamma of the GRM prefill's backward on bf16 MFMA (gfx950), d_k = d_v = 128.
//
// Memory Caching paper, Eq. (9)-(10) differentiated: for token t of segment s and a cached
// segment i < s, dL/dgamma_t^(i) = <dy_t, M^(i) phi(q_t)>.  One workgroup = 256 consecutive
// tokens of one (b, h), 4 waves, one wave per SIMD; wave w owns tokens 64 w .. + 63 as two
// blocks of 32.  Per state i, O^(i)[c][t] = sum_r M^(i)[c][r] phi(q_t)[r] runs on 32x32x16
// MFMAs (A: the state's rows from LDS, B: phi(q) in registers), and dgamma_t^(i) =
// sum_c dy_t[c] O^(i)[c][t] is reduced in registers (the lane of token t holds 16 of its
// rows per 32-row block; the two half-waves are added).  The states are streamed into LDS
// by direct global->LDS loads two states ahead (three buffers, rows XOR-swizzled in 16-byte
// chunks so the fragment reads fall on distinct banks).  A state's product runs as two
// halves of 64 rows with their own accumulator sets: the reduction of one half is
// interleaved with the MFMAs of the next (two products per MFMA), so the matrix unit hides
// it.  This file is compiled
// without the machine schedulers, so the issue order is the one written here.  The result
// is written segment-major, dGT[i][t].
#include <type_traits>

#include "common.cuh"
#include "mc_internal.h"

namespace mc {
namespace {

typedef __bf16 gbf16x8_t __attribute__((ext_vector_type(8)));
typedef float gf32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t gu32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t gu32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ gf32x16_t gmfma(const gu32x4_t& a, const gu32x4_t& b, const gf32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(gbf16x8_t, a),
                                                   __builtin_bit_cast(gbf16x8_t, b), c, 0, 0, 0);
}

// One 16-byte direct global->LDS load per lane: the 16 bytes at base + voff land at LDS
// address lds_base + 16 * lane (lds_base wave-uniform).  The kernel waits for these loads
// itself (s_waitcnt vmcnt) before the barrier that publishes a buffer.
__device__ __forceinline__ void gdma16(const void* base, uint32_t voff, uint32_t lds_base) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_base), "v"(voff), "s"(base)
                 : "memory", "m0");
#pragma clang diagnostic pop
}

constexpr int GT = 256;         // tokens per workgroup
constexpr int GD = 128;         // d_k = d_v
constexpr int SB = GD * GD;     // bf16 per state
constexpr int NBUF = 3;         // state buffers: the load of state i + 2 overlaps the read of i
constexpr int CPR = GD / 8;     // 16-byte chunks per state row
constexpr int STAGE = SB / 8 / 256;  // direct loads per lane per state
constexpr int KS = GD / 16;     // k steps of a state product

__global__ __launch_bounds__(256, 1) void bwd_dgamma_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ dY, const bf16_t* __restrict__ M_lo,
    int L, int C, int NS, int phi, float* __restrict__ dGT) {
    __shared__ __attribute__((aligned(16))) bf16_t ms[NBUF][SB];
    const int ntile = gridDim.x;
    const int tile = ntile - 1 - blockIdx.x;  // the tiles that read the most states first
    const size_t bh = blockIdx.y;
    const int t0 = tile * GT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, half = lane >> 5;
    const int s_hi = (min(L, t0 + GT) - 1) / C;
    if (s_hi == 0) return;  // uniform: no token of the tile reads a cached state

    // B operands phi(q_t) (k = 16 ks + 8 half + 0..7) and dy_t at the rows this lane holds
    // in a product (c = 32 cb + 8 g + 4 half + 0..3, bf16 pairs), for both token blocks
    gu32x4_t qb[2][KS];
    gu32x2_t dyp[2][4][4];
    int tok[2], stok[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int t = t0 + wave * 64 + tb * 32 + l32;
        const bool ok = t < L;
        tok[tb] = t;
        stok[tb] = ok ? t / C : 0;
        const size_t row = bh * L + (ok ? t : 0);
        const bf16_t* qr = Q + row * GD + half * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            gu32x4_t v = *reinterpret_cast<const gu32x4_t*>(qr + ks * 16);
            if (phi) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = pack_bf16x2(feature(__uint_as_float(v[e] << 16), 1),
                                       feature(__uint_as_float(v[e] & 0xffff0000u), 1));
            }
            qb[tb][ks] = v;
        }
        const bf16_t* dr = dY + row * GD + half * 4;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                dyp[tb][cb][g] = *reinterpret_cast<const gu32x2_t*>(dr + cb * 32 + 8 * g);
    }
    // every load above has landed before the first direct load is issued (the kernel's own
    // counts below assume only direct loads and the result stores are in flight)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // state i -> ms[buf]: direct load m of wave w fills chunks [(m * 4 + w) * 64, + 64), whole
    // rows, so each load reads contiguous memory; chunk (c, kc) sits at kc ^ (c % CPR)
    const bf16_t* Sbh = M_lo + bh * (size_t)NS * SB;
    uint32_t soff[STAGE];
#pragma unroll
    for (int mm = 0; mm < STAGE; ++mm) {
        const int p = (mm * 4 + wave) * 64 + lane;
        const int c = p / CPR, kc = (p % CPR) ^ (c % CPR);
        soff[mm] = (uint32_t)((c * GD + kc * 8) * 2);
    }
    auto stage = [&](int i, int buf) {
        const bf16_t* src = Sbh + (size_t)i * SB;
#pragma unroll
        for (int mm = 0; mm < STAGE; ++mm) {
            const uint32_t base = (uint32_t)(uintptr_t)&ms[buf][(mm * 4 + wave) * 64 * 8];
            gdma16(src, soff[mm], __builtin_amdgcn_readfirstlane(base));
        }
    };
    const int swz = l32 % CPR;
    const gf32x16_t zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                            0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // a state's product runs as two halves (rows 64 h .. + 63, blocks cb = 2 h, 2 h + 1);
    // the accumulator set of a half is its h
    gf32x16_t acc[2][2][2];  // [half][block in half][tb]
    float dg[2];             // dgamma of the state being reduced, per token block

    // the products of half H of the state in buffer buf; with RED the reduction of the other
    // half's accumulators (the previous half) interleaved, one piece per MFMA, into dg (reset
    // first with RESET)
    auto half_state = [&](auto Hc, auto REDc, auto RESETc, int buf) {
        constexpr int H = decltype(Hc)::value;
        constexpr bool RED = decltype(REDc)::value, RESET = decltype(RESETc)::value;
        const bf16_t* st = ms[buf];
        gu32x4_t af[3][2];
        auto load_a = [&](int ks) {
#pragma unroll
            for (int cl = 0; cl < 2; ++cl)
                af[ks % 3][cl] = *reinterpret_cast<const gu32x4_t*>(
                    &st[((2 * H + cl) * 32 + l32) * GD + (((2 * ks + half) ^ swz) * 8)]);
        };
        // piece q of the other half: values v, v + 1 of block (cl, tb)
        auto piece = [&](int q) {
            const int cl = q / 16, tb = (q / 8) % 2, v = (q % 8) * 2;
            const uint32_t w = dyp[tb][2 * (1 - H) + cl][v / 4][(v % 4) / 2];
            dg[tb] += __uint_as_float(w << 16) * acc[1 - H][cl][tb][v] +
                      __uint_as_float(w & 0xffff0000u) * acc[1 - H][cl][tb][v + 1];
        };
        if constexpr (RED && RESET) dg[0] = dg[1] = 0.f;
        load_a(0);
        load_a(1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const int cl = n / 2, tb = n % 2;
                acc[H][cl][tb] = gmfma(af[ks % 3][cl], qb[tb][ks], ks == 0 ? zero : acc[H][cl][tb]);
                if constexpr (RED) piece(ks * 4 + n);
                if (n == 1 && ks + 2 < KS) load_a(ks + 2);
            }
        }
    };
    // the reduction of half 1 of the last state, alone
    auto reduce_last = [&]() {
#pragma unroll
        for (int q = 0; q < 32; ++q) {
            const int cl = q / 16, tb = (q / 8) % 2, v = (q % 8) * 2;
            const uint32_t w = dyp[tb][2 + cl][v / 4][(v % 4) / 2];
            dg[tb] += __uint_as_float(w << 16) * acc[1][cl][tb][v] +
                      __uint_as_float(w & 0xffff0000u) * acc[1][cl][tb][v + 1];
        }
    };
    // state i's dgamma: both half-waves added, lanes of half 0 write
    auto finish = [&](int i) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const float v = dg[tb] + __shfl_xor(dg[tb], 32);
            if (half == 0 && tok[tb] < L && i < stok[tb]) dGT[(bh * NS + i) * (size_t)L + tok[tb]] = v;
        }
    };
    // state i has landed for this lane (the loads of state i + 1, issued later, may still be
    // in flight; so may the result stores, issued after them, which only makes the wait
    // stricter); after the barrier for every lane, and every wave is done with state i - 1
    auto publish = [&](int i) {
        if (i + 1 < s_hi)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(STAGE) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    stage(0, 0);
    if (s_hi > 1) stage(1, 1);
    publish(0);
    if (s_hi > 2) stage(2, 2);
    half_state(I0{}, std::false_type{}, std::false_type{}, 0);
    half_state(I1{}, std::true_type{}, std::true_type{}, 0);  // reduces half 0 of state 0
    for (int i = 1, buf = 1; i < s_hi; ++i, buf = buf == NBUF - 1 ? 0 : buf + 1) {
        publish(i);
        if (i + 2 < s_hi) stage(i + 2, buf == 0 ? NBUF - 1 : buf - 1);
        half_state(I0{}, std::true_type{}, std::false_type{}, buf);  // ends state i - 1
        finish(i - 1);
        half_state(I1{}, std::true_type{}, std::true_type{}, buf);   // half 0 of state i
    }
    reduce_last();
    finish(s_hi - 1);
}

}  // namespace

int launch_bwd_dgamma(const mc_dims& d, const void* Q, const void* dY, const uint16_t* M_lo,
                      float* dGT, void* stream) {
    const int NS = (d.L + d.seg_len - 1) / d.seg_len;
    hipLaunchKernelGGL(bwd_dgamma_kernel, dim3((d.L + GT - 1) / GT, d.B * d.H), dim3(256), 0,
                       (hipStream_t)stream, (const bf16_t*)Q, (const bf16_t*)dY,
                       (const bf16_t*)M_lo, d.L, d.seg_len, NS, d.phi, dGT);
    return (int)hipGetLastError();
}

}  // namespace mc
