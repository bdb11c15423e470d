// backward_mfma.hip -- the bf16, d_k = d_v = 128 backward of the GRM prefill on MFMA.
//
// The same gradients as backward.hip (Memory Caching paper, Eq. 4b / 9 / 10 differentiated
// token by token), organised around the dense contractions:
//   dphi(q_t) = sum_{i<s} gamma_i M^(i)^T dy_t + gamma_s M_t^(s)^T dy_t is the gated read of
//     Eq. 9 with the roles swapped -- queries dy, keys v, values phi(k), states M^(i)^T, the
//     same gate -- so it runs on the forward read kernel (grm_read_kernel) with transposed
//     bf16 states (transpose_states_kernel) and the forward gate pass's softmax numerators.
//   dgamma_t^(i) = <dy_t, M^(i) phi(q_t)>: launch_bwd_dgamma (dgamma_mfma.hip), per 256-token
//     tile, streams the states through LDS and contracts each with the tile's phi(q) on MFMA,
//     then reduces the products against dy in registers.
//   dM^(i) = sum_t gamma_t^(i) dy_t phi(q_t)^T: bwd_dm_mfma_kernel, per group of four cached
//     segments and range of later tokens, walks the tokens in chunks of 64 (the scan's
//     state-update contraction with phi(q) in place of phi(k) and gamma dy in place of v),
//     and dP_i = sum_t da_t^(i) u_t beside it; dM is stored transposed.
//   bwd_gate_mfma_kernel: the softmax backward from the gate numerators W, 1/l and the online
//     weight (gamma_i = W_i / l), dgamma of the online segment, du_t (on MFMA) and dq.
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

// M_lo [BH*NS][DV][DK] bf16 -> MT [BH*NS][DK][DV] bf16, 32 x 32 tiles through LDS.  The
// values are the bf16 states themselves (no rounding here), so the bf16 call reads M_lo only.
__global__ __launch_bounds__(256) void transpose_states_kernel(const bf16_t* __restrict__ M_lo,
                                                               int DV, int DK,
                                                               bf16_t* __restrict__ MT) {
    __shared__ bf16_t tile[32][34];
    const size_t st = blockIdx.x;
    const int r0 = blockIdx.y * 32, c0 = blockIdx.z * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    const bf16_t* src = M_lo + st * (size_t)DV * DK;
    bf16_t* dst = MT + st * (size_t)DV * DK;
    for (int y = ty; y < 32; y += 8) tile[y][tx] = src[(size_t)(c0 + y) * DK + r0 + tx];
    __syncthreads();
    for (int y = ty; y < 32; y += 8) dst[(size_t)(r0 + y) * DV + c0 + tx] = tile[tx][y];
}

constexpr int CHK = 64;    // tokens per chunk of the dM walk
constexpr int TPAD = 72;   // row stride (bf16) of the token-indexed LDS tiles: 144 bytes

constexpr int SPW = 4;          // cached segments per dM workgroup (8 waves: 2 per segment)
constexpr int DM_CHUNKS = 128;  // chunks of 64 tokens per token range of the dM walk

typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4_t mfma16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// dM^(i) (stored transposed, [r][c]) for d_k = d_v = 128 and d_g <= 128, SPW consecutive
// segments i0.. (a group) per workgroup: dM^T[r][c] += sum_t phi(q_t)[r] (gamma_t^(i) dy_t[c]),
// and dP_i of this head = sum_t da_t^(i) u_t.  A chunk of 64 later tokens is staged once in LDS
// for all the segments, transposed so that the token index (the contraction index) runs along
// the rows: phi(q)^T, dy^T, u^T (token pairs packed in 32-bit words), gamma_t^(i0+k) =
// W_t^(i0+k) / l_t from the forward gate pass (zero unless token t lies after segment i0+k)
// and da_t^(i0+k) split into a bf16 high part and the bf16 rest.  Wave w serves segment
// i0 + w / 2 and value columns c in [64 (w % 2), +64): it scales its own dy^T fragments by
// gamma in registers and keeps the four 32-row blocks of r for its two 32-column blocks in
// its accumulators.  dP runs on 16x16x32 MFMAs: rows 0..3 the high parts of the SPW segments'
// da, rows 4..7 the rest (rows 8..15 zero), columns the 16 gate columns of wave w; the two
// halves are added at the end.  The tiles are double-buffered and the next chunk's rows are
// loaded into registers while the current one is contracted, so a chunk takes one barrier.
//
// Work items: the token axis is cut into ranges of DM_CHUNKS chunks; a workgroup takes one
// (token range, group, head) and walks the range's tokens after the group (items whose range
// ends before the group's later tokens begin exit at once).  Items are numbered head fastest,
// so the workgroups dealt round-robin to the 8 XCDs run, on each XCD, the same range and
// groups of a few heads side by side: their token chunks are read from HBM about once per
// head and served to the other groups from that XCD's L2.  Every item adds its partial dM
// and dP into the zero-filled outputs (fp32 atomic adds, the order of the partial sums
// varies); dM^T puts the 32 lanes of a row block on one 128-byte line.
__global__ __launch_bounds__(512, 1) void bwd_dm_mfma_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ dY, const uint16_t* __restrict__ Wg,
    const float* __restrict__ inv_l, const bf16_t* __restrict__ U,
    const float* __restrict__ daT, int BH, int L, int C, int NS, int DG, int H, int xh, int phi,
    float* __restrict__ dM, float* __restrict__ dP) {
    __shared__ __attribute__((aligned(16))) bf16_t qt[2][128][TPAD];  // phi(q)^T [r][t]
    __shared__ __attribute__((aligned(16))) bf16_t yt[2][128][TPAD];  // dy^T [c][t]
    __shared__ __attribute__((aligned(16))) bf16_t ut[2][128][TPAD];  // u^T [e][t]
    __shared__ __attribute__((aligned(16))) float sg[2][SPW][CHK];     // gamma [segment][t]
    __shared__ __attribute__((aligned(16))) bf16_t sda[2][16][TPAD];   // da split [row][t]
    const int NG = (NS + SPW - 1) / SPW;
    const size_t bh = blockIdx.x % BH;
    const int grp = (blockIdx.x / BH) % NG, range = blockIdx.x / BH / NG;
    const int i0 = grp * SPW;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, half = lane >> 5;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int T = (L + kGateTile - 1) / kGateTile;
    const int nseg = min(SPW, NS - i0);

    // the chunks [c_lo, c_hi) of the range that hold tokens after the group (64-token chunks
    // from token 0; the tokens of the first chunk up to segment i0 + k have gamma = da = 0)
    const int first0 = (i0 + 1) * C;
    const int c_lo = max(range * DM_CHUNKS, first0 / CHK);
    const int c_hi = min((range + 1) * DM_CHUNKS, (L + CHK - 1) / CHK);
    if (first0 >= L || c_lo >= c_hi) return;  // uniform: no later token in this range
    const int first = c_lo * CHK;
    const int nchunk = c_hi - c_lo;

    // staging roles: token pair (2p, 2p + 1) and columns dc..dc + 7 of q, dy and u; threads
    // 0..255 one gamma (segment kg, token tg), threads 256..511 one da
    const int p = tid & 31, dc = (tid >> 5) * 8;
    const int dcu = min(dc, DG - 8);  // u columns clamped into the row (stored only if dc < DG)
    const int kg = (tid >> 6) & 3, tg = tid & 63;
    const int ig = min(i0 + kg, NS - 1);
    // one chunk in registers (raw loaded values only: anything computed from them here would
    // wait for the loads).  Rows past L are read at L - 1 and cancelled by gamma = da = 0.
    u32x4_t rq[2], ry[2], ru[2];
    uint32_t rw = 0u;
    float rx = 0.f;  // 1 / l_t (threads 0..255) or da (threads 256..511)
    auto load = [&](int j0) {
#pragma unroll
        for (int o = 0; o < 2; ++o) {
            const size_t row = bh * L + min(j0 + 2 * p + o, L - 1);
            rq[o] = *reinterpret_cast<const u32x4_t*>(Q + row * 128 + dc);
            ry[o] = *reinterpret_cast<const u32x4_t*>(dY + row * 128 + dc);
            ru[o] = *reinterpret_cast<const u32x4_t*>(U + row * DG + dcu);
        }
        // every thread issues the same loads (no branch around a load)
        const int t = min(j0 + tg, L - 1);
        rw = Wg[((bh * T + t / kGateTile) * NS + ig) * kGateTile + t % kGateTile];
        rx = *(tid < 256 ? inv_l + bh * L + t : daT + (bh * NS + ig) * L + t);
    };
    auto pack_pairs = [&](bf16_t (*dst)[TPAD], const u32x4_t& a, const u32x4_t& b) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            *reinterpret_cast<uint32_t*>(&dst[dc + 2 * e][2 * p]) = (a[e] & 0xffffu) | (b[e] << 16);
            *reinterpret_cast<uint32_t*>(&dst[dc + 2 * e + 1][2 * p]) =
                (a[e] >> 16) | (b[e] & 0xffff0000u);
        }
    };
    auto stage = [&](int buf, int j0) {
        pack_pairs(qt[buf], phi8(rq[0], phi), phi8(rq[1], phi));
        pack_pairs(yt[buf], ry[0], ry[1]);
        if (dc < DG) pack_pairs(ut[buf], ru[0], ru[1]);
        const int t = j0 + tg;
        const bool later = t < L && t / C > i0 + kg && kg < nseg;
        if (tid < 256) {
            sg[buf][kg][tg] = later ? bf16_to_f32((bf16_t)rw) * rx : 0.f;
        } else {
            const float da = later ? rx : 0.f;
            const bf16_t hi = f32_to_bf16(da);
            sda[buf][kg][tg] = hi;
            sda[buf][SPW + kg][tg] = f32_to_bf16(da - bf16_to_f32(hi));
        }
    };

    f32x16_t mt[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mt[db][cb][r] = 0.f;
    f32x4_t pacc = {0.f, 0.f, 0.f, 0.f};
    const int k = wave >> 1, c0 = (wave & 1) * 64, e0 = wave * 16;

    // rows 8..15 of the da tiles stay zero
    for (int e = tid; e < 2 * 8 * TPAD; e += 512)
        sda[e / (8 * TPAD)][8 + (e / TPAD) % 8][e % TPAD] = (bf16_t)0;
    load(first);
    stage(0, first);
    if (nchunk > 1) load(first + CHK);
    __syncthreads();
    for (int ch = 0; ch < nchunk; ++ch) {
        const int buf = ch & 1;
#pragma unroll
        for (int ks = 0; ks < CHK / 16; ++ks) {
            const int t8 = ks * 16 + half * 8;
            const float4 g0 = *reinterpret_cast<const float4*>(&sg[buf][k][t8]);
            const float4 g1 = *reinterpret_cast<const float4*>(&sg[buf][k][t8 + 4]);
            const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
            u32x4_t gb[2];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(&yt[buf][c0 + cb * 32 + l32][t8]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    gb[cb][e] = pack_bf16x2(g[2 * e] * bf_lo(raw[e]), g[2 * e + 1] * bf_hi(raw[e]));
            }
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const u32x4_t qa = *reinterpret_cast<const u32x4_t*>(&qt[buf][db * 32 + l32][t8]);
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) mt[db][cb] = mfma32(qa, gb[cb], mt[db][cb]);
            }
        }
        if (e0 < DG) {
#pragma unroll
            for (int ks = 0; ks < CHK / 32; ++ks) {
                const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&sda[buf][l16][ks * 32 + q4 * 8]);
                const u32x4_t b = *reinterpret_cast<const u32x4_t*>(&ut[buf][e0 + l16][ks * 32 + q4 * 8]);
                pacc = mfma16(a, b, pacc);
            }
        }
        if (ch + 1 < nchunk) {
            // the other buffer was last read before the previous barrier
            stage(buf ^ 1, first + (ch + 1) * CHK);
            if (ch + 2 < nchunk) load(first + (ch + 2) * CHK);
        }
        __syncthreads();
    }
    // dP: lane l16 of rows 0..3 (lanes 0..15) plus the rest in rows 4..7 (lanes 16..31)
    const int b = (int)(bh / H), h = (int)(bh % H);
    const size_t rgi = xh == 1 ? h : 0, bx = xh == 1 ? b : bh;
    const size_t nbx = (size_t)(BH / H) * xh;
    f32x4_t rest;
#pragma unroll
    for (int j = 0; j < 4; ++j) rest[j] = __shfl_down(pacc[j], 16);
    if (e0 < DG && q4 == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (j < nseg)
                unsafeAtomicAdd(&dP[((rgi * NS + i0 + j) * nbx + bx) * DG + e0 + l16], pacc[j] + rest[j]);
    }
    // dM^T[r][c]: lane holds c = c0 + 32 cb + l32 and r = 32 db + 8g + 4 half + e
    if (k >= nseg) return;
    float* out = dM + (bh * NS + i0 + k) * (size_t)(128 * 128) + c0 + l32;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    unsafeAtomicAdd(out + (size_t)(db * 32 + 8 * g + 4 * half + e) * 128 + cb * 32,
                                    mt[db][cb][4 * g + e]);
}

constexpr int OT = 64;     // tokens per t tile of the online-segment backward
constexpr int RT = 128;    // tokens per r tile
constexpr int NPAD = 136;  // row stride (bf16) of the token-major LDS tiles: 272 bytes

// dM^T (fp32, [r][c]) -> dM (bf16, [c][r]) per cached state, 32 x 32 tiles through LDS
__global__ __launch_bounds__(256) void dm_cr_kernel(const float* __restrict__ dMT,
                                                   bf16_t* __restrict__ dMc) {
    __shared__ float tile[32][33];
    const size_t st = blockIdx.x;
    const int r0 = blockIdx.y * 32, c0 = blockIdx.z * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    const float* src = dMT + st * (128 * 128);
    bf16_t* dst = dMc + st * (128 * 128);
    for (int y = ty; y < 32; y += 8) tile[y][tx] = src[(size_t)(r0 + y) * 128 + c0 + tx];
    __syncthreads();
    for (int y = ty; y < 32; y += 8) dst[(size_t)(c0 + y) * 128 + r0 + tx] = f32_to_bf16(tile[tx][y]);
}

// The online segment's share of dK and dV for d_k = d_v = 128 (bf16), on MFMA.  For token r
// of segment s, E_r = dM^(s) + sum_{t >= r in s} gamma_t^(s) dy_t phi(q_t)^T, dv_r = E_r phi(k_r)
// and dphi(k_r) = E_r^T v_r; over a tile of r tokens that is
//   dV^T[c][r]      = sum_j dM[c][j] phi(k_r)[j] + sum_{t >= r} dy_t[c] P[t][r],
//                     P[t][r] = gamma_t <phi(q_t), phi(k_r)>
//   dphi(K)^T[j][r] = sum_c dM[c][j] v_r[c]      + sum_{t >= r} phi(q_t)[j] B[t][r],
//                     B[t][r] = gamma_t <dy_t, v_r>
// (the flash-attention backward's dK/dV loop without the softmax).  A workgroup takes one
// tile of RT = 128 r tokens and walks the segment's 64-token t tiles from the r tile's start
// on; waves 0..3 form dV, waves 4..7 dphi(K), wave rb of each side the 32 r tokens
// 32 rb .. + 31.  Per t tile a wave forms the two 32 x 32 blocks P or B of its r block and
// the tile's two t blocks (8 MFMAs each over the features), masked (t >= r, t in the
// segment) and scaled in registers, where they are already the B operand of the token
// contraction: the k index of the second product is permuted the same way on both sides
// (the A operand, dy^T or phi(q)^T staged in LDS with tokens along the rows, is read as two
// 4-token runs per k step); its accumulators hold the four 32-row blocks (c or j) of its r
// block.  The dM term uses bf16 copies of dM ([c][j] for dV; the fp32 [j][c] rounded on load
// for dK).  phi(q) and dy of a t tile are staged twice (token-major for the first product,
// transposed for the second), double-buffered, the next tile loaded into registers during
// the current one.
__global__ __launch_bounds__(512, 1) void bwd_online_mfma_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kh, const bf16_t* __restrict__ K,
    const bf16_t* __restrict__ V, const bf16_t* __restrict__ dY, const float* __restrict__ gs,
    const float* __restrict__ dMT, const bf16_t* __restrict__ dMc, int BH, int L, int C, int NS,
    int phi, float* __restrict__ dK, float* __restrict__ dV) {
    // one LDS block: phi(q) [t][j] and dy [t][c] token-major, phi(q)^T [j][t] and dy^T [c][t],
    // gamma_t (0 past the segment), two buffers each
    constexpr int NB = 2 * OT * NPAD * 2, TB = 2 * 128 * TPAD * 2;
    __shared__ uint4 lds[(2 * NB + 2 * TB + 2 * OT * 4) / 16];
    unsigned char* lb = reinterpret_cast<unsigned char*>(lds);
    bf16_t(*qn)[OT][NPAD] = reinterpret_cast<bf16_t(*)[OT][NPAD]>(lb);
    bf16_t(*yn)[OT][NPAD] = reinterpret_cast<bf16_t(*)[OT][NPAD]>(lb + NB);
    bf16_t(*qtt)[128][TPAD] = reinterpret_cast<bf16_t(*)[128][TPAD]>(lb + 2 * NB);
    bf16_t(*ytt)[128][TPAD] = reinterpret_cast<bf16_t(*)[128][TPAD]>(lb + 2 * NB + TB);
    float(*sgo)[OT] = reinterpret_cast<float(*)[OT]>(lb + 2 * NB + 2 * TB);
    // r tiles slowest: the first r tiles of every segment (the most t tiles) go first
    const int nsb = NS * BH;
    const int R = blockIdx.x / nsb;
    const size_t bh = (blockIdx.x % nsb) % BH;
    const int s = (blockIdx.x % nsb) / BH;
    const int t0 = s * C, n = min(C, L - t0);
    const int r0 = R * RT;
    if (r0 >= n) return;  // uniform: the segment has no r tile R
    const int NT = (n + OT - 1) / OT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, half = lane >> 5;
    const bool kside = wave >= 4;  // waves 4..7: dphi(K); 0..3: dV
    const int rb = wave & 3;
    const int rbase = r0 + rb * 32;     // the wave's first r
    const int rr = rbase + l32;         // this lane's r (segment-relative; rows past the
                                        // segment are read clamped, their sums not stored)
    const size_t rrow = bh * L + min(t0 + rr, L - 1);

    // phi(k_r) (dV side) or v_r (dK side): the fixed B operand, k = 16 ks + 8 half + 0..7
    u32x4_t kv[8];
    {
        const bf16_t* src = (kside ? V : Kh) + rrow * 128 + half * 8;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) kv[ks] = *reinterpret_cast<const u32x4_t*>(src + ks * 16);
    }
    const f32x16_t zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                           0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    f32x16_t acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = zero;

    // staging roles: token pair (2p, 2p + 1) of the tile, features 8 fg .. + 7
    const int p = tid & 31, fg = tid >> 5;
    u32x4_t rq[2], ry[2];
    float rg = 0.f;
    auto load = [&](int tt0) {
#pragma unroll
        for (int o = 0; o < 2; ++o) {
            const size_t row = bh * L + min(t0 + tt0 + 2 * p + o, L - 1);
            rq[o] = *reinterpret_cast<const u32x4_t*>(Q + row * 128 + fg * 8);
            ry[o] = *reinterpret_cast<const u32x4_t*>(dY + row * 128 + fg * 8);
        }
        rg = gs[bh * L + min(t0 + tt0 + (tid & 63), L - 1)];
    };
    auto stage = [&](int buf, int tt0) {
        const u32x4_t a = phi8(rq[0], phi), b = phi8(rq[1], phi);
        *reinterpret_cast<u32x4_t*>(&qn[buf][2 * p][fg * 8]) = a;
        *reinterpret_cast<u32x4_t*>(&qn[buf][2 * p + 1][fg * 8]) = b;
        *reinterpret_cast<u32x4_t*>(&yn[buf][2 * p][fg * 8]) = ry[0];
        *reinterpret_cast<u32x4_t*>(&yn[buf][2 * p + 1][fg * 8]) = ry[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int rw = fg * 8 + 2 * e;
            *reinterpret_cast<uint32_t*>(&qtt[buf][rw][2 * p]) = (a[e] & 0xffffu) | (b[e] << 16);
            *reinterpret_cast<uint32_t*>(&qtt[buf][rw + 1][2 * p]) = (a[e] >> 16) | (b[e] & 0xffff0000u);
            *reinterpret_cast<uint32_t*>(&ytt[buf][rw][2 * p]) = (ry[0][e] & 0xffffu) | (ry[1][e] << 16);
            *reinterpret_cast<uint32_t*>(&ytt[buf][rw + 1][2 * p]) =
                (ry[0][e] >> 16) | (ry[1][e] & 0xffff0000u);
        }
        if (tid < OT) sgo[buf][tid] = tt0 + tid < n ? rg : 0.f;
    };

    const int T0 = r0 / OT;  // the t tile holding the r tile's first token
    load(T0 * OT);
    stage(0, T0 * OT);
    if (T0 + 1 < NT) load((T0 + 1) * OT);
    // the dM term over all four 32-row blocks of c (dV) or j (dK)
    // (the side is chosen outside the loops, so each block's fragment loads are all issued
    // before its MFMAs: loads under a per-fragment branch were waited for one by one)
    {
        const size_t st = (bh * NS + s) * (size_t)(128 * 128);
        if (!kside) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const bf16_t* row = dMc + st + (b * 32 + l32) * 128 + half * 8;
                u32x4_t a[8];
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) a[ks] = *reinterpret_cast<const u32x4_t*>(row + ks * 16);
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) acc[b] = mfma32(a[ks], kv[ks], acc[b]);
            }
        } else {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float* row = dMT + st + (b * 32 + l32) * 128 + half * 8;
#pragma unroll
                for (int k4 = 0; k4 < 8; k4 += 4) {  // four k-steps' loads at a time
                    float4 f[4][2];
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        f[ks][0] = *reinterpret_cast<const float4*>(row + (k4 + ks) * 16);
                        f[ks][1] = *reinterpret_cast<const float4*>(row + (k4 + ks) * 16 + 4);
                    }
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const u32x4_t a = {pack_bf16x2(f[ks][0].x, f[ks][0].y),
                                           pack_bf16x2(f[ks][0].z, f[ks][0].w),
                                           pack_bf16x2(f[ks][1].x, f[ks][1].y),
                                           pack_bf16x2(f[ks][1].z, f[ks][1].w)};
                        acc[b] = mfma32(a, kv[k4 + ks], acc[b]);
                    }
                }
            }
        }
    }
    __syncthreads();
    for (int T = T0; T < NT; ++T) {
        const int buf = (T - T0) & 1;
        const int tt0 = T * OT;
        // first products: D[t][r] over the 128 features (phi(q) phi(k)^T or dy v^T) for the
        // tile's two t blocks; a block wholly before the wave's r block is masked
        const bf16_t(*an)[NPAD] = kside ? yn[buf] : qn[buf];
        u32x4_t pf[2][2];
        bool live[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            live[tb] = tt0 + tb * 32 + 31 >= rbase;  // uniform
            if (!live[tb]) continue;
            f32x16_t sa = zero;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const u32x4_t a =
                    *reinterpret_cast<const u32x4_t*>(&an[tb * 32 + l32][ks * 16 + half * 8]);
                sa = mfma32(a, kv[ks], sa);
            }
            // lane holds r = rr and t = tt0 + 32 tb + 8 g + 4 half + e (value 4 g + e)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int tl = tb * 32 + 8 * g + 4 * half;
                const float4 gv = *reinterpret_cast<const float4*>(&sgo[buf][tl]);
                const float gg[4] = {gv.x, gv.y, gv.z, gv.w};
                float pv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) pv[e] = tt0 + tl + e >= rr ? sa[4 * g + e] * gg[e] : 0.f;
                pf[tb][g >> 1][(g & 1) * 2] = pack_bf16x2(pv[0], pv[1]);
                pf[tb][g >> 1][(g & 1) * 2 + 1] = pack_bf16x2(pv[2], pv[3]);
            }
        }
        // second products over the tile's tokens: k step kk of block tb holds, in slots 0..3
        // and 4..7, the tokens 32 tb + 16 kk + 4 half + 0..3 and 32 tb + 16 kk + 8 + 4 half + 0..3
        const bf16_t(*at)[TPAD] = kside ? qtt[buf] : ytt[buf];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            if (!live[tb]) continue;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int c0 = tb * 32 + 16 * kk + 4 * half;
                    const uint2 lo = *reinterpret_cast<const uint2*>(&at[b * 32 + l32][c0]);
                    const uint2 hi = *reinterpret_cast<const uint2*>(&at[b * 32 + l32][c0 + 8]);
                    const u32x4_t a = {lo.x, lo.y, hi.x, hi.y};
                    acc[b] = mfma32(a, pf[tb][kk], acc[b]);
                }
        }
        if (T + 1 < NT) {
            // the other buffer was last read before the previous barrier
            stage(buf ^ 1, tt0 + OT);
            if (T + 2 < NT) load(tt0 + 2 * OT);
        }
        __syncthreads();
    }
    if (rr >= n) return;
    const size_t orow = (bh * L + t0 + rr) * 128;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int m = b * 32 + 8 * g + 4 * half;  // c (dV) or j (dK) of values 4 g .. 4 g + 3
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = acc[b][4 * g + e];
            if (kside && phi) {
                const u32x2_t kw = *reinterpret_cast<const u32x2_t*>(K + orow + m);
                o[0] *= fminf(feature(bf_lo(kw[0]), 1), 1.f);
                o[1] *= fminf(feature(bf_hi(kw[0]), 1), 1.f);
                o[2] *= fminf(feature(bf_lo(kw[1]), 1), 1.f);
                o[3] *= fminf(feature(bf_hi(kw[1]), 1), 1.f);
            }
            *reinterpret_cast<float4*>((kside ? dK : dV) + orow + m) = make_float4(o[0], o[1], o[2], o[3]);
        }
}

constexpr int GTOK = 256;  // tokens per workgroup of the gate backward (one gate tile)
static_assert(GTOK == kGateTile, "the gate backward reads whole gate tiles");

// The means as B fragments of the du product (k = segment, n = gate column): for x head bx,
// k step ks, 32-column block eb and lane (l32, half) the 8 values P_i[32 eb + l32],
// i = 16 ks + 8 half + 0..7, as bf16 high parts then bf16 rests (2 x 16 bytes); zero past NS
// and d_g.
__global__ void ptf_kernel(const float* __restrict__ P, int NS, int DG, int NSK, size_t n,
                           u32x4_t* __restrict__ out) {
    const size_t d = blockIdx.x * (size_t)blockDim.x + threadIdx.x;  // (bx, ks, eb, lane)
    if (d >= n) return;
    const int lane = (int)(d % 64), eb = (int)((d / 64) % 4), ks = (int)((d / 256) % NSK);
    const size_t bx = d / 256 / NSK;
    const int e = 32 * eb + (lane & 31), i0 = 16 * ks + 8 * (lane >> 5);
    u32x4_t hi, lo;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float v[2];
#pragma unroll
        for (int o = 0; o < 2; ++o) {
            const int i = i0 + 2 * q + o;
            v[o] = i < NS && e < DG ? P[(bx * NS + i) * DG + e] : 0.f;
        }
        hi[q] = pack_bf16x2(v[0], v[1]);
        lo[q] = pack_bf16x2(v[0] - bf_lo(hi[q]), v[1] - bf_hi(hi[q]));
    }
    out[2 * d] = hi;
    out[2 * d + 1] = lo;
}

// The softmax backward of the gate for d_k = d_v = 128 and d_g <= 128, one 256-token gate
// tile per workgroup: gamma_i = W_t^(i) / l_t (i < s), gamma_s = won_t / l_t; dgamma of the
// online segment <dy_t, O_on[t]> (formed by the online scan); D_t = sum_i gamma_i dgamma_i;
// da_i = gamma_i (dgamma_i - D) written over dgamma (segment-major, [i][t]); da_s;
// du_t = sum_i da_i P_i on MFMA plus da_s times the prefix mean x_t; dq = dphi(q) phi'(q)
// with dphi(q) the bf16 output of the swapped read.  Wave w takes tokens 32 w .. + 31 (lane l32 = token): pass 1 sums D over the
// segments (half h of the wave the segments 16 ks + 8 h + 0..7), pass 2 forms da for the
// same segments, which are then the A fragment (bf16 high part and rest) of 32x32x16 MFMAs
// against the means' fragments (high and rest; the rest times the rest is dropped).
__global__ __launch_bounds__(512) void bwd_gate_mfma_kernel(
    const bf16_t* __restrict__ Q, const float* __restrict__ xps, const uint16_t* __restrict__ Wg,
    const float* __restrict__ won, const float* __restrict__ inv_l, const float* __restrict__ dgs_i,
    const bf16_t* __restrict__ dqh, const u32x4_t* __restrict__ ptf,
    int L, int C, int NS, int DG, int H, int xh, int phi, float* __restrict__ daT,
    float* __restrict__ das_o, float* __restrict__ gs_o, float* __restrict__ dU,
    float* __restrict__ dQ) {
    __shared__ float s_das[GTOK];
    const int T = (L + GTOK - 1) / GTOK;
    const int tile = T - 1 - blockIdx.x;  // the tiles that read the most segments first
    const size_t bh = blockIdx.y;
    const int b = (int)(bh / H), h = (int)(bh % H);
    const size_t bx = (size_t)b * xh + (xh == 1 ? 0 : h);
    const int t0 = tile * GTOK;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, half = lane >> 5;
    const int NSK = (NS + 15) / 16;
    const int s_hi = (min(L, t0 + GTOK) - 1) / C;  // segments read by the tile's last token
    const int nks = (s_hi + 15) / 16;
    const uint16_t* wt = Wg + (bh * T + tile) * (size_t)NS * GTOK;  // [i][t - t0]
    const float* dgt = daT + bh * (size_t)NS * L;                  // [i][t]

    const int tl = wave * 32 + l32;
    const int t = t0 + tl;
    const int tc = min(t, L - 1);
    const int sg = tc / C;
    const float il = inv_l[bh * L + tc];
    const float dgs = dgs_i[bh * L + tc];  // dgamma of the online segment
    // pass 1: sum_i W_i dgamma_i over this half's segments, then both halves
    // the eight (numerator, dgamma) pairs of a k-step are loaded together: the opaque uses
    // keep the compiler from sinking each load under its i < sg test, where every load was
    // waited for on its own
    auto load_wg = [&](int ks, float (&w)[8], float (&g)[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int ic = min(16 * ks + 8 * half + j, NS - 1);
            w[j] = bf16_to_f32((bf16_t)wt[(size_t)ic * GTOK + tl]);
            g[j] = dgt[(size_t)ic * L + tc];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(w[j]), "+v"(g[j]));
    };
    float dp = 0.f;
#pragma unroll 2
    for (int ks = 0; ks < nks; ++ks) {
        float w[8], g[8];
        load_wg(ks, w, g);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = 16 * ks + 8 * half + j;
            dp += i < sg ? w[j] * g[j] : 0.f;
        }
    }
    dp += __shfl_xor(dp, 32);
    const float gsv = won[bh * L + tc] * il;
    const float Dt = dp * il + gsv * dgs;
    const float das = gsv * (dgs - Dt);
    if (half == 0) {
        s_das[tl] = das;
        if (t < L) {
            das_o[bh * L + t] = das;
            gs_o[bh * L + t] = gsv;
        }
    }
    // pass 2: da (written over dgamma) and du on MFMA
    const f32x16_t zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                           0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    f32x16_t acc[4];
#pragma unroll
    for (int eb = 0; eb < 4; ++eb) acc[eb] = zero;
    const int neb = (DG + 31) / 32;
    const u32x4_t* pb = ptf + (bx * NSK) * 4 * 64 * 2;
    for (int ks = 0; ks < nks; ++ks) {
        float da[8], w[8], g[8];
        load_wg(ks, w, g);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = 16 * ks + 8 * half + j;
            da[j] = i < sg ? w[j] * il * (g[j] - Dt) : 0.f;
        }
        u32x4_t bhi[4], blo[4];
#pragma unroll
        for (int eb = 0; eb < 4; ++eb) {
            const u32x4_t* src = pb + ((size_t)(ks * 4 + eb) * 64 + lane) * 2;
            bhi[eb] = src[0];
            blo[eb] = src[1];
        }
        if (t < L) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = 16 * ks + 8 * half + j;
                if (i < sg) daT[(bh * NS + i) * (size_t)L + t] = da[j];
            }
        }
        u32x4_t ahi, alo;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            ahi[q] = pack_bf16x2(da[2 * q], da[2 * q + 1]);
            alo[q] = pack_bf16x2(da[2 * q] - bf_lo(ahi[q]), da[2 * q + 1] - bf_hi(ahi[q]));
        }
#pragma unroll
        for (int eb = 0; eb < 4; ++eb) {
            if (eb >= neb) continue;  // uniform
            acc[eb] = mfma32(ahi, bhi[eb], acc[eb]);
            acc[eb] = mfma32(ahi, blo[eb], acc[eb]);
            acc[eb] = mfma32(alo, bhi[eb], acc[eb]);
        }
    }
    // du_t: lane holds e = 32 eb + l32 and token 32 w + 8 g + 4 half + e' (value 4 g + e');
    // plus da_s x_t with x_t the prefix mean (prefix sum / (j + 1)) of the token's segment
#pragma unroll
    for (int eb = 0; eb < 4; ++eb) {
        const int e = 32 * eb + l32;
        if (eb >= neb || e >= DG) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int tt = wave * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
            const int tv = t0 + tt;
            if (tv >= L) continue;
            const int j = tv - (tv / C) * C;
            dU[(bh * L + tv) * DG + e] =
                acc[eb][v] + s_das[tt] * xps[(bx * L + tv) * DG + e] / (float)(j + 1);
        }
    }
    // dq = dphi(q) phi'(q), 8 columns per thread and step
    for (int idx = tid; idx < GTOK * 16; idx += 512) {
        const int tq = t0 + idx / 16, c8 = (idx % 16) * 8;
        if (tq >= L) break;
        const size_t o = (bh * L + tq) * 128 + c8;
        const u32x4_t g = *reinterpret_cast<const u32x4_t*>(dqh + o);
        const u32x4_t q = *reinterpret_cast<const u32x4_t*>(Q + o);
        float r[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            r[2 * e] = bf_lo(g[e]) * (phi ? fminf(feature(bf_lo(q[e]), 1), 1.f) : 1.f);
            r[2 * e + 1] = bf_hi(g[e]) * (phi ? fminf(feature(bf_hi(q[e]), 1), 1.f) : 1.f);
        }
        *reinterpret_cast<float4*>(dQ + o) = make_float4(r[0], r[1], r[2], r[3]);
        *reinterpret_cast<float4*>(dQ + o + 4) = make_float4(r[4], r[5], r[6], r[7]);
    }
}

__global__ void zero_kernel(float* __restrict__ p, size_t n) {
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n;
         e += (size_t)gridDim.x * blockDim.x)
        p[e] = 0.f;
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
                       0, st, (const bf16_t*)M_lo, d.d_v, d.d_k, (bf16_t*)w.mt);
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
    rc = launch_bwd_dgamma(d, Q, dY, M_lo, w.daT, stream);
    if (rc) return rc;
    // the means as the du product's B fragments, then the gate backward (da over dgamma;
    // da of the online segment into dG, used as [B,H,L])
    const int nsk = (NS + 15) / 16;
    const size_t nptf = (size_t)d.B * d.x_heads * nsk * 4 * 64;
    hipLaunchKernelGGL(ptf_kernel, dim3((unsigned)((nptf + 255) / 256)), dim3(256), 0, st, P, NS,
                       d.d_g, nsk, nptf, (u32x4_t*)w.ptf);
    hipLaunchKernelGGL(bwd_gate_mfma_kernel, dim3((d.L + GTOK - 1) / GTOK, BH), dim3(512), 0, st,
                       (const bf16_t*)Q, w.xps, w.W, w.won, w.inv_l, w.on,
                       (const bf16_t*)w.dqh, (const u32x4_t*)w.ptf, d.L, d.seg_len, NS, d.d_g,
                       d.H, d.x_heads, d.phi, w.daT, w.dG, w.gs, dU, dQ);
    // dM and dP take the partial sums of the split workgroups: zero them first (a kernel, so
    // the sequence stays capturable)
    const size_t ndm = (size_t)BH * NS * d.d_v * d.d_k;
    const size_t ndp = (size_t)d.B * d.H * NS * d.d_g;  // [H or 1][NS][B*xh][dg]
    hipLaunchKernelGGL(zero_kernel, dim3(2048), dim3(256), 0, st, w.dM, ndm);
    hipLaunchKernelGGL(zero_kernel, dim3(256), dim3(256), 0, st, w.dpp, ndp);
    const int nranges = ((d.L + CHK - 1) / CHK + DM_CHUNKS - 1) / DM_CHUNKS;
    hipLaunchKernelGGL(bwd_dm_mfma_kernel, dim3(nranges * ((NS + SPW - 1) / SPW) * BH), dim3(512),
                       0, st, (const bf16_t*)Q, (const bf16_t*)dY, w.W, w.inv_l, (const bf16_t*)U,
                       w.daT, BH, d.L, d.seg_len, NS, d.d_g, d.H, d.x_heads, d.phi, w.dM, w.dpp);
    return (int)hipGetLastError();
}

int launch_bwd_online_mfma(const mc_dims& d, const BwdBuffers& w, const void* Q, const void* K,
                           const void* V, const void* dY, float* dK, float* dV, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    const int NS = (d.L + d.seg_len - 1) / d.seg_len;
    const int BH = d.B * d.H;
    // dM in bf16, [c][j], over the transposed states of the swapped read (no longer needed)
    hipLaunchKernelGGL(dm_cr_kernel, dim3(BH * NS, 4, 4), dim3(256), 0, st, w.dM, (bf16_t*)w.mt);
    const int rt = (d.seg_len + RT - 1) / RT;  // r tiles of a segment
    hipLaunchKernelGGL(bwd_online_mfma_kernel, dim3(rt * NS * BH), dim3(512), 0, st,
                       (const bf16_t*)Q, (const bf16_t*)(d.phi ? w.khat : K), (const bf16_t*)K,
                       (const bf16_t*)V, (const bf16_t*)dY, w.gs, w.dM, (const bf16_t*)w.mt, BH,
                       d.L, d.seg_len, NS, d.phi, dK, dV);
    return (int)hipGetLastError();
}

}  // namespace mc
