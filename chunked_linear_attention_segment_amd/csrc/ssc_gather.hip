// ssc_gather.hip -- the Sparse Selective Caching read, routed by segment (gitcode explainer
// §3.4: only the selected memories are loaded and read).
//
// For token t of segment s with selected segments R_t (the Top-k of its router scores),
//     y_t = w_on(t) M_t^(s) phi(q_t) + sum_{i in R_t} w_t^(i) M^(i) phi(q_t),
// w being the softmax over R_t and the online segment, normalised (Memory Caching paper §3.1,
// Eq. (9) restricted to R_t).  The selection pass has sorted every read tile's (token, i)
// pairs by segment i.  Here one workgroup takes one tile of one (b, h): it walks the segments
// that have pairs, in ascending order, and applies each state to its pairs 32 at a time, the
// pairs being the columns of one MFMA block:
//     Y^T[c, token_j] += M^(i)[c, :] . bf16(w_j phi(q_{token_j})),   j = 0..31,
// so the work follows the number of pairs, sum_t min(k, s_t), and not the number of states.
//
// 8 waves (two per SIMD); wave w owns value rows 16 w .. 16 w + 15, so its share of a state
// (16 rows x d_k, bf16, read from a copy of the states in MFMA fragment order) is the A
// operand of 16x16x32 MFMAs, held in registers and loaded when the previous segment begins.
// The B operand of a pair block is built once in LDS (two buffers) by all threads and read by
// every wave.  The tile's output accumulates in fp32 in LDS, every wave in its own columns,
// starting from the weighted online term and then adding the states in ascending order, so
// the result is the same on every run.  The tile's pair blocks are listed in LDS when the
// workgroup starts, so walking them costs no memory round trip on the way.
#include <type_traits>

#include "common.cuh"
#include "mc_internal.h"

namespace mc {
namespace {

typedef __bf16 sbf16x8_t __attribute__((ext_vector_type(8)));
typedef float sf32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t su32x4_t __attribute__((ext_vector_type(4)));

constexpr int GT = kSscTile;  // tokens per tile
constexpr int GD = 128;       // d_k = d_v
constexpr int NW = 8;         // waves per workgroup (two per SIMD)
constexpr int RW = GD / NW;   // value rows per wave
constexpr int KS = GD / 32;   // k-steps of a 16x16x32 MFMA
constexpr int OSTR = GD + 4;  // output row stride (floats)
constexpr int PB = 32;        // pairs per block (two MFMA column tiles of 16)

__device__ __forceinline__ sf32x4_t mfma_g(const su32x4_t& a, const su32x4_t& b,
                                           const sf32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sbf16x8_t, a),
                                                   __builtin_bit_cast(sbf16x8_t, b), c, 0, 0, 0);
}

// Blocks are dealt round-robin to the 8 XCDs; when B*H is a multiple of 8 an XCD takes whole
// heads, so the states a head's tiles share stay in that XCD's L2.  Later tiles (more
// candidate segments) go first.
__device__ __forceinline__ void gather_tile(int bid, int BH, int T, int& bh, int& tile) {
    if (BH % 8 == 0) {
        const int xcd = bid % 8, local = bid / 8;
        bh = xcd + 8 * (local / T);
        tile = T - 1 - local % T;
    } else {
        bh = bid / T;
        tile = T - 1 - bid % T;
    }
}

// Slot of (k group G of 8, pair j) in a B-operand buffer: the pair index is XOR-swizzled with
// the group, so both the staging writes (16 groups of one pair per 16 lanes) and the MFMA
// reads (16 pairs of one group per 16 lanes) fall in distinct LDS banks.
__device__ __forceinline__ int bslot(int G, int j) { return G * PB + (j ^ G); }

// The cached states in MFMA fragment order for the routed read: for state (bh, i), wave w
// (value rows RW w ..), k-step ks and lane (l16, q4 = lane / 16), the 8 values
// M[RW w + l16][32 ks + 8 q4 + 0..7] are 16 contiguous bytes, so one k-step of a wave's rows
// is 1 KB.
__global__ void frag_states_kernel(const uint4* __restrict__ S, size_t n16, uint4* __restrict__ Sf) {
    const size_t d = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // destination 16-byte unit
    if (d >= n16) return;
    const int lane = (int)(d % 64), ks = (int)((d / 64) % KS), w = (int)((d / 64 / KS) % NW);
    const size_t st = d / (64 * KS * NW);  // state (bh, i)
    const int row = RW * w + (lane & 15), col = 32 * ks + 8 * (lane >> 4);
    Sf[d] = S[(st * GD + row) * (GD / 8) + col / 8];
}

// the most segments a tile's run starts are staged for (LDS)
constexpr int GNS_MAX = 512;

// A pair block: pairs [p0, min(p0 + PB, pe)) of segment i's run [.., pe); nx is the next
// segment with pairs after i (i itself for the last).  i == s_end: no block.
struct Blk {
    int i, nx, p0, pe;
};
// the most pair blocks of a tile: a block per 32 pairs plus at most one partial block per
// segment
constexpr int NB_MAX = GT * 16 / PB + GNS_MAX;

template <int PHI>
__global__ __launch_bounds__(64 * NW, 1) void ssc_gather_kernel(
    const bf16_t* __restrict__ Q, const uint4* __restrict__ Sf, const float* __restrict__ O_on,
    const float* __restrict__ won, const int32_t* __restrict__ ptok,
    const float* __restrict__ pw, const int32_t* __restrict__ poff, int BH, int L, int C, int NS,
    int top_k, bf16_t* __restrict__ Y, const SegArg sg) {
    constexpr int NT = 64 * NW;
    __shared__ __attribute__((aligned(16))) float out[GT * OSTR];
    // B operand of a pair block: [k group of 8 (16 groups)][pair] 16 bytes each
    __shared__ __attribute__((aligned(16))) su32x4_t bst[2][(GD / 8) * PB];
    __shared__ int rtok[2][PB];
    __shared__ int offs[GNS_MAX + 1];
    // the tile's pair blocks in order: (i | nx << 16, p0 | pe << 16)
    __shared__ int2 blks[NB_MAX];
    __shared__ int nblk_sh;
    const int T = (L + GT - 1) / GT;
    int bh, tile;
    gather_tile(blockIdx.x, BH, T, bh, tile);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int t0 = tile * GT, ntok = min(GT, L - t0);
    const size_t tb = (size_t)bh * T + tile;
    const int32_t* pt = ptok + tb * GT * top_k;
    const float* pwt = pw + tb * GT * top_k;
    const size_t row0 = (size_t)bh * L + t0;
    const int s_end = seg_of(sg, t0 + ntok - 1, C);  // pairs exist only for segments below this
    for (int x = tid; x <= s_end; x += NT) offs[x] = poff[tb * (NS + 1) + x];
    __syncthreads();
    if (wave == 0) {  // the block table: one lane per segment, 64 segments at a time
        int carry = 0, last_nz = -1;
        for (int base = 0; base < s_end; base += 64) {
            const int i = base + lane;
            const int n = i < s_end ? min(max(offs[i + 1] - offs[i], 0), GT * 16) : 0;
            const int nb = (n + PB - 1) / PB;
            int x = nb;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(x, o, 64);
                if (lane >= o) x += y;
            }
            // the next segment with pairs after i: the lowest non-empty lane above, else the
            // first non-empty segment of a later group (patched below through last_nz)
            const unsigned long long nzm = __ballot(nb > 0);
            const unsigned long long above = lane < 63 ? nzm & (~0ull << (lane + 1)) : 0ull;
            int nx = above ? base + __ffsll((long long)above) - 1 : -1;
            const int start = carry + x - nb;
            for (int q = 0; q < nb && start + q < NB_MAX; ++q)
                blks[start + q] = make_int2(i | ((nx < 0 ? i : nx) << 16),
                                            (offs[i] + PB * q) | (offs[i + 1] << 16));
            // the previous group's last non-empty segment learns its successor
            if (nzm && last_nz >= 0 && lane == 0) {
                const int first = base + __ffsll((long long)nzm) - 1;
                // every block of last_nz precedes 'carry'; patch them
                for (int b = min(carry, NB_MAX) - 1; b >= 0 && (blks[b].x & 0xffff) == last_nz; --b)
                    blks[b].x = last_nz | (first << 16);
            }
            if (nzm) last_nz = base + 63 - __clzll((long long)nzm);
            carry += __shfl(x, 63, 64);
        }
        if (lane == 0) nblk_sh = min(carry, NB_MAX);
    }

    // the online term, weighted; several rows' loads in flight per thread before any is used
    // (rows past the tile's tokens read row 0 and are zeroed)
    constexpr int OB = 4;
    for (int e0 = tid; e0 < GT * (GD / 4); e0 += NT * OB) {
        float4 o[OB];
        float wo[OB];
#pragma unroll
        for (int u = 0; u < OB; ++u) {
            const int e = e0 + NT * u, r = e / (GD / 4), c4 = e % (GD / 4);
            const int rr = r < ntok ? r : 0;
            o[u] = *reinterpret_cast<const float4*>(O_on + (row0 + rr) * GD + 4 * c4);
            wo[u] = r < ntok ? won[row0 + rr] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < OB; ++u) {
            const int e = e0 + NT * u, r = e / (GD / 4), c4 = e % (GD / 4);
            *reinterpret_cast<float4*>(&out[r * OSTR + 4 * c4]) =
                make_float4(o[u].x * wo[u], o[u].y * wo[u], o[u].z * wo[u], o[u].w * wo[u]);
        }
    }
    __syncthreads();

    // staging role of this thread: pair j of a block, k = 8 g .. 8 g + 7 (sixteen lanes read
    // one q row, so a load instruction covers whole rows).  A pair index or token outside the
    // tile's ranges is dropped, never dereferenced; the loads themselves are unconditional,
    // from clamped indices, so the code has no branches for the memory counters' bookkeeping
    // to merge.
    const int j = tid >> 4, g = tid & 15;
    const int pmax = GT * top_k;
    auto pair_index = [&](const Blk& b, bool& pv) {
        const int p = b.p0 + j;
        pv = b.i < s_end && p >= 0 && p < b.pe && p < pmax;
        return min(max(p, 0), pmax - 1);
    };
    // the raw token of pair j of block b (tested only where it is used, a block later: a test
    // here would wait for the load)
    auto ld_tok = [&](const Blk& b, bool& pv) {
        const int pc = pair_index(b, pv);
        return pt[pc];
    };
    auto token = [&](int tv, bool pv) { return pv && tv < ntok ? tv : -1; };
    // q values and weight of pair j of block b, whose token is tok
    auto ld_qw = [&](const Blk& b, int tok, su32x4_t& q, float& w) {
        bool pv;
        const int pc = pair_index(b, pv);
        const float wv = pwt[pc];
        w = tok >= 0 ? wv : 0.f;
        q = *reinterpret_cast<const su32x4_t*>(Q + (row0 + (tok >= 0 ? tok : 0)) * GD + 8 * g);
    };
    auto build = [&](const su32x4_t& q, float w) {
        su32x4_t r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo = feature(__uint_as_float(q[e] << 16), PHI) * w;
            const float hv = feature(__uint_as_float(q[e] & 0xffff0000u), PHI) * w;
            r[e] = pack_bf16x2(lo, hv);
        }
        return r;
    };
    // the wave's rows of state i as A fragments (fragment-major copy: 1 KB per k-step)
    auto ld_a = [&](int i, su32x4_t (&a)[KS]) {
        const su32x4_t* sr = reinterpret_cast<const su32x4_t*>(Sf) +
                             (((size_t)bh * NS + i) * NW + wave) * KS * 64 + lane;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a[ks] = sr[ks * 64];
    };
    // the products of a column tile: column l16 is pair (16 nt + l16)'s token tk, rows
    // 4 q4 + 0..3 of the wave's rows
    auto add_out = [&](const sf32x4_t& a, int tk) {
        if (tk < 0) return;
        float* o = &out[tk * OSTR + RW * wave + 4 * q4];
        float4 v = *reinterpret_cast<float4*>(o);
        v.x += a[0];
        v.y += a[1];
        v.z += a[2];
        v.w += a[3];
        *reinterpret_cast<float4*>(o) = v;
    };

    // Pipeline over the pair blocks D0 (read now), D1, D2.  The q values and weights of a
    // block are loaded one block ahead and its tokens two ahead, each into one register set
    // that is consumed before it is reloaded.  The state fragments form a two-slot ring
    // indexed by the parity of the segment (the segment loop is unrolled by two, so the index
    // is known at compile time and no load result is ever copied, which would wait for the
    // load); the next segment's fragments are loaded when a segment begins.  A block's
    // products are added into the output while the next block's MFMAs run.
    const int NB = nblk_sh;
    auto blk = [&](int b) {
        if (b >= NB) return Blk{s_end, s_end, 0, 0};
        const int2 e = blks[b];
        return Blk{e.x & 0xffff, e.x >> 16, e.y & 0xffff, e.y >> 16};
    };
    int bn = 0;  // index of block D0
    Blk D0 = blk(0), D1 = blk(1), D2 = blk(2);
    su32x4_t Qr, Ar[2][KS];
    float Wc = 0.f;
    int tokc = -1, Tn = 0, tk0 = -1, tk1 = -1;
    bool Tv = false;
    sf32x4_t p0, p1;  // the previous block's products (column tiles 0 and 1)
#pragma unroll
    for (int r = 0; r < 4; ++r) p0[r] = p1[r] = 0.f;
    if (D0.i < s_end) {
        bool v0;
        const int t0r = ld_tok(D0, v0);
        tokc = token(t0r, v0);
        ld_qw(D0, tokc, Qr, Wc);
        Tn = ld_tok(D1, Tv);
        ld_a(D0.i, Ar[0]);
    }
    int buf = 0;
    auto run_segment = [&](auto Sc) {
        constexpr int S = decltype(Sc)::value;
        const int cur = D0.i;
        ld_a(D0.nx, Ar[S ^ 1]);  // the next segment with pairs (the last one reloads itself)
        do {
            const Blk D3 = blk(bn + 3);  // read early: its wait then falls behind other work
            bst[buf][bslot(g, j)] = build(Qr, Wc);
            if (g == 0) rtok[buf][j] = tokc;
            // block D1's q values and weights (its token loaded a block ago), block D2's tokens
            tokc = token(Tn, Tv);
            ld_qw(D1, tokc, Qr, Wc);
            Tn = ld_tok(D2, Tv);
            __syncthreads();
            const int n0 = rtok[buf][l16], n1 = rtok[buf][16 + l16];
            sf32x4_t c0, c1;
#pragma unroll
            for (int r = 0; r < 4; ++r) c0[r] = c1[r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                c0 = mfma_g(Ar[S][ks], bst[buf][bslot(4 * ks + q4, l16)], c0);
                c1 = mfma_g(Ar[S][ks], bst[buf][bslot(4 * ks + q4, 16 + l16)], c1);
            }
            // the previous block's products go out while these MFMAs run
            add_out(p0, tk0);
            add_out(p1, tk1);
            p0 = c0;
            p1 = c1;
            tk0 = n0;
            tk1 = n1;
            buf ^= 1;
            D0 = D1;
            D1 = D2;
            D2 = D3;
            ++bn;
        } while (D0.i == cur);
    };
    while (D0.i < s_end) {
        run_segment(std::integral_constant<int, 0>{});
        if (D0.i >= s_end) break;
        run_segment(std::integral_constant<int, 1>{});
    }
    add_out(p0, tk0);
    add_out(p1, tk1);
    __syncthreads();
    for (int e = tid; e < GT * (GD / 8); e += NT) {
        const int r = e / (GD / 8), c8 = e % (GD / 8);
        if (r >= ntok) continue;
        const float* src = &out[r * OSTR + 8 * c8];
        su32x4_t v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = pack_bf16x2(src[2 * q], src[2 * q + 1]);
        *reinterpret_cast<su32x4_t*>(Y + (row0 + r) * GD + 8 * c8) = v;
    }
}

}  // namespace

static int num_segs(const mc_dims& d, int NS) { return NS ? NS : (d.L + d.seg_len - 1) / d.seg_len; }

bool ssc_gather_covers(const mc_dims& d, int top_k, int n_seg) {
    const int NS = num_segs(d, n_seg);
    return read_mfma_covers(d) && d.d_k == GD && d.d_v == GD && top_k >= 1 && top_k <= 16 &&
           NS <= GNS_MAX;
}

size_t ssc_frag_states_bytes(const mc_dims& d, int n_seg) {
    const int NS = num_segs(d, n_seg);
    return sizeof(uint16_t) * (size_t)d.B * d.H * NS * GD * GD;
}

static const SegArg kConstSegS{};  // constant segment length

int launch_ssc_gather(const mc_dims& d, int top_k, const void* Q, const uint16_t* M_lo,
                      const float* O_on, const SscRoute& rt, void* Y, void* stream,
                      const SegArg* sgp) {
    const SegArg& sg = sgp ? *sgp : kConstSegS;
    const int NS = num_segs(d, sg.n);
    if (!ssc_gather_covers(d, top_k, sg.n) || !rt.Sf) return (int)hipErrorInvalidValue;
    const int T = (d.L + GT - 1) / GT;
    const int BH = d.B * d.H;
    const size_t n16 = ssc_frag_states_bytes(d, sg.n) / 16;
    hipLaunchKernelGGL(frag_states_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, (const uint4*)M_lo, n16, (uint4*)rt.Sf);
    const dim3 grid(T * BH);
    if (d.phi)
        hipLaunchKernelGGL(ssc_gather_kernel<1>, grid, dim3(64 * NW), 0, (hipStream_t)stream,
                           (const bf16_t*)Q, (const uint4*)rt.Sf, O_on, rt.won, rt.ptok, rt.pw,
                           rt.poff, BH, d.L, d.seg_len, NS, top_k, (bf16_t*)Y, sg);
    else
        hipLaunchKernelGGL(ssc_gather_kernel<0>, grid, dim3(64 * NW), 0, (hipStream_t)stream,
                           (const bf16_t*)Q, (const uint4*)rt.Sf, O_on, rt.won, rt.ptok, rt.pw,
                           rt.poff, BH, d.L, d.seg_len, NS, top_k, (bf16_t*)Y, sg);
    return (int)hipGetLastError();
}

}  // namespace mc
