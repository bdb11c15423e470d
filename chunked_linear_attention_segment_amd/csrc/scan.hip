// scan.hip -- the MC write path: per-segment linear-attention scan, cached states, segment
// means and the ungated online read.
//
// Memory Caching paper §3, Eq. (4b): inside segment s the memory starts from zero and runs
// M_t = M_{t-1} + v_t phi(k_t)^T (the linear-attention update of §2, Eq. 2); the state after
// the segment's last token is cached.  The online read M_t^(s) phi(q_t) (§3.1, Eq. 6/8) is
// taken after token t has updated the memory.  MeanPooling(S^(i)) (§3.1, Eq. 10) averages X.
// With SWLA gates (the paper's sliding-window linear attention with window 2, Eq. 28) the
// update is M_t = alpha_t M_{t-1} + beta_t v_{t-1} phi(k_{t-1})^T + lam_t v_t phi(k_t)^T,
// the previous token taken only from the same segment.
#include "common.cuh"
#include "mc_internal.h"

namespace mc {

// One workgroup per (segment, b*H+h).  The d_v x d_k fp32 state lives in registers: thread
// `tid` owns row c = tid / TPR and the CPT consecutive columns starting at (tid % TPR) * CPT.
// Tokens are staged TT at a time in LDS (phi applied on load); each token updates the state
// and then reads it with phi(q_t) -- the read is reduced over the TPR threads of a row.
template <typename T, int DK, int DV, bool SW>
__global__ __launch_bounds__(256) void scan_valu_kernel(const T* __restrict__ Q,
                                                        const T* __restrict__ K,
                                                        const T* __restrict__ V, int L, int C,
                                                        int NS, int phi, float* __restrict__ M,
                                                        bf16_t* __restrict__ M_lo,
                                                        float* __restrict__ O_on,
                                                        const SegArg sg, SwlaGates gt) {
    constexpr int TPR = 256 / DV;
    constexpr int CPT = DK / TPR;
    constexpr int TT = 32;
    __shared__ float sk[TT][DK];
    __shared__ float sq[TT][DK];
    __shared__ float sv[TT][DV];
    __shared__ float sga[SW ? TT : 1], sgb[SW ? TT : 1], sgl[SW ? TT : 1];

    const int s = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int t0 = seg_first(sg, s, C);
    const int len = seg_length(sg, s, C, L);
    const int tid = threadIdx.x;
    const int c = tid / TPR;
    const int r0 = (tid % TPR) * CPT;

    float m[CPT];
    float kp[SW ? CPT : 1];  // SWLA: phi(k) and v of the previous token of the segment
    float vp = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) m[i] = 0.f;
#pragma unroll
    for (int i = 0; i < (SW ? CPT : 1); ++i) kp[i] = 0.f;

    const size_t kbase = (bh * L + t0) * DK;
    const size_t vbase = (bh * L + t0) * DV;
    for (int j0 = 0; j0 < len; j0 += TT) {
        const int n = min(TT, len - j0);
        __syncthreads();
        for (int e = tid; e < n * DK; e += 256) {
            sk[e / DK][e % DK] = feature(ld(K, kbase + (size_t)j0 * DK + e), phi);
            sq[e / DK][e % DK] = feature(ld(Q, kbase + (size_t)j0 * DK + e), phi);
        }
        for (int e = tid; e < n * DV; e += 256) sv[e / DV][e % DV] = ld(V, vbase + (size_t)j0 * DV + e);
        if (SW && tid < n) {
            const size_t gi = bh * L + t0 + j0 + tid;
            sga[tid] = gt.alpha[gi];
            sgb[tid] = gt.beta[gi];
            sgl[tid] = gt.lam[gi];
        }
        __syncthreads();
        for (int j = 0; j < n; ++j) {
            const float vc = sv[j][c];
            float acc = 0.f;
            if (SW) {
                // the segment's first token has no previous token: vp and kp are still zero
                const float al = sga[j], bv = sgb[j] * vp, lv = sgl[j] * vc;
#pragma unroll
                for (int i = 0; i < CPT; ++i) {
                    const float kc = sk[j][r0 + i];
                    m[i] = al * m[i] + bv * kp[i] + lv * kc;
                    kp[i] = kc;
                    acc += m[i] * sq[j][r0 + i];
                }
                vp = vc;
            } else {
#pragma unroll
                for (int i = 0; i < CPT; ++i) {
                    m[i] += vc * sk[j][r0 + i];
                    acc += m[i] * sq[j][r0 + i];
                }
            }
            acc = warp_sum(acc, TPR);
            if (O_on && tid % TPR == 0) O_on[(bh * L + t0 + j0 + j) * DV + c] = acc;
        }
    }
    const size_t mo = (bh * NS + s) * (size_t)(DV * DK) + (size_t)c * DK + r0;
    if (M) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) M[mo + i] = m[i];
    }
    if (M_lo) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) M_lo[mo + i] = f32_to_bf16(m[i]);
    }
}

// MeanPooling(S^(i)) = mean of X over segment i (a trailing partial segment averages the
// tokens it has).  One workgroup per (segment, b*xh+hx): 256 threads = 16 token lanes x 16
// column groups of 8; each thread sums its column group over every 16th token (16-byte
// loads), then the 16 token lanes are combined in a fixed order through LDS.
template <typename T>
__global__ __launch_bounds__(256) void seg_means_kernel(const T* __restrict__ X, int L, int C,
                                                        int NS, int DG, float* __restrict__ P,
                                                        const SegArg sg) {
    __shared__ float part[16][257];
    const int s = blockIdx.x;
    const size_t bx = blockIdx.y;
    const int t0 = seg_first(sg, s, C);
    const int len = seg_length(sg, s, C, L);
    const int tl = threadIdx.x / 16, cg = threadIdx.x % 16;
    for (int e0 = cg * 8; e0 < DG; e0 += 128) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        int j = tl;
        for (; j + 48 < len; j += 64) {  // four rows in flight per thread
            float v0[8], v1[8], v2[8], v3[8];
            ld8(X, (bx * L + t0 + j) * DG + e0, v0);
            ld8(X, (bx * L + t0 + j + 16) * DG + e0, v1);
            ld8(X, (bx * L + t0 + j + 32) * DG + e0, v2);
            ld8(X, (bx * L + t0 + j + 48) * DG + e0, v3);
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] += ((v0[k] + v1[k]) + (v2[k] + v3[k]));
        }
        for (; j < len; j += 16) {
            float v[8];
            ld8(X, (bx * L + t0 + j) * DG + e0, v);
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] += v[k];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) part[tl][e0 + k] = acc[k];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < DG; e += 256) {
        float acc = 0.f;
        for (int r = 0; r < 16; ++r) acc += part[r][e];
        P[(bx * NS + s) * DG + e] = acc / (float)len;
    }
}

static const SegArg kConstSeg{};  // constant segment length

static const SwlaGates kNoGates{};

template <typename T, int DK, int DV>
static int launch_scan_t(const mc_dims& d, const void* Q, const void* K, const void* V,
                         float* M, uint16_t* M_lo, float* O_on, const SegArg& sg,
                         const SwlaGates& gt, hipStream_t st) {
    const int NS = sg.n ? sg.n : (d.L + d.seg_len - 1) / d.seg_len;
    dim3 grid(NS, d.B * d.H);
    if (gt.alpha)
        hipLaunchKernelGGL((scan_valu_kernel<T, DK, DV, true>), grid, dim3(256), 0, st,
                           (const T*)Q, (const T*)K, (const T*)V, d.L, d.seg_len, NS, d.phi, M,
                           (bf16_t*)M_lo, O_on, sg, gt);
    else
        hipLaunchKernelGGL((scan_valu_kernel<T, DK, DV, false>), grid, dim3(256), 0, st,
                           (const T*)Q, (const T*)K, (const T*)V, d.L, d.seg_len, NS, d.phi, M,
                           (bf16_t*)M_lo, O_on, sg, gt);
    return (int)hipGetLastError();
}

template <typename T>
static int launch_scan_dt(const mc_dims& d, const void* Q, const void* K, const void* V,
                          float* M, uint16_t* M_lo, float* O_on, const SegArg& sg,
                          hipStream_t st, const SwlaGates& gt = kNoGates) {
    if (d.d_k == 128 && d.d_v == 128) return launch_scan_t<T, 128, 128>(d, Q, K, V, M, M_lo, O_on, sg, gt, st);
    if (d.d_k == 128 && d.d_v == 64) return launch_scan_t<T, 128, 64>(d, Q, K, V, M, M_lo, O_on, sg, gt, st);
    if (d.d_k == 64 && d.d_v == 128) return launch_scan_t<T, 64, 128>(d, Q, K, V, M, M_lo, O_on, sg, gt, st);
    return launch_scan_t<T, 64, 64>(d, Q, K, V, M, M_lo, O_on, sg, gt, st);
}

int launch_scan_online(const mc_dims& d, const void* Q, const void* K, const void* V,
                       float* O_on, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    return d.dtype == MC_BF16
               ? launch_scan_dt<bf16_t>(d, Q, K, V, nullptr, nullptr, O_on, kConstSeg, st)
               : launch_scan_dt<float>(d, Q, K, V, nullptr, nullptr, O_on, kConstSeg, st);
}

template <typename T>
static int launch_means(const mc_dims& d, const void* X, float* P, const SegArg& sg,
                        hipStream_t st) {
    const int NS = sg.n ? sg.n : (d.L + d.seg_len - 1) / d.seg_len;
    hipLaunchKernelGGL(seg_means_kernel<T>, dim3(NS, d.B * d.x_heads), dim3(256), 0, st,
                       (const T*)X, d.L, d.seg_len, NS, d.d_g, P, sg);
    return (int)hipGetLastError();
}

int launch_scan_mfma_segs(const mc_dims& d, const SegArg& sg, const void* Q, const void* K,
                          const void* V, float* M, uint16_t* M_lo, float* O_on, void* stream,
                          const float* M0 = nullptr);

__device__ __forceinline__ bool piece_first(const PieceArg& pa, int j) {
    return (pa.first[j >> 5] >> (j & 31)) & 1u;
}

// The first piece of segment s (the (s+1)-th set bit of the first-piece table), and one past
// the last piece of the segment that starts at piece j.
__device__ __forceinline__ int segment_first_piece(const PieceArg& pa, int s) {
    for (int w = 0;; ++w) {
        uint32_t bits = pa.first[w];
        const int c = __popc(bits);
        if (s < c) {
            for (; s > 0; --s) bits &= bits - 1u;  // drop the lower set bits
            return 32 * w + __ffs(bits) - 1;
        }
        s -= c;
    }
}
__device__ __forceinline__ int piece_end(const PieceArg& pa, int j, int NP) {
    int e = j + 1;
    while (e < NP && !piece_first(pa, e)) ++e;
    return e;
}

// Prefix sums of the piece states inside each segment: the memory restarts only at a
// segment start (Eq. 4b), so the memory before piece j is the sum of the earlier pieces of
// its segment (Pref_j, zero for a segment's first piece) and the segment's state is the sum
// of all of them.  One workgroup per (segment, b*H+h, 512-element slice of the d_v x d_k
// state) walks the segment's pieces in order, sixteen pieces at a time: every load of a batch
// is issued before the first sum (rows past the segment's last piece are read clamped to it
// and not used).  The segment is the slowest grid index, so the workgroups of the first
// segments, which walk the most pieces when the segments shrink along the sequence, are
// dispatched first.  Pref (fp32, for the online scan) and Pref_lo (bf16, for a read that
// forms the online term itself) are each written when given; so is pfirst[s], the index of
// segment s's first piece.
template <int DK, int DV>
__global__ __launch_bounds__(128) void piece_prefix_kernel(const float* __restrict__ Msub,
                                                           int NP, const PieceArg pa, int NS,
                                                           float* __restrict__ Pref,
                                                           float* __restrict__ M,
                                                           bf16_t* __restrict__ M_lo,
                                                           bf16_t* __restrict__ Pref_lo,
                                                           int32_t* __restrict__ pfirst) {
    constexpr int N = DV * DK;
    constexpr int BATCH = 16;
    const int seg = blockIdx.z;  // slowest: the longest segments (the first) start first
    const int j = segment_first_piece(pa, seg);
    const size_t bh = blockIdx.y;
    const int e0 = blockIdx.x * 512 + 4 * threadIdx.x;
    const int jend = piece_end(pa, j, NP);
    if (pfirst && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) pfirst[seg] = j;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int b = j; b < jend; b += BATCH) {
        float4 v[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
            v[i] = *reinterpret_cast<const float4*>(Msub + (bh * NP + min(b + i, jend - 1)) * (size_t)N + e0);
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
            if (b + i < jend) {
                if (Pref)
                    *reinterpret_cast<float4*>(Pref + (bh * NP + b + i) * (size_t)N + e0) = acc;
                if (Pref_lo) {
                    uint2 a;
                    a.x = pack_bf16x2(acc.x, acc.y);
                    a.y = pack_bf16x2(acc.z, acc.w);
                    *reinterpret_cast<uint2*>(Pref_lo + (bh * NP + b + i) * (size_t)N + e0) = a;
                }
                acc.x += v[i].x;
                acc.y += v[i].y;
                acc.z += v[i].z;
                acc.w += v[i].w;
            }
    }
    *reinterpret_cast<float4*>(M + (bh * NS + seg) * (size_t)N + e0) = acc;
    uint2 lo;
    lo.x = pack_bf16x2(acc.x, acc.y);
    lo.y = pack_bf16x2(acc.z, acc.w);
    *reinterpret_cast<uint2*>(M_lo + (bh * NS + seg) * (size_t)N + e0) = lo;
}

// Segment means from the means of its pieces (P_s = sum over the segment's pieces, in order, of
// length x mean, over the segment's length).  One workgroup per (segment, b*x_heads).
__global__ __launch_bounds__(256) void piece_means_kernel(const float* __restrict__ Pm, int NP,
                                                          const PieceArg pa, int NS, int DG,
                                                          float* __restrict__ P) {
    const int seg = blockIdx.x;
    const int j = segment_first_piece(pa, seg);
    const size_t bx = blockIdx.y;
    const int jend = piece_end(pa, j, NP);
    const float inv_len = 1.f / (float)(pa.sg.off[jend] - pa.sg.off[j]);
    for (int e = threadIdx.x; e < DG; e += 256) {
        float acc = 0.f;
        for (int q0 = j; q0 < jend; q0 += 8) {  // eight pieces' loads in flight, summed in order
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = Pm[(bx * NP + min(q0 + u, jend - 1)) * DG + e];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (q0 + u < jend)
                    acc += v[u] * (float)(pa.sg.off[q0 + u + 1] - pa.sg.off[q0 + u]);
        }
        P[(bx * NS + seg) * DG + e] = acc * inv_len;
    }
}

int scan_piece_len(int L, int n_seg, int pl_min) {
    for (int pl = pl_min; pl > 0 && pl <= (1 << 30); pl <<= 1)
        if (n_seg + (L + pl - 1) / pl <= MC_MAX_SEGS) return pl;
    return 0;
}

// two fp32 state arrays (pieces, prefix sums) and the pieces' means of X, for at most
// n_seg + ceil(L / piece) pieces; only the bf16 MFMA scan splits segments
static size_t segs_state_bytes(const mc_dims& d, size_t np) {
    return align256(sizeof(float) * (size_t)d.B * d.H * np * d.d_v * d.d_k);
}
size_t segs_scan_ws_bytes(const mc_dims& d, int n_seg, int pl_min) {
    const bool mfma = d.dtype == MC_BF16 && (d.d_k == 64 || d.d_k == 128) &&
                      (d.d_v == 64 || d.d_v == 128);
    const int pl = scan_piece_len(d.L, n_seg, pl_min);
    if (!mfma || !pl) return 0;
    const size_t np = (size_t)n_seg + (d.L + pl - 1) / pl;
    return 2 * segs_state_bytes(d, np) +
           align256(sizeof(float) * (size_t)d.B * d.x_heads * np * d.d_g);
}

size_t segs_pref_lo_bytes(const mc_dims& d, int n_seg, int pl_min) {
    const int pl = scan_piece_len(d.L, n_seg, pl_min);
    if (!pl) return 0;
    const size_t np = (size_t)n_seg + (d.L + pl - 1) / pl;
    return align256(sizeof(uint16_t) * (size_t)d.B * d.H * np * d.d_v * d.d_k);
}

template <int DK, int DV>
static int launch_pieces_t(const mc_dims& d, const PieceArg& pa, int NS, float* Msub,
                           float* Pref, float* M, uint16_t* M_lo, uint16_t* Pref_lo,
                           int32_t* pfirst, hipStream_t st) {
    const int NP = pa.sg.n;
    static_assert(DV * DK % 512 == 0, "512-element slices");
    hipLaunchKernelGGL((piece_prefix_kernel<DK, DV>), dim3(DV * DK / 512, d.B * d.H, NS),
                       dim3(128), 0, st, Msub, NP, pa, NS, Pref, M, (bf16_t*)M_lo,
                       (bf16_t*)Pref_lo, pfirst);
    return (int)hipGetLastError();
}

// Arbitrary boundaries: the MFMA scan for bf16 widths 64/128 (segments longer than a piece
// split into pieces scanned in parallel, then combined), else the generic scan (any dtype);
// then the means over each segment (split: over the pieces, then combined per segment).
int launch_scan_prefill_segs(const mc_dims& d, const SegArg& sg, const void* Q, const void* K,
                             const void* V, const void* X, float* M, uint16_t* M_lo, float* P,
                             float* O_on, void* ws, size_t ws_bytes, void* stream,
                             PieceOnline* pon, uint16_t* pref_lo, int32_t* pfirst, int pl_min) {
    hipStream_t st = (hipStream_t)stream;
    int rc = -1;
    const int pl = scan_piece_len(d.L, sg.n, pl_min);
    bool split = false;
    for (int i = 0; pl && i < sg.n; ++i) split |= sg.off[i + 1] - sg.off[i] > pl;
    const size_t need = segs_scan_ws_bytes(d, sg.n, pl_min);
    PieceArg piece{};
    float* Pm = nullptr;  // the pieces' means of X, when the scan ran over pieces
    if (split && need && ws && ws_bytes >= need) {
        int np = 0;
        for (int i = 0; i < sg.n; ++i)
            for (int a = sg.off[i]; a < sg.off[i + 1]; a += pl) {
                if (a == sg.off[i]) piece.first[np >> 5] |= 1u << (np & 31);
                piece.sg.off[np++] = a;
            }
        piece.sg.off[np] = d.L;
        piece.sg.n = np;
        // the pieces' own states; their prefix sums per segment (and the segments' states);
        // then, for the online read, the pieces again from the memory before each
        const size_t sb = segs_state_bytes(d, (size_t)sg.n + (d.L + pl - 1) / pl);
        float* Msub = (float*)ws;
        float* Pref = (float*)((char*)ws + sb);
        rc = launch_scan_mfma_segs(d, piece.sg, Q, K, V, Msub, nullptr, nullptr, stream);
        if (rc >= 0) {
            if (rc) return rc;
            // the fp32 memory before each piece for the online scan, or its bf16 copy for a
            // read that forms the online term itself
            float* pr = O_on ? Pref : nullptr;
            uint16_t* pl16 = pon ? pref_lo : nullptr;
            int32_t* pf = pon ? pfirst : nullptr;
            if (d.d_k == 128 && d.d_v == 128)
                rc = launch_pieces_t<128, 128>(d, piece, sg.n, Msub, pr, M, M_lo, pl16, pf, st);
            else if (d.d_k == 128)
                rc = launch_pieces_t<128, 64>(d, piece, sg.n, Msub, pr, M, M_lo, pl16, pf, st);
            else if (d.d_v == 128)
                rc = launch_pieces_t<64, 128>(d, piece, sg.n, Msub, pr, M, M_lo, pl16, pf, st);
            else
                rc = launch_pieces_t<64, 64>(d, piece, sg.n, Msub, pr, M, M_lo, pl16, pf, st);
            if (!rc && pon) {
                pon->M0 = pref_lo;
                pon->pfirst = pfirst;
                pon->PL = pl;
                pon->NP = np;
            }
            if (!rc && O_on)
                rc = launch_scan_mfma_segs(d, piece.sg, Q, K, V, nullptr, nullptr, O_on, stream,
                                           Pref);
            if (!rc) Pm = (float*)((char*)ws + 2 * sb);
        }
    }
    if (rc < 0) rc = launch_scan_mfma_segs(d, sg, Q, K, V, M, M_lo, O_on, stream);
    if (rc < 0)
        rc = d.dtype == MC_BF16 ? launch_scan_dt<bf16_t>(d, Q, K, V, M, M_lo, O_on, sg, st)
                                : launch_scan_dt<float>(d, Q, K, V, M, M_lo, O_on, sg, st);
    if (rc) return rc;
    if (Pm) {  // bf16 (the pieced scan is the MFMA one)
        if ((rc = launch_means<bf16_t>(d, X, Pm, piece.sg, st))) return rc;
        hipLaunchKernelGGL(piece_means_kernel, dim3(sg.n, d.B * d.x_heads), dim3(256), 0,
                           st, Pm, piece.sg.n, piece, sg.n, d.d_g, P);
        return (int)hipGetLastError();
    }
    return d.dtype == MC_BF16 ? launch_means<bf16_t>(d, X, P, sg, st)
                              : launch_means<float>(d, X, P, sg, st);
}

int launch_scan_mfma(const mc_dims& d, const void* Q, const void* K, const void* V, float* M,
                     uint16_t* M_lo, float* O_on, const SwlaGates& gt, void* stream,
                     const SegArg* sg = nullptr);

// SWLA write path: the MFMA scan for bf16 widths 64/128 (constant segments or offsets), the
// generic scan otherwise, then the means.
int launch_scan_prefill_swla(const mc_dims& d, const SegArg& sg, const SwlaGates& gt,
                             const void* Q, const void* K, const void* V, const void* X,
                             float* M, uint16_t* M_lo, float* P, float* O_on, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    int rc = -1;
    if (d.dtype == MC_BF16) rc = launch_scan_mfma(d, Q, K, V, M, M_lo, O_on, gt, stream, &sg);
    if (rc >= 0) {
        if (rc) return rc;
    } else if (d.dtype == MC_BF16)
        rc = launch_scan_dt<bf16_t>(d, Q, K, V, M, M_lo, O_on, sg, st, gt);
    else
        rc = launch_scan_dt<float>(d, Q, K, V, M, M_lo, O_on, sg, st, gt);
    if (rc) return rc;
    return d.dtype == MC_BF16 ? launch_means<bf16_t>(d, X, P, sg, st)
                              : launch_means<float>(d, X, P, sg, st);
}

int launch_scan_prefill(const mc_dims& d, const void* Q, const void* K, const void* V,
                        const void* X, float* M, uint16_t* M_lo, float* P, float* O_on,
                        void* stream) {
    hipStream_t st = (hipStream_t)stream;
    int rc = -1;
    if (d.dtype == MC_BF16) rc = launch_scan_mfma(d, Q, K, V, M, M_lo, O_on, kNoGates, stream);
    if (rc >= 0) {
        if (rc) return rc;
    } else if (d.dtype == MC_BF16)
        rc = launch_scan_dt<bf16_t>(d, Q, K, V, M, M_lo, O_on, kConstSeg, st);
    else
        rc = launch_scan_dt<float>(d, Q, K, V, M, M_lo, O_on, kConstSeg, st);
    if (rc) return rc;
    return d.dtype == MC_BF16 ? launch_means<bf16_t>(d, X, P, kConstSeg, st)
                              : launch_means<float>(d, X, P, kConstSeg, st);
}

}  // namespace mc
