// mc_internal.h -- launchers shared between the ABI layer (abi.cpp) and the HIP kernels.
// Every launcher enqueues on `stream` and returns the hipError_t of its launches as int.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/mc.h"

namespace mc {

// Byte sizes of the workspace regions, in the order they are carved out of `ws`.
struct GrmWorkspace {
    size_t aon;   // fp32 [B,H,L]: online gate logit <u_t, prefix mean of X> (generic kernels)
    size_t on;    // fp32 [B,H,L,dv]: online read, for the generic kernels when O_on is NULL
    size_t xps;   // fp32 [B,xh,L,dg]: segment-causal prefix sums of X (MFMA read)
    size_t w;     // bf16 [B,H,T,NS,kGateTile]: gate numerators per read tile (gate pass)
    size_t won;   // fp32 [B,H,L]: online weight exp(a_on - m) (gate pass)
    size_t inv_l; // fp32 [B,H,L]: 1 / softmax denominator (gate pass)
    size_t pf;    // the means as MFMA fragments (gate pass)
    size_t total;
};

// The gate pass (gate.hip) writes the softmax numerators per read tile of kGateTile tokens;
// the gated read then only loads them.  Used for d_k = d_v = 128 bf16 GRM while the
// numerators fit kGateMaxBytes (longer sequences keep the gate inside the read).
constexpr int kGateTile = 256;
constexpr size_t kGateMaxBytes = size_t(4) << 30;
// the gate as its own pass (bf16, d_k = d_v = 128) for NS segments (0: the constant length's)
bool gate_pass(const mc_dims& d, int NS = 0);
struct GateWeights {
    const uint16_t* W = nullptr;   // null: the read computes the gate itself
    const float* won = nullptr;
    const float* inv_l = nullptr;
};
size_t gate_pfrag_bytes(const mc_dims& d, int NS = 0);  // the means as MFMA fragments (bf16 high + rest)
// idx (with top_k) given: the SSC gate, every logit but the token's selected segments and the
// online one masked out
struct SegArg;
int launch_gate_w(const mc_dims& d, const void* U, const float* xps, const float* P,
                  void* pfrag, uint16_t* W, float* won, float* inv_l, void* stream,
                  const int32_t* idx = nullptr, int top_k = 0, const SegArg* sg = nullptr);
struct SscWorkspace {
    size_t aon;    // fp32 [B,H,L] (generic kernels)
    size_t on;     // fp32 [B,H,L,dv] (generic kernels only)
    size_t xps;    // fp32 [B,xh,L,dg] (MFMA read)
    size_t xsum64; // fp64 [B,xh,dg,NS rounded up to 16]: segment means of X (ssc_means_bytes)
    size_t w, won, inv_l, pf;  // the gate pass (as GrmWorkspace), masked to the selections
    size_t ptok, pw, poff, sf;  // the routed read: the tiles' pairs by segment, fragment-order states
    size_t total;
};
// Decode: each (b, h) has one partial softmax for the online segment and one per run of
// kDecodeRun cached states (one workgroup each: many short runs keep every compute unit
// streaming to the end of the launch); `slots` = 1 + runs at n_cached = n_cap.
constexpr int kDecodeRun = 8;
struct DecodeWorkspace {
    size_t partial;  // fp32 [B,H,slots,dv]: unnormalised reads of the runs
    size_t ml;       // fp32 [B,H,slots,2]: max logit and sum of exp of each run
    size_t total;
    int slots;
};

// n_seg > 0: sized for that many segment offsets (the gate pass's buffers included when they
// fit), else for the constant segment length
GrmWorkspace grm_workspace(const mc_dims& d, int n_seg = 0);
// n_seg > 0: for that many segment offsets (the online read is the caller's, the read is the
// routed one or the generic kernels)
SscWorkspace ssc_workspace(const mc_dims& d, int top_k, int n_seg = 0);
DecodeWorkspace decode_workspace(const mc_dims& d, int n_cap, int n_cached);

inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Segment boundaries for the generic kernels, passed to them by value: n = 0 means constant
// length C; otherwise segment i is [off[i], off[i+1]) for i < n.
struct SegArg {
    int32_t n;
    int32_t off[MC_MAX_SEGS + 1];
};

// SWLA gates ([B,H,L] fp32 each, device): alpha == nullptr means the linear-attention update.
struct SwlaGates {
    const float* alpha = nullptr;
    const float* beta = nullptr;
    const float* lam = nullptr;
};
int launch_scan_prefill_swla(const mc_dims& d, const SegArg& sg, const SwlaGates& gt,
                             const void* Q, const void* K, const void* V, const void* X,
                             float* M, uint16_t* M_lo, float* P, float* O_on, void* stream);

// Backward of the GRM prefill (backward.hip): device buffers carved from the workspace.
struct BwdBuffers {
    float* aon;    // [B,H,L] online logits
    float* xps;    // [B,xh,L,dg] segment-causal prefix sums of X
    float* xtail;  // their per-chunk partial sums
    float* on;     // [B,H,L,dv] online read M_t^(s) phi(q_t) (MFMA path: [B,H,L] <dy_t, it>)
    float* ot;     // [B,H,L,dk] M_t^(s)T dy_t
    void* khat;    // [B,H,L,dk] phi(K) in the input dtype (elu + 1 only)
    float* lse;    // [B,H,L] log of the softmax denominator
    float* D;      // [B,H,L] sum_i gamma_i dgamma_i
    float* gs;     // [B,H,L] online weight gamma_s
    float* dG;     // [B,H,L,NS] dgamma, then da (MFMA path: [B,H,L] da of the online segment)
    float* dM;     // [B,H,NS,dv,dk] gradient of each cached state ([B,H,NS,dk,dv] on MFMA)
    float* dpp;    // [NR,NS,B*xh,dg] partial sums of dP_i over token ranges
    // the MFMA path (bf16, d_k = d_v = 128 with the forward gate pass):
    uint16_t* W;   // gate numerators per read tile (gate pass layout)
    float* won;    // [B,H,L] online numerator
    float* inv_l;  // [B,H,L] 1 / softmax denominator
    void* pf;      // the means as MFMA fragments
    void* mt;      // [B,H,NS,dk,dv] bf16 transposed states
    void* dqh;     // [B,H,L,dk] bf16 dphi(q) from the swapped read
    float* daT;    // [B,H,NS,L] dgamma_t^(i), then da_t^(i), segment-major
    void* ptf;     // the means as B fragments of the du product
};
struct BwdWorkspace {
    size_t aon, xps, xtail, on, ot, khat, lse, D, gs, dG, dM, dpp;
    size_t W, won, inv_l, pf, mt, dqh, daT, ptf, total;
};
// The MFMA backward applies where the forward uses the gate pass (bf16, d_k = d_v = 128).
inline bool bwd_fast(const mc_dims& d) { return gate_pass(d); }
int launch_bwd_fast(const mc_dims& d, const BwdBuffers& w, const void* Q, const void* K,
                    const void* V, const void* U, const float* M, const uint16_t* M_lo,
                    const float* P, const void* dY, float* dQ, float* dU, void* stream);
// dgamma_t^(i) = <dy_t, M^(i) phi(q_t)> (bf16, d_k = d_v = 128), segment-major [B,H,NS,L]
int launch_bwd_dgamma(const mc_dims& d, const void* Q, const void* dY, const uint16_t* M_lo,
                      float* dGT, void* stream);
// the online segment's dK and dV for the MFMA backward (dM stored transposed)
int launch_bwd_online_mfma(const mc_dims& d, const BwdBuffers& w, const void* Q, const void* K,
                           const void* V, const void* dY, float* dK, float* dV, void* stream);
// tokens per range of the dP partial sums: a multiple of 64, at most 64 ranges
inline int bwd_dp_range(int L) {
    const int r = (L + 63) / 64;
    return (r + 63) / 64 * 64;
}
BwdWorkspace bwd_workspace(const mc_dims& d);
int launch_scan_mfma_online(const mc_dims& d, const void* Q, const void* K, const void* V,
                            float* O_on, void* stream);
// dgs[t] = <dy_t, O_on[t]> ([B,H,L]) from the online read, which is not stored
int launch_scan_mfma_dgs(const mc_dims& d, const void* Q, const void* K, const void* V,
                         const void* dY, float* dgs, void* stream);
int launch_grm_backward(const mc_dims& d, const BwdBuffers& w, const void* Q, const void* K,
                        const void* V, const void* U, const void* X, const float* M,
                        const uint16_t* M_lo, const float* P, const void* dY, float* dQ,
                        float* dK, float* dV, float* dU, float* dX, void* stream);

// The online term of a read over segment offsets formed in the read from K and V, with long
// segments cut into pieces of PL tokens from each segment's start: the read walks a token's
// piece up to the token and adds M0 of the piece, the memory of the segment's earlier pieces
// (bf16 [B*H][NP][d_v][d_k]; a segment's first piece has none and its entry is not read);
// pfirst[s] is the index of segment s's first piece.  PL >= L: no segment is cut.
struct PieceOnline {
    const uint16_t* M0 = nullptr;
    const int32_t* pfirst = nullptr;
    int PL = 1 << 30;
    int NP = 0;
};

// Long segments of the offsets scan are cut into pieces (at most scan_piece_len tokens, each
// inside one segment) that are scanned in parallel; `first` marks the pieces that start a
// segment.  The pieces' states and their prefix sums within a segment take workspace.
struct PieceArg {
    SegArg sg;
    uint32_t first[(MC_MAX_SEGS + 32) / 32];
};
// pieces of at least pl_min tokens (a power of two)
int scan_piece_len(int L, int n_seg, int pl_min = 512);  // 0: no piece table fits MC_MAX_SEGS
size_t segs_scan_ws_bytes(const mc_dims& d, int n_seg, int pl_min = 512);
// pon given (with O_on NULL): the bf16 memory before each piece goes to pref_lo (half of a
// state array of the pieces) and the first-piece table to pfirst (n_seg entries), and pon is
// filled for the read; left as it is when no segment is cut.
int launch_scan_prefill_segs(const mc_dims& d, const SegArg& sg, const void* Q, const void* K,
                             const void* V, const void* X, float* M, uint16_t* M_lo, float* P,
                             float* O_on, void* ws, size_t ws_bytes, void* stream,
                             PieceOnline* pon = nullptr, uint16_t* pref_lo = nullptr,
                             int32_t* pfirst = nullptr, int pl_min = 512);
// the bf16 memories before the pieces (launch_scan_prefill_segs with pon)
size_t segs_pref_lo_bytes(const mc_dims& d, int n_seg, int pl_min = 512);
// xps / xtail (nullable: the per-segment walk of aon_kernel is used instead) are workspace for
// the segment-causal prefix sums of X.
// the gate pass's buffers for a read with segment offsets (W == nullptr: the in-kernel gate)
struct SegGate {
    uint16_t* W = nullptr;
    float* won = nullptr;
    float* inv_l = nullptr;
    void* pf = nullptr;
};
int launch_grm_readout_segs(const mc_dims& d, const SegArg& sg, const void* Q, const void* U,
                            const void* X, const float* M, const uint16_t* M_lo, const float* P,
                            const float* O_on, float* aon, float* xps, float* xtail, void* Y,
                            float* gamma, void* stream, const SegGate& gate = SegGate{},
                            const void* K = nullptr, const void* V = nullptr,
                            const PieceOnline* pon = nullptr);

int launch_scan_prefill(const mc_dims& d, const void* Q, const void* K, const void* V,
                        const void* X, float* M, uint16_t* M_lo, float* P, float* O_on,
                        void* stream);

// The online read M_t^(s) phi(q_t) alone (generic fp32-accumulating kernel), into O_on.
int launch_scan_online(const mc_dims& d, const void* Q, const void* K, const void* V,
                       float* O_on, void* stream);

int launch_aon(const mc_dims& d, const void* X, const void* U, float* a_on, void* stream);

// xps[b, xh, t, :] = sum of X over t's segment from its first token up to t (fp32); `tails`
// holds xps_tail_floats(d) floats of per-chunk partial sums
size_t xps_tail_floats(const mc_dims& d);
int launch_xps(const mc_dims& d, const void* X, float* xps, float* tails, void* stream);

// true when the bf16 MFMA read kernel handles these sizes (given K and V instead of O_on it
// forms the online term and the online logit itself); otherwise the generic kernels run and
// need O_on and a_on
bool read_mfma_covers(const mc_dims& d);

// The MFMA read forms the online logit itself from xps (launch_xps); the generic kernels
// and the optional gamma output use a_on (launch_aon).
bool read_mfma_ssc_covers(const mc_dims& d, bool online_given);
int launch_read_mfma(const mc_dims& d, bool ssc, int top_k, const void* Q, const void* K,
                     const void* V, const void* U, const float* xps, const uint16_t* M_lo,
                     const float* P, const float* O_on, const int32_t* idx,
                     const GateWeights& gw, void* Y, void* stream,
                     const SegArg* sg = nullptr, const PieceOnline* pon = nullptr);

int launch_grm_readout(const mc_dims& d, const void* Q, const void* K, const void* V,
                       const void* U, const float* aon, const float* xps, const float* M,
                       const uint16_t* M_lo, const float* P, const float* O_on,
                       const GateWeights& gw, void* Y, float* gamma, void* stream);

// Outputs of the selection for the routed SSC read (launch_ssc_gather): the normalised online
// weight per token, and per read tile of kSscTile tokens the (token, selected segment) pairs
// sorted by segment with their normalised weights, and each segment's start in that list.
constexpr int kSscTile = 256;
struct SscRoute {
    const float* aon;  // [B, H, L] the online logits (input, launch_aon)
    float* won;        // [B, H, L]
    int32_t* ptok;     // [B*H, T, kSscTile * top_k] tile-local token numbers
    float* pw;         // [B*H, T, kSscTile * top_k]
    int32_t* poff;     // [B*H, T, NS + 1]
    void* Sf;          // the states in MFMA fragment order (ssc_frag_states_bytes)
};
// n_seg (or sg->n) = 0 below: segments of the constant length
size_t ssc_frag_states_bytes(const mc_dims& d, int n_seg = 0);
int launch_ssc_select(const mc_dims& d, int top_k, const void* U, const void* X,
                      double* xsum64, int32_t* idx, void* stream,
                      const SscRoute* route = nullptr, const SegArg* sg = nullptr);
size_t ssc_means_bytes(const mc_dims& d, int n_seg = 0);
// the routed SSC read: per tile, only the selected segments' states, each applied to the
// tokens that chose it; y = won * O_on + sum of pw * S^T phi(q) (bf16, d_k = d_v = 128)
bool ssc_gather_covers(const mc_dims& d, int top_k, int n_seg = 0);
int launch_ssc_gather(const mc_dims& d, int top_k, const void* Q, const uint16_t* M_lo,
                      const float* O_on, const SscRoute& rt, void* Y, void* stream,
                      const SegArg* sg = nullptr);
// segment offsets: the online logits, and the generic read restricted to idx
// (xps given: through the segment-causal prefix sums of X, tails as for launch_xps, else one
// workgroup walks each segment)
int launch_aon_segs(const mc_dims& d, const SegArg& sg, const void* X, const void* U,
                    float* a_on, void* stream, float* xps = nullptr, float* tails = nullptr);
int launch_ssc_readout_segs(const mc_dims& d, const SegArg& sg, int top_k, const void* Q,
                            const void* U, const float* aon, const float* M,
                            const uint16_t* M_lo, const float* P, const float* O_on,
                            const int32_t* idx, void* Y, void* stream);

int launch_ssc_readout(const mc_dims& d, int top_k, const void* Q, const void* K,
                       const void* V, const void* U, const float* aon, const float* xps,
                       const float* M,
                       const uint16_t* M_lo, const float* P, const float* O_on,
                       const int32_t* idx, void* Y, void* stream);

// ws is laid out for a cache of ws_cap states (decode_workspace(d, ws_cap, .)); ws_cap >=
// n_cached.  The workspace entry point passes n_cap, the scratch entry point n_cached.
int launch_decode_step(const mc_dims& d, const void* q, const void* k, const void* v,
                       const void* u, const void* x, float* M_on, float* xsum_on,
                       int count_on, void* M_cache, float* P_cache, int n_cached, int n_cap,
                       int emit, void* y, void* ws, int ws_cap, void* stream);
// Device address of the fixed decode scratch (MC_NOALLOC_SCRATCH_BYTES) on the current
// device, taken with hipGetSymbolAddress on the first call per device.  Returns a hipError_t.
int noalloc_scratch(void** out);

}  // namespace mc
