// abi.cpp -- the C ABI of libmc: argument validation, workspace sizing and dispatch.
//
// Validation runs before any HIP call, so every error path is observable without a GPU.
// The operations themselves are documented in include/mc.h.
#include <stdint.h>
#include <string.h>

#include "mc_internal.h"

namespace mc {

static int num_segments(const mc_dims& d) { return (d.L + d.seg_len - 1) / d.seg_len; }

static size_t online_ws(const mc_dims& d) {
    return read_mfma_covers(d) ? 0 : align256(sizeof(float) * (size_t)d.B * d.H * d.L * d.d_v);
}

// prefix sums of X for the MFMA read, then the per-chunk partial sums that form them
static size_t xps_only(const mc_dims& d) {
    return align256(sizeof(float) * (size_t)d.B * d.x_heads * d.L * d.d_g);
}
static size_t xps_ws(const mc_dims& d) {
    return read_mfma_covers(d) ? xps_only(d) + align256(sizeof(float) * xps_tail_floats(d)) : 0;
}

// the gate pass's numerators for NS segments (NS = 0: the constant segment length's count)
static size_t gate_w_bytes(const mc_dims& d, int NS = 0) {
    const size_t T = ((size_t)d.L + kGateTile - 1) / kGateTile;
    return sizeof(uint16_t) * (size_t)d.B * d.H * T * (NS ? NS : num_segments(d)) * kGateTile;
}

bool gate_pass(const mc_dims& d, int NS) {
    return read_mfma_covers(d) && d.d_k == 128 && d.d_v == 128 &&
           gate_w_bytes(d, NS) <= kGateMaxBytes;
}

GrmWorkspace grm_workspace(const mc_dims& d, int n_seg) {
    GrmWorkspace w{};
    w.aon = align256(sizeof(float) * (size_t)d.B * d.H * d.L);
    w.on = online_ws(d);
    w.xps = xps_ws(d);
    if (gate_pass(d, n_seg)) {
        w.w = align256(gate_w_bytes(d, n_seg));
        w.won = align256(sizeof(float) * (size_t)d.B * d.H * d.L);
        w.inv_l = w.won;
        w.pf = align256(gate_pfrag_bytes(d, n_seg));
    }
    w.total = w.aon + w.on + w.xps + w.w + w.won + w.inv_l + w.pf;
    return w;
}

SscWorkspace ssc_workspace(const mc_dims& d, int top_k, int n_seg) {
    SscWorkspace w{};
    const size_t bhl = (size_t)d.B * d.H * d.L;
    w.aon = align256(sizeof(float) * bhl);
    if (n_seg > 0) {
        // offsets: the caller's online read; the online logits, the means, and the routed
        // read's tables where it applies (else the generic read needs nothing more)
        w.xsum64 = align256(ssc_means_bytes(d, n_seg));
        w.xps = xps_only(d) + align256(sizeof(float) * xps_tail_floats(d));
        if (ssc_gather_covers(d, top_k, n_seg)) {
            const size_t tiles = (size_t)d.B * d.H * ((d.L + kSscTile - 1) / kSscTile);
            w.won = align256(sizeof(float) * bhl);
            w.ptok = align256(sizeof(int32_t) * tiles * kSscTile * top_k);
            w.pw = align256(sizeof(float) * tiles * kSscTile * top_k);
            w.poff = align256(sizeof(int32_t) * tiles * (n_seg + 1));
            w.sf = align256(ssc_frag_states_bytes(d, n_seg));
        }
        w.total = w.aon + w.xsum64 + w.xps + w.won + w.ptok + w.pw + w.poff + w.sf;
        return w;
    }
    w.on = online_ws(d);
    w.xps = xps_ws(d);
    w.xsum64 = align256(ssc_means_bytes(d));
    if (ssc_gather_covers(d, top_k)) {
        // the routed read: the online term (formed here when the caller passes none), the
        // normalised online weights, and every tile's pairs sorted by segment
        const size_t tiles = (size_t)d.B * d.H * ((d.L + kSscTile - 1) / kSscTile);
        w.on = align256(sizeof(float) * bhl * d.d_v);
        w.won = align256(sizeof(float) * bhl);
        w.ptok = align256(sizeof(int32_t) * tiles * kSscTile * top_k);
        w.pw = align256(sizeof(float) * tiles * kSscTile * top_k);
        w.poff = align256(sizeof(int32_t) * tiles * (num_segments(d) + 1));
        w.sf = align256(ssc_frag_states_bytes(d));
    } else if (gate_pass(d)) {
        w.w = align256(gate_w_bytes(d));
        w.won = align256(sizeof(float) * (size_t)d.B * d.H * d.L);
        w.inv_l = w.won;
        w.pf = align256(gate_pfrag_bytes(d));
    }
    w.total = w.aon + w.on + w.xps + w.xsum64 + w.w + w.won + w.inv_l + w.pf + w.ptok + w.pw +
              w.poff + w.sf;
    return w;
}

// The whole prefill over segment offsets in one call: the offsets scan's workspace, then
// either the bf16 memories before the pieces and the first-piece table (the read forms the
// online term itself) or the online read O_on (fp32), whichever is larger, then the read's.
struct PrefillSegsWorkspace {
    size_t scan, mid, read, total;
};
// The pieces over which the read forms the online term: those of the offsets scan (at least
// 512 tokens; pieces of one 256-token read tile measured no faster, their scan and prefix
// passes taking what the shorter walks save).
constexpr int kFusedPiece = 512;
static PrefillSegsWorkspace prefill_segs_workspace(const mc_dims& d, int n_seg) {
    PrefillSegsWorkspace w{};
    w.scan = align256(segs_scan_ws_bytes(d, n_seg) > segs_scan_ws_bytes(d, n_seg, kFusedPiece)
                          ? segs_scan_ws_bytes(d, n_seg)
                          : segs_scan_ws_bytes(d, n_seg, kFusedPiece));
    const size_t pieces =
        segs_pref_lo_bytes(d, n_seg, kFusedPiece) + align256(sizeof(int32_t) * n_seg);
    const size_t on = align256(sizeof(float) * (size_t)d.B * d.H * d.L * d.d_v);
    w.mid = pieces > on ? pieces : on;
    w.read = grm_workspace(d, n_seg).total;
    w.total = w.scan + w.mid + w.read;
    return w;
}

BwdWorkspace bwd_workspace(const mc_dims& d) {
    BwdWorkspace w{};
    const size_t bhl = (size_t)d.B * d.H * d.L;
    const size_t esz = d.dtype == MC_BF16 ? 2 : 4;
    w.aon = align256(sizeof(float) * bhl);
    w.xps = xps_only(d);
    w.xtail = align256(sizeof(float) * xps_tail_floats(d));
    w.on = align256(sizeof(float) * bhl * d.d_v);
    w.ot = align256(sizeof(float) * bhl * d.d_k);
    w.khat = d.phi ? align256(esz * bhl * d.d_k) : 0;
    w.lse = w.D = w.gs = align256(sizeof(float) * bhl);
    w.dG = align256(sizeof(float) * bhl * num_segments(d));
    w.dM = align256(sizeof(float) * (size_t)d.B * d.H * num_segments(d) * d.d_v * d.d_k);
    const int RL = bwd_dp_range(d.L);
    const size_t nr = (size_t)((d.L + RL - 1) / RL);  // token ranges (at most 64)
    w.dpp = align256(sizeof(float) * (bwd_fast(d) ? (size_t)d.H * d.B : nr * d.B * d.x_heads) *
                     num_segments(d) * d.d_g);
    if (bwd_fast(d)) {  // the swapped read and the gate numerators replace Ot, lse and D
        w.ot = w.lse = w.D = 0;
        w.W = align256(gate_w_bytes(d));
        w.won = w.inv_l = align256(sizeof(float) * bhl);
        w.pf = align256(gate_pfrag_bytes(d));
        w.mt = align256(sizeof(uint16_t) * (size_t)d.B * d.H * num_segments(d) * d.d_v * d.d_k);
        w.dqh = align256(sizeof(uint16_t) * bhl * d.d_k);
        w.daT = align256(sizeof(float) * bhl * num_segments(d));
        // B fragments of the means: per x head, k step of 16 segments, 4 column blocks, lane
        w.ptf = align256((size_t)d.B * d.x_heads * ((num_segments(d) + 15) / 16) * 4 * 64 * 32);
    }
    w.total = w.aon + w.xps + w.xtail + w.on + w.ot + w.khat + w.lse + w.D + w.gs + w.dG + w.dM +
              w.dpp + w.W + w.won + w.inv_l + w.pf + w.mt + w.dqh + w.daT + w.ptf;
    return w;
}

// The cached states of a decode step are read in runs of kDecodeRun states (one workgroup
// each); the workspace holds the partial softmaxes of a full cache, so its size depends only
// on n_cap.
DecodeWorkspace decode_workspace(const mc_dims& d, int n_cap, int /*n_cached*/) {
    DecodeWorkspace w{};
    w.slots = 1 + (n_cap + kDecodeRun - 1) / kDecodeRun;
    const size_t bh = (size_t)d.B * d.H;
    w.partial = align256(sizeof(float) * bh * (size_t)w.slots * d.d_v);
    w.ml = align256(sizeof(float) * bh * (size_t)w.slots * 2);
    w.total = w.partial + w.ml;
    return w;
}

}  // namespace mc

using namespace mc;

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shared size checks; `need_L` is false for decode, which ignores L.
static mc_status check_dims(const mc_dims* d, bool need_L) {
    if (!d) return MC_ERR_NULL;
    if (d->B <= 0 || d->H <= 0 || d->d_k <= 0 || d->d_v <= 0 || d->d_g <= 0 ||
        d->seg_len <= 0)
        return MC_ERR_DIMS;
    if (need_L && d->L <= 0) return MC_ERR_DIMS;
    if (!(d->x_heads == 1 || d->x_heads == d->H)) return MC_ERR_DIMS;
    if (!(d->dtype == MC_F32 || d->dtype == MC_BF16)) return MC_ERR_UNSUPPORTED;
    if (!(d->phi == MC_PHI_IDENTITY || d->phi == MC_PHI_ELU1)) return MC_ERR_UNSUPPORTED;
    if (!(d->d_k == 64 || d->d_k == 128) || !(d->d_v == 64 || d->d_v == 128))
        return MC_ERR_UNSUPPORTED;
    if (d->d_g > 256 || d->d_g % 8 != 0) return MC_ERR_UNSUPPORTED;
    // element offsets are formed in 64-bit, but a single sequence must index in 32-bit
    if (need_L && (int64_t)d->L * 256 > INT32_MAX) return MC_ERR_UNSUPPORTED;
    return MC_OK;
}

extern "C" {

int mc_abi_version(void) { return MC_ABI_VERSION; }

const char* mc_status_str(mc_status s) {
    switch (s) {
        case MC_OK: return "ok";
        case MC_ERR_NULL: return "a required pointer is NULL";
        case MC_ERR_DIMS: return "invalid or inconsistent sizes";
        case MC_ERR_UNSUPPORTED: return "sizes or types not supported by this library";
        case MC_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case MC_ERR_WORKSPACE: return "workspace too small";
        case MC_ERR_HIP: return "HIP launch failed";
        case MC_ERR_CAPACITY: return "decode cache is full";
        case MC_ERR_SCRATCH:
            return "the step needs more scratch than the fixed buffer of "
                   "mc_decode_step_noalloc holds";
    }
    return "unknown status";
}

size_t mc_workspace_bytes(const mc_dims* d, mc_op op, int32_t top_k, int32_t n_cap) {
    if (op == MC_OP_DECODE) {
        if (check_dims(d, false) != MC_OK || n_cap < 0) return 0;
        return decode_workspace(*d, n_cap, 0).total;
    }
    if (check_dims(d, true) != MC_OK) return 0;
    switch (op) {
        case MC_OP_PREFILL: return 0;
        case MC_OP_GRM: return grm_workspace(*d).total;
        case MC_OP_GRM_SEGS:
            return top_k >= 1 && top_k <= MC_MAX_SEGS ? grm_workspace(*d, top_k).total : 0;
        case MC_OP_SSC: return top_k >= 1 ? ssc_workspace(*d, top_k).total : 0;
        case MC_OP_GRM_PREFILL_SEGS:
            return top_k >= 1 && top_k <= MC_MAX_SEGS ? prefill_segs_workspace(*d, top_k).total
                                                      : 0;
        case MC_OP_SSC_SEGS:
            return top_k >= 1 && top_k <= 16 && n_cap >= 1 && n_cap <= MC_MAX_SEGS
                       ? ssc_workspace(*d, top_k, n_cap).total
                       : 0;
        case MC_OP_GRM_BACKWARD: return bwd_workspace(*d).total;
        case MC_OP_SCAN_SEGS:
            return top_k >= 1 && top_k <= MC_MAX_SEGS ? segs_scan_ws_bytes(*d, top_k) : 0;
        default: return 0;
    }
}

mc_status mc_scan_prefill(const mc_dims* d, const void* Q, const void* K, const void* V,
                          const void* X, float* M, uint16_t* M_lo, float* P, float* O_on,
                          void* ws, size_t ws_bytes, void* stream) {
    (void)ws;
    (void)ws_bytes;
    mc_status st = check_dims(d, true);
    if (st != MC_OK) return st;
    if (!Q || !K || !V || !X || !M || !P) return MC_ERR_NULL;
    if (d->dtype == MC_BF16 && !M_lo) return MC_ERR_NULL;
    const void* ptrs[] = {Q, K, V, X, M, M_lo, P, O_on};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MC_ERR_ALIGN;
    return launch_scan_prefill(*d, Q, K, V, X, M, M_lo, P, O_on, stream) ? MC_ERR_HIP : MC_OK;
}

mc_status mc_grm_readout(const mc_dims* d, const void* Q, const void* K, const void* V,
                         const void* U, const void* X, const float* M, const uint16_t* M_lo,
                         const float* P, const float* O_on, void* Y, float* gamma, void* ws,
                         size_t ws_bytes, void* stream) {
    mc_status st = check_dims(d, true);
    if (st != MC_OK) return st;
    if (!Q || !U || !X || !P || !Y) return MC_ERR_NULL;
    if (!O_on && (!K || !V)) return MC_ERR_NULL;
    if (d->dtype == MC_BF16 ? !M_lo : !M) return MC_ERR_NULL;
    const GrmWorkspace w = grm_workspace(*d);
    if (!ws || ws_bytes < w.total) return MC_ERR_WORKSPACE;
    const void* ptrs[] = {Q, K, V, U, X, M, M_lo, P, O_on, Y, gamma, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MC_ERR_ALIGN;
    float* aon = (float*)ws;
    float* xps = (float*)((char*)ws + w.aon + w.on);
    if (!O_on && w.on) {  // generic kernels: form the online read first
        float* on = (float*)((char*)ws + w.aon);
        if (launch_scan_online(*d, Q, K, V, on, stream)) return MC_ERR_HIP;
        O_on = on;
    }
    const bool mfma = read_mfma_covers(*d);
    if (mfma && launch_xps(*d, X, xps, (float*)((char*)xps + xps_only(*d)), stream))
        return MC_ERR_HIP;
    if ((!mfma || gamma) && launch_aon(*d, X, U, aon, stream)) return MC_ERR_HIP;
    GateWeights gw;
    if (gate_pass(*d)) {  // the gate as its own pass; the read loads its numerators
        char* g = (char*)ws + w.aon + w.on + w.xps;
        uint16_t* W = (uint16_t*)g;
        float* won = (float*)(g + w.w);
        float* inv_l = (float*)(g + w.w + w.won);
        void* pf = g + w.w + w.won + w.inv_l;
        if (launch_gate_w(*d, U, xps, P, pf, W, won, inv_l, stream)) return MC_ERR_HIP;
        gw.W = W;
        gw.won = won;
        gw.inv_l = inv_l;
    }
    if (launch_grm_readout(*d, Q, K, V, U, aon, xps, M, M_lo, P, O_on, gw, Y, gamma, stream))
        return MC_ERR_HIP;
    return MC_OK;
}

mc_status mc_ssc_readout(const mc_dims* d, int32_t top_k, const void* Q, const void* K,
                         const void* V, const void* U, const void* X, const float* M,
                         const uint16_t* M_lo, const float* P, const float* O_on, void* Y,
                         int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
    mc_status st = check_dims(d, true);
    if (st != MC_OK) return st;
    if (top_k < 1) return MC_ERR_DIMS;
    if (top_k > 16) return MC_ERR_UNSUPPORTED;
    if (!Q || !U || !X || !P || !Y || !idx) return MC_ERR_NULL;
    if (!O_on && (!K || !V)) return MC_ERR_NULL;
    if (d->dtype == MC_BF16 ? !M_lo : !M) return MC_ERR_NULL;
    const SscWorkspace w = ssc_workspace(*d, top_k);
    if (!ws || ws_bytes < w.total) return MC_ERR_WORKSPACE;
    const void* ptrs[] = {Q, K, V, U, X, M, M_lo, P, O_on, Y, idx, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MC_ERR_ALIGN;
    float* aon = (float*)ws;
    float* xps = (float*)((char*)ws + w.aon + w.on);
    double* xsum64 = (double*)((char*)ws + w.aon + w.on + w.xps);
    if (ssc_gather_covers(*d, top_k)) {
        // routed: the online term, the selection with its weights and the tiles' pairs sorted
        // by segment, then only the selected states are read
        if (!O_on) {
            float* on = (float*)((char*)ws + w.aon);
            if (launch_scan_mfma_online(*d, Q, K, V, on, stream)) return MC_ERR_HIP;
            O_on = on;
        }
        if (launch_aon(*d, X, U, aon, stream)) return MC_ERR_HIP;
        char* g = (char*)ws + w.aon + w.on + w.xps + w.xsum64;
        SscRoute rt;
        rt.aon = aon;
        rt.won = (float*)g;
        rt.ptok = (int32_t*)(g + w.won);
        rt.pw = (float*)(g + w.won + w.ptok);
        rt.poff = (int32_t*)(g + w.won + w.ptok + w.pw);
        rt.Sf = g + w.won + w.ptok + w.pw + w.poff;
        if (launch_ssc_select(*d, top_k, U, X, xsum64, idx, stream, &rt)) return MC_ERR_HIP;
        if (launch_ssc_gather(*d, top_k, Q, M_lo, O_on, rt, Y, stream)) return MC_ERR_HIP;
        return MC_OK;
    }
    if (!O_on && w.on) {
        float* on = (float*)((char*)ws + w.aon);
        if (launch_scan_online(*d, Q, K, V, on, stream)) return MC_ERR_HIP;
        O_on = on;
    }
    const bool mfma = read_mfma_covers(*d);
    if (mfma && launch_xps(*d, X, xps, (float*)((char*)xps + xps_only(*d)), stream))
        return MC_ERR_HIP;
    // the generic read needs the online logits
    const bool generic = !gate_pass(*d) && !read_mfma_ssc_covers(*d, O_on != nullptr);
    if (generic && launch_aon(*d, X, U, aon, stream)) return MC_ERR_HIP;
    if (launch_ssc_select(*d, top_k, U, X, xsum64, idx, stream)) return MC_ERR_HIP;
    if (gate_pass(*d)) {
        // the gate as its own pass, masked to the selections; the read then loads its
        // numerators (the GRM read with zero weight on every segment not selected)
        char* g = (char*)ws + w.aon + w.on + w.xps + w.xsum64;
        uint16_t* W = (uint16_t*)g;
        float* won = (float*)(g + w.w);
        float* inv_l = (float*)(g + w.w + w.won);
        void* pf = g + w.w + w.won + w.inv_l;
        if (launch_gate_w(*d, U, xps, P, pf, W, won, inv_l, stream, idx, top_k)) return MC_ERR_HIP;
        GateWeights gw;
        gw.W = W;
        gw.won = won;
        gw.inv_l = inv_l;
        if (launch_grm_readout(*d, Q, K, V, U, aon, xps, M, M_lo, P, O_on, gw, Y, nullptr,
                               stream))
            return MC_ERR_HIP;
        return MC_OK;
    }
    if (launch_ssc_readout(*d, top_k, Q, K, V, U, aon, xps, M, M_lo, P, O_on, idx, Y, stream))
        return MC_ERR_HIP;
    return MC_OK;
}

// Host checks of a segmentation; fills the by-value kernel argument.
static mc_status check_segs(const mc_dims* d, const int32_t* off, int32_t n_seg, SegArg* sg) {
    if (!off) return MC_ERR_NULL;
    if (n_seg < 1) return MC_ERR_DIMS;
    if (n_seg > MC_MAX_SEGS) return MC_ERR_UNSUPPORTED;
    if (off[0] != 0 || off[n_seg] != d->L) return MC_ERR_DIMS;
    for (int i = 0; i < n_seg; ++i)
        if (off[i + 1] <= off[i]) return MC_ERR_DIMS;
    sg->n = n_seg;
    for (int i = 0; i <= n_seg; ++i) sg->off[i] = off[i];
    return MC_OK;
}

mc_status mc_scan_prefill_segs(const mc_dims* d, const int32_t* seg_off, int32_t n_seg,
                               const void* Q, const void* K, const void* V, const void* X,
                               float* M, uint16_t* M_lo, float* P, float* O_on, void* ws,
                               size_t ws_bytes, void* stream) {
    mc_status st = check_dims(d, true);
    if (st != MC_OK) return st;
    SegArg sg;
    if ((st = check_segs(d, seg_off, n_seg, &sg)) != MC_OK) return st;
    if (!Q || !K || !V || !X || !M || !P) return MC_ERR_NULL;
    if (d->dtype == MC_BF16 && !M_lo) return MC_ERR_NULL;
    const size_t need = segs_scan_ws_bytes(*d, n_seg);
    if (need && (!ws || ws_bytes < need)) return MC_ERR_WORKSPACE;
    const void* ptrs[] = {Q, K, V, X, M, M_lo, P, O_on, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MC_ERR_ALIGN;
    return launch_scan_prefill_segs(*d, sg, Q, K, V, X, M, M_lo, P, O_on, ws, ws_bytes, stream)
               ? MC_ERR_HIP
               : MC_OK;
}

mc_status mc_grm_readout_segs(const mc_dims* d, const int32_t* seg_off, int32_t n_seg,
                              const void* Q, const void* U, const void* X, const float* M,
                              const uint16_t* M_lo, const float* P, const float* O_on, void* Y,
                              float* gamma, void* ws, size_t ws_bytes, void* stream) {
    mc_status st = check_dims(d, true);
    if (st != MC_OK) return st;
    SegArg sg;
    if ((st = check_segs(d, seg_off, n_seg, &sg)) != MC_OK) return st;
    if (!Q || !U || !X || !P || !O_on || !Y) return MC_ERR_NULL;
    if (d->dtype == MC_BF16 ? !M_lo : !M) return MC_ERR_NULL;
    // with the workspace for n_seg segments (MC_OP_GRM_SEGS) the gate runs as its own pass;
    // with the constant-length one (MC_OP_GRM) the read forms it in-kernel
    const GrmWorkspace w = grm_workspace(*d, n_seg);
    const bool own_gate = w.w && ws && ws_bytes >= w.total;
    if (!ws || ws_bytes < (own_gate ? w.total : w.aon + w.on + w.xps)) return MC_ERR_WORKSPACE;
    const void* ptrs[] = {Q, U, X, M, M_lo, P, O_on, Y, gamma, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MC_ERR_ALIGN;
    char* b = (char*)ws;
    float* xps = w.xps ? (float*)(b + w.aon + w.on) : nullptr;
    float* xtail = xps ? (float*)((char*)xps + xps_only(*d)) : nullptr;
    SegGate gate;  // the gate pass's buffers (none: the in-kernel gate)
    if (own_gate) {
        char* g = b + w.aon + w.on + w.xps;
        gate.W = (uint16_t*)g;
        gate.won = (float*)(g + w.w);
        gate.inv_l = (float*)(g + w.w + w.won);
        gate.pf = g + w.w + w.won + w.inv_l;
    }
    return launch_grm_readout_segs(*d, sg, Q, U, X, M, M_lo, P, O_on, (float*)ws, xps, xtail, Y,
                                   gamma, stream, gate)
               ? MC_ERR_HIP
               : MC_OK;
}

mc_status mc_grm_prefill_segs(const mc_dims* d, const int32_t* seg_off, int32_t n_seg,
                              const void* Q, const void* K, const void* V, const void* U,
                              const void* X, float* M, uint16_t* M_lo, float* P, void* Y,
                              float* gamma, void* ws, size_t ws_bytes, void* stream) {
    mc_status st = check_dims(d, true);
    if (st != MC_OK) return st;
    SegArg sg;
    if ((st = check_segs(d, seg_off, n_seg, &sg)) != MC_OK) return st;
    if (!Q || !K || !V || !U || !X || !M || !P || !Y) return MC_ERR_NULL;
    if (d->dtype == MC_BF16 && !M_lo) return MC_ERR_NULL;
    const PrefillSegsWorkspace w = prefill_segs_workspace(*d, n_seg);
    if (!ws || ws_bytes < w.total) return MC_ERR_WORKSPACE;
    const void* ptrs[] = {Q, K, V, U, X, M, M_lo, P, Y, gamma, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MC_ERR_ALIGN;
    char* b = (char*)ws;
    char* mid = b + w.scan;
    char* rd = mid + w.mid;
    const GrmWorkspace rw = grm_workspace(*d, n_seg);
    float* xps = rw.xps ? (float*)(rd + rw.aon + rw.on) : nullptr;
    float* xtail = xps ? (float*)((char*)xps + xps_only(*d)) : nullptr;
    SegGate gate;
    if (rw.w) {
        char* g = rd + rw.aon + rw.on + rw.xps;
        gate.W = (uint16_t*)g;
        gate.won = (float*)(g + rw.w);
        gate.inv_l = (float*)(g + rw.w + rw.won);
        gate.pf = g + rw.w + rw.won + rw.inv_l;
    }
    // the read forms the online term itself after the gate pass (bf16, d = 128), walking each
    // token's piece, when no segment is longer than a piece or the scan cuts the long ones
    const int pl = scan_piece_len(d->L, n_seg, kFusedPiece);
    int longest = 0;
    for (int i = 0; i < n_seg; ++i)
        if (seg_off[i + 1] - seg_off[i] > longest) longest = seg_off[i + 1] - seg_off[i];
    const bool fused = gate.W && (pl > 0 || longest <= 1024);
    if (fused) {
        uint16_t* pref_lo = (uint16_t*)mid;
        int32_t* pfirst = (int32_t*)(mid + segs_pref_lo_bytes(*d, n_seg, kFusedPiece));
        PieceOnline pon;
        pon.M0 = pref_lo;
        pon.pfirst = pfirst;
        if (launch_scan_prefill_segs(*d, sg, Q, K, V, X, M, M_lo, P, nullptr, b, w.scan, stream,
                                     &pon, pref_lo, pfirst, kFusedPiece))
            return MC_ERR_HIP;
        return launch_grm_readout_segs(*d, sg, Q, U, X, M, M_lo, P, nullptr, (float*)rd, xps,
                                       xtail, Y, gamma, stream, gate, K, V, &pon)
                   ? MC_ERR_HIP
                   : MC_OK;
    }
    float* O_on = (float*)mid;
    if (launch_scan_prefill_segs(*d, sg, Q, K, V, X, M, M_lo, P, O_on, b, w.scan, stream))
        return MC_ERR_HIP;
    return launch_grm_readout_segs(*d, sg, Q, U, X, M, M_lo, P, O_on, (float*)rd, xps, xtail, Y,
                                   gamma, stream, gate)
               ? MC_ERR_HIP
               : MC_OK;
}

mc_status mc_ssc_readout_segs(const mc_dims* d, const int32_t* seg_off, int32_t n_seg,
                              int32_t top_k, const void* Q, const void* U, const void* X,
                              const float* M, const uint16_t* M_lo, const float* P,
                              const float* O_on, void* Y, int32_t* idx, void* ws,
                              size_t ws_bytes, void* stream) {
    mc_status st = check_dims(d, true);
    if (st != MC_OK) return st;
    SegArg sg;
    if ((st = check_segs(d, seg_off, n_seg, &sg)) != MC_OK) return st;
    if (top_k < 1) return MC_ERR_DIMS;
    if (top_k > 16) return MC_ERR_UNSUPPORTED;
    if (!Q || !U || !X || !P || !O_on || !Y || !idx) return MC_ERR_NULL;
    if (d->dtype == MC_BF16 ? !M_lo : !M) return MC_ERR_NULL;
    const SscWorkspace w = ssc_workspace(*d, top_k, n_seg);
    if (!ws || ws_bytes < w.total) return MC_ERR_WORKSPACE;
    const void* ptrs[] = {Q, U, X, M, M_lo, P, O_on, Y, idx, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MC_ERR_ALIGN;
    float* aon = (float*)ws;
    double* xsum64 = (double*)((char*)ws + w.aon);
    float* xps = (float*)((char*)ws + w.aon + w.xsum64);
    if (launch_aon_segs(*d, sg, X, U, aon, stream, xps, (float*)((char*)xps + xps_only(*d))))
        return MC_ERR_HIP;
    if (ssc_gather_covers(*d, top_k, n_seg)) {
        // routed: the selection with its weights and the tiles' pairs sorted by segment, then
        // only the selected states are read
        char* g = (char*)ws + w.aon + w.xsum64 + w.xps;
        SscRoute rt;
        rt.aon = aon;
        rt.won = (float*)g;
        rt.ptok = (int32_t*)(g + w.won);
        rt.pw = (float*)(g + w.won + w.ptok);
        rt.poff = (int32_t*)(g + w.won + w.ptok + w.pw);
        rt.Sf = g + w.won + w.ptok + w.pw + w.poff;
        if (launch_ssc_select(*d, top_k, U, X, xsum64, idx, stream, &rt, &sg)) return MC_ERR_HIP;
        if (launch_ssc_gather(*d, top_k, Q, M_lo, O_on, rt, Y, stream, &sg)) return MC_ERR_HIP;
        return MC_OK;
    }
    if (launch_ssc_select(*d, top_k, U, X, xsum64, idx, stream, nullptr, &sg)) return MC_ERR_HIP;
    return launch_ssc_readout_segs(*d, sg, top_k, Q, U, aon, M, M_lo, P, O_on, idx, Y, stream)
               ? MC_ERR_HIP
               : MC_OK;
}

mc_status mc_scan_prefill_swla(const mc_dims* d, const int32_t* seg_off, int32_t n_seg,
                               const float* alpha, const float* beta, const float* lambda,
                               const void* Q, const void* K, const void* V, const void* X,
                               float* M, uint16_t* M_lo, float* P, float* O_on, void* stream) {
    mc_status st = check_dims(d, true);
    if (st != MC_OK) return st;
    SegArg sg{};
    if (seg_off && (st = check_segs(d, seg_off, n_seg, &sg)) != MC_OK) return st;
    if (!alpha || !beta || !lambda || !Q || !K || !V || !X || !M || !P || !O_on)
        return MC_ERR_NULL;
    if (d->dtype == MC_BF16 && !M_lo) return MC_ERR_NULL;
    const void* ptrs[] = {alpha, beta, lambda, Q, K, V, X, M, M_lo, P, O_on};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MC_ERR_ALIGN;
    SwlaGates gt;
    gt.alpha = alpha;
    gt.beta = beta;
    gt.lam = lambda;
    return launch_scan_prefill_swla(*d, sg, gt, Q, K, V, X, M, M_lo, P, O_on, stream)
               ? MC_ERR_HIP
               : MC_OK;
}

mc_status mc_grm_backward(const mc_dims* d, const void* Q, const void* K, const void* V,
                          const void* U, const void* X, const float* M, const uint16_t* M_lo,
                          const float* P, const void* dY, float* dQ, float* dK, float* dV,
                          float* dU, float* dX, void* ws, size_t ws_bytes, void* stream) {
    mc_status st = check_dims(d, true);
    if (st != MC_OK) return st;
    if (!Q || !K || !V || !U || !X || !P || !dY || !dQ || !dK || !dV || !dU || !dX)
        return MC_ERR_NULL;
    if (d->dtype == MC_BF16 ? !M_lo : !M) return MC_ERR_NULL;
    const BwdWorkspace w = bwd_workspace(*d);
    if (!ws || ws_bytes < w.total) return MC_ERR_WORKSPACE;
    const void* ptrs[] = {Q, K, V, U, X, M, M_lo, P, dY, dQ, dK, dV, dU, dX, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MC_ERR_ALIGN;
    char* b = (char*)ws;
    BwdBuffers bw;
    bw.aon = (float*)b;
    b += w.aon;
    bw.xps = (float*)b;
    b += w.xps;
    bw.xtail = (float*)b;
    b += w.xtail;
    bw.on = (float*)b;
    b += w.on;
    bw.ot = (float*)b;
    b += w.ot;
    bw.khat = w.khat ? (void*)b : nullptr;
    b += w.khat;
    bw.lse = (float*)b;
    b += w.lse;
    bw.D = (float*)b;
    b += w.D;
    bw.gs = (float*)b;
    b += w.gs;
    bw.dG = (float*)b;
    b += w.dG;
    bw.dM = (float*)b;
    b += w.dM;
    bw.dpp = (float*)b;
    b += w.dpp;
    bw.W = (uint16_t*)b;
    b += w.W;
    bw.won = (float*)b;
    b += w.won;
    bw.inv_l = (float*)b;
    b += w.inv_l;
    bw.pf = b;
    b += w.pf;
    bw.mt = b;
    b += w.mt;
    bw.dqh = b;
    b += w.dqh;
    bw.daT = (float*)b;
    b += w.daT;
    bw.ptf = b;
    return launch_grm_backward(*d, bw, Q, K, V, U, X, M, M_lo, P, dY, dQ, dK, dV, dU, dX,
                               stream)
               ? MC_ERR_HIP
               : MC_OK;
}

}  // extern "C"

// Validation shared by the two decode entry points (before any HIP call).
static mc_status check_decode(const mc_dims* d, const void* q, const void* k, const void* v,
                              const void* u, const void* x, const float* M_on,
                              const float* xsum_on, const int32_t* count_on,
                              const void* M_cache, const float* P_cache,
                              const int32_t* n_cached, int32_t n_cap, const void* y) {
    mc_status st = check_dims(d, false);
    if (st != MC_OK) return st;
    // u may be NULL: uniform weights over the memories (post-training memory caching)
    if (!q || !k || !v || !x || !M_on || !xsum_on || !count_on || !P_cache || !n_cached || !y)
        return MC_ERR_NULL;
    if (n_cap < 0) return MC_ERR_DIMS;
    if (n_cap > 0 && !M_cache) return MC_ERR_NULL;
    const int cnt = *count_on, n = *n_cached;
    if (cnt < 0 || cnt >= d->seg_len || n < 0 || n > n_cap) return MC_ERR_DIMS;
    if (cnt + 1 == d->seg_len && n == n_cap) return MC_ERR_CAPACITY;
    const void* ptrs[] = {q, k, v, u, x, M_on, xsum_on, M_cache, P_cache, y};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MC_ERR_ALIGN;
    return MC_OK;
}

// The host counters after an enqueued step.
static void decode_advance(const mc_dims* d, int32_t* count_on, int32_t* n_cached) {
    if (*count_on + 1 == d->seg_len) {
        *count_on = 0;
        *n_cached += 1;
    } else {
        *count_on += 1;
    }
}

extern "C" {

mc_status mc_decode_step(const mc_dims* d, const void* q, const void* k, const void* v,
                         const void* u, const void* x, float* M_on, float* xsum_on,
                         int32_t* count_on, void* M_cache, float* P_cache, int32_t* n_cached,
                         int32_t n_cap, void* y, void* ws, size_t ws_bytes, void* stream) {
    mc_status st = check_decode(d, q, k, v, u, x, M_on, xsum_on, count_on, M_cache, P_cache,
                                n_cached, n_cap, y);
    if (st != MC_OK) return st;
    const int cnt = *count_on, n = *n_cached;
    const DecodeWorkspace w = decode_workspace(*d, n_cap, n);
    if (!ws || ws_bytes < w.total) return MC_ERR_WORKSPACE;
    if (!aligned16(ws)) return MC_ERR_ALIGN;
    if (launch_decode_step(*d, q, k, v, u, x, M_on, xsum_on, cnt, M_cache, P_cache, n, n_cap,
                           cnt + 1 == d->seg_len, y, ws, n_cap, stream))
        return MC_ERR_HIP;
    decode_advance(d, count_on, n_cached);
    return MC_OK;
}

mc_status mc_decode_step_noalloc(const mc_dims* d, const void* q, const void* k, const void* v,
                                 const void* u, const void* x, float* M_on, float* xsum_on,
                                 int32_t* count_on, void* M_cache, float* P_cache,
                                 int32_t* n_cached, int32_t n_cap, void* y, void* stream) {
    mc_status st = check_decode(d, q, k, v, u, x, M_on, xsum_on, count_on, M_cache, P_cache,
                                n_cached, n_cap, y);
    if (st != MC_OK) return st;
    const int cnt = *count_on, n = *n_cached;
    // the scratch is laid out for the n cached states this step reads
    if (decode_workspace(*d, n, n).total > MC_NOALLOC_SCRATCH_BYTES) return MC_ERR_SCRATCH;
    void* scratch = nullptr;
    if (noalloc_scratch(&scratch)) return MC_ERR_HIP;
    if (launch_decode_step(*d, q, k, v, u, x, M_on, xsum_on, cnt, M_cache, P_cache, n, n_cap,
                           cnt + 1 == d->seg_len, y, scratch, n, stream))
        return MC_ERR_HIP;
    decode_advance(d, count_on, n_cached);
    return MC_OK;
}

}  // extern "C"
