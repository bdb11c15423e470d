/*
 * mc.h -- C ABI of libmc: Memory Caching (MC) over a linear-attention memory on MI355X.
 *
 * The operations are those of the Memory Caching paper ("Memory Caching: RNNs with growing
 * memory", Behrouz et al.; zh-TW / ja renderings) and of its gitcode explainer
 * ("给 RNN 装上“会增长的记忆”：解读 Google 的 Memory Caching"):
 *   - the sequence is split into segments of constant length C; inside segment s the
 *     memory runs the linear-attention recurrence M_t = M_{t-1} + v_t phi(k_t)^T from zero
 *     (paper §3, Eq. 4b with the update of §2, Eq. 2), and the state after the segment's
 *     last token is cached;
 *   - Gated Residual Memory (paper §3.1, Eq. 9):
 *         y_t = gamma_t^(s) M_t^(s) phi(q_t) + sum_{i<s} gamma_t^(i) M^(i) phi(q_t)
 *     with gamma_t = softmax_i <u_t, MeanPooling(S^(i))> (paper §3.1, Eq. 10);
 *   - Sparse Selective Caching (explainer §3.4): only the Top-k cached segments by the
 *     router score <u_t, MeanPooling(S^(i))> are read, plus the online memory;
 *   - decode: one new token per sequence reads the online memory and every cached state.
 *
 * Readings where the pages leave a step open (fixed by this ABI):
 *   - no normaliser 1/Z (the paper's Miras remark: the inner-product objective gives the
 *     unnormalised linear attention);
 *   - the state is M = sum_r v_r phi(k_r)^T, d_v x d_k, row-major, read as y = M phi(q);
 *   - token t updates the memory before it reads it;
 *   - MeanPooling averages the layer input X; the online segment uses the causal prefix
 *     mean over its tokens up to t;
 *   - the softmax runs over all cached segments and the online segment, no temperature;
 *   - SSC ties in the router score go to the lower segment index.
 *
 * Conventions shared by every entry point
 *   Memory: every tensor argument is a DEVICE pointer owned by the caller, dense row-major
 *     with the last dimension contiguous, 16-byte aligned.  The library allocates, frees
 *     and retains nothing; scratch memory is the caller's workspace `ws` of at least
 *     mc_workspace_bytes() bytes (16-byte aligned; NULL allowed when that size is 0).  The
 *     one exception is mc_decode_step_noalloc, whose scratch is a fixed buffer the library
 *     holds on each GPU it runs on until the process ends.
 *   Streams: `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *     work on it and never synchronise.  Host scalars passed by pointer are read and
 *     updated on the host when the call is made.
 *   Errors: every argument is validated before any HIP call; on error nothing is enqueued,
 *     nothing is written and the MC_ERR_* code is returned.  A failed kernel launch
 *     returns MC_ERR_HIP.  Faults inside kernels surface at the caller's next sync.  The
 *     library never prints, aborts or throws.
 *   Threads: no global mutable state; calls are re-entrant (except that calls of
 *     mc_decode_step_noalloc on one GPU share its scratch buffer, see there).
 *
 * Token layout: t = 0..L-1 is 0-based; s = t / C is its segment, j = t % C its position.
 * NS = ceil(L / C) segments; if L % C != 0 the last segment is partial.
 */
#ifndef MC_H
#define MC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MC_ABI_VERSION 1

typedef enum {
    MC_OK = 0,
    MC_ERR_NULL = 1,        /* a required pointer is NULL                                 */
    MC_ERR_DIMS = 2,        /* a size is non-positive or inconsistent                     */
    MC_ERR_UNSUPPORTED = 3, /* valid, but outside what this library implements            */
    MC_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                           */
    MC_ERR_WORKSPACE = 5,   /* ws_bytes < mc_workspace_bytes()                            */
    MC_ERR_HIP = 6,         /* a HIP launch failed                                        */
    MC_ERR_CAPACITY = 7,    /* decode: the cache is full and the step would append to it  */
    MC_ERR_SCRATCH = 8      /* mc_decode_step_noalloc: the step needs more scratch than
                               MC_NOALLOC_SCRATCH_BYTES                                    */
} mc_status;

/* Size of the fixed per-GPU scratch buffer of mc_decode_step_noalloc (64 MiB). */
#define MC_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

typedef enum { MC_F32 = 0, MC_BF16 = 1 } mc_dtype;           /* storage type of Q,K,V,U,X,Y */
typedef enum { MC_PHI_IDENTITY = 0, MC_PHI_ELU1 = 1 } mc_phi; /* feature map on Q and K     */
typedef enum {
    MC_OP_PREFILL = 0,
    MC_OP_GRM = 1,
    MC_OP_SSC = 2,
    MC_OP_DECODE = 3,
    MC_OP_GRM_BACKWARD = 4,
    MC_OP_SCAN_SEGS = 5,
    MC_OP_GRM_SEGS = 6,
    MC_OP_SSC_SEGS = 7,
    MC_OP_GRM_PREFILL_SEGS = 8
} mc_op;

/* Problem sizes.  Supported by this library: d_k, d_v in {64, 128}; 1 <= d_g <= 256 and
 * d_g % 8 == 0; C >= 1; x_heads in {1, H}; dtype MC_F32 or MC_BF16.                      */
typedef struct mc_dims {
    int32_t B, H;       /* sequences, heads                                                 */
    int32_t L;          /* tokens per sequence in this call (prefill); ignored by decode    */
    int32_t d_k, d_v;   /* query/key width, value width                                     */
    int32_t d_g;        /* gate width = width of U and X                                    */
    int32_t seg_len;    /* C, the segment length                                            */
    int32_t x_heads;    /* 1: X is [B,1,L,d_g], shared by the heads; H: X is [B,H,L,d_g]    */
    int32_t dtype;      /* mc_dtype of Q, K, V, U, X and Y                                  */
    int32_t phi;        /* mc_phi applied to Q and K inside the kernels                     */
} mc_dims;

/* Returns MC_ABI_VERSION. */
int mc_abi_version(void);

/* Static description of a status code (never NULL). */
const char* mc_status_str(mc_status status);

/* Workspace bytes an operation needs for these sizes (top_k is used by MC_OP_SSC, n_cap by
 * MC_OP_DECODE; MC_OP_SCAN_SEGS, the segment-offset write path, and MC_OP_GRM_SEGS, the
 * segment-offset read, take the number of segments in top_k; MC_OP_SSC_SEGS, the
 * segment-offset SSC read, takes top_k in top_k and the number of segments in n_cap;
 * MC_OP_GRM_PREFILL_SEGS, the one-call prefill over offsets, the number of segments in top_k).
 * Returns 0 when no workspace is needed or the sizes are invalid. */
size_t mc_workspace_bytes(const mc_dims* dims, mc_op op, int32_t top_k, int32_t n_cap);

/*
 * mc_scan_prefill -- the write path: per-segment scan, cached states, segment means and the
 * ungated online read (paper §3 Eq. 4b; §3.1 Eq. 6 / Eq. 8 for the online memory).
 *
 *   Q, K  [B,H,L,d_k]  dtype          V [B,H,L,d_v] dtype          X [B,x_heads,L,d_g] dtype
 *   M      out [B,H,NS,d_v,d_k] fp32   M^(i) = sum_{r in segment i} v_r phi(k_r)^T; the slot
 *                                      of a trailing partial segment holds its state after
 *                                      token L-1 (the online state a decode continues from)
 *   M_lo   out, nullable: the same states rounded to bf16 (the operand copy the bf16 read
 *                                      paths and the decode cache use); required when
 *                                      dtype == MC_BF16
 *   P      out [B,x_heads,NS,d_g] fp32 MeanPooling(S^(i)); a partial segment averages the
 *                                      tokens it has
 *   O_on   out, nullable [B,H,L,d_v] fp32  M_t^(s) phi(q_t), the online read with weight 1.
 *          The read calls form this term themselves when given K and V instead, so a caller
 *          that only wants y passes NULL here and in the read call (the fast path).
 */
mc_status mc_scan_prefill(const mc_dims* dims, const void* Q, const void* K, const void* V,
                          const void* X, float* M, uint16_t* M_lo, float* P, float* O_on,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * mc_grm_readout -- Gated Residual Memory read (paper §3.1, Eq. 9 with the gate of Eq. 10):
 *     a_t^(i) = <u_t, P_i> (i < s),  a_t^(s) = <u_t, prefix mean of X over t's segment>,
 *     gamma_t = softmax(a_t^(0..s)),
 *     y_t = gamma^(s) M_t^(s) phi(q_t) + sum_{i<s} gamma^(i) M^(i) phi(q_t)
 *
 *   Q, K [B,H,L,d_k], V [B,H,L,d_v], U [B,H,L,d_g], X [B,x_heads,L,d_g]: dtype
 *   M, M_lo, P: as written by mc_scan_prefill for the same Q,K,V,X (M_lo is read when
 *     dtype == MC_BF16, M when MC_F32; the other may be NULL)
 *   O_on   nullable: the online read written by mc_scan_prefill.  When NULL the online term
 *     M_t^(s) phi(q_t) is formed here from K and V (then required); K and V are ignored when
 *     O_on is given.
 *   Y      out [B,H,L,d_v] dtype
 *   gamma  out, nullable [B,H,L,NS] fp32: gamma_t^(i) for i <= s, 0 beyond
 */
mc_status mc_grm_readout(const mc_dims* dims, const void* Q, const void* K, const void* V,
                         const void* U, const void* X, const float* M, const uint16_t* M_lo,
                         const float* P, const float* O_on, void* Y, float* gamma, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * mc_ssc_readout -- Sparse Selective Caching read (explainer §3.4):
 *     R_t = Top-k of {a_t^(i)}_{i<s} (larger score first, lower index on ties; all of them
 *     when s <= k); gamma_t = softmax over R_t and the online segment;
 *     y_t = gamma^(s) M_t^(s) phi(q_t) + sum_{i in R_t} gamma^(i) M^(i) phi(q_t)
 *   The selection is exact: every score is formed in fp64 in the definition's order -- the
 *   segment's x values summed token by token, divided by its length, then the dot product
 *   with u_t summed term by term with no fused multiply-add -- and ranked on those values,
 *   ties going to the lower index.
 *
 *   Arguments as mc_grm_readout, plus
 *   top_k  1 <= top_k <= 16
 *   idx    out [B,H,L,top_k] int32: R_t in ascending order, -1 padded
 *   ws     mc_workspace_bytes(dims, MC_OP_SSC, top_k, 0) bytes
 */
mc_status mc_ssc_readout(const mc_dims* dims, int32_t top_k, const void* Q, const void* K,
                         const void* V, const void* U, const void* X, const float* M,
                         const uint16_t* M_lo, const float* P, const float* O_on, void* Y,
                         int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * mc_decode_step -- one new token per sequence (paper §3 applied to token t+1): for every
 * (b, h) the online memory is updated with the token (Eq. 4b), the gate runs over the
 * *n_cached cached segments plus the online one (Eq. 10), and y reads all of them (Eq. 9).
 * If the online segment then holds C tokens, its state (rounded to the cache dtype) and its
 * mean are appended at slot *n_cached, the online state and x sum restart from zero, and
 * *n_cached is incremented.  All sequences share *count_on and *n_cached.
 *
 *   dims: B, H, d_k, d_v, d_g, seg_len, x_heads, dtype, phi (L is ignored)
 *   q, k [B,H,d_k]; v [B,H,d_v]; u [B,H,d_g]; x [B,x_heads,d_g]: dtype
 *   u may be NULL: every logit is then 0 and y is the plain mean of the n_cached + 1
 *            memories -- memory caching applied after pre-training (the paper's appendix on
 *            the MC variants: decoding averages the cached memories, no learned weights).
 *            The cache bookkeeping (x sums, means, emission) is unchanged.
 *   M_on     in/out [B,H,d_v,d_k] fp32  online state before / after the token
 *   xsum_on  in/out [B,x_heads,d_g] fp32 sum of x over the online segment
 *   count_on host in/out: tokens in the online segment, 0..C-1 on entry
 *   M_cache  in/out [B,H,n_cap,d_v,d_k]  bf16 (MC_BF16) or fp32 (MC_F32)
 *   P_cache  in/out [B,x_heads,n_cap,d_g] fp32
 *   n_cached host in/out: cached segments, 0..n_cap
 *   y        out [B,H,d_v] dtype
 *   ws       mc_workspace_bytes(dims, MC_OP_DECODE, 0, n_cap) bytes
 *   Returns MC_ERR_CAPACITY (and changes nothing) if the step would append to a full cache.
 */
mc_status mc_decode_step(const mc_dims* dims, const void* q, const void* k, const void* v,
                         const void* u, const void* x, float* M_on, float* xsum_on,
                         int32_t* count_on, void* M_cache, float* P_cache, int32_t* n_cached,
                         int32_t n_cap, void* y, void* ws, size_t ws_bytes, void* stream);

/*
 * mc_decode_step_noalloc -- mc_decode_step without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  It runs the same kernels on the same arguments (all of
 * them as mc_decode_step, minus ws / ws_bytes) and gives the same results; the scratch they
 * need (the partial softmaxes of the runs of cached states) is a fixed buffer of
 * MC_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on until the process
 * ends.  The call allocates and frees nothing.
 *
 *   The scratch needed is mc_workspace_bytes(dims, MC_OP_DECODE, 0, *n_cached) bytes; if
 *   that exceeds MC_NOALLOC_SCRATCH_BYTES the call returns MC_ERR_SCRATCH and changes
 *   nothing (64 sequences x 32 heads x d_v = 128 fit up to 496 cached states).
 *   The buffer is that of the current device, which must be the device of `stream`.  Every
 *   call on one GPU uses the same buffer and every region of it that a step reads is first
 *   written by that step, so nothing carries over between calls; but calls that may run at
 *   the same time on one GPU (on different streams, or from several host threads without
 *   ordering) race on it and must be serialised by the caller.
 *   Errors otherwise as mc_decode_step; a failure to obtain the buffer's device address
 *   returns MC_ERR_HIP.
 */
mc_status mc_decode_step_noalloc(const mc_dims* dims, const void* q, const void* k,
                                 const void* v, const void* u, const void* x, float* M_on,
                                 float* xsum_on, int32_t* count_on, void* M_cache,
                                 float* P_cache, int32_t* n_cached, int32_t n_cap, void* y,
                                 void* stream);

/*
 * Arbitrary segment boundaries (Memory Caching paper §3, Eq. 4b: segment s has its own
 * length L^(s); gitcode explainer §4.2: the logarithmic segmentation, one segment per set bit
 * of L, largest first).  The same write path and GRM read, with segment i holding the tokens
 * [seg_off[i], seg_off[i+1]) instead of a constant length:
 *
 *   seg_off  HOST array of n_seg + 1 int32: 0 = seg_off[0] < seg_off[1] < ... < seg_off[n_seg]
 *            = L.  It is read when the call is made (passed to the kernels by value), so the
 *            caller may reuse it at once.  dims->seg_len is ignored (it must still be >= 1).
 *   n_seg    1 <= n_seg <= MC_MAX_SEGS; NS = n_seg below.
 *   The other arguments are those of mc_scan_prefill / mc_grm_readout with NS = n_seg, except
 *   that the read takes the online read O_on written by mc_scan_prefill_segs (required), not
 *   K and V.  Its workspace is mc_workspace_bytes(dims, MC_OP_GRM_SEGS, n_seg, 0) bytes; with
 *   that much (bf16, d_k = d_v = 128) the gate runs as its own pass over the offsets ahead of
 *   the read, as in mc_grm_readout.  mc_workspace_bytes(dims, MC_OP_GRM, 0, 0) bytes are
 *   also accepted; the read then forms the gate itself.
 *   The write path's workspace is mc_workspace_bytes(dims, MC_OP_SCAN_SEGS, n_seg, 0) bytes
 *   (0 for fp32: NULL allowed): bf16 segments longer than a piece (512 tokens, or the
 *   smallest power of two above it that keeps the pieces within MC_MAX_SEGS) are scanned as
 *   pieces in parallel, whose states and prefix sums it holds, with the pieces' means of X
 *   (a segment's mean is then combined from its pieces' in order).
 *   bf16 inputs of width 64/128 run on MFMA (scan and read); the rest on the
 *   fp32-accumulating kernels that take any segmentation.
 *   Errors as the constant-length calls; offsets that are not strictly increasing from 0 to L
 *   return MC_ERR_DIMS, more than MC_MAX_SEGS segments MC_ERR_UNSUPPORTED.
 */
#define MC_MAX_SEGS 512

mc_status mc_scan_prefill_segs(const mc_dims* dims, const int32_t* seg_off, int32_t n_seg,
                               const void* Q, const void* K, const void* V, const void* X,
                               float* M, uint16_t* M_lo, float* P, float* O_on, void* ws,
                               size_t ws_bytes, void* stream);

mc_status mc_grm_readout_segs(const mc_dims* dims, const int32_t* seg_off, int32_t n_seg,
                              const void* Q, const void* U, const void* X, const float* M,
                              const uint16_t* M_lo, const float* P, const float* O_on, void* Y,
                              float* gamma, void* ws, size_t ws_bytes, void* stream);

/*
 * mc_grm_prefill_segs -- the whole GRM prefill over segment offsets in one call: the write
 * path of mc_scan_prefill_segs (M, M_lo, P) and the read of mc_grm_readout_segs (Y, gamma),
 * with the same offsets, arguments and errors, except that no online read O_on is handed over:
 * for bf16 with d_k = d_v = 128 (after the gate pass) the read forms the online term
 * M_t^(s) phi(q_t) itself from K and V (Memory Caching paper §3.1, Eq. 8), walking the keys of
 * the token's piece -- long segments are cut into pieces as in mc_scan_prefill_segs -- and
 * adding the memory of the segment's earlier pieces, so the sequence is scanned once.  Other
 * sizes, and segmentations with a segment longer than 1024 tokens that no piece length
 * cuts, form O_on in the workspace and read it.
 *   ws  mc_workspace_bytes(dims, MC_OP_GRM_PREFILL_SEGS, n_seg, 0) bytes (it holds the scan's
 *       pieces, the memories before them or O_on, and the read's buffers).
 */
mc_status mc_grm_prefill_segs(const mc_dims* dims, const int32_t* seg_off, int32_t n_seg,
                              const void* Q, const void* K, const void* V, const void* U,
                              const void* X, float* M, uint16_t* M_lo, float* P, void* Y,
                              float* gamma, void* ws, size_t ws_bytes, void* stream);

/*
 * mc_ssc_readout_segs -- the Sparse Selective Caching read of mc_ssc_readout (explainer §3.4)
 * over arbitrary segment boundaries (Memory Caching paper §3, Eq. 4b: segment s has its own
 * length).  Token t of segment s selects among the segments i < s; every router score is
 * formed in fp64 with the segment's x values summed in token order and divided by that
 * segment's own length, then ranked as in mc_ssc_readout (ties to the lower index).
 *
 *   seg_off, n_seg  host offsets as for mc_scan_prefill_segs (NS = n_seg).
 *   top_k    1 <= top_k <= 16
 *   Q, U, X, M, M_lo, P  as for mc_grm_readout_segs with NS = n_seg.
 *   O_on     [B,H,L,d_v] fp32, required: the online read written by mc_scan_prefill_segs
 *            (or mc_scan_prefill_swla).
 *   Y        out [B,H,L,d_v] dtype;  idx  out [B,H,L,top_k] int32, ascending, -1 padded
 *   ws       mc_workspace_bytes(dims, MC_OP_SSC_SEGS, top_k, n_seg) bytes
 *   bf16 with d_k = d_v = 128 runs the routed read (only the selected states are loaded);
 *   the rest runs the fp32-accumulating read restricted to the selections.
 *   Errors as mc_ssc_readout and mc_grm_readout_segs.
 */
mc_status mc_ssc_readout_segs(const mc_dims* dims, const int32_t* seg_off, int32_t n_seg,
                              int32_t top_k, const void* Q, const void* U, const void* X,
                              const float* M, const uint16_t* M_lo, const float* P,
                              const float* O_on, void* Y, int32_t* idx, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * SWLA memory under Memory Caching (Memory Caching paper, the sliding-window linear
 * attention paragraph: Eq. 26 with window c = 2, i.e. Eq. 28 for the segment memories and
 * Eq. 29 for the read).  The write path with the update
 *     M_t = alpha_t M_{t-1} + beta_t v_{t-1} phi(k_{t-1})^T + lambda_t v_t phi(k_t)^T
 * in place of the linear-attention one.  The window stays inside the segment: a segment's
 * first token has no previous token to write, its memory starting from zero (Eq. 4b).  The
 * read is unchanged (Eq. 29): pass the O_on written here to mc_grm_readout (constant
 * segments) or mc_grm_readout_segs (offsets), or to mc_ssc_readout.
 *
 *   seg_off, n_seg  NULL for segments of dims->seg_len; else host offsets as for
 *                   mc_scan_prefill_segs.
 *   alpha, beta, lambda  [B,H,L] fp32 device arrays: the decay and the two window weights of
 *                   every token of every head (any finite values; alpha = 1, beta = 0,
 *                   lambda = 1 is the linear-attention memory).
 *   Q, K, V, X, M, M_lo, P  as for mc_scan_prefill.
 *   O_on     out [B,H,L,d_v] fp32, required: the online read M_t^(s) phi(q_t); the gated
 *            read cannot form a decayed online term itself.
 *   Constant bf16 segments with d_k, d_v in {64, 128} run on MFMA; everything else on the
 *   fp32-accumulating kernels.  Errors as mc_scan_prefill and mc_scan_prefill_segs.
 */
mc_status mc_scan_prefill_swla(const mc_dims* dims, const int32_t* seg_off, int32_t n_seg,
                               const float* alpha, const float* beta, const float* lambda,
                               const void* Q, const void* K, const void* V, const void* X,
                               float* M, uint16_t* M_lo, float* P, float* O_on, void* stream);

/*
 * Backward of the GRM prefill (training): the gradients of a loss with respect to Q, K, V,
 * U and X, given its gradient dY with respect to the output Y of mc_grm_readout (Memory
 * Caching paper: the Eq. 4b segment memories, the Eq. 10 softmax gate and the Eq. 9 read,
 * differentiated token by token; the chain rule through phi, the softmax, the segment
 * means and the causal prefix means of the online segment).  Constant segments of
 * dims->seg_len.
 *
 *   Q, K, V, U, X       the forward inputs (dtype, layouts as mc_grm_readout)
 *   M, M_lo, P          the states and means mc_scan_prefill wrote for them (M_lo is read
 *                       for MC_BF16, M for MC_F32; the other may be NULL)
 *   dY       [B,H,L,d_v] dtype
 *   dQ, dK   out [B,H,L,d_k] fp32;  dV out [B,H,L,d_v] fp32;  dU out [B,H,L,d_g] fp32
 *   dX       out [B,x_heads,L,d_g] fp32 (with x_heads = 1 the heads' gradients are summed)
 *   ws       mc_workspace_bytes(dims, MC_OP_GRM_BACKWARD, 0, 0) bytes
 *   The forward states are recomputed where needed (the online read and its transpose);
 *   every sum accumulates in fp32.  Errors as mc_grm_readout.
 */
mc_status mc_grm_backward(const mc_dims* dims, const void* Q, const void* K, const void* V,
                          const void* U, const void* X, const float* M, const uint16_t* M_lo,
                          const float* P, const void* dY, float* dQ, float* dK, float* dV,
                          float* dU, float* dX, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MC_H */
