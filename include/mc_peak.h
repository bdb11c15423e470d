/*
 * mc_peak.h -- C ABI of libmcpeak: in-run ceilings for the benchmark of libmc.
 *
 * Not part of the Memory Caching operations (those are in mc.h).  The gated prefill read of
 * Memory Caching is a dense bf16 contraction and its decode read streams every cached state
 * from HBM; these calls measure the two ceilings on the GPU the benchmark runs on.
 *
 * Every pointer is a device pointer owned by the caller; calls only enqueue a kernel on
 * `stream` (a hipStream_t, NULL = default) and never synchronise; the caller times them with
 * events on that stream.  Return value: 0 ok, 1 invalid argument (nothing enqueued), 2 the
 * launch failed.
 */
#ifndef MC_PEAK_H
#define MC_PEAK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core loop: n_blocks workgroups of 4 waves, each wave issuing 16 * iters
 * v_mfma_f32_32x32x16_bf16 from registers.  out: mcpeak_mfma_out_floats(n_blocks) floats.
 * mcpeak_mfma_flops gives the launch's floating-point operations (2 per multiply-add). */
int mcpeak_mfma_out_floats(int n_blocks);
double mcpeak_mfma_flops(int n_blocks, int iters);
int mcpeak_mfma(int n_blocks, int iters, float* out, void* stream);

/* Streaming read of `bytes` (multiple of 16, 16-byte aligned) with n_blocks workgroups of 256
 * threads.  out: mcpeak_stream_out_words(n_blocks) words (a fold of what was read). */
int mcpeak_stream_out_words(int n_blocks);
int mcpeak_stream_read(const void* src, size_t bytes, int n_blocks, uint32_t* out, void* stream);

/* dst[0:bytes] = src[0:bytes] (multiple of 16, both 16-byte aligned, not overlapping): the
 * kernel of known traffic that HBM byte counters are scaled by. */
int mcpeak_copy(const void* src, void* dst, size_t bytes, int n_blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MC_PEAK_H */
