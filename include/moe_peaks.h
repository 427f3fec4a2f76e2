/*
 * moe_peaks.h -- C ABI of libmoe_peaks, measurement probes for MI355X
 * (gfx950) that give the achievable peaks a roofline is drawn against.
 *
 * They are not part of the MoE layer.  A roofline of the expert GEMMs needs
 * its ceilings (the TritonMoE review, pith.science verdict for arXiv
 * 2605.23911, minor comments: its Figure 1 roofline lacks the peak lines);
 * the datasheet gives HBM3E 8 TB/s and 2.5 PFLOP/s of dense bf16 MFMA, and
 * these probes measure what plain kernels reach on the device at hand:
 *  - a streaming read and a streaming copy of a large buffer (HBM ceiling);
 *  - a loop of independent bf16 MFMAs with register operands (matrix-core
 *    ceiling).
 * Each probe leaves a result the caller can check exactly, so a probe that
 * skipped work would be caught.
 *
 * Conventions: pointers are DEVICE pointers; the caller allocates every
 * buffer; work is enqueued on `stream` (NULL = the null stream) and the call
 * returns at once; the caller times it (HIP events on the same stream).
 * Arguments are checked on the host first: on an invalid argument nothing is
 * enqueued and the call returns 1; a launch failure reported by
 * hipGetLastError returns 5 (the codes of moe_status_t in moe.h).
 */
#ifndef MOE_PEAKS_H
#define MOE_PEAKS_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` bytes at `buf` (bytes a positive multiple of
 * 1024, buf 16-byte aligned).  `blocks` workgroups of 512 threads; each
 * wavefront reads whole 1 KB chunks (lane l: bytes 16l..16l+15 of a chunk),
 * issuing the loads of 8 (strided) or 16 (regions) chunks before using any.
 * flags (0..3): bit 0 = loads with the non-temporal cache policy; bit 1 =
 * each wavefront reads one contiguous region of the buffer (nch / (8*blocks)
 * chunks, nch = bytes / 1024, the chunks left over going one to each of the
 * first wavefronts), else chunk c goes to wavefront c mod (8*blocks).
 * sink[b] (sink: `blocks` words) receives the XOR of every 32-bit word
 * workgroup b read, so the XOR of all of sink equals the XOR of every word of
 * the buffer. */
int moe_peak_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, int flags, hipStream_t stream);

/* Streaming copy: dst[i] = src[i] for `bytes` bytes (a positive multiple of
 * 1024; both 16-byte aligned, not overlapping), with the chunk order and
 * flags of moe_peak_read (bit 0 also makes the stores non-temporal). */
int moe_peak_copy(const void* src, void* dst, size_t bytes, int blocks, int flags, hipStream_t stream);

/* Matrix-core loop: `blocks` workgroups of 256 threads (one wavefront per
 * SIMD); each wavefront runs `iters` rounds of 8 independent
 * v_mfma_f32_16x16x32_bf16 (16x16x32 products, 16384 FLOPs each) on operands
 * whose every element is the bf16 value of `a` and `b` (truncated to bf16).
 * sink[4*blk + w] (sink: 4*blocks floats) receives the sum of element 0 of
 * wavefront w's eight accumulators: exactly 256 * iters * a * b when a and b
 * are small integers and that value is at most 2^24 (for example a = b = 1,
 * iters <= 65536).  FLOPs launched: blocks * 4 * 8 * iters * 16384.
 * iters >= 1. */
int moe_peak_mfma(float a, float b, int iters, float* sink, int blocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PEAKS_H */
