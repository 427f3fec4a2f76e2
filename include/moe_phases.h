/*
 * moe_phases.h -- C ABI of libmoe_phases, a measurement build of libmoe.
 *
 * libmoe_phases.so exports everything libmoe.so exports (moe.h), with the same
 * behaviour and the same results; its bf16 grouped-GEMM kernels also read the
 * shader clock around each phase of every main-loop iteration and store, per
 * wavefront, how many cycles it spent
 *   [0] waiting for its own loads (activation tile and weights),
 *   [1] waiting at the workgroup barrier,
 *   [2] issuing the activation loads and its MFMAs (including the LDS reads
 *       of the activation fragments and any wait for the matrix core),
 *   [3] issuing its weight loads,
 * (in the ping-pong main loop of the compute-heavy tiles: [0] waits for its
 * loads and LDS reads, [1] barriers, [2] its MFMA phases, [3] issuing its
 * loads and LDS fragment reads), followed by [4] the cycles of the whole
 * loop, [5] its iterations, [6] the loop's duration in ticks of the constant
 * 100 MHz counter (so [4] / [6] * 100 MHz is the shader clock over the loop)
 * and [7] = 1, as 8 uint64 per slot.  Slot =
 * (workgroup id * wavefronts per workgroup + wavefront) modulo
 * MOE_PHASE_SLOTS.  Only main loops without a K split inside the workgroup
 * (tiles of 96 rows and more) record.  It is for measuring where a GEMM's
 * time goes; the product library is libmoe.so, which has none of this.
 *
 * Both calls act on the device that is current.  dst: HOST memory of
 * MOE_PHASE_SLOTS * 8 uint64, written when clear == 0; clear != 0 zeroes the
 * device buffer instead (dst unused).  Synchronous.  Return 0 on success,
 * 1 on a HIP error.  Calls that overlap a GEMM launch race with it.
 */
#ifndef MOE_PHASES_H
#define MOE_PHASES_H

#define MOE_PHASE_SLOTS (1 << 17)

#ifdef __cplusplus
extern "C" {
#endif

/* phase sums of the last bf16 fused gate+up launches */
int moe_loop_phases_gateup(void* dst, int clear);
/* phase sums of the last bf16 down-projection launches */
int moe_loop_phases_down(void* dst, int clear);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PHASES_H */
