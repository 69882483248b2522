/* MFMA throughput probe (libflce_probe.so), a measuring aid beside libflce.so.
 *
 * The fused cross-entropy kernels are contractions on the bf16 matrix
 * instructions; their roofline is the chip's dense bf16 peak.  This probe
 * measures what those instructions sustain alone -- operands in registers,
 * no memory traffic -- with random or zero operands, so that the gap
 * between a kernel's rate and the peak can be split into what the clock
 * (power) takes and what the kernel's own schedule takes.  It is not part of
 * the fused path and computes nothing the method needs.
 */
#ifndef FLCE_PROBE_H
#define FLCE_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue one launch of `blocks` blocks of 4 waves on `stream` (a
 * hipStream_t, NULL = the default stream); every wave issues `iters` rounds
 * of bf16 MFMAs into independent accumulators:
 *   shape 16: v_mfma_f32_16x16x32_bf16, 16 accumulators per round;
 *   shape 32: v_mfma_f32_32x32x16_bf16, 8 accumulators per round.
 * random_operands != 0 fills the operand registers with pseudo-random bf16
 * values (full mantissas, both signs, magnitudes in [2^-8, 2^8)); 0 leaves
 * them zero.  `sink` is caller-owned device memory of blocks*256 floats; each
 * thread writes the sum of its accumulators there (0 for zero operands), so
 * the work cannot be optimised away.
 * Returns 0 on success, 1 for a bad argument (shape not 16 or 32, blocks or
 * iters not positive, sink NULL: nothing is launched), 3 if the launch
 * failed.  The call does not synchronise. */
int32_t flce_probe_mfma_stream(int32_t shape, int32_t blocks, int32_t iters,
                               int32_t random_operands, float* sink, void* stream);

/* Floating-point operations of one such launch (2 per multiply-add; the two
 * shapes do the same work per round), or 0 for an unknown shape. */
double flce_probe_mfma_flops(int32_t shape, int32_t blocks, int32_t iters);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_PROBE_H */
