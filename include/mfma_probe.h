/*
 * mfma_probe.h -- C ABI of libmfma_probe.so: a pure matrix-core loop that
 * measures what the MI355X bf16 MFMA pipes sustain on this device, with
 * random operand data and no memory traffic, and at what shader clock.
 *
 * It is a measurement aid for the attention benchmark (the sustainable
 * ceiling under the board's power limit is well below the 2.5 PFLOP/s
 * datasheet figure, which assumes the 2.4 GHz peak clock); it computes
 * nothing the attention path uses.
 *
 * mfma_probe_launch: enqueues `blocks` work-groups of 256 threads on
 * `stream`; each wave runs 16 * iters v_mfma_f32_32x32x16_bf16 on operands
 * drawn from a hash of its indices (bf16 values of magnitude 0.5 .. 1 with
 * random sign and mantissa, like N(0,1) data), i.e.
 *     flops = blocks * 4 waves * iters * 16 * 32768.
 *   sink   : device float [blocks * 256], written (keeps the results live)
 *   clocks : device uint64 [2 * blocks]: per block, shader-clock cycles and
 *            100 MHz reference ticks spent in the loop (clock = ratio * 100 MHz)
 * Returns 0, -1 for a null pointer or non-positive count, or -100 when the
 * launch fails.  Allocates nothing; the caller owns both buffers.
 */
#ifndef MFMA_PROBE_H_
#define MFMA_PROBE_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int mfma_probe_launch(float* sink, uint64_t* clocks, int blocks, int iters, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MFMA_PROBE_H_ */
