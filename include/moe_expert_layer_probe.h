/*
 * moe_expert_layer_probe.h - the one extra entry point of the probe library
 * (libmoe_expert_layer_probe.so), a build of the same sources with MOE_PHASE_PROBE defined.
 *
 * In that build the large-tile bf16 grouped GEMMs (fc1, fc2 and the backward's recompute of g and
 * u), the backward's LDS-DMA GEMMs (weight gradients, down and gate/up dgrads) and the large-tile
 * MX-FP8 grouped GEMMs (fc1, fc2) read the cycle
 * counter at fixed points of their task loop and add per-workgroup sums to device arrays; every
 * kernel does the same work as in the product library (the stamps only add instructions).  The
 * product library does not export this function.
 *
 * For callers that measure where a GEMM launch spends its cycles, not for the compute path.
 */
#ifndef MOE_EXPERT_LAYER_PROBE_H
#define MOE_EXPERT_LAYER_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Fields per kernel kind, in order: 0 cycles from the previous task's epilogue end (or the
 * kernel's start) past the task's top barrier; 1 K loops; 2 K loops of full-height, full-width
 * tasks; 3 from the K loop's end past the barrier that ends it; 4 the next task's setup (its
 * first copies); 5 epilogues; 6 tasks; 7 full-height, full-width tasks; 8 cycles from the kernel's
 * start to the workgroup's end; 9 the same span in ticks of the 100 MHz real-time counter;
 * 10 workgroups; 11 K steps over all tasks (32 bf16 or 64 fp8 elements of K; either issues 1024
 * cycles of MFMAs per SIMD).
 * Counts of cycles are wave 0's, summed over workgroups and launches.
 */
#define MOE_PROBE_FIELDS 12
/*
 * Kernel kinds: 0 fc2 (down projection), 1 fc1 (gate and up), 2 the backward's recompute of g and u,
 * 3 the weight gradients, 4 the down dgrad (with the SwiGLU backward), 5 the gate/up dgrad,
 * 6 MX-FP8 fc2, 7 MX-FP8 fc1.
 */
#define MOE_PROBE_KINDS 8

/*
 * Copies the sums since the last reset into out (host, MOE_PROBE_KINDS * MOE_PROBE_FIELDS
 * unsigned 64-bit values, kind-major) unless out is null, then zeroes them when reset is non-zero.
 * Waits for all work on the current device first.  Returns 0, or 1 when a runtime call failed.
 * Launches that run while it executes are not counted reliably.
 */
int moe_probe_phases(unsigned long long* out, int reset);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EXPERT_LAYER_PROBE_H */
