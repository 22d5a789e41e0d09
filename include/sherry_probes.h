/* sherry_probes.h -- measured ceilings for the rooflines of the products in
 * sherry.h (streaming HBM reads, the int8 matrix-core and v_dot4 rates, and
 * whether the two overlap).  Same conventions as sherry.h: extern "C",
 * device pointers owned by the caller, host-side validation (a status and
 * nothing enqueued on error), asynchronous on `stream`.  Measurement aids
 * beside the published peaks; the products do not use them. */
#ifndef SHERRY_PROBES_H
#define SHERRY_PROBES_H

#include "sherry.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (> 0, a multiple of 16) from `src` (16-byte aligned device
 * memory) once, with 16-byte non-temporal loads: up to 64 workgroups per CU,
 * each streaming one contiguous chunk.  `sink`: device buffer of 256
 * uint32 (4-byte aligned), written only in the practically impossible case
 * that the XOR of a thread's data equals a fixed constant (the store keeps
 * the loads).  Time it with events: the
 * achieved read bandwidth is bytes / time. */
sherry_status sherry_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Rate probe: `blocks` workgroups of 4 waves each run `iters` iterations
 * (1 .. 2^24; blocks 1 .. 2^20).  Per iteration a working wave issues
 *   matrix-core work: 4 independent v_mfma_i32_16x16x64_i8 (4 x 32768 ops),
 *   VALU work:        16 independent v_dot4_i32_i8 (16 x 512 ops),
 * by mode (also SHERRY_PROBE_MFMA32 below): SHERRY_PROBE_MFMA (every wave, matrix cores only),
 * SHERRY_PROBE_DOT4 (every wave, VALU only), SHERRY_PROBE_SAME_WAVE (every
 * wave does both, interleaved), SHERRY_PROBE_ALT_WAVES (even waves of a
 * workgroup the matrix-core work, odd waves the VALU work).  `sink` as in
 * sherry_probe_read.  If the two kinds of work overlap, the SAME_WAVE time
 * is close to the larger of the MFMA and DOT4 times; if not, to their sum. */
enum { SHERRY_PROBE_MFMA = 0, SHERRY_PROBE_DOT4 = 1, SHERRY_PROBE_SAME_WAVE = 2, SHERRY_PROBE_ALT_WAVES = 3,
       SHERRY_PROBE_MFMA32 = 4, SHERRY_PROBE_ALU = 5, SHERRY_PROBE_SAME_ALU = 6 };
/* SHERRY_PROBE_MFMA32: every wave, matrix cores only, as 2 independent
 * v_mfma_i32_32x32x32_i8 per iteration (the same 2 x 65536 ops per iteration
 * as the MFMA mode's four 16 x 16 x 64 products).
 * SHERRY_PROBE_ALU: every wave, plain 32-bit VALU only: 16 independent
 * chains of shift, mask and add per iteration (48 operations).
 * SHERRY_PROBE_SAME_ALU: every wave issues both the MFMA mode's matrix-core
 * work and the ALU mode's operations, interleaved. */
sherry_status sherry_probe_rates(int32_t mode, int32_t iters, int32_t blocks, uint32_t* sink, hipStream_t stream);

/* The rate probe with a clock record: thread 0 of workgroup b writes the
 * shader-clock counter (s_memtime) and the constant 100 MHz counter
 * (s_memrealtime) read before and after its wave's loop to ticks[4 b + 0]
 * (clock, start), [4 b + 1] (clock, end), [4 b + 2] (100 MHz, start) and
 * [4 b + 3] (100 MHz, end).  ticks: device buffer of 4 * blocks uint64,
 * 8-byte aligned.  The ratio of the two spans gives the shader clock while
 * the probe ran, so a rate can be compared with the peak at that clock.
 * Errors as sherry_probe_rates, plus EINVAL for a null ticks and EALIGN for
 * a misaligned one. */
sherry_status sherry_probe_clock(int32_t mode, int32_t iters, int32_t blocks, uint32_t* sink, uint64_t* ticks,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SHERRY_PROBES_H */
