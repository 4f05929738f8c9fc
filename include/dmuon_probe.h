/* dmuon_probe.h — a measurement probe that sits beside the Muon step library
 * (libdmuon_probe.so, built with it).  It is not part of the step.
 *
 * The step's bf16 contractions run on v_mfma_f32_16x16x32_bf16.  Under a sustained
 * load the board's power limit, not the 2.5 PFLOP/s dense bf16 figure, decides
 * how fast those instructions can go on operands with random bits.  The probe
 * measures that ceiling: every wave issues only matrix-core instructions on
 * register operands (no memory traffic inside the loop), so a caller that times
 * it for a few seconds sees what the matrix cores alone sustain at the limit.
 *
 * Conventions: device pointers, asynchronous on the given stream (NULL = the
 * default stream), return value DMUON_OK or a negative DMUON_E_* code from
 * dmuon_ns.h; dmuon_probe_last_error() describes the last failure of this
 * library's calls on the calling thread.
 */
#ifndef DMUON_PROBE_H
#define DMUON_PROBE_H

#include <stdint.h>

#include "dmuon_ns.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Operand contents of the probe's instructions. */
typedef enum {
  DMUON_PROBE_RANDOM = 0, /* bf16 with random sign and mantissa, exponents 2^-7 .. 2^6 */
  DMUON_PROBE_ZERO = 1    /* all-zero operands (the unloaded bound) */
} dmuon_probe_operands;

/* Launch `blocks` workgroups of 256 threads; every wave runs `iters` rounds of
 * 8 independent v_mfma_f32_32x32x16_bf16 (shape 32) or 16 independent
 * v_mfma_f32_16x16x32_bf16 (shape 16) on register operands.  One round is
 * 131072 multiply-adds per wave for either shape, so a launch performs
 * blocks × 4 × iters × 262144 floating-point operations.  Each thread writes the
 * sum of its accumulators to sink[global thread index] (sink: blocks × 256
 * floats, device), which keeps the work from being optimised away; with
 * DMUON_PROBE_ZERO every sink entry is 0.
 * shape ∈ {16, 32}, 1 ≤ blocks ≤ 65536, 4 ≤ iters ≤ 2^24 and a multiple of 4,
 * operands a dmuon_probe_operands value; otherwise DMUON_E_SHAPE (DMUON_E_NULL
 * for a NULL sink) before anything is enqueued. */
int dmuon_probe_mfma(int32_t shape, int32_t operands, int32_t blocks, int32_t iters, float* sink, void* stream);

/* Text of the last failure of a call of this library on this thread ("" after a
 * success). */
const char* dmuon_probe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DMUON_PROBE_H */
