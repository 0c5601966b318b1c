/*
 * la_probe.h -- measurement aid beside the GEMM library (same shared library,
 * liblagemm.so), not part of any computation in la_gemm.h.
 *
 * The matrix cores' power depends on the operand bits, and the chip lowers
 * its clock to stay inside its power limit, so the rate an MFMA-bound kernel
 * can reach on a given workload is set by that workload's values as well as
 * by the nominal peak.  This probe measures that rate so that benchmarks can
 * report it next to the nominal roofline.
 */
#ifndef LA_PROBE_H
#define LA_PROBE_H

#include <stdint.h>

#include "la_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core rate probe -- a measurement aid, not part of any computation
 * above.  Launches `workgroups` workgroups of 4 waves (one wave per SIMD of a
 * CU); every lane loads eight 16-byte operand fragments from `operands`
 * (fragment f at byte 16 * (f mod (operand_bytes / 16))) and issues
 * mfma_per_wave v_mfma_f32_32x32x16 instructions (bf16 or f16 per in_type),
 * v_mfma_f32_32x32x2_f32 on the first word of each fragment (GEMM_F32), or
 * v_mfma_f32_32x32x64_f8f6f4 on E4M3 codes (GEMM_F8E4M3; operand i of each side
 * is fragments i and (i + 1) mod 4 of that side), in 16 independent accumulator chains, with no other memory traffic, then
 * writes the sum of its accumulators to sink[lane id] (workgroups * 256
 * floats, device memory).  Timed by the caller, it gives the rate the matrix
 * cores sustain on those operand values at the clock the chip settles to
 * under that load, the practical ceiling for the MFMA-bound kernels next to
 * the nominal peak.  operands: device pointer, 16-byte aligned,
 * operand_bytes a positive multiple of 16; 1 <= workgroups <= 2^20;
 * mfma_per_wave a positive multiple of 16, <= 2^24.  Asynchronous on
 * `stream`, allocates nothing. */
gemm_status la_probe_mfma(const void* operands, int64_t operand_bytes, float* sink, int64_t workgroups,
                          int64_t mfma_per_wave, int32_t in_type, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LA_PROBE_H */
