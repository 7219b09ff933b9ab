/*
 * atlasmem calibration -- measuring instruments for the rooflines the kernels are reported
 * against.  These are not steps of the neural-memory update: they time what the chip itself
 * reaches, so that each kernel's rate can be put next to a measured ceiling as well as the vendor
 * one.  Same conventions as atlasmem.h (device pointers, stream as void*, status codes).
 */
#ifndef ATLASMEM_CALIBRATION_H
#define ATLASMEM_CALIBRATION_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The dense bf16 matrix-core rate: n_workgroups workgroups of eight waves (two per SIMD) each run
 * `iters` rounds of eight independent v_mfma_f32_32x32x16_bf16 chains (32768 FLOP per
 * instruction), so the chip's matrix cores stay busy without memory traffic.  One float per
 * workgroup is written to `sink` ([n_workgroups] fp32, device) so that the work is not removed.
 * FLOPs of one call = n_workgroups * 8 waves * iters * 8 * 32768.
 * Errors: E_INVALID for iters < 1, n_workgroups < 1 or a null sink. */
int atlasmem_calibrate_mfma(int64_t iters, int32_t n_workgroups, float* sink, void* stream);

/* A plain streaming copy of `bytes` bytes (a multiple of 16) from src to dst (device, not
 * overlapping), 16-byte loads and stores: the reference for HBM read / write counters and for the
 * copy bandwidth the chip reaches.  Errors: E_INVALID for bad sizes or null pointers. */
int atlasmem_calibrate_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATLASMEM_CALIBRATION_H */
