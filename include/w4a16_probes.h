/*
 * w4a16_probes.h -- measurement probes of libw4a16_probes.so (a separate
 * library; nothing in the GEMM library uses it).
 *
 * They measure what the chip sustains on the two resources that bound a
 * weight-only INT4 GEMM -- the HBM rate at which weights stream in the
 * memory-bound regime and the FP16 matrix-instruction rate in the
 * compute-bound one ("Quant Marlin kernel" explainer, "The architecture",
 * bottom rows: check a kernel against the roofline of the hardware) -- so
 * that measured GEMM rates can be set beside achievable ceilings as well as
 * the published peaks.  The caller times them (HIP events on `stream`).
 *
 * All launches are asynchronous on `stream` (a hipStream_t; NULL is the
 * null stream).  Return 0, -1 for a bad argument (nothing launched), -6 for
 * a launch failure.  Nothing allocates.
 */
#ifndef W4A16_PROBES_H
#define W4A16_PROBES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a multiple of 16, >= 16) of device memory at `buf` (16-byte
 * aligned) once, with 16-byte non-temporal loads, over `blocks` workgroups
 * of 512 threads.  `sink` (device, one uint32) is written only for a value
 * the reads cannot be expected to produce; it must be valid device memory. */
int w4a16_probe_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, void* stream);

/* Run `iters` rounds of sixteen independent v_mfma_f32_16x16x32_f16 in each
 * of the four waves of `blocks` workgroups, on register operands.  `sink`
 * (device, one float) as above. */
int w4a16_probe_mfma(float* sink, int blocks, int iters, void* stream);

/* Floating-point operations of one w4a16_probe_mfma launch. */
double w4a16_probe_mfma_flops(int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_PROBES_H */
