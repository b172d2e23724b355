/*
 * moe_peaks.h — probes of the MI355X ceilings that the MoE layer's roofline
 * fractions are quoted against (not an operation of the layer).
 *
 * The layer's expert GEMMs run the gfx950 scaled matrix instruction
 * V_MFMA_SCALE_F32_32X32X64_F8F6F4 on MXFP4 weights ("gpt-oss architecture
 * walk-through", section "Quantization": 4-bit values, one 8-bit scale per 32)
 * and, at decode sizes, stream those weights from HBM.  These probes measure
 * what the chip sustains for each: the issue rate of the matrix instruction for
 * one pair of operand formats, and the rate of a plain streaming read.  The
 * caller times a launch (HIP events on `stream`) and divides the work below by
 * the time.  libmoe_peaks.so, built beside libmoe_mxfp4.so; it shares no code
 * with the layer.
 *
 * Conventions: device pointers are caller-owned; arguments are checked on the
 * host before the launch (MOE_PEAK_EINVAL, nothing launched); a launch error
 * returns MOE_PEAK_EHIP.
 */
#ifndef MOE_PEAKS_H
#define MOE_PEAKS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_PEAK_OK = 0, MOE_PEAK_EINVAL = 1, MOE_PEAK_EHIP = 4 } moe_peak_status;

/* Operand formats of the probes. */
typedef enum {
  MOE_PEAK_FP6_FP4 = 0,     /* scaled 32x32x64, A FP6 E2M3, B FP4 E2M1 (the layer's default path) */
  MOE_PEAK_FP4_FP4 = 1,     /* scaled 32x32x64, A and B FP4 E2M1 (the MXFP4-activation path) */
  MOE_PEAK_FP8_FP4 = 2,     /* scaled 32x32x64, A FP8 E4M3, B FP4 E2M1 */
  MOE_PEAK_BF16 = 3         /* 32x32x16 bf16 (the router) */
} moe_peak_format;

/*
 * Matrix-instruction rate: `workgroups` workgroups of 4 wavefronts, each
 * wavefront issuing iters x 4 independent instructions of `format` back to back.
 *   work = workgroups * 4 * iters * 4 * flops_per_instruction, with
 *   flops_per_instruction = 2*32*32*64 (scaled formats) or 2*32*32*16 (bf16),
 *   as moe_peak_mfma_flops returns.
 *   sink: device float[workgroups * 256], written (keeps the results live).
 */
double moe_peak_mfma_flops(moe_peak_format format, int32_t workgroups, int32_t iters);
moe_peak_status moe_peak_mfma(moe_peak_format format, int32_t workgroups, int32_t iters, float* sink,
                              hipStream_t stream);

/*
 * Streaming read of `bytes` bytes (a multiple of 16, 16-byte aligned) with
 * 16-byte buffer loads, the non-temporal hint when `nontemporal` is non-zero
 * (as the layer's weight stream uses), `workgroups` workgroups of 256 threads
 * in a grid-stride loop.  work = bytes.
 *   sink: device uint32[workgroups * 256], written (keeps the loads live).
 */
moe_peak_status moe_peak_stream_read(const void* buf, size_t bytes, int32_t nontemporal, int32_t workgroups,
                                     uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PEAKS_H */
