/*
 * dg_ceiling.h - measurement helper of libdg.so: the FP8 matrix-core
 * throughput this device reaches, against which the GEMMs' times are
 * reported besides the published peak. Not part of the GEMM contract of
 * dg.h (same status codes and conventions).
 */
#ifndef DG_CEILING_H
#define DG_CEILING_H

#include "dg.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Enqueues on `stream` (a hipStream_t; NULL = the null stream) one kernel
 * with the GEMM kernels' launch shape -- one workgroup of 8 waves (two per
 * SIMD) on each of dg_get_num_cus() CUs -- in which every wave issues FP8
 * MFMAs into independent float32 accumulators and nothing else:
 *   variant 0: iters * 16 v_mfma_f32_16x16x128_f8f6f4 (65536 FLOP each), the
 *              instruction of the GEMM kernels;
 *   variant 1: the same plus the float32 promotion of the float32-scale
 *              GEMMs (four FMAs per MFMA);
 *   variant 2: iters * 16 v_mfma_f32_32x32x64_f8f6f4 (131072 FLOP each, two
 *              per 128-K block), for comparison;
 *   variant 3: 32x32x64 with the promotion: per 128-K block two chained
 *              MFMAs into a partial and 16 FMAs promoting the previous one,
 *              4 chains per wave (iters * 8 MFMAs);
 *   variant 4: variant 0 plus the promotion of the K-grouped GEMM, whose
 *              weights differ per column (four multiplications and four
 *              FMAs per MFMA).
 *   fragments  device memory, 16-byte aligned, >= 4096 bytes: the operand
 *              bytes every wave multiplies (E4M3 codes; random, non-NaN
 *              values make the clock behave as in a GEMM on random data)
 *   sink       device memory, >= 2048 * dg_get_num_cus() bytes; written
 *              only if the accumulators reach a value the data used never
 *              gives (it keeps the loop from being removed)
 *   flops      host: receives the FLOP count of the launch
 * Time it with events on `stream`. Errors: DG_ERR_NULL, DG_ERR_SHAPE
 * (iters outside [1, 2^24], unknown variant), DG_ERR_ALIGN, DG_ERR_DEVICE,
 * DG_ERR_LAUNCH; nothing is enqueued on error. The library allocates
 * nothing.
 */
dg_status dg_mfma_fp8_ceiling(const void* fragments, float* sink, int iters, int variant,
                              long long* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DG_CEILING_H */
