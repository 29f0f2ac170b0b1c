/*
 * bsg_testing.h -- element-wise access to the device-side decoders that the GEMM kernels use,
 * so that tests can compare them bit for bit with a CPU decoding of every code.
 *
 * Element formats are OCP Microscaling v1.0 E4M3 (FN variant) and E2M1; the NVFP4 operand
 * decode multiplies each E2M1 element by its block's E4M3 scale, the dequantisation that the
 * CUTLASS issue #3003 page's NVFP4 GEMM (runNvfp4Gemm) applies per 16-element block.
 *
 * All buffers are device pointers owned by the caller; stream is a hipStream_t (NULL = null
 * stream); calls are asynchronous.  Errors: BSG_ERR_NULL, BSG_ERR_SHAPE (bad n), BSG_ERR_ALIGN,
 * BSG_ERR_HIP.
 */
#ifndef BSG_TESTING_H
#define BSG_TESTING_H

#include "bsg.h"

#ifdef __cplusplus
extern "C" {
#endif

/* out[i] = fp32 value of E4M3 code codes[i] (exact; code 0x7F/0xFF gives a NaN), i < n. */
bsg_status bsg_test_decode_e4m3(const uint8_t* codes, float* out, int64_t n, void* stream);

/* Dequantise n_elements NVFP4 elements laid out as one operand row: packed[n/2] (element 2t in the
 * low nibble of byte t), scale_codes[n/16] (one E4M3 code per 16 elements).  out_bf16[k] = bf16
 * bits of e2m1(element k) * e4m3(scale_codes[k / 16]), which is exact.  This runs the GEMM kernels'
 * own in-register routine, one dword (8 elements) per thread.  n_elements must be a multiple of
 * 16 (BSG_ERR_SHAPE) and `packed` 4-byte aligned (BSG_ERR_ALIGN). */
bsg_status bsg_test_decode_nvfp4(const uint8_t* packed, const uint8_t* scale_codes, uint16_t* out_bf16,
                                 int64_t n_elements, void* stream);

/* Same layout as bsg_test_decode_nvfp4, through the tiled NVFP4 kernels' fp16 routine:
 * out_f16[k] = fp16 bits of e2m1(element k) * e4m3(scale_codes[k / 16]) * 2^-7, exact (the factor
 * 2^-7 keeps every scale inside fp16's range; the GEMM restores it in the epilogue).  A NaN scale
 * code gives a NaN for its 16 elements.  n_elements: a multiple of 32; packed and out_f16 16-byte
 * aligned.  Errors: BSG_ERR_SHAPE, BSG_ERR_NULL, BSG_ERR_ALIGN, BSG_ERR_HIP. */
bsg_status bsg_test_decode_nvfp4_f16(const uint8_t* packed, const uint8_t* scale_codes, uint16_t* out_f16,
                                     int64_t n_elements, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSG_TESTING_H */
