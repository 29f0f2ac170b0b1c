/*
 * bsg_testing.h -- element-wise access to the device-side NVFP4 dequantisation that the GEMM
 * kernels use, so that tests can compare it bit for bit with a CPU decoding of every code.
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

/* Dequantise n_elements NVFP4 elements laid out as one operand row -- packed[n/2] (element 2t in the
 * low nibble of byte t), scale_codes[n/16] (one E4M3 code per 16 elements) -- through the GEMM
 * kernels' own routine: out_f16[k] = fp16 bits of e2m1(element k) * e4m3(scale_codes[k / 16]) * 2^-8,
 * which is exact (the factor 2^-8 keeps every product inside fp16's range; the GEMM restores it in
 * its epilogue).  A NaN scale code gives NaN for its 16 elements.  n_elements: a multiple of 32
 * (else BSG_ERR_SHAPE); packed and out_f16 16-byte aligned (else BSG_ERR_ALIGN). */
bsg_status bsg_test_decode_nvfp4_f16(const uint8_t* packed, const uint8_t* scale_codes, uint16_t* out_f16,
                                     int64_t n_elements, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSG_TESTING_H */
