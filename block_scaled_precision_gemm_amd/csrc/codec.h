// Device-side decoders of the OCP MX element formats used by the GEMM kernels.
//
// E4M3 (FN variant): sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0; exponent 0
// is subnormal (m * 2^-9); 0x7F / 0xFF are NaN; no infinities.
// E2M1: sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0; values +-{0,.5,1,1.5,2,3,4,6}.
// NVFP4 dequantisation multiplies each E2M1 element by its 16-element block's E4M3 scale.  That
// product has at most 6 significant bits and lies in [2^-10, 2688], so it is exact in bf16: the
// bf16 MFMA then sees exactly the dequantised operand.
#pragma once

#include "common.h"

namespace bsg {

// E4M3 code -> fp32, exact.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  const uint32_t em = code & 0x7Fu;
  const uint32_t e = em >> 3, m = em & 7u;
  // normal: 2^(e-7) (1 + m/8) -> fp32 exponent field e - 7 + 127, mantissa m in its top 3 bits
  const float normal = __uint_as_float(((e + 120u) << 23) | (m << 20));
  const float sub = (float)m * 0x1p-9f;
  float v = e ? normal : sub;
  v = (em == 0x7Fu) ? __builtin_nanf("") : v;
  return __uint_as_float(__float_as_uint(v) | ((code & 0x80u) << 24));
}

}  // namespace bsg

namespace bsg {

// E2M1 nibble -> fp32 by bit assembly (exact).
__device__ __forceinline__ float e2m1_to_f32(uint32_t nib) {
  const uint32_t mag = nib & 7u;
  // exponent field e = mag >> 1 (bias 1) -> fp32 exponent e - 1 + 127; mantissa bit -> fp32 bit 22
  const uint32_t normal = (((mag >> 1) + 126u) << 23) | ((mag & 1u) << 22);
  const uint32_t bits = mag >= 2u ? normal : (mag ? 0x3F000000u : 0u);  // e = 0: 0 or 0.5
  return __uint_as_float(bits | ((nib & 8u) << 28));
}

}  // namespace bsg

namespace bsg {

// Two fp32 values that are exactly representable in bf16 -> one dword of two bf16 (low half = lo).
__device__ __forceinline__ uint32_t pack_bf16x2_exact(float lo, float hi) {
  // exact inputs: dropping the low 16 bits of each fp32 is the value itself
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

// Eight E2M1 codes of one dword (nibble j = element j), each times `scale`, as four dwords of
// bf16 pairs (dword i holds elements 2i, 2i+1).  The fp32 product is exact (<= 6 significant
// bits), hence so is the bf16 value.
__device__ __forceinline__ v4i e2m1x8_scaled_bf16x8(uint32_t packed, float scale) {
  v4i r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = e2m1_to_f32(packed >> (8 * i)) * scale;
    const float hi = e2m1_to_f32(packed >> (8 * i + 4)) * scale;
    r[i] = (int)pack_bf16x2_exact(lo, hi);
  }
  return r;
}

}  // namespace bsg
