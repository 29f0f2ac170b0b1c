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

namespace bsg {

// ---------------------------------------------------------------------------------------------
// fp16 route (tiled NVFP4 kernels).  An E2M1 nibble placed at fp16 bits [11:9] (magnitude) and
// [15] (sign) is the fp16 number q * 2^-14, exactly: E2M1's exponent field lands in fp16's low
// exponent bits (bias 15 instead of 1), and E2M1's subnormal 0.5 becomes the fp16 subnormal 2^-15.
// Multiplying by s * 2^7 (s the E4M3 block scale; s * 2^7 <= 57344 fits fp16) gives q * s * 2^-7,
// exact in fp16 (<= 6 significant bits, smallest 2^-17 >= the fp16 subnormal step 2^-24).  Both
// v_pk_mul_f16 and the fp16 MFMA keep fp16 subnormals (checked on the device), and the factor 2^14
// of a product of two such operands is restored in the epilogue.
// ---------------------------------------------------------------------------------------------
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Two E4M3 scale codes (bits 7:0 and 15:8 of `sc`) -> two fp16 (s0 * 2^7, s1 * 2^7), exact.
// Placing an E4M3 code's exponent and mantissa at fp16 bits [13:7] gives the fp16 number s * 2^-8
// for normal and subnormal codes alike (E4M3 bias 7, fp16 bias 15, both with 3 leading mantissa
// bits in place); one multiplication by 2^15 then yields s * 2^7 (<= 57344, exact).  The NaN codes
// 0x7F / 0xFF map to an fp16 NaN.
__device__ __forceinline__ uint32_t e4m3x2_scale_f16x2(uint32_t sc) {
  const uint32_t placed = ((sc & 0x7Fu) << 7) | ((sc & 0x80u) << 8) | ((sc & 0x7F00u) << 15) | ((sc & 0x8000u) << 16);
  const v2h k = {(_Float16)32768.0f, (_Float16)32768.0f};
  uint32_t r = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, placed) * k);
  if ((sc & 0x7Fu) == 0x7Fu) r = (r & 0xFFFF0000u) | 0x7E00u;
  if ((sc & 0x7F00u) == 0x7F00u) r = (r & 0x0000FFFFu) | 0x7E000000u;
  return r;
}

// fp16 pair (x.lo, x.lo) and (x.hi, x.hi) of a dword of two fp16.
__device__ __forceinline__ uint32_t f16x2_splat_lo(uint32_t x) { return __builtin_amdgcn_perm(x, x, 0x01000100u); }
__device__ __forceinline__ uint32_t f16x2_splat_hi(uint32_t x) { return __builtin_amdgcn_perm(x, x, 0x03020302u); }

// Eight E2M1 codes of one dword (nibble j = element j) times the fp16 pair `s2` (= s * 2^7 twice):
// four dwords of fp16 pairs, dword i = elements (2i, 2i+1), each q * s * 2^-7.
__device__ __forceinline__ v4i e2m1x8_scaled_f16x8(uint32_t w, uint32_t s2) {
  // fp16 high byte of q * 2^-14: magnitude bits at [3:1], sign at bit 7.  Byte i of `lo` serves
  // element 2i (nibble at bits 8i+3..8i), byte i of `hi` element 2i+1 (bits 8i+7..8i+4).
  const uint32_t lo = ((w << 1) & 0x0E0E0E0Eu) | ((w << 4) & 0x80808080u);
  const uint32_t hi = ((w >> 3) & 0x0E0E0E0Eu) | (w & 0x80808080u);
  const v2h s = __builtin_bit_cast(v2h, s2);
  v4i r;
  // v_perm_b32 selector bytes: 0..3 pick bytes of `lo`, 4..7 bytes of `hi`, 0x0C gives 0x00.
  r[0] = __builtin_bit_cast(int, __builtin_bit_cast(v2h, __builtin_amdgcn_perm(hi, lo, 0x040C000Cu)) * s);
  r[1] = __builtin_bit_cast(int, __builtin_bit_cast(v2h, __builtin_amdgcn_perm(hi, lo, 0x050C010Cu)) * s);
  r[2] = __builtin_bit_cast(int, __builtin_bit_cast(v2h, __builtin_amdgcn_perm(hi, lo, 0x060C020Cu)) * s);
  r[3] = __builtin_bit_cast(int, __builtin_bit_cast(v2h, __builtin_amdgcn_perm(hi, lo, 0x070C030Cu)) * s);
  return r;
}

// A 16-byte chunk of packed E2M1 (32 elements, two scale blocks) and its two scale codes (bits 7:0:
// elements 0..15, bits 15:8: elements 16..31) -> 32 fp16 values q * s * 2^-7 in four v4i (v4i d =
// elements 8d .. 8d+7).
__device__ __forceinline__ void e2m1x32_scaled_f16(v4i q, uint32_t sc, v4i out[4]) {
  const uint32_t s = e4m3x2_scale_f16x2(sc);
  const uint32_t s0 = f16x2_splat_lo(s), s1 = f16x2_splat_hi(s);
  out[0] = e2m1x8_scaled_f16x8((uint32_t)q[0], s0);
  out[1] = e2m1x8_scaled_f16x8((uint32_t)q[1], s0);
  out[2] = e2m1x8_scaled_f16x8((uint32_t)q[2], s1);
  out[3] = e2m1x8_scaled_f16x8((uint32_t)q[3], s1);
}

}  // namespace bsg
