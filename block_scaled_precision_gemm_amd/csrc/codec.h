// Device-side dequantisation of NVFP4 operands for the fp16 MFMA route.
//
// NVFP4 (OCP Microscaling v1.0 element types): E2M1 elements (sign bit 3, exponent bits 2..1 with
// bias 1, mantissa bit 0; values +-{0, .5, 1, 1.5, 2, 3, 4, 6}), one E4M3 scale per 16 elements
// (sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0; exponent 0 is subnormal,
// m * 2^-9; codes 0x7F / 0xFF are NaN).  Dequantisation multiplies each element by its block's scale.
//
// Each element becomes the fp16 number q * s * 2^-8, which is exact:
// * q * s has at most 2 + 4 = 6 significant bits and lies in [2^-10, 2688] (or is zero), so
//   q * s * 2^-8 lies in [2^-18, 10.5]; its lowest set bit is at least 2^-23, above the fp16
//   subnormal step 2^-24.
// * v_cvt_scalef32_pk_f16_fp4 turns two E2M1 codes into two fp16 q (exact; its fp32 scale operand
//   contributes only its exponent, here 2^0).
// * s * 2^-8 is an E4M3 code's exponent and mantissa placed at fp16 bits [13:7]: E4M3 bias 7 vs fp16
//   bias 15, 3 leading mantissa bits in both, and E4M3 subnormals land on fp16 subnormals.
// * one v_pk_mul_f16 forms q * (s * 2^-8); fp16 subnormals are kept (not flushed) by both the
//   multiply and the MFMA.
// A product of two such operands is the exact dequantised product times 2^-16; the GEMM epilogue
// multiplies by 2^16.
#pragma once

#include "common.h"

namespace bsg {

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Two E4M3 scale codes (bits 7:0 and 15:8 of `sc`) -> fp16 pair (s0 * 2^-8, s1 * 2^-8), exact; a
// NaN code gives an fp16 NaN.  A byte permute puts code i at bits 8..15 of half i; shifted right by
// one, its magnitude bits land on fp16 bits 13..7 and its sign stays at bit 15.  The NaN magnitude
// 0x7F lands on 0x3F80, an fp16 NaN but for bit 14, which the carry of 0x3F80 + 0x80 supplies (for
// that magnitude only).  Seven VALU operations for the pair.
__device__ __forceinline__ uint32_t e4m3x2_scale_f16x2(uint32_t sc) {
  const uint32_t y = __builtin_amdgcn_perm(0u, sc, 0x010C000Cu);  // (c0 << 8) | (c1 << 24)
  const uint32_t t = (y >> 1) & 0x3F803F80u;
  const uint32_t nan = (t + 0x00800080u) & 0x40004000u;
  return t | nan | (y & 0x80008000u);
}

// The same for the code pair a byte-permute selector picks from a dword of four codes: sel =
// 0x010C000C takes bytes 0, 1 (as e4m3x2_scale_f16x2), 0x030C020C bytes 2, 3.
__device__ __forceinline__ uint32_t e4m3x2_scale_f16x2_sel(uint32_t w, uint32_t sel) {
  const uint32_t y = __builtin_amdgcn_perm(0u, w, sel);
  const uint32_t t = (y >> 1) & 0x3F803F80u;
  const uint32_t nan = (t + 0x00800080u) & 0x40004000u;
  return t | nan | (y & 0x80008000u);
}

// fp16 pair (x.lo, x.lo) and (x.hi, x.hi) of a dword of two fp16.
__device__ __forceinline__ uint32_t f16x2_splat_lo(uint32_t x) { return __builtin_amdgcn_perm(x, x, 0x01000100u); }
__device__ __forceinline__ uint32_t f16x2_splat_hi(uint32_t x) { return __builtin_amdgcn_perm(x, x, 0x03020302u); }

// Eight E2M1 codes of one dword (nibble j = element j) times the fp16 pair `s2` (the block scale
// twice): four dwords of fp16 pairs, dword i = elements (2i, 2i+1).
__device__ __forceinline__ v4i e2m1x8_scaled_f16x8(uint32_t w, uint32_t s2) {
  const v2h s = __builtin_bit_cast(v2h, s2);
  v4i r;
  r[0] = __builtin_bit_cast(int, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0)) * s);
  r[1] = __builtin_bit_cast(int, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1)) * s);
  r[2] = __builtin_bit_cast(int, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2)) * s);
  r[3] = __builtin_bit_cast(int, __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3)) * s);
  return r;
}

// A 16-byte chunk of packed E2M1 (32 elements, two scale blocks) and its two scale codes (bits 7:0:
// elements 0..15, bits 15:8: elements 16..31) -> 32 fp16 values q * s * 2^-8 in four v4i (v4i d =
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
