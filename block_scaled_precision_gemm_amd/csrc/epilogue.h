// Fused epilogue: y = alpha * acc (+ bias[n]), optional SiLU, one rounding to bf16/fp16.
//
// The epilogue of runNvfp4Gemm<T, kEnableSilu, kEnableBias> on the CUTLASS issue #3003 page (alpha,
// bias, SiLU) and the alpha_ptr of the nvFuser PR #5736 page, applied in registers so that the fp32
// accumulators never leave the kernel.
#pragma once

#include "common.h"

namespace bsg {

// SiLU(y) = y / (1 + e^-y) with the hardware exp2 and reciprocal (each about 1 ulp of fp32, far below
// the bf16 / fp16 rounding that follows).
// * FP16 output: y * rcp(1 + e^-y).  Where e^-y overflows (y < -88.7) this gives -0, which is also
//   the fp16 rounding of SiLU(y) there (|SiLU(y)| < 2^-25 from y ~ -21 down).
// * BF16 output, whose range is fp32's: SiLU's negative tail is a bf16 subnormal down to y ~ -97,
//   so e^-y must not overflow.  For y < 0 both denominator terms are scaled by c = 2^-64:
//   SiLU(y) = (y * rcp(c + c e^-y)) * c, with c e^-y = 2^(-y log2 e - 64) finite down to y ~ -132
//   (below, rcp(inf) = 0, and SiLU(y) rounds to zero anyway); c = 1 for y >= 0.  The final
//   multiply by c rounds once into fp32's subnormal range.
template <bool SILU, Out O>
__device__ __forceinline__ float epi_value(float acc, float alpha, float bias) {
  float y = __builtin_fmaf(alpha, acc, bias);
  if constexpr (SILU) {
    constexpr float kLog2e = 1.44269504088896341f, kTwoM64 = 5.42101086242752217e-20f;  // 2^-64
    if constexpr (O == Out::F16) {
      y = y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-y * kLog2e));
    } else {
      const bool neg = y < 0.0f;
      const float c = neg ? kTwoM64 : 1.0f;
      const float v = __builtin_amdgcn_exp2f(__builtin_fmaf(-y, kLog2e, neg ? -64.0f : 0.0f));
      y = (y * __builtin_amdgcn_rcpf(c + v)) * c;
    }
  }
  return y;
}

template <Out O>
__device__ __forceinline__ uint16_t to_out_bits(float y) {
  if constexpr (O == Out::BF16) {
    const __bf16 b = (__bf16)y;  // round to nearest even
    return __builtin_bit_cast(uint16_t, b);
  } else {
    const _Float16 h = (_Float16)y;  // round to nearest even
    return __builtin_bit_cast(uint16_t, h);
  }
}

// Two outputs in one dword (lo in bits 0..15).  BF16: one paired conversion (the same round to
// nearest even as two single ones, without the shift and or that join them).  FP16: single
// conversions, which the compiler fuses with a preceding multiply or fma into one rounding.
template <Out O>
__device__ __forceinline__ uint32_t pack2_out(float lo, float hi) {
  if constexpr (O == Out::BF16) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
  } else {
    return (uint32_t)to_out_bits<O>(lo) | ((uint32_t)to_out_bits<O>(hi) << 16);
  }
}

// f16(a0 * b0 + c0) | f16(a1 * b1 + c1) << 16, each product-sum rounded once from the exact value
// (v_fma_mixlo_f16, then v_fma_mixhi_f16 writing the high half in place: no shift and or).
__device__ __forceinline__ uint32_t f16x2_fma_rounded(float a0, float b0, float c0, float a1, float b1, float c1) {
  uint32_t d;
  asm("v_fma_mixlo_f16 %0, %1, %2, %3" : "=v"(d) : "v"(a0), "v"(b0), "v"(c0));
  asm("v_fma_mixhi_f16 %0, %1, %2, %3" : "+v"(d) : "v"(a1), "v"(b1), "v"(c1));
  return d;
}

// Two epilogue outputs in one dword (acc0's in bits 0..15).  FP16: the last step of each --
// alpha * acc + bias, or y * 1/(1 + e^-y) for SiLU -- is one fused multiply-add rounded once to fp16.
// BF16: epi_value in fp32, then the paired conversion.
template <bool SILU, Out O>
__device__ __forceinline__ uint32_t epi_pack2(float acc0, float acc1, float alpha, float bias0, float bias1) {
  if constexpr (O == Out::F16) {
    if constexpr (SILU) {
      constexpr float kLog2e = 1.44269504088896341f;
      const float y0 = __builtin_fmaf(alpha, acc0, bias0), y1 = __builtin_fmaf(alpha, acc1, bias1);
      const float r0 = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-y0 * kLog2e));
      const float r1 = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-y1 * kLog2e));
      return f16x2_fma_rounded(y0, r0, 0.0f, y1, r1, 0.0f);
    } else {
      return f16x2_fma_rounded(alpha, acc0, bias0, alpha, acc1, bias1);
    }
  } else {
    return pack2_out<O>(epi_value<SILU, O>(acc0, alpha, bias0), epi_value<SILU, O>(acc1, alpha, bias1));
  }
}

__device__ __forceinline__ float load_alpha(const GemmArgs& p) {
  return p.alpha_ptr ? *p.alpha_ptr : p.alpha;
}

}  // namespace bsg
