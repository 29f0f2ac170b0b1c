// Fused epilogue: y = alpha * acc (+ bias[n]), optional SiLU, one rounding to bf16/fp16.
//
// The epilogue of runNvfp4Gemm<T, kEnableSilu, kEnableBias> on the CUTLASS issue #3003 page (alpha,
// bias, SiLU) and the alpha_ptr of the nvFuser PR #5736 page, applied in registers so that the fp32
// accumulators never leave the kernel.
#pragma once

#include "common.h"

namespace bsg {

// SiLU as y * rcp(1 + exp(-y)) with the hardware exp2 and reciprocal (each about 1 ulp of fp32):
// far below the bf16 / fp16 rounding that follows, and a handful of VALU operations instead of an
// IEEE division.  Large -y gives exp = inf, rcp(inf) = 0 and y * 0 = -0.
template <bool SILU>
__device__ __forceinline__ float epi_value(float acc, float alpha, float bias) {
  float y = __builtin_fmaf(alpha, acc, bias);
  if constexpr (SILU) y = y * __builtin_amdgcn_rcpf(1.0f + __expf(-y));
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

template <Out O>
__device__ __forceinline__ uint32_t pack2_out(float lo, float hi) {
  return (uint32_t)to_out_bits<O>(lo) | ((uint32_t)to_out_bits<O>(hi) << 16);
}

__device__ __forceinline__ float load_alpha(const GemmArgs& p) {
  return p.alpha_ptr ? *p.alpha_ptr : p.alpha;
}

}  // namespace bsg
