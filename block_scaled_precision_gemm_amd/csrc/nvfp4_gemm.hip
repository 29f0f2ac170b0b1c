// NVFP4 block-scaled GEMM kernels for gfx950.
//
// D = epi(alpha * A x B^T (+ bias)), A [M][K/2] and B [N][K/2] packed E2M1 (element 2t in the low
// nibble of byte t), one E4M3 scale per 16 K elements, global fp32 alpha (the NVFP4 GEMM
// runNvfp4Gemm<T, kEnableSilu, kEnableBias> of the CUTLASS issue #3003 page).
//
// CDNA4's scaled MFMAs take E8M0 (power-of-two) scales per 32 elements; an E4M3 scale per 16 does
// not fit them exactly.  Instead each element is dequantised in registers to the exact bf16 value
// e2m1 * e4m3 (at most 6 significant bits, range [2^-10, 2688]) and fed to the bf16 MFMA
// v_mfma_f32_32x32x16_bf16, so the products the hardware accumulates are exactly the dequantised
// ones.  The global alpha is applied once, in the epilogue.
//
// K order inside the contraction is free as long as A and B use the same order and each element
// carries its own block's scale.  Each lane therefore loads one contiguous 16-byte chunk (32
// elements = two scale blocks) per 64-K step and spreads it over four MFMAs:
//   lane l (r = l % 32, h = l / 32), step c, MFMA t: K elements 64c + 32h + 8t .. +8
// Register layout of v_mfma_f32_32x32x16_bf16: A lane l holds row r, eight K slots [8h, 8h+8);
// B likewise for column r; accumulator element i: column r, row 8*(i/4) + 4*h + (i%4).
#include "codec.h"
#include "common.h"
#include "epilogue.h"

namespace bsg {
namespace {

__device__ __forceinline__ v16f mfma_bf16_32x32x16(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------------------------
// Direct kernel: 4 waves, 64x64 tile per workgroup, 32x32 per wave, operands decoded straight
// from global memory.  Any M >= 1, N % 16 == 0, K % 32 == 0.
// ---------------------------------------------------------------------------------------------
template <Out O, bool BIAS, bool SILU>
__global__ __launch_bounds__(256) void nvfp4_direct_kernel(GemmArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int m0 = blockIdx.y * 64 + (wave >> 1) * 32;
  const int n0 = blockIdx.x * 64 + (wave & 1) * 32;
  const int K = p.K, KH = K >> 1, KB = K >> 4;
  const int arow = min(m0 + r, p.M - 1);
  const int brow = min(n0 + r, p.N - 1);
  const uint8_t* ap = p.A + (size_t)arow * KH + 16 * h;
  const uint8_t* bp = p.B + (size_t)brow * KH + 16 * h;
  const uint8_t* sap = p.sA + (size_t)arow * KB + 2 * h;
  const uint8_t* sbp = p.sB + (size_t)brow * KB + 2 * h;
  v16f acc = {};
  for (int k0 = 0; k0 < K; k0 += 64) {
    v4i qa = {0, 0, 0, 0}, qb = {0, 0, 0, 0};
    float sa0 = 0.f, sa1 = 0.f, sb0 = 0.f, sb1 = 0.f;
    if (k0 + 32 * h < K) {  // K % 32 == 0: a lane's 32-element chunk is all in or all out
      qa = *(const v4i*)(ap + (k0 >> 1));
      qb = *(const v4i*)(bp + (k0 >> 1));
      const int kb = k0 >> 4;
      sa0 = e4m3_to_f32(sap[kb]);
      sa1 = e4m3_to_f32(sap[kb + 1]);
      sb0 = e4m3_to_f32(sbp[kb]);
      sb1 = e4m3_to_f32(sbp[kb + 1]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const v4i a = e2m1x8_scaled_bf16x8((uint32_t)qa[t], t < 2 ? sa0 : sa1);
      const v4i b = e2m1x8_scaled_bf16x8((uint32_t)qb[t], t < 2 ? sb0 : sb1);
      acc = mfma_bf16_32x32x16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), acc);
    }
  }
  const int n = n0 + r;
  if (n >= p.N) return;
  const float alpha = load_alpha(p);
  const float bv = BIAS ? p.bias[n] : 0.0f;
  uint16_t* D = (uint16_t*)p.D;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = m0 + 8 * (i >> 2) + 4 * h + (i & 3);
    if (m < p.M) D[(size_t)m * p.N + n] = to_out_bits<O>(epi_value<SILU>(acc[i], alpha, bv));
  }
}

template <Out O, bool BIAS, bool SILU>
hipError_t launch_direct(const GemmArgs& args, dim3 grid, dim3 block, hipStream_t stream) {
  void* kargs[] = {(void*)&args};
  return hipLaunchKernel((const void*)&nvfp4_direct_kernel<O, BIAS, SILU>, grid, block, kargs, 0, stream);
}

#define BSG_NV_DIRECT(O, B, S) \
  { "nvfp4_direct_64x64", &launch_direct<O, B, S>, 64, 64, 64, 256, 0, false }
const KernelVariant kDirect[8] = {
    BSG_NV_DIRECT(Out::BF16, false, false), BSG_NV_DIRECT(Out::BF16, false, true),
    BSG_NV_DIRECT(Out::BF16, true, false),  BSG_NV_DIRECT(Out::BF16, true, true),
    BSG_NV_DIRECT(Out::F16, false, false),  BSG_NV_DIRECT(Out::F16, false, true),
    BSG_NV_DIRECT(Out::F16, true, false),   BSG_NV_DIRECT(Out::F16, true, true),
};
#undef BSG_NV_DIRECT

}  // namespace

const KernelVariant* nvfp4_variants(int64_t M, int64_t N, int64_t /*K*/) { return nvfp4_tiled_variants(M, N); }

}  // namespace bsg
