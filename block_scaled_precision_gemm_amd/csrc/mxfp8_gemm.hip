// MXFP8 block-scaled GEMM kernels for gfx950.
//
// D = epi(alpha * A x B^T (+ bias)), A [M][K] and B [N][K] E4M3 codes (K contiguous), one E8M0 scale
// per 32 K elements (the mx_float8_t<float_e4m3_t> operands with float_ue8m0_t scale factors of the
// nvFuser PR #5736 page, MxFp8GemmSm100), fp32 accumulation, bf16/fp16 output.
//
// CDNA4's scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4 consumes exactly this format: each lane
// holds 32 consecutive K bytes of one row of A (and of B) plus that block's E8M0 code, and the
// hardware applies both scales to every product before fp32 accumulation.  So the block scaling
// costs nothing beyond one scale byte per lane per instruction.
//
// Register layout of v_mfma_scale_f32_32x32x64_f8f6f4 (lane l, r = l % 32, h = l / 32), as measured
// on the device with one-hot operands and distinct per-lane scales:
//   A operand bytes 0..15:  row r, K [16h, 16h+16)       (inside 32-block 0)
//   A operand bytes 16..31: row r, K [32+16h, 32+16h+16)  (inside 32-block 1)
//   A scale (byte 0 of the lane's scale VGPR): E8M0 of (row r, 32-block h)
//   B operand and scale: the same with column r (= row r of our N x K B)
//   accumulator element i: column r, row 8*(i/4) + 4*h + (i%4)
// So each lane's 32 bytes straddle both 32-blocks while its scale byte names one of them; within
// a block the K order is free, as long as A and B agree.
#include "common.h"
#include "epilogue.h"

namespace bsg {
namespace {

__device__ __forceinline__ v16f mfma_mx_e4m3_32x32x64(v8i a, v8i b, v16f c, int sa, int sb) {
  // format codes 0 = E4M3 for both operands; op_sel 0 = scale byte 0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ v8i join(v4i lo, v4i hi) {
  return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ---------------------------------------------------------------------------------------------
// Direct kernel: 4 waves, 64x64 output tile per workgroup, each wave a 32x32 tile; operands go
// straight from global memory into MFMA registers.  Any M >= 1, N % 16 == 0, K % 32 == 0.
// ---------------------------------------------------------------------------------------------
template <Out O, bool BIAS, bool SILU>
__global__ __launch_bounds__(256) void mxfp8_direct_kernel(GemmArgs p) {
  select_batch(p);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int m0 = blockIdx.y * 64 + (wave >> 1) * 32;
  const int n0 = blockIdx.x * 64 + (wave & 1) * 32;
  const int K = p.K, KB = K >> 5;
  // rows past the edge load a valid row and are never stored
  const int arow = min(m0 + r, p.M - 1);
  const int brow = min(n0 + r, p.N - 1);
  const uint8_t* ap = p.A + (size_t)arow * K + 16 * h;
  const uint8_t* bp = p.B + (size_t)brow * K + 16 * h;
  v16f acc = {};
  for (int k0 = 0; k0 < K; k0 += 64) {
    // block k0/32 always exists; block k0/32 + 1 is missing in the last step when K % 64 == 32
    const bool second = (k0 >> 5) + 1 < KB;
    const v4i z = {0, 0, 0, 0};
    const v4i a0 = *(const v4i*)(ap + k0), b0 = *(const v4i*)(bp + k0);
    v4i a1 = z, b1 = z;
    if (second) {
      a1 = *(const v4i*)(ap + k0 + 32);
      b1 = *(const v4i*)(bp + k0 + 32);
    }
    const bool mine = (k0 >> 5) + h < KB;
    const int blk = (k0 >> 5) + h;
    const int sa = mine ? p.sA[scale_offset(p.scale_ktile, arow, blk, p.M, KB)] : 127;
    const int sb = mine ? p.sB[scale_offset(p.scale_ktile, brow, blk, p.N, KB)] : 127;
    acc = mfma_mx_e4m3_32x32x64(join(a0, a1), join(b0, b1), acc, sa, sb);
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
  return hipLaunchKernel((const void*)&mxfp8_direct_kernel<O, BIAS, SILU>, grid, block, kargs, 0, stream);
}

#define BSG_MX_DIRECT(O, B, S) \
  { "mxfp8_direct_64x64", &launch_direct<O, B, S>, 64, 64, 64, 256, 0, false }
const KernelVariant kDirect[8] = {
    BSG_MX_DIRECT(Out::BF16, false, false), BSG_MX_DIRECT(Out::BF16, false, true),
    BSG_MX_DIRECT(Out::BF16, true, false),  BSG_MX_DIRECT(Out::BF16, true, true),
    BSG_MX_DIRECT(Out::F16, false, false),  BSG_MX_DIRECT(Out::F16, false, true),
    BSG_MX_DIRECT(Out::F16, true, false),   BSG_MX_DIRECT(Out::F16, true, true),
};
#undef BSG_MX_DIRECT

}  // namespace

// Kernel choice by shape: the 8-wave ping-pong kernel for K % 512 == 0 once 256 x 256 tiles give at
// least one workgroup per CU; the direct kernel for short K (<= 512: at most 4 K tiles of 128, where
// the LDS pipeline's fixed costs dominate) while its 64 x 64 tiles number at most one workgroup per
// CU (measured: 256^3 4.4 vs 10.7 us, 1024x1024x512 7.2 vs 11.7 us; with more workgroups the tiled
// kernels win, 2048x2048x512 13.4 vs 21.0 us); the two-stage tiled kernels otherwise.
const KernelVariant* mxfp8_variants(int64_t M, int64_t N, int64_t K, int64_t batch) {
  const int64_t large_tiles = ((M + 255) / 256) * ((N + 255) / 256) * batch;
  if (K % 512 == 0 && large_tiles >= 256) return mxfp8_pp_variants();
  const int64_t direct_tiles = ((M + 63) / 64) * ((N + 63) / 64) * batch;
  if (K <= 512 && direct_tiles <= 256) return kDirect;
  return mxfp8_tiled_variants(M, N, batch);
}

}  // namespace bsg
