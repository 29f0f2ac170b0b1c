// MXFP8 block-scaled GEMM for gfx950: the format, the scaled MFMA's register layout, and the
// plan-time kernel choice (the kernels are in mxfp8_pp.hip and mxfp8_tiled.hip).
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

namespace bsg {

// Kernel choice by shape: the 8-wave ping-pong kernel for K % 512 == 0 with packed A and B rows once
// 256 x 256 tiles give at least one workgroup per CU; the tiled kernels (256 x 256 or 128 x 128
// tiles, split K for small tile grids, a partial last K tile for K % 128 != 0, any row pitch) for
// every other K % 32 == 0.
const KernelVariant* mxfp8_variants(int64_t M, int64_t N, int64_t K, int64_t batch, bool packed_ab) {
  const int64_t large_tiles = ((M + 255) / 256) * ((N + 255) / 256) * batch;
  if (packed_ab && K % 512 == 0 && large_tiles >= 256) return mxfp8_pp_variants();
  return mxfp8_tiled_variants(M, N, batch);
}

}  // namespace bsg
