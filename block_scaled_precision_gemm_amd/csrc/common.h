// Shared host/device definitions of the block-scaled GEMM kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsg {

// MFMA operand/accumulator register vectors.
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

enum class Fmt : int { MXFP8 = 1, NVFP4 = 2 };
enum class Out : int { BF16 = 1, F16 = 2 };

// Kernel arguments, filled once at plan time; the per-call pointers and alpha are patched into a
// copy by the run entry point.  Passed by value (kernarg segment).
struct GemmArgs {
  const uint8_t* A;       // MXFP8: [M][K] E4M3; NVFP4: [M][K/2] packed E2M1
  const uint8_t* B;       // MXFP8: [N][K] E4M3; NVFP4: [N][K/2] packed E2M1
  const uint8_t* sA;      // MXFP8: [M][K/32] E8M0; NVFP4: [M][K/16] E4M3
  const uint8_t* sB;      // MXFP8: [N][K/32] E8M0; NVFP4: [N][K/16] E4M3
  const float* bias;      // [N] fp32 or null
  const float* alpha_ptr; // device alpha, or null to use `alpha`
  void* D;                // [M][N] bf16/fp16
  float alpha;
  int M, N, K;
  // Row pitches: bytes per row of A and of B, elements per row of D (packed: K or K/2, and N).
  // Split-K partials stay packed [M][N].  (Next to the shape: read in the same kernel-argument load.)
  int row_a, row_b, ldd;
  int tiles_m, tiles_n;   // output tile grid
  int splits;             // split-K factor (1: none)
  int scale_ktile;        // 0: sA / sB row-major [rows][KB]; 1: K-tile-major [ceil(KB/4)][rows][4]
  int ws_through;         // NVFP4 split plans: 1 = partial stores write through the L2 (store_partials)
  float* ws;              // split-K partials [batch][splits][M][N] fp32 (plan-owned), or null
  // Batched problems: grid.z = batch count; batch z uses each pointer advanced by z * its stride
  // (bytes; a stride of 0 shares one matrix / bias vector among all batches).
  int64_t stride_a, stride_b, stride_sa, stride_sb, stride_bias, stride_d;
};

// Byte offset of scale code `blk` (K block) of operand row `row` in either scale layout: row-major
// [rows][KB], or K-tile-major, where the 4 codes of K-block group g of every row are stored
// together: group g, row r, code c at byte (g * rows + r) * 4 + c.
__device__ __forceinline__ size_t scale_offset(bool ktile, int row, int blk, int rows, int KB) {
  return ktile ? ((size_t)(blk >> 2) * rows + row) * 4 + (blk & 3) : (size_t)row * KB + blk;
}

// Move this workgroup's operand, output and workspace pointers to its batch (blockIdx.z).
__device__ __forceinline__ void select_batch(GemmArgs& p) {
  const int64_t z = blockIdx.z;
  p.A += z * p.stride_a;
  p.B += z * p.stride_b;
  p.sA += z * p.stride_sa;
  p.sB += z * p.stride_sb;
  p.bias = (const float*)((const uint8_t*)p.bias + z * p.stride_bias);
  p.D = (uint8_t*)p.D + z * p.stride_d;
  if (p.ws) p.ws += z * (int64_t)p.splits * p.M * p.N;
}

// A launcher: enqueues one kernel on `stream` with a precomputed launch shape.  Kernels use static
// LDS only; no dynamic LDS is requested at launch.
typedef hipError_t (*LaunchFn)(const GemmArgs& args, dim3 grid, dim3 block, hipStream_t stream);

struct KernelVariant {
  const char* name;
  LaunchFn launch;
  int tile_m, tile_n, tile_k;
  int block_threads;
  uint32_t lds_bytes;    // static LDS of the kernel (informational)
  bool linear_grid;      // grid = (tiles_m * tiles_n * splits) workgroups in x; else (tiles_n, tiles_m)
  int max_splits = 1;    // > 1: the kernel supports split-K up to this factor (needs a workspace)
  // Split-K cost model of a split-capable kernel (microseconds, fitted to timings on MI355X): one K
  // tile of a workgroup's loop while the grid fills at most one workgroup per CU, one MiB of fp32
  // partials per split (stored by the GEMM kernel, read back by the finish kernel), and the fixed
  // cost of splitting at all (the finish kernel's launch and ramp, the split kernel's own prologue).
  float ktile_us = 0.0f, partial_us_per_mib = 0.0f, split_fixed_us = 0.0f;
  bool persistent = false;  // the kernel loops over tiles: launch at most one workgroup per CU
};

// Variant tables, one per format: index = out dtype (0 bf16, 1 f16) * 4 + bias * 2 + silu.
// Each kernel family returns its table for the M bucket it serves.
// `batch`: problems per launch (the grid holds tiles x batch workgroups).  `packed_ab`: A and B rows
// are K bytes apart (the large-shape MXFP8 kernel's copies assume it).
const KernelVariant* mxfp8_variants(int64_t M, int64_t N, int64_t K, int64_t batch, bool packed_ab);
const KernelVariant* mxfp8_tiled_variants(int64_t M, int64_t N, int64_t batch);
const KernelVariant* mxfp8_pp_variants();
const KernelVariant* nvfp4_variants(int64_t M, int64_t N, int64_t K, int64_t batch);

inline int variant_index(Out out, bool bias, bool silu) {
  return (out == Out::F16 ? 4 : 0) + (bias ? 2 : 0) + (silu ? 1 : 0);
}

}  // namespace bsg
