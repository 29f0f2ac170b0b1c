// MXFP8 block-scaled GEMM, LDS-tiled kernel for gfx950 (the main path for K % 128 == 0).
//
// Same operation as mxfp8_gemm.hip (E4M3 operands with one E8M0 scale per 32 K elements, the
// mx_float8_t / float_ue8m0_t operands of the nvFuser PR #5736 page), organised for CDNA4:
//
// * Workgroup tile 256 x 256, K tile 128, 4 waves in a 2 x 2 arrangement, each wave owning a
//   128 x 128 block of D as 4 x 4 accumulators of v_mfma_scale_f32_32x32x64_f8f6f4 (256 fp32
//   accumulator registers per lane).
// * A and B K-tiles are copied global -> LDS with global_load_lds_dwordx4 (16 bytes per lane, no
//   register staging) into a two-stage ring (2 x 64 KiB), so the copy of tile k+1 runs while the
//   MFMAs consume tile k; one workgroup barrier per K tile.
// * LDS rows are 128 bytes = 8 chunks of 16 bytes; chunk c of row R is stored at chunk
//   c ^ f(R), f(R) = (R & 7) ^ ((R >> 3) & 1).  The MFMA fragment reads (ds_read_b128 of one
//   chunk from 8 or 16 consecutive rows) then hit distinct banks.
// * E8M0 scales go straight from global memory to registers, one dword (the 4 blocks of a K tile)
//   per row and K tile, prefetched one tile ahead.
// * Workgroups are dispatched round-robin over the 8 XCDs; the tile order gives each XCD a
//   contiguous range of tiles, walked in groups of 8 tile-rows, so that concurrently resident
//   workgroups of one XCD share A and B panels in its L2.
//
// Operand register layout of the scaled MFMA (measured on the device): lane l (r = l % 32,
// h = l / 32) holds K bytes [16h, 16h+16) and [32+16h, 32+16h+16) of its row, and its scale
// byte is the E8M0 code of 32-block h.  Accumulator element e: row 8*(e/4) + 4*h + e%4, column r.
#include "common.h"
#include "epilogue.h"

namespace bsg {
namespace {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int A_TILE = BM * BK;            // bytes per stage
constexpr int B_TILE = BN * BK;
constexpr int STAGE = A_TILE + B_TILE;     // 64 KiB
constexpr int THREADS = 256;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ v16f mfma_mx(v8i a, v8i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ int2 tile_of(int bid, int tiles_m, int tiles_n) {
  const int T = tiles_m * tiles_n;
  int id = bid;
  if ((T & 7) == 0) id = (bid & 7) * (T >> 3) + (bid >> 3);  // contiguous range per XCD
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int group = id / per_group;
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int in_group = id - group * per_group;
  return make_int2(first_m + in_group % gsize, in_group / gsize);
}

// Copy one 256 x 128-byte operand tile (rows row0.., K bytes k0..k0+127) into LDS `dst`.
// Wave w issues 8 instructions; instruction q fills LDS rows 8*(8w+q) .. +8 (1 KiB).  Lane j of
// an instruction writes LDS bytes [16j, 16j+16) of that KiB: row R = 8*(8w+q) + j/8, physical chunk
// j%8, which holds logical chunk (j%8) ^ swz(R).
__device__ __forceinline__ void copy_tile(const uint8_t* __restrict__ src, int ld, int row0, int rows_valid, int k0,
                                          uint8_t* dst, int wave, int lane) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int R0 = 8 * (8 * wave + q);
    const int R = R0 + (lane >> 3);
    const int c = (lane & 7) ^ swz(R);
    const int grow = min(R, rows_valid - 1);  // rows past the edge re-read a valid row; never stored
    const uint8_t* g = src + (size_t)(row0 + grow) * ld + k0 + 16 * c;
    __builtin_amdgcn_global_load_lds((const void*)g, (lds_void*)(dst + R0 * BK), 16, 0, 0);
  }
}

template <Out O, bool BIAS, bool SILU>
__global__ __launch_bounds__(THREADS, 1) void mxfp8_tiled_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int2 t = tile_of(blockIdx.x, p.tiles_m, p.tiles_n);
  const int m0 = t.x * BM, n0 = t.y * BN;
  const int K = p.K, KB = K >> 5, KT = K / BK;
  const int m_valid = min(BM, p.M - m0), n_valid = min(BN, p.N - n0);

  // per-lane LDS offsets of the two 16-byte chunks of k-step ks (see the layout comment above)
  const int f = swz(r);
  int off[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    off[ks][0] = 16 * ((4 * ks + h) ^ f);
    off[ks][1] = 16 * ((4 * ks + 2 + h) ^ f);
  }
  const int a_row = (wm * 128 + r) * BK;  // LDS byte offset of this lane's row in row-tile 0
  const int b_row = (wn * 128 + r) * BK;

  // scale pointers: one dword = the 4 E8M0 codes of a K tile, per row-tile
  const uint32_t* sa_ptr[4];
  const uint32_t* sb_ptr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int am = min(wm * 128 + 32 * i + r, m_valid - 1);
    const int bn = min(wn * 128 + 32 * i + r, n_valid - 1);
    sa_ptr[i] = (const uint32_t*)(p.sA + (size_t)(m0 + am) * KB);
    sb_ptr[i] = (const uint32_t*)(p.sB + (size_t)(n0 + bn) * KB);
  }

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v16f){};

  // prologue: tile 0 -> stage 0, scales of tile 0 -> registers
  copy_tile(p.A, K, m0, m_valid, 0, lds, wave, lane);
  copy_tile(p.B, K, n0, n_valid, 0, lds + A_TILE, wave, lane);
  uint32_t sa_next[4], sb_next[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sa_next[i] = sa_ptr[i][0];
    sb_next[i] = sb_ptr[i][0];
  }

  for (int kt = 0; kt < KT; ++kt) {
    uint32_t sa_cur[4], sb_cur[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa_cur[i] = sa_next[i];
      sb_cur[i] = sb_next[i];
    }
    __syncthreads();  // tile kt is in LDS stage kt&1; everyone is done reading stage (kt+1)&1
    if (kt + 1 < KT) {
      uint8_t* nxt = lds + ((kt + 1) & 1) * STAGE;
      copy_tile(p.A, K, m0, m_valid, (kt + 1) * BK, nxt, wave, lane);
      copy_tile(p.B, K, n0, n_valid, (kt + 1) * BK, nxt + A_TILE, wave, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa_next[i] = sa_ptr[i][kt + 1];
        sb_next[i] = sb_ptr[i][kt + 1];
      }
    }
    const uint8_t* sa_lds = lds + (kt & 1) * STAGE;
    const uint8_t* sb_lds = sa_lds + A_TILE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8i af[4], bf[4];
      int sa[4], sb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint8_t* pa = sa_lds + a_row + i * 32 * BK;
        const uint8_t* pb = sb_lds + b_row + i * 32 * BK;
        const v4i a0 = *(const v4i*)(pa + off[ks][0]), a1 = *(const v4i*)(pa + off[ks][1]);
        const v4i b0 = *(const v4i*)(pb + off[ks][0]), b1 = *(const v4i*)(pb + off[ks][1]);
        af[i] = (v8i){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        bf[i] = (v8i){b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        // block 2*ks + h of this K tile, moved to byte 0
        sa[i] = (int)(sa_cur[i] >> (8 * (2 * ks + h)));
        sb[i] = (int)(sb_cur[i] >> (8 * (2 * ks + h)));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_mx(af[i], bf[j], acc[i][j], sa[i], sb[j]);
    }
  }

  // epilogue
  const float alpha = load_alpha(p);
  uint16_t* D = (uint16_t*)p.D;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * 128 + 32 * j + r;
    if (n >= p.N) continue;
    const float bv = BIAS ? p.bias[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 128 + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
        if (m < p.M) D[(size_t)m * p.N + n] = to_out_bits<O>(epi_value<SILU>(acc[i][j][e], alpha, bv));
      }
    }
  }
}

template <Out O, bool BIAS, bool SILU>
hipError_t launch_tiled(const GemmArgs& args, dim3 grid, dim3 block, hipStream_t stream) {
  void* kargs[] = {(void*)&args};
  return hipLaunchKernel((const void*)&mxfp8_tiled_kernel<O, BIAS, SILU>, grid, block, kargs, 0, stream);
}

#define BSG_MX_TILED(O, B, S) \
  { "mxfp8_tiled_256x256x128", &launch_tiled<O, B, S>, BM, BN, BK, THREADS, 2 * STAGE, true }
const KernelVariant kTiled[8] = {
    BSG_MX_TILED(Out::BF16, false, false), BSG_MX_TILED(Out::BF16, false, true),
    BSG_MX_TILED(Out::BF16, true, false),  BSG_MX_TILED(Out::BF16, true, true),
    BSG_MX_TILED(Out::F16, false, false),  BSG_MX_TILED(Out::F16, false, true),
    BSG_MX_TILED(Out::F16, true, false),   BSG_MX_TILED(Out::F16, true, true),
};
#undef BSG_MX_TILED

}  // namespace

const KernelVariant* mxfp8_tiled_variants() { return kTiled; }

}  // namespace bsg
