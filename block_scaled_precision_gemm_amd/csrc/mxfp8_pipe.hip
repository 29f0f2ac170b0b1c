// MXFP8 block-scaled GEMM, deep-pipelined kernel for gfx950 (K % 512 == 0, large M x N).
//
// Same operation as mxfp8_gemm.hip (E4M3 operands, one E8M0 scale per 32 K elements: the
// mx_float8_t / float_ue8m0_t operands of the nvFuser PR #5736 page).  Measured on MI355X, the
// two-stage kernel (mxfp8_tiled.hip) spends most of its time waiting for global memory: one tile of
// prefetch does not cover the load latency, and per-row scale loads (one scattered dword per row and
// K tile) cost as much again.  This kernel keeps more bytes in flight and gathers the scales in bulk:
//
// * Workgroup tile 256 x 256, K tile 64, 8 waves (2 x 4), each wave 128 x 64 of D as 4 x 2
//   accumulators of v_mfma_scale_f32_32x32x64_f8f6f4 (two waves per SIMD).
// * A 4-stage LDS ring (4 x 32 KiB) filled by buffer_load_dwordx4 ... lds: the copy of tile k+3 is
//   issued while tile k is consumed.  Each wave waits only for its own copy of tile k
//   (s_waitcnt vmcnt(n) with n = the loads it issued after that copy), then one barrier.
// * E8M0 scales: every 8 K tiles (512 K elements = 16 bytes per row), each wave issues one 16-byte
//   LDS-DMA load covering 64 rows of A or B; lanes then read their rows' 16 bytes once per 8 tiles.
// * The K loop is unrolled by 8 tiles so stage offsets and wait counts are compile-time constants.
//   Past the last tile the copies still run (re-reading the last tile into a stage nobody reads),
//   which keeps every wave's load count uniform.
// * LDS rows are 64 bytes = 4 chunks of 16; chunk c of row R is stored at chunk c ^ g(R),
//   g(R) = ((R >> 1) & 3) ^ ((R >> 3) & 1): the fragment reads (one chunk of 8 or 16 consecutive rows
//   per ds_read_b128 pass) hit distinct banks for 32- and for 64-bank LDS.
// * XCD-aware tile order as in mxfp8_tiled.hip.
//
// Scaled-MFMA operand layout (measured on the device): lane l (r = l % 32, h = l / 32) holds K bytes
// [16h, 16h+16) and [32+16h, 32+16h+16) of its row; its scale byte is the E8M0 code of 32-block h.
// Accumulator element e: row 8*(e/4) + 4*h + e%4, column r.
#include <type_traits>

#include "common.h"
#include "epilogue.h"

namespace bsg {
namespace mxp {

constexpr int BM = 256, BN = 256, BK = 64, NS = 4, UNROLL = 8;
constexpr int WM = 2, WN = 4, WAVES = WM * WN, THREADS = 64 * WAVES;
constexpr int TM = BM / WM / 32, TN = BN / WN / 32;  // 4 x 2 MFMA tiles per wave
constexpr int A_TILE = BM * BK, B_TILE = BN * BK, STAGE = A_TILE + B_TILE;  // 32 KiB
constexpr int SCALE_BYTES = 16;                                            // per row per 8 K tiles
constexpr int SCALE_A = BM * SCALE_BYTES, SCALE_B = BN * SCALE_BYTES;      // 4 KiB each
constexpr int MAIN_LDS = NS * STAGE + SCALE_A + SCALE_B;                   // 136 KiB
// epilogue staging: each wave's 128 x 64 output block, rows padded to 144 bytes (16-byte aligned)
constexpr int EPI_ROW = 144, EPI_WAVE = 128 * EPI_ROW;
constexpr int LDS_BYTES = MAIN_LDS > WAVES * EPI_WAVE ? MAIN_LDS : WAVES * EPI_WAVE;  // 144 KiB
constexpr int COPIES = (BM + BN) / 16 / WAVES;  // 16-row copy instructions per wave per tile: 4
constexpr uint32_t kRsrcWord3 = 0x00020000u;     // raw buffer, 32-bit data format (gfx9 family)
static_assert(COPIES == 4, "copy split");
static_assert(LDS_BYTES <= 160 * 1024, "LDS");

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }

__device__ __forceinline__ v16f mfma_mx(v8i a, v8i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Wait until at most N of this wave's vector-memory loads are outstanding, then meet the other waves
// at the workgroup barrier.  Written as one asm block with a memory clobber so that no LDS access is
// moved across it, and so that no full vmcnt(0) wait (which would drain the prefetches) is implied.
template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
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

// Loads a wave issues after the copy of tile t and before the wait for tile t at the start of
// iteration t: the copies of tiles t+1 and t+2 (4 each) plus the scale load that follows the copy of
// every tile u with u % 8 == 4 when u is in [t, t+2].
constexpr int loads_after(int t_mod8) {
  int n = 2 * COPIES;
  for (int u = t_mod8; u <= t_mod8 + 2; ++u)
    if (u % UNROLL == 4) n += 1;
  return n;
}

template <Out O, bool BIAS, bool SILU>
__global__ __launch_bounds__(THREADS, 1) void mxfp8_pipe_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
  uint8_t* const scale_lds = lds + NS * STAGE;  // [A rows][16] then [B rows][16]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 31, h = lane >> 5;
  const int wm = wave / WN, wn = wave % WN;
  const int2 t = tile_of(blockIdx.x, p.tiles_m, p.tiles_n);
  const int m0 = t.x * BM, n0 = t.y * BN;
  const int K = p.K, KB = K >> 5, KT = K / BK;
  const int m_valid = min(BM, p.M - m0), n_valid = min(BN, p.N - n0);

  const __amdgpu_buffer_rsrc_t rsA =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.A + (size_t)m0 * K), (short)0, m_valid * K, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsB =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.B + (size_t)n0 * K), (short)0, n_valid * K, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsSA =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.sA + (size_t)m0 * KB), (short)0, m_valid * KB, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsSB =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.sB + (size_t)n0 * KB), (short)0, n_valid * KB, kRsrcWord3);

  // Copy plan.  Per tile the workgroup issues 16 A and 16 B instructions of 16 rows x 64 bytes; wave w
  // issues A instructions 2w, 2w+1 and B instructions 2w, 2w+1.  Lane j of an instruction writes LDS
  // bytes [16j, 16j+16) of its KiB: row R = 16*ins + j/4, physical chunk j%4 = logical (j%4) ^ swz(R).
  uint32_t voff[2];
  int lds_row[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    lds_row[q] = 16 * (2 * wave + q);
    const int R = lds_row[q] + (lane >> 2);
    voff[q] = (uint32_t)R * (uint32_t)K + 16u * (uint32_t)((lane & 3) ^ swz(R));
  }
  // Scale plan: waves 0..3 load 64 A rows each, waves 4..7 64 B rows each: 16 bytes per row.
  const bool scale_a = wave < 4;
  const int srow0 = 64 * (wave & 3);
  const uint32_t soff = (uint32_t)(srow0 + lane) * (uint32_t)KB;
  uint8_t* const sdst = scale_lds + (scale_a ? 0 : SCALE_A) + srow0 * SCALE_BYTES;

  auto copy_tile = [&](int kt, int stage) {
    uint8_t* a_dst = lds + stage * STAGE;
    uint8_t* b_dst = a_dst + A_TILE;
    // past the last tile, re-read the last tile (in bounds, never consumed) so that every wave issues
    // the same number of loads per step
    const uint32_t k0 = (uint32_t)min(kt, KT - 1) * BK;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_void*)(a_dst + lds_row[q] * BK), 16, voff[q], k0, 0, 0);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_void*)(b_dst + lds_row[q] * BK), 16, voff[q], k0, 0, 0);
  };
  auto copy_scales = [&](int batch) {
    const uint32_t k0 = (uint32_t)min(batch, KT / UNROLL - 1) * SCALE_BYTES;
    if (scale_a)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsSA, (lds_void*)sdst, 16, soff, k0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsSB, (lds_void*)sdst, 16, soff, k0, 0, 0);
  };

  // per-lane LDS offsets of the fragment chunks h and 2 + h
  const int f = swz(r);
  const int off0 = 16 * (h ^ f), off1 = 16 * ((2 + h) ^ f);
  const int a_row = (wm * TM * 32 + r) * BK;
  const int b_row = (wn * TN * 32 + r) * BK;

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (v16f){};

  // prologue: scales of batch 0, tiles 0..2
  copy_scales(0);
  copy_tile(0, 0);
  copy_tile(1, 1);
  copy_tile(2, 2);

  uint32_t sa[TM][4], sb[TN][4];  // this batch's 16 scale bytes per row-tile
  int kb = 0;
  // one K tile; U = position in the batch of 8 (compile-time: stage, wait count, scale byte)
  auto step = [&](auto uc) {
    constexpr int u = decltype(uc)::value;
    const int kt = kb + u;
    // tile kt is in stage u%4 for all waves; everyone is done with stage (u+3)%4
    wait_vmcnt_barrier<loads_after(u)>();
    copy_tile(kt + 3, (u + 3) % NS);
    if constexpr (u == 0) {
      // scales of this batch (landed with the wait above); read once per 8 tiles
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const v4i v = *(const v4i*)(scale_lds + (wm * TM * 32 + 32 * i + r) * SCALE_BYTES);
        sa[i][0] = v[0]; sa[i][1] = v[1]; sa[i][2] = v[2]; sa[i][3] = v[3];
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v4i v = *(const v4i*)(scale_lds + SCALE_A + (wn * TN * 32 + 32 * j + r) * SCALE_BYTES);
        sb[j][0] = v[0]; sb[j][1] = v[1]; sb[j][2] = v[2]; sb[j][3] = v[3];
      }
    }
    if constexpr (u == 1) copy_scales(kb / UNROLL + 1);  // every wave read this batch's scales at u == 0
    const uint8_t* a_lds = lds + (u % NS) * STAGE;
    const uint8_t* b_lds = a_lds + A_TILE;
    v8i af[TM], bf[TN];
    int ssa[TM], ssb[TN];
    const int shift = 8 * (2 * (u & 1) + h);  // byte 2u + h of the 16 is in dword u/2
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const uint8_t* pa = a_lds + a_row + i * 32 * BK;
      const v4i x0 = *(const v4i*)(pa + off0), x1 = *(const v4i*)(pa + off1);
      af[i] = (v8i){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      ssa[i] = (int)(sa[i][u >> 1] >> shift);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const uint8_t* pb = b_lds + b_row + j * 32 * BK;
      const v4i x0 = *(const v4i*)(pb + off0), x1 = *(const v4i*)(pb + off1);
      bf[j] = (v8i){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      ssb[j] = (int)(sb[j][u >> 1] >> shift);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma_mx(bf[j], af[i], acc[i][j], ssb[j], ssa[i]);
  };
  for (; kb < KT; kb += UNROLL) {
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
    step(std::integral_constant<int, 4>{});
    step(std::integral_constant<int, 5>{});
    step(std::integral_constant<int, 6>{});
    step(std::integral_constant<int, 7>{});
  }
  // Epilogue.  acc[i][j] holds the 32 x 32 block (rows 32i.., columns 32j.. of the wave's 128 x 64)
  // transposed: lane (r, h), element 4g + c is row r, column 8g + 4h + c.  Each lane applies alpha,
  // bias and SiLU to its values, converts them, writes 4-column pieces into the wave's LDS block, and
  // the wave then stores its block row by row with 16 bytes per lane (128-byte row segments).
  wait_vmcnt_barrier<0>();  // no LDS-DMA write in flight, every wave done with the pipeline buffers
  const float alpha = load_alpha(p);
  uint8_t* const eb = lds + wave * EPI_WAVE;
  const int nw = n0 + wn * TN * 32;  // first column of the wave's block
#pragma unroll
  for (int j = 0; j < TN; ++j) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c0 = 32 * j + 8 * g + 4 * h;  // first of this lane's 4 columns in the block
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BIAS) {
        if (nw + c0 < p.N) {
          const v4f b4 = *(const v4f*)(p.bias + nw + c0);
          bv[0] = b4[0]; bv[1] = b4[1]; bv[2] = b4[2]; bv[3] = b4[3];
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const v16f& a = acc[i][j];
        const uint32_t lo = pack2_out<O>(epi_value<SILU>(a[4 * g + 0], alpha, bv[0]),
                                         epi_value<SILU>(a[4 * g + 1], alpha, bv[1]));
        const uint32_t hi = pack2_out<O>(epi_value<SILU>(a[4 * g + 2], alpha, bv[2]),
                                         epi_value<SILU>(a[4 * g + 3], alpha, bv[3]));
        *(uint2*)(eb + (32 * i + r) * EPI_ROW + 2 * c0) = make_uint2(lo, hi);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done (block is wave-private)
  uint16_t* D = (uint16_t*)p.D;
  const int mw = m0 + wm * TM * 32;  // first row of the wave's block
  const int cc = 8 * (lane & 7);     // this lane's 8 columns
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int row = 8 * q + (lane >> 3);
    const v4i v = *(const v4i*)(eb + row * EPI_ROW + 2 * cc);
    const int m = mw + row, n = nw + cc;
    if (m < p.M && n < p.N) *(v4i*)(D + (size_t)m * p.N + n) = v;
  }
}

template <Out O, bool BIAS, bool SILU>
hipError_t launch_pipe(const GemmArgs& args, dim3 grid, dim3 block, hipStream_t stream) {
  void* kargs[] = {(void*)&args};
  return hipLaunchKernel((const void*)&mxfp8_pipe_kernel<O, BIAS, SILU>, grid, block, kargs, 0, stream);
}

#define BSG_MX_PIPE(O, B, S) \
  { "mxfp8_pipe_256x256x64_s4", &launch_pipe<O, B, S>, BM, BN, BK, THREADS, (uint32_t)LDS_BYTES, true }
const KernelVariant kPipe[8] = {
    BSG_MX_PIPE(Out::BF16, false, false), BSG_MX_PIPE(Out::BF16, false, true),
    BSG_MX_PIPE(Out::BF16, true, false),  BSG_MX_PIPE(Out::BF16, true, true),
    BSG_MX_PIPE(Out::F16, false, false),  BSG_MX_PIPE(Out::F16, false, true),
    BSG_MX_PIPE(Out::F16, true, false),   BSG_MX_PIPE(Out::F16, true, true),
};
#undef BSG_MX_PIPE

}  // namespace mxp

const KernelVariant* mxfp8_pipe_variants() { return mxp::kPipe; }

}  // namespace bsg
