// MXFP8 block-scaled GEMM: 4-wave kernel with prefetched fragment reads, for gfx950
// (K % 512 == 0, large M x N).
//
// Same operation as mxfp8_gemm.hip (E4M3 operands with one E8M0 scale per 32 K elements: the
// mx_float8_t / float_ue8m0_t operands of the nvFuser PR #5736 page).
//
// * Workgroup tile 256 x 256, K tile 64, 4 waves (2 x 2), each wave 128 x 128 of D as 4 x 4
//   accumulators of v_mfma_scale_f32_32x32x64_f8f6f4 (256 accumulator registers, one wave per SIMD).
// * A 4-stage LDS ring (4 x 32 KiB) filled by buffer_load_dwordx4 ... lds; the copy of tile k+4 is
//   issued while tile k is consumed.
// * Fragment reads are prefetched: right after the barrier that publishes tile k+1, a wave issues the
//   ds_reads of tile k+1 into a second register set and then runs the 16 MFMAs of tile k from the set
//   read one iteration earlier, so no MFMA waits on LDS latency.  (With a barrier per tile, waves
//   that read their fragments after the barrier all stall at once.)
// * E8M0 scales arrive every 8 tiles as 16 bytes per row by LDS-DMA; each wave loads 64 rows of A and
//   64 rows of B.  The K loop is unrolled by 8 so stage offsets and wait counts are compile-time.
//   Past the last tile the copies re-read the last tile so every wave's load count stays uniform.
// * LDS rows are 64 bytes = 4 chunks of 16; chunk c of row R is stored at chunk c ^ g(R),
//   g(R) = ((R >> 1) & 3) ^ ((R >> 3) & 1) (conflict-free fragment reads for 32- and 64-bank LDS).
// * Epilogue: MFMA operands are swapped (B_j x A_i^T) so a lane's accumulators run along 4
//   consecutive columns; values are finished in registers (alpha, bias, SiLU, rounding), staged in
//   LDS and stored row-wise, 16 bytes per lane.
// * XCD-aware tile order as in mxfp8_tiled.hip.
//
// Scaled-MFMA operand layout (measured on the device): lane l (r = l % 32, h = l / 32) holds K bytes
// [16h, 16h+16) and [32+16h, 32+16h+16) of its row; its scale byte is the E8M0 code of 32-block h.
#include <type_traits>

#include "common.h"
#include "epilogue.h"

namespace bsg {
namespace mxq {

constexpr int BM = 256, BN = 256, BK = 64, NS = 4, UNROLL = 8;
constexpr int WM = 2, WN = 2, WAVES = WM * WN, THREADS = 64 * WAVES;
constexpr int TM = BM / WM / 32, TN = BN / WN / 32;  // 4 x 4 MFMA tiles per wave
constexpr int A_TILE = BM * BK, B_TILE = BN * BK, STAGE = A_TILE + B_TILE;  // 32 KiB
constexpr int SCALE_BYTES = 16;                                            // per row per 8 K tiles
constexpr int SCALE_A = BM * SCALE_BYTES, SCALE_B = BN * SCALE_BYTES;      // 4 KiB each
constexpr int MAIN_LDS = NS * STAGE + SCALE_A + SCALE_B;                   // 136 KiB
constexpr int EPI_ROW = 272, EPI_WAVE = 128 * EPI_ROW;                     // 128 cols + pad
constexpr int LDS_BYTES = MAIN_LDS > WAVES * EPI_WAVE ? MAIN_LDS : WAVES * EPI_WAVE;
constexpr int CPO = BM / 16 / WAVES;  // copy instructions per operand per wave per tile: 4
constexpr int COPY_LOADS = 2 * CPO;   // per tile per wave: 8
constexpr int SCALE_LOADS = 2;        // per batch per wave
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)
static_assert(LDS_BYTES <= 160 * 1024, "LDS");
static_assert(CPO * 16 * WAVES == BM && BM == BN, "copy split");

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }

__device__ __forceinline__ v16f mfma_mx(v8i a, v8i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Wait for this wave's LDS reads and for all but N of its vector-memory loads, then meet the other
// waves at the barrier.  One asm block with a memory clobber: no LDS access moves across it and no
// full vmcnt(0) drain is implied.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
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

// Loads a wave has issued after the copy of tile t+1 when it waits for that tile at the start of
// iteration t (t % 8 == u): the copies of tiles t+2 and t+3, plus the scale loads that follow the
// copy of tile 8b+5 (issued in iteration 8b+1) when that tile is one of t+1 .. t+3.
constexpr int loads_after(int u) {
  int n = 2 * COPY_LOADS;
  for (int v = u + 1; v <= u + 3; ++v)
    if (v % UNROLL == 5) n += SCALE_LOADS;
  return n;
}

template <Out O, bool BIAS, bool SILU>
__global__ __launch_bounds__(THREADS, 1) void mxfp8_plr_kernel(GemmArgs p) {
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

  // Copy plan: per tile each operand needs 16 instructions of 16 rows x 64 bytes; wave w issues
  // instructions 4w .. 4w+3 of A and of B.  Lane j writes LDS bytes [16j, 16j+16) of the KiB: row
  // R = 16*ins + j/4, physical chunk j%4, holding logical chunk (j%4) ^ swz(R).
  uint32_t voff[CPO];
#pragma unroll
  for (int q = 0; q < CPO; ++q) {
    const int R = 16 * (CPO * wave + q) + (lane >> 2);
    voff[q] = (uint32_t)R * (uint32_t)K + 16u * (uint32_t)((lane & 3) ^ swz(R));
  }
  const int lds_row0 = 16 * CPO * wave;
  // Scale plan: wave w loads rows 64w .. 64w+63 of A and of B, 16 bytes each.
  const uint32_t soff = (uint32_t)(64 * wave + lane) * (uint32_t)KB;
  uint8_t* const sdst_a = scale_lds + 64 * wave * SCALE_BYTES;
  uint8_t* const sdst_b = sdst_a + SCALE_A;

  auto copy_tile = [&](int kt, int stage) {
    uint8_t* a_dst = lds + stage * STAGE + lds_row0 * BK;
    uint8_t* b_dst = a_dst + A_TILE;
    // past the last tile, re-read the last tile (in bounds, never consumed): uniform load counts
    const uint32_t k0 = (uint32_t)min(kt, KT - 1) * BK;
#pragma unroll
    for (int q = 0; q < CPO; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_void*)(a_dst + 16 * q * BK), 16, voff[q], k0, 0, 0);
#pragma unroll
    for (int q = 0; q < CPO; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_void*)(b_dst + 16 * q * BK), 16, voff[q], k0, 0, 0);
  };
  auto copy_scales = [&](int batch) {
    const uint32_t k0 = (uint32_t)min(batch, KT / UNROLL - 1) * SCALE_BYTES;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsSA, (lds_void*)sdst_a, 16, soff, k0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsSB, (lds_void*)sdst_b, 16, soff, k0, 0, 0);
  };

  // per-lane LDS offsets of the fragment chunks h and 2 + h
  const int f = swz(r);
  const int off0 = 16 * (h ^ f), off1 = 16 * ((2 + h) ^ f);
  const int a_row = (wm * TM * 32 + r) * BK;
  const int b_row = (wn * TN * 32 + r) * BK;

  v8i af[2][TM], bf[2][TN];        // fragment sets, alternating by tile
  uint32_t sa[TM][4], sb[TN][4];   // 16 scale bytes per row-tile for the current batch

  auto read_frags = [&](int stage, int set) {
    const uint8_t* a_lds = lds + stage * STAGE;
    const uint8_t* b_lds = a_lds + A_TILE;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const uint8_t* pa = a_lds + a_row + i * 32 * BK;
      const v4i x0 = *(const v4i*)(pa + off0), x1 = *(const v4i*)(pa + off1);
      af[set][i] = (v8i){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const uint8_t* pb = b_lds + b_row + j * 32 * BK;
      const v4i x0 = *(const v4i*)(pb + off0), x1 = *(const v4i*)(pb + off1);
      bf[set][j] = (v8i){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    }
  };
  auto read_scales = [&]() {
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
  };

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (v16f){};

  // prologue: scales of batch 0 and tiles 0..3 in flight; tile 0's fragments and the scales in registers
  copy_scales(0);
  copy_tile(0, 0);
  copy_tile(1, 1);
  copy_tile(2, 2);
  copy_tile(3, 3);
  wait_barrier<3 * COPY_LOADS>();
  read_frags(0, 0);
  read_scales();

  int kb = 0;
  auto step = [&](auto uc) {
    constexpr int u = decltype(uc)::value;
    constexpr int cur = u & 1, nxt = cur ^ 1;
    const int kt = kb + u;
    // this tile's scale operands (byte 2u + h of the batch's 16 is in dword u/2)
    int ssa[TM], ssb[TN];
    const int shift = 8 * (2 * (u & 1) + h);
#pragma unroll
    for (int i = 0; i < TM; ++i) ssa[i] = (int)(sa[i][u >> 1] >> shift);
#pragma unroll
    for (int j = 0; j < TN; ++j) ssb[j] = (int)(sb[j][u >> 1] >> shift);
    // tile kt+1 is in stage (u+1)%4 for every wave; every wave has finished reading stage u%4.
    // MFMAs touch no memory, so without a scheduling barrier the previous tile's would sink below
    // this wait and push this tile's fragment reads towards the next one.
    __builtin_amdgcn_sched_barrier(0);
    wait_barrier<loads_after(u)>();
    copy_tile(kt + 4, u % NS);
    if constexpr (u == 1) copy_scales(kb / UNROLL + 1);
    read_frags((u + 1) % NS, nxt);
    if constexpr (u == UNROLL - 1) read_scales();  // next batch, for tile kt+1
    // keep those reads ahead of this tile's MFMAs: issued late, they would still be in flight at the
    // next barrier, whose lgkmcnt(0) would then stall on them
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma_mx(bf[cur][j], af[cur][i], acc[i][j], ssb[j], ssa[i]);
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

  // Epilogue.  acc[i][j] holds rows 32i.., columns 32j.. of the wave's 128 x 128 block, transposed:
  // lane (r, h), element 4g + c is row r, column 8g + 4h + c.  Finish in registers, stage in LDS,
  // store rows with 16 bytes per lane.
  wait_barrier<0>();  // no LDS-DMA write in flight; every wave done with the pipeline buffers
  const float alpha = load_alpha(p);
  uint8_t* const eb = lds + wave * EPI_WAVE;
  const int nw = n0 + wn * TN * 32;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c0 = 32 * j + 8 * g + 4 * h;
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
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the block is private to this wave
  uint16_t* D = (uint16_t*)p.D;
  const int mw = m0 + wm * TM * 32;
  const int cc = 8 * (lane & 15);  // this lane's 8 columns; 16 lanes per 256-byte row
#pragma unroll
  for (int q = 0; q < 32; ++q) {
    const int row = 4 * q + (lane >> 4);
    const v4i v = *(const v4i*)(eb + row * EPI_ROW + 2 * cc);
    const int m = mw + row, n = nw + cc;
    if (m < p.M && n < p.N) *(v4i*)(D + (size_t)m * p.N + n) = v;
  }
}

template <Out O, bool BIAS, bool SILU>
hipError_t launch_plr(const GemmArgs& args, dim3 grid, dim3 block, hipStream_t stream) {
  void* kargs[] = {(void*)&args};
  return hipLaunchKernel((const void*)&mxfp8_plr_kernel<O, BIAS, SILU>, grid, block, kargs, 0, stream);
}

#define BSG_MX_PLR(O, B, S) \
  { "mxfp8_plr_256x256x64_w4", &launch_plr<O, B, S>, BM, BN, BK, THREADS, (uint32_t)LDS_BYTES, true }
const KernelVariant kPlr[8] = {
    BSG_MX_PLR(Out::BF16, false, false), BSG_MX_PLR(Out::BF16, false, true),
    BSG_MX_PLR(Out::BF16, true, false),  BSG_MX_PLR(Out::BF16, true, true),
    BSG_MX_PLR(Out::F16, false, false),  BSG_MX_PLR(Out::F16, false, true),
    BSG_MX_PLR(Out::F16, true, false),   BSG_MX_PLR(Out::F16, true, true),
};
#undef BSG_MX_PLR

}  // namespace mxq

const KernelVariant* mxfp8_plr_variants() { return mxq::kPlr; }

}  // namespace bsg
