// MXFP8 block-scaled GEMM, LDS-tiled kernels for gfx950 (every shape the large-shape kernel does not
// take: fewer than 256 tiles of 256 x 256, or K % 512 != 0; any K % 32 == 0).
//
// Same operation as mxfp8_gemm.hip (E4M3 operands with one E8M0 scale per 32 K elements, the
// mx_float8_t / float_ue8m0_t operands of the nvFuser PR #5736 page), organised for CDNA4:
//
// * Workgroup tile BM x BN, K tile 128, WM x WN waves, each wave owning a (BM/WM) x (BN/WN) block
//   of D as 32 x 32 accumulators of v_mfma_scale_f32_32x32x64_f8f6f4.  With 8 waves two waves
//   share each SIMD, so one wave's LDS reads overlap the other's MFMAs.
// * A and B K-tiles are copied global -> LDS with buffer_load_dwordx4 ... lds (16 bytes per lane,
//   no register staging) into a two-stage ring (three stages for split plans of 128 x 128 tiles with
//   at least 8 K tiles per workgroup), so the copies of the next tiles run while the MFMAs consume
//   tile k; one workgroup barrier per K tile.  Each lane's buffer offsets are computed once; the K
//   position is a scalar offset.  Rows past M (or N) lie outside the buffer range and read as 0.
// * LDS rows are 128 bytes = 8 chunks of 16 bytes; chunk c of row R is stored at chunk
//   c ^ f(R), f(R) = (R & 7) ^ ((R >> 3) & 1).  The MFMA fragment reads (ds_read_b128 of one
//   chunk from 8 or 16 consecutive rows) then hit distinct banks.
// * E8M0 scales (4 codes per row per K tile) are copied into LDS with the operands, one 4-byte copy
//   per row, and read from there (see the scale modes below for the row-major K % 512 == 0 and the
//   partial-tile cases, which keep them in registers).
// * K % 128 != 0: the last K tile is partial.  Its chunks past K are copied from an out-of-range
//   offset (zeros) and its missing 32-blocks get scale code 127 (2^0), so they add exact zeros.
// * Workgroups are dispatched round-robin over the 8 XCDs; the tile order gives each XCD a
//   contiguous range of tiles, walked in groups of 8 tile-rows, so that concurrently resident
//   workgroups of one XCD share A and B panels in its L2.
// * Row-major scales with K % 512 == 0 (BULK, 128 x 128 tiles): a row's codes for 4 K tiles are one
//   aligned 16-byte piece, loaded once per 4 K tiles instead of a dword per K tile (the per-tile
//   loads touch one cache line per row each time, more line requests than the operand copies).
// * Epilogue through LDS: with B as the MFMAs' first operand each lane holds 4 consecutive output
//   columns per group; each wave finishes 32 rows at a time in registers, stages them in its own
//   padded LDS block and stores 16-byte row pieces (2-byte scattered stores were the largest cost
//   of short-K shapes).
// * Split-K (SPLIT, small tile grids): workgroup id = split * tiles + tile; split s covers a
//   contiguous range of K tiles and writes its fp32 sums to the plan's workspace ws[s][m][n], which
//   splitk.h's finish kernel adds in split order and finishes (alpha, bias, SiLU, rounding).
//
// Operand register layout of the scaled MFMA (measured on the device): lane l (r = l % 32,
// h = l / 32) holds K bytes [16h, 16h+16) and [32+16h, 32+16h+16) of its row, and its scale
// byte is the E8M0 code of 32-block h.  Accumulator element e: row 8*(e/4) + 4*h + e%4, column r.
#include "common.h"
#include "epilogue.h"
#include "splitk.h"

namespace bsg {
// Named (not anonymous) namespace: kernel templates instantiated on these configuration types need
// external linkage for their host-side launch stubs to be emitted.
namespace mxt {

constexpr int BK = 128;
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)
constexpr uint32_t kOutOfRange = 0x80000000u;  // a buffer offset past any range: the load returns zeros

typedef __attribute__((address_space(3))) void lds_void;

template <int BM_, int BN_, int WM_, int WN_, int MAX_SPLITS_, int NS_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, MAX_SPLITS = MAX_SPLITS_;
  static constexpr int NS = NS_;  // LDS stages: copies run NS - 1 K tiles ahead
  static constexpr int WAVES = WM * WN, THREADS = 64 * WAVES;
  static constexpr int TM = BM / WM / 32, TN = BN / WN / 32;  // 32x32 MFMA tiles per wave
  static constexpr int A_TILE = BM * BK, B_TILE = BN * BK, STAGE = A_TILE + B_TILE;
  static constexpr int A_COPIES = BM / 8 / WAVES, B_COPIES = BN / 8 / WAVES;  // per wave per K tile
  static_assert(TM >= 1 && TN >= 1, "wave tile must hold at least one 32x32 MFMA tile");
  static_assert(A_COPIES * 8 * WAVES == BM && B_COPIES * 8 * WAVES == BN, "copy split");
  static_assert(NS >= 2 && NS * STAGE <= 160 * 1024, "LDS");
  static constexpr int COPIES = A_COPIES + B_COPIES;
  static constexpr int SSTAGE = (BM + BN) * 4;  // scale codes of a K tile staged in LDS (kScaleLds)
  static_assert(BM + BN == 64 * WAVES && NS * (STAGE + SSTAGE) <= 160 * 1024, "scale staging");
};

using Large = Cfg<256, 256, 2, 4, 1, 2>;    // 8 waves of 128 x 64 (enough tiles to fill the chip: no split)
using Small = Cfg<128, 128, 2, 2, 16, 2>;   // 4 waves of 64 x 64, for problems with few large tiles
using Small3 = Cfg<128, 128, 2, 2, 16, 3>;  // the same with a third stage (twice the bytes in flight per
                                            // CU), for K ranges of 8 K tiles or more

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

// The same order for the split-K finish kernel's blocks (splitk.h).
struct TiledOrder {
  __device__ static int2 of(int t, int tiles_m, int tiles_n) { return tile_of(t, tiles_m, tiles_n); }
};

// Copy plan for one operand tile (ROWS rows x 128 bytes): wave w issues COPIES instructions; its
// instruction q fills LDS rows 8*(COPIES*w + q) .. +8 (1 KiB).  Lane j of an instruction writes LDS
// bytes [16j, 16j+16) of that KiB: row R = 8*(COPIES*w+q) + j/8, physical chunk j%8, which holds
// logical chunk (j%8) ^ swz(R).  voff[q] is the lane's byte offset of that chunk in the operand
// buffer (relative to the tile's first row, at K position 0).
template <int COPIES>
struct CopyPlan {
  uint32_t voff[COPIES];
  int kpos[COPIES];  // K offset of the lane's chunk within the tile
  int lds_row0;      // first LDS row of the wave's first instruction (wave-uniform)

  __device__ __forceinline__ void init(int wave, int lane, int ld) {
    lds_row0 = 8 * COPIES * wave;
#pragma unroll
    for (int q = 0; q < COPIES; ++q) {
      const int R = lds_row0 + 8 * q + (lane >> 3);
      kpos[q] = 16 * ((lane & 7) ^ swz(R));
      voff[q] = (uint32_t)R * (uint32_t)ld + (uint32_t)kpos[q];
    }
  }

  // Copy the K tile at byte k0 of each row; `left` = K - k0.  TAIL (K % 128 != 0): in the last,
  // partial tile the chunks past K take an out-of-range offset and read as zeros (branch-free: a
  // select per copy).
  template <bool TAIL>
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rsrc, uint32_t k0, int left, uint8_t* tile) const {
#pragma unroll
    for (int q = 0; q < COPIES; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(tile + (lds_row0 + 8 * q) * BK), 16,
                                               TAIL && kpos[q] >= left ? kOutOfRange : voff[q], k0, 0, 0);
  }
};

// Scale handling of a launch (template argument SM):
//   kScaleLds   K % 128 == 0 (either layout; not the group case): the tile's codes are copied into
//               LDS with the operands, one 4-byte copy per row and K tile (64 rows per wave), and
//               read from there.  Per-tile dword loads by every wave that needs a row touched one
//               cache line per row and wave (4096x4096x4224 row-major: 72.8 -> 62.6 us);
//   kScaleGroup row-major, K % 512 == 0, 128 x 128 tiles: one 16-byte group per row per 4 K tiles
//               held in registers;
//   kScaleTail  K % 128 != 0: a partial last K tile (zero-filled chunks; missing blocks' codes 127),
//               codes loaded per row and K tile (row-major rows are not dword-aligned);
//   kScaleTile  K-tile-major, three-stage split plans: one dword per row per K tile in registers,
//               loaded a tile ahead (already one cache line per 32 rows; an LDS round trip at the
//               head of each short K tile cost 9% at 128x8192x8192).
enum : int { kScaleLds = 0, kScaleGroup = 1, kScaleTail = 2, kScaleTile = 3 };

template <class C, Out O, bool BIAS, bool SILU, bool SPLIT, int SM>
__global__ __launch_bounds__(C::THREADS, 1) void mxfp8_tiled_kernel(GemmArgs p) {
  constexpr bool BULK = SM == kScaleGroup, TAIL = SM == kScaleTail, LDSS = SM == kScaleLds;
  constexpr int TILE_LOADS = C::COPIES + (LDSS ? 1 : 0);  // memory instructions per K tile and wave
  select_batch(p);
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::NS * C::STAGE + (LDSS ? C::NS * C::SSTAGE : 0)];
  constexpr int TM = C::TM, TN = C::TN;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 31, h = lane >> 5;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int T = p.tiles_m * p.tiles_n;
  int bid = blockIdx.x, kt_begin = 0, kt_end = (p.K + BK - 1) / BK;
  if constexpr (SPLIT) {  // split-major ids; split s gets K tiles [s KT / S, (s + 1) KT / S)
    const int s = bid / T;
    bid -= s * T;
    kt_begin = (int)((int64_t)s * kt_end / p.splits);
    kt_end = (int)((int64_t)(s + 1) * kt_end / p.splits);
  }
  const int2 t = tile_of(bid, p.tiles_m, p.tiles_n);
  const int m0 = t.x * C::BM, n0 = t.y * C::BN;
  const int K = p.K, KB = K >> 5;
  const int m_valid = min(C::BM, p.M - m0), n_valid = min(C::BN, p.N - n0);

  // operand buffers start at the tile's first row and end at the last valid row
  const __amdgpu_buffer_rsrc_t rsA =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.A + (size_t)m0 * p.row_a), (short)0, (m_valid - 1) * p.row_a + K,
                                        kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsB =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.B + (size_t)n0 * p.row_b), (short)0, (n_valid - 1) * p.row_b + K,
                                        kRsrcWord3);
  CopyPlan<C::A_COPIES> cpA;
  CopyPlan<C::B_COPIES> cpB;
  cpA.init(wave, lane, p.row_a);
  cpB.init(wave, lane, p.row_b);

  // per-lane LDS offsets of the two 16-byte chunks of k-step ks (see the layout comment above)
  const int f = swz(r);
  int off[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    off[ks][0] = 16 * ((4 * ks + h) ^ f);
    off[ks][1] = 16 * ((4 * ks + 2 + h) ^ f);
  }
  const int a_row = (wm * TM * 32 + r) * BK;  // LDS byte offset of this lane's row in row-tile 0
  const int b_row = (wn * TN * 32 + r) * BK;

  // scale pointers: one dword = the 4 E8M0 codes of a K tile, dword kt * step of a row's pointer
  // (row-major: consecutive dwords; K-tile-major: one dword per row per K tile); rows past the edge
  // re-read a valid row
  size_t sa_row[TM], sb_row[TN];  // byte offset of the row's first code (K tile 0)
#pragma unroll
  for (int i = 0; i < TM; ++i)
    sa_row[i] = scale_offset(p.scale_ktile, m0 + min(wm * TM * 32 + 32 * i + r, m_valid - 1), 0, p.M, KB);
#pragma unroll
  for (int j = 0; j < TN; ++j)
    sb_row[j] = scale_offset(p.scale_ktile, n0 + min(wn * TN * 32 + 32 * j + r, n_valid - 1), 0, p.N, KB);
  // TAIL: scale word of K tile kt (4 codes, code c in byte c), loaded per row; codes of 32-blocks
  // past K become 127 (2^0): their data are zeros, so they add nothing, whatever the padding holds.
  // K-tile-major: the dword at row + 4 kt rows.  Row-major rows are not dword-aligned (KB % 4 != 0):
  // the codes come from the aligned dword holding the first one and, only when they run into it,
  // the next dword, joined with a byte-align shift (no load reaches a dword past the last code).
  auto scale_word = [&](const uint8_t* base, size_t row, int rows, int kt) -> uint32_t {
    if constexpr (SM == kScaleTile) return *(const uint32_t*)(base + row + (size_t)kt * rows * 4);
    const int blk0 = 4 * kt, valid = KB - blk0;
    uint32_t w = 0;
    if (p.scale_ktile) {
      w = *(const uint32_t*)(base + row + (size_t)kt * rows * 4);
    } else {
      const size_t at = row + blk0;
      const uint32_t* d = (const uint32_t*)(base + (at & ~(size_t)3));
      const int sh = (int)(at & 3);
      const uint32_t lo = d[0];
      const uint32_t hi = sh + min(valid, 4) > 4 ? d[1] : 0u;
      w = __builtin_amdgcn_alignbyte(hi, lo, sh);
    }
    if (valid < 4) w = (w & ((1u << (8 * valid)) - 1u)) | (0x7F7F7F7Fu << (8 * valid));
    return w;
  };

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (v16f){};

  // BULK: the 16-byte group of 4 K tiles holding tile kt, per row-tile
  v4i sa_grp[TM], sb_grp[TN];
  auto load_group = [&](int g) {
#pragma unroll
    for (int i = 0; i < TM; ++i) sa_grp[i] = *(const v4i*)(p.sA + sa_row[i] + 16 * g);
#pragma unroll
    for (int j = 0; j < TN; ++j) sb_grp[j] = *(const v4i*)(p.sB + sb_row[j] + 16 * g);
  };

  // LDSS: wave w copies the codes of rows 64w .. 64w+63 of the tile's [A rows | B rows] (4 bytes per
  // row and K tile; rows past M / N lie outside the buffer range and read as zeros).
  uint8_t* const sc_lds = lds + C::NS * C::STAGE;
  auto sc_stage_of = [&](int t) { return sc_lds + ((t - kt_begin) % C::NS) * C::SSTAGE; };
  const bool s_is_a = 64 * wave < C::BM;  // wave-uniform
  // Row-major: row r's codes of K tile t at r * KB + 4t; K-tile-major: at 4r + 4t * rows (the range
  // then ends at the array's end: rows past the operand's last read other rows' codes, which only
  // reach outputs never stored).
  const int s_all = s_is_a ? p.M : p.N, s_first = s_is_a ? m0 : n0;
  const uint32_t s_rowb = p.scale_ktile ? 4u : (uint32_t)KB, s_tb = p.scale_ktile ? 4u * (uint32_t)s_all : 4u;
  const uint32_t s_range = p.scale_ktile ? (uint32_t)KB * (uint32_t)s_all - 4u * (uint32_t)s_first
                                         : (uint32_t)(s_is_a ? m_valid : n_valid) * (uint32_t)KB;
  const __amdgpu_buffer_rsrc_t rsS = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((s_is_a ? p.sA : p.sB) + (size_t)s_first * s_rowb), (short)0, (int)s_range, kRsrcWord3);
  const uint32_t s_voff = (uint32_t)(64 * wave + lane - (s_is_a ? 0 : C::BM)) * s_rowb;
  auto issue_scales = [&](int t) {
    if constexpr (LDSS)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsS, (lds_void*)(sc_stage_of(t) + 256 * wave), 4, s_voff,
                                               t < kt_end ? (uint32_t)t * s_tb : kOutOfRange, 0, 0);
  };

  // Copies of K tile t into its ring stage; with three stages, tiles past the split's range are
  // issued with an out-of-range offset (zeros, no traffic), so every iteration issues the same
  // number of copies and a fixed vmcnt proves a tile has landed.
  auto stage_of = [&](int t) { return lds + ((t - kt_begin) % C::NS) * C::STAGE; };
  auto issue_tile = [&](int t) {
    const bool real = t < kt_end;
    const uint32_t k0 = real ? (uint32_t)t * BK : kOutOfRange;
    const int left = real ? K - t * BK : 0;
    cpA.template issue<TAIL>(rsA, k0, left, stage_of(t));
    cpB.template issue<TAIL>(rsB, k0, left, stage_of(t) + C::A_TILE);
    issue_scales(t);
  };
  uint32_t sa_next[TM], sb_next[TN];
  auto load_scales = [&](int t) {
#pragma unroll
    for (int i = 0; i < TM; ++i) sa_next[i] = scale_word(p.sA, sa_row[i], p.M, t);
#pragma unroll
    for (int j = 0; j < TN; ++j) sb_next[j] = scale_word(p.sB, sb_row[j], p.N, t);
  };

  // prologue: the first NS - 1 K tiles -> stages 0 .., the first tile's scales -> registers
  if constexpr (BULK) load_group(kt_begin >> 2);
  else if constexpr (!LDSS) load_scales(kt_begin);
  if constexpr (C::NS == 2) {
    cpA.template issue<TAIL>(rsA, (uint32_t)kt_begin * BK, K - kt_begin * BK, lds);
    cpB.template issue<TAIL>(rsB, (uint32_t)kt_begin * BK, K - kt_begin * BK, lds + C::A_TILE);
    issue_scales(kt_begin);
  } else {
#pragma unroll
    for (int t = 0; t < C::NS - 1; ++t) issue_tile(kt_begin + t);
  }

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    // LDS-DMA copies count in vmcnt only; the barrier does not wait for them, and the compiler waits
    // only before this wave's own LDS reads, so each wave drains its copies of tile kt here: after
    // the barrier the whole tile is in its stage and everyone is done reading the stage that the
    // next copies overwrite.  NS >= 3 stages: the copies of tiles kt+1 .. kt+NS-2 (the last
    // (NS - 2) * TILE_LOADS memory instructions issued) may stay in flight.
    if constexpr (C::NS == 2) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      static_assert((C::NS - 2) * TILE_LOADS < 64, "tiles in flight at the barrier");
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((C::NS - 2) * TILE_LOADS) : "memory");
    }
    __syncthreads();
    uint32_t sa_cur[TM], sb_cur[TN];
    if constexpr (LDSS) {
      const uint8_t* sc = sc_stage_of(kt);
#pragma unroll
      for (int i = 0; i < TM; ++i) sa_cur[i] = *(const uint32_t*)(sc + 4 * (wm * TM * 32 + 32 * i + r));
#pragma unroll
      for (int j = 0; j < TN; ++j) sb_cur[j] = *(const uint32_t*)(sc + 4 * (C::BM + wn * TN * 32 + 32 * j + r));
    } else if constexpr (BULK) {
      const int u = kt & 3;
#pragma unroll
      for (int i = 0; i < TM; ++i) sa_cur[i] = (uint32_t)sa_grp[i][u];
#pragma unroll
      for (int j = 0; j < TN; ++j) sb_cur[j] = (uint32_t)sb_grp[j][u];
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i) sa_cur[i] = sa_next[i];
#pragma unroll
      for (int j = 0; j < TN; ++j) sb_cur[j] = sb_next[j];
    }
    if constexpr (C::NS >= 3) {
      // next tile's scales first, then tile kt+NS-1's copies (into the stage tile kt-1 used)
      if constexpr (BULK) {
        if (((kt + 1) & 3) == 0 && kt + 1 < kt_end) load_group((kt + 1) >> 2);
      } else if constexpr (!LDSS) {
        load_scales(min(kt + 1, kt_end - 1));
      }
      // keep the scale loads here, a whole K tile ahead of their use (left to itself the scheduler
      // sinks them below the MFMAs, and the next barrier then waits out their latency)
      __builtin_amdgcn_sched_barrier(0);
      issue_tile(kt + C::NS - 1);
    } else if (kt + 1 < kt_end) {
      uint8_t* nxt = lds + ((kt + 1 - kt_begin) & 1) * C::STAGE;
      const uint32_t k1 = (uint32_t)(kt + 1) * BK;
      cpA.template issue<TAIL>(rsA, k1, K - (int)k1, nxt);
      cpB.template issue<TAIL>(rsB, k1, K - (int)k1, nxt + C::A_TILE);
      issue_scales(kt + 1);
      if constexpr (BULK) {
        if (((kt + 1) & 3) == 0) load_group((kt + 1) >> 2);  // lands before the next barrier
      } else if constexpr (!LDSS) {
#pragma unroll
        for (int i = 0; i < TM; ++i) sa_next[i] = scale_word(p.sA, sa_row[i], p.M, kt + 1);
#pragma unroll
        for (int j = 0; j < TN; ++j) sb_next[j] = scale_word(p.sB, sb_row[j], p.N, kt + 1);
      }
    }
    const uint8_t* a_lds = stage_of(kt);
    const uint8_t* b_lds = a_lds + C::A_TILE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8i af[TM], bf[TN];
      int sa[TM], sb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const uint8_t* pa = a_lds + a_row + i * 32 * BK;
        const v4i x0 = *(const v4i*)(pa + off[ks][0]), x1 = *(const v4i*)(pa + off[ks][1]);
        af[i] = (v8i){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        sa[i] = (int)(sa_cur[i] >> (8 * (2 * ks + h)));  // block 2*ks + h of this K tile, in byte 0
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint8_t* pb = b_lds + b_row + j * 32 * BK;
        const v4i x0 = *(const v4i*)(pb + off[ks][0]), x1 = *(const v4i*)(pb + off[ks][1]);
        bf[j] = (v8i){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        sb[j] = (int)(sb_cur[j] >> (8 * (2 * ks + h)));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_mx(bf[j], af[i], acc[i][j], sb[j], sa[i]);
    }
  }

  // Epilogue, staged through LDS.  B is the MFMAs' first operand, so acc[i][j] holds the transposed
  // block: lane (r, h) element e is row 32i + r, column 32j + 8(e/4) + 4h + e%4 of the wave's block,
  // four consecutive columns per e/4.  One pass per row-tile i: the wave finishes its 32 rows in
  // registers (alpha, bias, SiLU, rounding; split: the raw fp32 sums), writes them to its own padded
  // LDS block, and reads them back as 16-byte row pieces for the global stores (rows past M and
  // pieces past N are not stored).
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();  // every wave is done with both stages
  constexpr int ES = SPLIT ? 4 : 2;     // bytes per output element
  constexpr int ECOLS = 32 * TN;        // columns of the wave's block
  constexpr int EROW = ECOLS * ES + 16;  // padded LDS row, bytes
  constexpr int PPR = ECOLS * ES / 16;  // 16-byte pieces per row
  constexpr int RPI = 64 / PPR;         // rows per read-back instruction
  static_assert(C::WAVES * 32 * EROW <= C::NS * C::STAGE && RPI * PPR == 64, "epilogue staging");
  uint8_t* const eb = lds + wave * 32 * EROW;
  const int mw = m0 + wm * TM * 32, nw = n0 + wn * TN * 32;
  const float alpha = SPLIT ? 1.0f : load_alpha(p);
  uint8_t* const out = SPLIT ? (uint8_t*)(p.ws + (size_t)(blockIdx.x / T) * p.M * p.N) : (uint8_t*)p.D;
  float bv[TN][4][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int n = nw + 32 * j + 8 * g + 4 * h + c;
        bv[j][g][c] = BIAS && n < p.N ? p.bias[n] : 0.0f;
      }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const v16f& a = acc[i][j];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint8_t* const dst = eb + r * EROW + (32 * j + 8 * g + 4 * h) * ES;
        if constexpr (SPLIT) {
          *(v4f*)dst = (v4f){a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
        } else {
          const uint32_t lo = epi_pack2<SILU, O>(a[4 * g + 0], a[4 * g + 1], alpha, bv[j][g][0], bv[j][g][1]);
          const uint32_t hi = epi_pack2<SILU, O>(a[4 * g + 2], a[4 * g + 3], alpha, bv[j][g][2], bv[j][g][3]);
          *(uint2*)dst = make_uint2(lo, hi);
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the block is private to this wave
#pragma unroll
    for (int q = 0; q < 32 / RPI; ++q) {
      const int row = RPI * q + lane / PPR, pc = lane % PPR;
      const v4i v = *(const v4i*)(eb + row * EROW + 16 * pc);
      const int m = mw + 32 * i + row, n = nw + pc * (16 / ES);
      if (m < p.M && n < p.N) {
        v4i* const dst = (v4i*)(out + ((size_t)m * (SPLIT ? p.N : p.ldd) + n) * ES);
        if constexpr (SPLIT)
          __builtin_nontemporal_store(v, dst);  // partials: streaming store, read once by the finish kernel
        else
          *dst = v;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read back before the next pass rewrites it
  }
}

// The kernel of one configuration for a launch's scale mode and split.
template <class C, Out O, bool BIAS, bool SILU>
const void* tiled_kernel_for(int sm, bool split) {
  constexpr int kGroupOrTile = C::BM == 128 ? kScaleGroup : kScaleLds;  // no group mode for 256 x 256
  constexpr int kTileOrLds = C::NS >= 3 ? kScaleTile : kScaleLds;        // register mode: deep rings only
  if (sm == kScaleTile) return split ? (const void*)&mxfp8_tiled_kernel<C, O, BIAS, SILU, true, kTileOrLds>
                                     : (const void*)&mxfp8_tiled_kernel<C, O, BIAS, SILU, false, kTileOrLds>;
  if (!split)
    return sm == kScaleTail    ? (const void*)&mxfp8_tiled_kernel<C, O, BIAS, SILU, false, kScaleTail>
           : sm == kScaleGroup ? (const void*)&mxfp8_tiled_kernel<C, O, BIAS, SILU, false, kGroupOrTile>
                               : (const void*)&mxfp8_tiled_kernel<C, O, BIAS, SILU, false, kScaleLds>;
  return sm == kScaleTail    ? (const void*)&mxfp8_tiled_kernel<C, O, BIAS, SILU, true, kScaleTail>
         : sm == kScaleGroup ? (const void*)&mxfp8_tiled_kernel<C, O, BIAS, SILU, true, kGroupOrTile>
                             : (const void*)&mxfp8_tiled_kernel<C, O, BIAS, SILU, true, kScaleLds>;
}

template <class C, Out O, bool BIAS, bool SILU>
hipError_t launch_tiled(const GemmArgs& args, dim3 grid, dim3 block, hipStream_t stream) {
  void* kargs[] = {(void*)&args};
  // bulk scale loads: row-major scales, 16-byte aligned groups of 4 K tiles (128 x 128 tiles only: the
  // 256 x 256 configuration never sees K % 512 == 0, which goes to the large-shape kernel); the scale
  // buffers and strides must then be 16-byte aligned (the ABI promises 4), checked per call
  const bool bulk = C::BM == 128 && !args.scale_ktile && args.K % 512 == 0 &&
                    (((uintptr_t)args.sA | (uintptr_t)args.sB | (uintptr_t)args.stride_sa | (uintptr_t)args.stride_sb) &
                     15) == 0;
  int sm = args.K % BK ? kScaleTail : bulk ? kScaleGroup : kScaleLds;
  const bool split = args.splits > 1;
  // 128 x 128 tiles, split K: three LDS stages (two K tiles in flight) when each workgroup runs at
  // least 8 K tiles.  Split plans are the under-filled grids whose workgroups stream long B panels
  // from HBM with little reuse (128x8192x8192: 24.2 -> 23.2 us); unsplit grids (2048^3: 14.4 vs
  // 15.2 us) and short K ranges (256^3: 4.3 vs 4.7 us) are faster with two.
  const int tiles_per_wg = (args.K + BK - 1) / BK / args.splits;
  const bool three = C::BM == 128 && split && tiles_per_wg >= 8;
  if (three && sm == kScaleLds && args.scale_ktile) sm = kScaleTile;
  const void* k = three ? tiled_kernel_for<Small3, O, BIAS, SILU>(sm, split) : tiled_kernel_for<C, O, BIAS, SILU>(sm, split);
  const hipError_t e = hipLaunchKernel(k, grid, block, kargs, 0, stream);
  if (e != hipSuccess || !split) return e;
  // split-major ids with a multiple of 8 tiles put every split of a tile on one XCD (id % 8 is the
  // same for all of them): the finish kernel's blocks follow (splitk.h)
  if ((args.tiles_m * args.tiles_n) % 8 == 0)
    return launch_splitk_finish<O, BIAS, SILU, 0, C::BM, C::BN, TiledOrder>(args, grid.z, stream);
  return launch_splitk_finish<O, BIAS, SILU, 0>(args, grid.z, stream);
}

#define BSG_MX_TILED(NAME, C, O, B, S) \
  { NAME, &launch_tiled<C, O, B, S>, C::BM, C::BN, BK, C::THREADS, C::NS * C::STAGE, true, C::MAX_SPLITS, \
    kSplitKtileUs, kSplitPartialUsPerMib, kSplitFixedUs }
#define BSG_MX_TABLE(NAME, C)                                                                    \
  {                                                                                              \
    BSG_MX_TILED(NAME, C, Out::BF16, false, false), BSG_MX_TILED(NAME, C, Out::BF16, false, true), \
    BSG_MX_TILED(NAME, C, Out::BF16, true, false), BSG_MX_TILED(NAME, C, Out::BF16, true, true),   \
    BSG_MX_TILED(NAME, C, Out::F16, false, false), BSG_MX_TILED(NAME, C, Out::F16, false, true),   \
    BSG_MX_TILED(NAME, C, Out::F16, true, false), BSG_MX_TILED(NAME, C, Out::F16, true, true)      \
  }


// Explicit instantiations: taking a kernel template's address only inside another template does not
// make the compiler emit its host-side launch stub when the template argument is a class type.
#define BSG_MX_INST(C, SP, BU)                                                            \
  template __global__ void mxfp8_tiled_kernel<C, Out::BF16, false, false, SP, BU>(GemmArgs); \
  template __global__ void mxfp8_tiled_kernel<C, Out::BF16, false, true, SP, BU>(GemmArgs);  \
  template __global__ void mxfp8_tiled_kernel<C, Out::BF16, true, false, SP, BU>(GemmArgs);  \
  template __global__ void mxfp8_tiled_kernel<C, Out::BF16, true, true, SP, BU>(GemmArgs);   \
  template __global__ void mxfp8_tiled_kernel<C, Out::F16, false, false, SP, BU>(GemmArgs);  \
  template __global__ void mxfp8_tiled_kernel<C, Out::F16, false, true, SP, BU>(GemmArgs);   \
  template __global__ void mxfp8_tiled_kernel<C, Out::F16, true, false, SP, BU>(GemmArgs);   \
  template __global__ void mxfp8_tiled_kernel<C, Out::F16, true, true, SP, BU>(GemmArgs);
BSG_MX_INST(Large, false, kScaleTail)
BSG_MX_INST(Large, true, kScaleTail)
BSG_MX_INST(Small, false, kScaleGroup)
BSG_MX_INST(Small, true, kScaleGroup)
BSG_MX_INST(Small, false, kScaleTail)
BSG_MX_INST(Small, true, kScaleTail)
BSG_MX_INST(Small3, false, kScaleGroup)
BSG_MX_INST(Small3, true, kScaleGroup)
BSG_MX_INST(Small3, false, kScaleTail)
BSG_MX_INST(Small3, true, kScaleTail)
BSG_MX_INST(Large, false, kScaleLds)
BSG_MX_INST(Large, true, kScaleLds)
BSG_MX_INST(Small, false, kScaleLds)
BSG_MX_INST(Small, true, kScaleLds)
BSG_MX_INST(Small3, false, kScaleLds)
BSG_MX_INST(Small3, true, kScaleLds)
BSG_MX_INST(Small3, false, kScaleTile)
BSG_MX_INST(Small3, true, kScaleTile)
#undef BSG_MX_INST

// Split-K cost model of the 128 x 128 kernel (see choose_splits): fitted to split sweeps of shapes
// with 16 to 64 tiles and 8 to 64 K tiles on MI355X (the fixed cost from the unsplit timings of the
// same shapes).  The 256 x 256 configuration never splits.
constexpr float kSplitKtileUs = 0.645f, kSplitPartialUsPerMib = 0.31f, kSplitFixedUs = 4.5f;
static_assert(Small::MAX_SPLITS <= kMaxFinishSplits && Small3::MAX_SPLITS == Small::MAX_SPLITS,
              "the finish kernel sums at most kMaxFinishSplits partials");
const KernelVariant kLarge[8] = BSG_MX_TABLE("mxfp8_tiled_256x256x128_w8", Large);
const KernelVariant kSmall[8] = BSG_MX_TABLE("mxfp8_tiled_128x128x128_w4", Small);
#undef BSG_MX_TABLE
#undef BSG_MX_TILED

}  // namespace mxt

// Large tiles once they give at least one workgroup per CU (256 CUs); smaller tiles otherwise.
const KernelVariant* mxfp8_tiled_variants(int64_t M, int64_t N, int64_t batch) {
  const int64_t large_tiles = ((M + 255) / 256) * ((N + 255) / 256) * batch;
  return large_tiles >= 256 ? mxt::kLarge : mxt::kSmall;
}

}  // namespace bsg
