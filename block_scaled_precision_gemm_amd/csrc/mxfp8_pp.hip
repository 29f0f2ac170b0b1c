// MXFP8 block-scaled GEMM: 8-wave ping-pong kernel for gfx950 (K % 512 == 0, large M x N).
//
// Same operation as mxfp8_gemm.hip (E4M3 operands with one E8M0 scale per 32 K elements: the
// mx_float8_t / float_ue8m0_t operands of the nvFuser PR #5736 page).
//
// * Workgroup tile 256 x 256, eight waves, two per SIMD.  Wave w = 4g + s (g = group, s = SIMD)
//   owns rows 128g .. 128g+127 and columns 64s .. 64s+63 of the tile: 4 x 2 accumulators of
//   v_mfma_scale_f32_32x32x64_f8f6f4 (128 registers).
// * Ping-pong: the two waves of a SIMD alternate between a memory phase (fragment reads of the next
//   64-wide K slice from LDS, and copies) and a compute phase (its 8 MFMAs on one 64-wide K slice,
//   512 cycles).  Group 1 starts one phase late, so in every phase one group computes while the
//   other moves data, and one barrier per phase keeps them in step.  With a single wave per SIMD
//   the copies, fragment reads and barriers could not overlap that wave's own MFMAs.
// * Global -> LDS: K tiles of 128 bytes per row (64 KiB per 256 x 256 tile pair), two LDS stages,
//   filled by buffer_load_dwordx4 ... lds with 8 lanes per 128-byte row piece.  Full 128-byte row
//   pieces stream about 1.7x faster than 64-byte ones (measured in this access pattern), which is
//   what lets the copies keep up with the MFMAs.  Every memory phase issues one quarter of the next
//   K tile (4 instructions per wave), so the address work of the copies is spread evenly: issuing a
//   whole tile in one phase held that phase's memory waves back.
// * E8M0 scales arrive every 512 K as 16 bytes per row (double-buffered; A's copied by group 0, B's
//   by group 1); the K loop is unrolled over those 512 K so stage offsets and wait counts are
//   compile-time.  Copies past the last K tile use an offset beyond the buffer's range: zero-filled,
//   no memory traffic.
// * LDS rows are 128 bytes = 8 chunks of 16; chunk c of row R is stored at chunk c ^ ((R >> 1) & 7),
//   which makes every 16-lane group of a fragment read hit 64 distinct banks.
// * Epilogue: MFMA operands are swapped (B_j x A_i^T) so a lane's accumulators run along 4
//   consecutive columns; values are finished in registers (alpha, bias, SiLU, rounding), staged in
//   LDS and stored along rows, 16 bytes per lane.
// * XCD-aware tile order: workgroups go to the 8 XCDs round-robin, so each XCD gets a contiguous
//   range of tile ids, walked in groups of 8 tile-rows; the tiles an XCD runs at once share A and B
//   panels in its L2.
// * Persistent: the plan launches at most one workgroup per CU; workgroup b computes the tiles of
//   virtual ids b, b + grid, b + 2 grid, ... (with a grid that is a multiple of 8 each keeps its
//   XCD, and every round covers the same tiles as a one-tile-per-workgroup launch), which saves
//   the workgroup relaunch between tiles.
//
// Scaled-MFMA operand layout (measured on the device): lane l (r = l % 32, h = l / 32) holds K bytes
// [16h, 16h+16) and [32+16h, 32+16h+16) of its row's 64-byte slice; its scale byte is the E8M0
// code of 32-block h.
#include <type_traits>

#include "common.h"
#include "epilogue.h"

namespace bsg {
namespace mxp {

constexpr int BM = 256, BN = 256;
constexpr int BK = 128;                          // K bytes per row per LDS stage
constexpr int HK = 64;                           // K per phase (one MFMA K step)
constexpr int NS = 2, UNROLL = 8;                // LDS stages; phases per 512 K (one scale batch)
constexpr int WAVES = 8, THREADS = 64 * WAVES;
constexpr int WROWS = 128, WCOLS = 64;           // a wave's block of D
constexpr int TM = WROWS / 32, TN = WCOLS / 32;  // 4 x 2 MFMA tiles per wave
constexpr int A_TILE = BM * BK, B_TILE = BN * BK;  // 32 KiB each; LDS: A stages, then B stages
constexpr int B_BASE = NS * A_TILE;
constexpr int SCALE_BYTES = 16;                                            // per row per 512 K
constexpr int SCALE_BUF = (BM + BN) * SCALE_BYTES;                         // 8 KiB: A rows, B rows
constexpr int MAIN_LDS = NS * (A_TILE + B_TILE) + 2 * SCALE_BUF;          // 144 KiB
constexpr int EPI_ROW = 2 * WCOLS + 16, EPI_WAVE = WROWS * EPI_ROW;        // 64 cols + pad
constexpr int LDS_BYTES = MAIN_LDS > WAVES * EPI_WAVE ? MAIN_LDS : WAVES * EPI_WAVE;
constexpr int CPW = BM * BK / 1024 / 8;  // copy instructions per wave per 64-wide K slice: 4
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)
// An offset past any operand buffer (operands have < 2^31 bytes, so no 32-bit wrap): the load
// returns zeros without touching memory.
constexpr uint32_t kOutOfRange = 0x80000000u;
static_assert(LDS_BYTES <= 160 * 1024, "LDS");
static_assert(CPW * 8 * 4 * 2 == BM && BM == BN, "copy split: 2 row halves x 4 waves x 4 instructions x 8 rows");
static_assert(4 * 64 == BM && 4 * 64 == BN, "scale split: 4 waves x 64 rows per operand");
static_assert(TM == 4 && TN == 2, "the accumulator pin lists 4 x 2 tiles");

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Scaled MFMA; SEL picks byte SEL of each 32-bit scale operand.
template <int SEL>
__device__ __forceinline__ v16f mfma_mx(v8i a, v8i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, SEL, sa, SEL, sb);
}

__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

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

// vmcnt wait with an LDS wait, then the barrier; the barrier alone.
template <int N>
__device__ __forceinline__ void phase_end() {
  if constexpr (N < 0)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <Out O, bool BIAS, bool SILU, bool KTILE>
__global__ __launch_bounds__(THREADS, 1) void mxfp8_pp_kernel(GemmArgs p) {
  select_batch(p);
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
  // two buffers, each A's 256 rows then B's, 16 scale bytes per row for 512 K: row-major scales as
  // [row][16] (dword d = K tile d of the 512), K-tile-major scales as [d][row][4]
  uint8_t* const scale_lds = lds + NS * (A_TILE + B_TILE);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2, ws = wave & 3;
  const int r = lane & 31, h = lane >> 5;
  const int n_tiles = p.tiles_m * p.tiles_n;
#pragma unroll 1
  for (int vb = blockIdx.x; vb < n_tiles; vb += gridDim.x) {  // one tile per pass
    const int2 t = tile_of(vb, p.tiles_m, p.tiles_n);
    const int m0 = t.x * BM, n0 = t.y * BN;
    const int K = p.K, KB = K >> 5, KT = K / BK;  // K tiles of 128
    const int m_valid = min(BM, p.M - m0), n_valid = min(BN, p.N - n0);

    const __amdgpu_buffer_rsrc_t rsA =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.A + (size_t)m0 * K), (short)0, m_valid * K, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rsB =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.B + (size_t)n0 * K), (short)0, n_valid * K, kRsrcWord3);
    // Copies of K tile k+1 are spread over the four memory phases of K tile k (slices u even / odd of
    // group 0 / group 1), one quarter each: operand g ^ (u & 1), rows 128 (u & 1) .. +127.  So group 0
    // copies A rows 0..127 (even u) and B rows 128..255 (odd u), group 1 B rows 0..127 and A rows
    // 128..255.  Every wave issues the same instruction mix (copies under a branch make the compiler
    // drain them before LDS reads); group 0 copies A's scales, group 1 B's.
    const __amdgpu_buffer_rsrc_t rsT0 = grp == 0 ? rsA : rsB, rsT1 = grp == 0 ? rsB : rsA;
    // Scale buffer of operand g from the tile's first row.  K-tile-major: up to the array's end (rows
    // past the operand's last row read other rows' codes, which only reach outputs never stored).
    const int s_all = grp == 0 ? p.M : p.N, s_first = grp == 0 ? m0 : n0;
    const uint8_t* const s_base = grp == 0 ? p.sA : p.sB;
    const __amdgpu_buffer_rsrc_t rsS =
        KTILE ? __builtin_amdgcn_make_buffer_rsrc((void*)(s_base + (size_t)s_first * 4), (short)0,
                                                  KB * s_all - 4 * s_first, kRsrcWord3)
              : __builtin_amdgcn_make_buffer_rsrc((void*)(s_base + (size_t)s_first * KB), (short)0,
                                                  (grp == 0 ? m_valid : n_valid) * KB, kRsrcWord3);

    // Copy plan: a quarter is 128 rows x 128 bytes = 16 instructions of 8 rows; wave 4g + s issues
    // instructions 4s .. 4s+3 (rows 32s + 8q .. +7 of the half).  Lane j writes LDS bytes
    // [16j, 16j+16) of the instruction's KiB: row R = 8*ins + j/8, physical chunk j%8, holding logical
    // chunk (j%8) ^ swz(R), so the 8 lanes of a row read its whole 128-byte piece.  swz(R) =
    // (4q + lane / 16) & 7 depends on q only through its parity, so the lane part of the offset takes
    // two values; the row part (128 half + 8q) K goes to the scalar offset.
    uint32_t voff[2];
#pragma unroll
    for (int qp = 0; qp < 2; ++qp) {
      const int R = 32 * ws + 8 * qp + (lane >> 3);
      voff[qp] = (uint32_t)(R - 8 * qp) * (uint32_t)K + 16u * (uint32_t)((lane & 7) ^ swz(R));
    }
    uint8_t* const copy_dst0 = lds + grp * B_BASE + CPW * ws * 1024;              // operand g, rows 0..127
    uint8_t* const copy_dst1 = lds + (1 - grp) * B_BASE + (16 + CPW * ws) * 1024;  // the other, 128..255
    // Scale plan: wave 4g + s copies 1 KiB of operand g's scales per 512 K: row-major, rows 64s ..
    // 64s+63, 16 bytes each; K-tile-major, K tile s of the 512 for all 256 rows (4 rows per lane).
    const uint32_t soff = KTILE ? 16u * (uint32_t)lane : (uint32_t)(64 * ws + lane) * (uint32_t)KB;
    uint8_t* const sdst = scale_lds + grp * BM * SCALE_BYTES + 64 * ws * SCALE_BYTES;

    auto copy_quarter = [&](auto sc, auto pc, int kt) {
      constexpr int stage = decltype(sc)::value;
      constexpr int par = decltype(pc)::value;
      static_assert(A_TILE == B_TILE, "one stage stride for both operands");
      uint8_t* dst = (par ? copy_dst1 : copy_dst0) + stage * A_TILE;
      const __amdgpu_buffer_rsrc_t rs = par ? rsT1 : rsT0;
      const uint32_t k0 = kt < KT ? (uint32_t)kt * BK + (uint32_t)(128 * par) * (uint32_t)K : kOutOfRange;
#pragma unroll
      for (int q = 0; q < CPW; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + q * 1024), 16, voff[q & 1],
                                                 k0 + (uint32_t)(8 * q) * (uint32_t)K, 0, 0);
    };
    auto copy_scales = [&](auto bc, int batch) {
      constexpr int buf = decltype(bc)::value;
      const uint32_t k0 = batch >= KT * BK / 512 ? kOutOfRange
                          : KTILE                 ? (uint32_t)(4 * batch + ws) * 4u * (uint32_t)s_all
                                                  : (uint32_t)batch * SCALE_BYTES;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsS, (lds_void*)(sdst + buf * SCALE_BUF), 16, soff, k0, 0, 0);
    };

    // per-lane LDS offsets of the fragment chunks h and 2 + h of the first 64-byte half of a row
    // (rows 32i + r share r's swizzle); the second half uses chunks 4 + h and 6 + h
    const int f = swz(r);
    const int off00 = 16 * (h ^ f), off01 = 16 * ((2 + h) ^ f);
    const int off10 = 16 * ((4 + h) ^ f), off11 = 16 * ((6 + h) ^ f);
    const int a_row = (WROWS * grp + r) * BK;
    const int b_row = (WCOLS * ws + r) * BK;

    v8i af[TM], bf[TN];
    uint32_t sa[TM][4], sb[TN][4];  // 16 scale bytes per row-tile for the current 512 K

    auto read_frags = [&](auto sc, auto hc) {
      constexpr int stage = decltype(sc)::value;
      constexpr int half = decltype(hc)::value;
      const int o0 = half ? off10 : off00, o1 = half ? off11 : off01;
      const uint8_t* a_lds = lds + stage * A_TILE;
      const uint8_t* b_lds = lds + B_BASE + stage * B_TILE;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const uint8_t* pa = a_lds + a_row + i * 32 * BK;
        const v4i x0 = *(const v4i*)(pa + o0), x1 = *(const v4i*)(pa + o1);
        af[i] = (v8i){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint8_t* pb = b_lds + b_row + j * 32 * BK;
        const v4i x0 = *(const v4i*)(pb + o0), x1 = *(const v4i*)(pb + o1);
        bf[j] = (v8i){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
    };
    // Dword d of a row's 16 scale bytes holds the 32-blocks of K tile d of the batch; shifted right by
    // 8h, slice 2d + e finds the byte of its block h at byte 2e, which the MFMA selects itself (no
    // per-slice shifts ahead of the MFMAs).
    auto read_scales = [&](auto bc) {
      constexpr int buf = decltype(bc)::value;
      const uint8_t* s = scale_lds + buf * SCALE_BUF;
      const int hs = 8 * h;
      auto row_scales = [&](const uint8_t* base, int row, uint32_t* out) {
        if constexpr (KTILE) {
#pragma unroll
          for (int d = 0; d < 4; ++d) out[d] = *(const uint32_t*)(base + d * 1024 + row * 4) >> hs;
        } else {
          const v4i v = *(const v4i*)(base + row * SCALE_BYTES);
#pragma unroll
          for (int d = 0; d < 4; ++d) out[d] = v[d] >> hs;
        }
      };
#pragma unroll
      for (int i = 0; i < TM; ++i) row_scales(s, WROWS * grp + 32 * i + r, sa[i]);
#pragma unroll
      for (int j = 0; j < TN; ++j) row_scales(s + BM * SCALE_BYTES, WCOLS * ws + 32 * j + r, sb[j]);
    };

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = (v16f){};

    // Prologue: K tile 0 and the scales of the first 512 K become visible at the barrier.  Group 1 then
    // waits one phase.
    copy_quarter(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, 0);
    copy_quarter(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}, 0);
    copy_scales(std::integral_constant<int, 0>{}, 0);
    phase_end<0>();
    if (grp == 1) barrier_only();

    // Phase u (0..7) of a 512-K batch works on K slice kb + 64u: K tile (kb + 64u) / 128 in stage
    // (u / 2) % 2, half u % 2.  With global phases 2h .. 2h+3 for the memory / compute phases of
    // slices 2t and 2t+1 (group 0 at 2h, 2h+2; group 1 at 2h+1, 2h+3), group 0 reads the next K tile
    // at 2h+4 and group 1 at 2h+5; A rows 128..255 are read only by group 1.  Waits (before the barrier
    // that ends a phase): group 0 drains its copies at the end of its compute phase of odd u (2h+3);
    // group 1 drains its even-u quarter at the end of its memory phase of odd u (2h+3) and everything
    // at the end of its compute phase of odd u (2h+4).  The scale share, issued at u == 1 with the
    // odd quarter, is drained with it.
    int kb = 0;  // in 64-wide K slices
    auto step = [&](auto uc, auto bc) {
      constexpr int u = decltype(uc)::value;
      constexpr int buf = decltype(bc)::value;  // scale buffer of this batch
      constexpr int stage = (u >> 1) & 1;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (u == 0) read_scales(bc);
      read_frags(std::integral_constant<int, stage>{}, std::integral_constant<int, u & 1>{});
      copy_quarter(std::integral_constant<int, stage ^ 1>{}, std::integral_constant<int, u & 1>{}, (kb + u) / 2 + 1);
      if constexpr (u == 1) copy_scales(std::integral_constant<int, buf ^ 1>{}, kb / UNROLL + 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (u & 1) {
        if (grp == 1)
          phase_end<CPW + (u == 1 ? 1 : 0)>();  // the quarter copied at u - 1
        else
          phase_end<-1>();
      } else {
        phase_end<-1>();
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = mfma_mx<2 * (u & 1)>(bf[j], af[i], acc[i][j], (int)sb[j][u >> 1], (int)sa[i][u >> 1]);
      // The MFMAs have no memory effects; this empty asm that reads their results keeps them inside
      // this phase (otherwise they can sink past the group-dependent barrier branches below).
      asm volatile("" ::"v"(acc[0][0]), "v"(acc[0][1]), "v"(acc[1][0]), "v"(acc[1][1]), "v"(acc[2][0]),
                   "v"(acc[2][1]), "v"(acc[3][0]), "v"(acc[3][1]));
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (u & 1)
        phase_end<0>();  // both quarters (and at u == 1 the scales)
      else
        barrier_only();
    };
    auto batch = [&](auto bc) {
      step(std::integral_constant<int, 0>{}, bc);
      step(std::integral_constant<int, 1>{}, bc);
      step(std::integral_constant<int, 2>{}, bc);
      step(std::integral_constant<int, 3>{}, bc);
      step(std::integral_constant<int, 4>{}, bc);
      step(std::integral_constant<int, 5>{}, bc);
      step(std::integral_constant<int, 6>{}, bc);
      step(std::integral_constant<int, 7>{}, bc);
      kb += UNROLL;
    };
    const int KS = K / HK;  // 64-wide K slices, a multiple of 8
    for (; kb + 2 * UNROLL <= KS;) {
      batch(std::integral_constant<int, 0>{});
      batch(std::integral_constant<int, 1>{});
    }
    if (kb < KS) batch(std::integral_constant<int, 0>{});

    // Epilogue.  Group 0 catches up with group 1's last compute phase; then every wave has drained
    // its copies and LDS reads before the stages are reused for staging.
    // acc[i][j] holds rows 32i.., columns 32j.. of the wave's 128 x 64 block, transposed: lane (r, h),
    // element 4g + c is row r, column 8g + 4h + c.
    __builtin_amdgcn_sched_barrier(0);
    if (grp == 0) barrier_only();
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const float alpha = load_alpha(p);
    uint8_t* const eb = lds + wave * EPI_WAVE;
    const int nw = n0 + WCOLS * ws;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = 32 * j + 8 * g + 4 * h;
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BIAS) {
          if (nw + c0 < p.N) {  // bias is 4-byte aligned (the ABI's promise): four dword loads
            const float* b = p.bias + nw + c0;
            bv[0] = b[0]; bv[1] = b[1]; bv[2] = b[2]; bv[3] = b[3];
          }
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const v16f& a = acc[i][j];
          const uint32_t lo = epi_pack2<SILU, O>(a[4 * g + 0], a[4 * g + 1], alpha, bv[0], bv[1]);
          const uint32_t hi = epi_pack2<SILU, O>(a[4 * g + 2], a[4 * g + 3], alpha, bv[2], bv[3]);
          *(uint2*)(eb + (32 * i + r) * EPI_ROW + 2 * c0) = make_uint2(lo, hi);
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the block is private to this wave
    uint16_t* D = (uint16_t*)p.D;
    const int mw = m0 + WROWS * grp;
    const int cc = 8 * (lane & 7);  // this lane's 8 columns; 8 lanes per 128-byte row
#pragma unroll
    for (int q = 0; q < WROWS / 8; ++q) {
      const int row = 8 * q + (lane >> 3);
      const v4i v = *(const v4i*)(eb + row * EPI_ROW + 2 * cc);
      const int m = mw + row, n = nw + cc;
      if (m < p.M && n < p.N) *(v4i*)(D + (size_t)m * p.ldd + n) = v;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // staging read before the next prologue
  }
}

template <Out O, bool BIAS, bool SILU>
hipError_t launch_pp(const GemmArgs& args, dim3 grid, dim3 block, hipStream_t stream) {
  void* kargs[] = {(void*)&args};
  const void* k = args.scale_ktile ? (const void*)&mxfp8_pp_kernel<O, BIAS, SILU, true>
                                   : (const void*)&mxfp8_pp_kernel<O, BIAS, SILU, false>;
  return hipLaunchKernel(k, grid, block, kargs, 0, stream);
}

#define BSG_MX_PP(O, B, S) \
  { "mxfp8_pp_256x256x64_w8", &launch_pp<O, B, S>, BM, BN, BK, THREADS, (uint32_t)LDS_BYTES, true, 1, 0.0f, 0.0f, \
    0.0f, true }
const KernelVariant kPp[8] = {
    BSG_MX_PP(Out::BF16, false, false), BSG_MX_PP(Out::BF16, false, true),
    BSG_MX_PP(Out::BF16, true, false),  BSG_MX_PP(Out::BF16, true, true),
    BSG_MX_PP(Out::F16, false, false),  BSG_MX_PP(Out::F16, false, true),
    BSG_MX_PP(Out::F16, true, false),   BSG_MX_PP(Out::F16, true, true),
};
#undef BSG_MX_PP

}  // namespace mxp

const KernelVariant* mxfp8_pp_variants() { return mxp::kPp; }

}  // namespace bsg
