// NVFP4 block-scaled GEMM for gfx950.
//
// D = epi(alpha * A x B^T (+ bias)): A [M][K/2] and B [N][K/2] packed E2M1 (element 2t in the low
// nibble of byte t), one E4M3 scale per 16 K elements, a global fp32 alpha (the operation of
// runNvfp4Gemm<T, kEnableSilu, kEnableBias> on the CUTLASS issue #3003 page).
//
// CDNA4's scaled MFMAs take power-of-two (E8M0) scales per 32 elements, which cannot carry an E4M3
// scale per 16 elements exactly.  The operands are therefore dequantised on the fly into fp16 and
// contracted on v_mfma_f32_32x32x16_f16:
// * element value q * s * 2^-8, exact in fp16 (codec.h): v_cvt_scalef32_pk_f16_fp4 gives q, one
//   v_pk_mul_f16 applies s * 2^-8; each MFMA product is the exact dequantised product times 2^-16,
//   accumulated in fp32, and the epilogue multiplies by alpha * 2^16.
//
// Work split.  A workgroup tile has a "shared" side of 128 or 256 rows and a "private" side of 256
// rows: with SHARED_A the tile is 128 (M) x 256 (N), otherwise 256 (M) x 128 (N) or, for grids of at
// least one tile per CU, 256 x 256.  Eight waves (two per SIMD: one wave alone issues VALU work at
// about half rate) each compute all 128 shared x 32 private outputs (128-row shared side: 4 x 1
// accumulators of 32 x 32) or 128 shared x 64 private outputs (256-row shared side: 4 x 2).
// * The shared operand is decoded once per K tile by all 512 threads (16 or 32 elements each) into a
//   double-buffered fp16 LDS tile, read by the waves as MFMA fragments.
// * Each wave decodes its private rows straight into MFMA registers: with the K order inside a
//   64-element tile permuted so that lane l (r = l % 32, h = l / 32) covers elements 32h .. 32h+31,
//   one 16-byte chunk per lane per 32-row block holds exactly the four fragments of that block.  The
//   shared fragments use the same permutation.  (With the 256-row shared side each private row is
//   decoded by the two waves that share it.)
// * Packed bytes and scale codes of K tile k+DIST are copied global -> LDS by buffer_load ... lds
//   (ring of DIST+1 stages) while tile k is computed and tile k+1's shared rows are decoded; one
//   barrier per K tile, after each wave has waited for its own copies of tile k+2.  Row-major scale
//   codes come 16 bytes per row for 4 K tiles (K % 256 == 0): every row's codes are a separate
//   piece of memory, and the copies cost per piece far more than per byte.  Rows past M / N
//   read as zeros through the buffer range check; the missing half of a final half tile
//   (K % 64 == 32) decodes with scale code 0, i.e. as zeros.
// * Split-K for small M x N: the grid holds tiles x S workgroups; split s covers K tiles
//   [s KT / S, (s+1) KT / S) and writes its raw fp32 accumulators to a plan-owned workspace
//   [S][M][N]; a second kernel sums the S partials in split order (deterministic), applies the
//   epilogue and writes D.  With S == 1 the epilogue runs in the GEMM kernel.
// * With the 128-row shared side and K % 256 == 0 a warp-specialised variant runs instead
//   (nvfp4_ws_kernel): four waves copy and decode the shared rows, four compute.
//
// v_mfma_f32_32x32x16_f16 register layout: A lane l (r = l % 32, h = l / 32) holds row r, K
// slots [8h, 8h+8) of the 16-slot slice; B likewise for column r; accumulator element e of lane l:
// row 8*(e/4) + 4h + e%4, column r.  Here slice s of a tile maps slot 8h + t to tile element
// 32h + 8s + t, the same for A and B, so the contraction covers each element once.
//
// LDS layouts (bank-conflict free for the access patterns named):
// * raw stage: row R's 32 packed bytes at 32R, its half h at +16 (h ^ ((R >> 3) & 1)) (fragment
//   reads: 16 lanes = 16 rows x one half); the two scale codes of row R, half h at 8R + 4h (a
//   2-byte buffer_load ... lds fills a 4-byte LDS slot per lane, zero-extended).
// * decoded shared stage: row R = 128 bytes = 8 pieces of 8 fp16 (piece p = elements 8p .. 8p+7),
//   piece p stored at p ^ dec_row_swizzle(R) (decode stores: 8 rows x 2 halves per 16 lanes;
//   fragment reads: 16 rows x one piece).
#include "codec.h"
#include "common.h"
#include "epilogue.h"
#include "splitk.h"

namespace bsg {
namespace nvr {

constexpr int BK = 64;                       // K elements per tile
constexpr int THREADS = 512, WAVES = 8;      // two waves per SIMD
constexpr int DIST = 3, NR = DIST + 1;       // copies run DIST tiles ahead; raw ring stages
constexpr int COPIES = 4;                    // buffer_load ... lds per wave per K tile
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)
constexpr float kRescale = 65536.0f;           // 2^16: undoes the 2^-8 of both fp16 operands

// Tile configuration: BS shared rows (128 or 256) x 256 private rows, and how the eight waves divide
// them.  ALL_SHARED: each wave takes all BS shared rows and 32 private rows of its own (TS = BS/32,
// TP = 1), so every private row is decoded by exactly one wave; otherwise each wave takes half the
// shared rows and 64 private rows (TS = BS/64, TP = 2), and every private row is decoded by the two
// waves that share it.  Either way a wave owns TS x TP accumulators of 32 x 32 and issues 16 (BS =
// 128) or 32 (BS = 256) MFMAs per K tile.  On this route the decode's VALU work adds to the MFMA
// time rather than hiding under it (measured: ~1870 cycles per K tile for 1024 cycles of MFMA and
// ~880 of decode VALU per SIMD), so decoding each private row once is worth the shared fragments'
// extra LDS reads.
template <int BS_, bool ALL_SHARED_>
struct Cfg {
  static constexpr int BS = BS_, BP = 256;
  static constexpr bool ALL_SHARED = ALL_SHARED_;
  static constexpr int ROWS = BS + BP;                   // rows copied per K tile
  static constexpr int RAW_DATA = ROWS * 32;             // packed bytes of a K tile
  static constexpr int RAW_STAGE = RAW_DATA + ROWS * 8;  // + scale codes, 8 bytes per row
  static constexpr int DEC_STAGE = BS * 128;             // decoded shared rows (fp16)
  static constexpr int TS = ALL_SHARED ? BS / 32 : BS / 64, TP = ALL_SHARED ? 1 : 2;
  static constexpr int WSH_ROWS = 32 * TS, WP_ROWS = 32 * TP;  // a wave's shared and private rows
  static constexpr int NSC = BS / 32;                    // shared data copies (32 rows each)
  static constexpr int EPI_STRIDE = 32 * (TS > TP ? TS : TP) + 8;  // floats; 4 rows = 32 mod 64 banks
  static constexpr int SRING = ROWS * 16;                // scale codes of 4 K tiles, 16 bytes per row
  static constexpr int MAIN_LDS = NR * RAW_STAGE + 2 * DEC_STAGE + 2 * SRING;
  static constexpr int EPI_LDS = WAVES * 32 * EPI_STRIDE * 4;   // epilogue staging, 32 rows per wave
  static constexpr int LDS_BYTES = MAIN_LDS > EPI_LDS ? MAIN_LDS : EPI_LDS;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(EPI_STRIDE % 16 == 8, "two rows 4 apart start 32 banks apart");
  static_assert(BS == 128 || BS == 256, "copy plan");
};
using Cfg128 = Cfg<128, true>;   // 128 x 256 (A shared, small M) or 256 x 128 (B shared)
using Cfg256 = Cfg<256, false>;  // 256 x 256, B shared, for grids of at least one tile per CU

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ v16f mfma_f16(v4i a, v4i b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}

// Wait until at most N of this wave's buffer loads (here: global -> LDS copies) are in flight.  The
// compiler does not see the LDS writes of those copies; the memory clobber keeps every LDS access
// on its side of the wait.
template <int N>
__device__ __forceinline__ void wait_copies() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait for this wave's LDS accesses, then meet the other waves (outstanding copies stay in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// XCD-aware order for the unsplit grid: consecutive workgroup ids go to different XCDs, so give each
// XCD a contiguous range of tile ids, walked in groups of 8 tile-rows.
__device__ __forceinline__ int2 tile_of(int bid, int tiles_m, int tiles_n) {
  const int T = tiles_m * tiles_n;
  int id = bid;
  if ((T & 7) == 0) id = (bid & 7) * (T >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int group = id / per_group;
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int in_group = id - group * per_group;
  return make_int2(first_m + in_group % gsize, in_group / gsize);
}

// Decoded shared rows (fp16, 128 bytes per row of a K tile): 16-byte piece j of row R sits at
// position j ^ dec_row_swizzle(R).  16 lanes reading piece j of 16 consecutive rows (16-byte reads
// resolve 16 lanes per 256 bytes) and 8 lanes storing into 8 consecutive rows (16-byte stores resolve
// 8 lanes per 128 bytes) both touch distinct banks (measured: no conflict cycles either way, where
// j ^ ((R >> 1) & 7) left the stores conflicting two ways).
__device__ __forceinline__ int dec_row_swizzle(int R) { return (R & 7) ^ ((R >> 3) & 1); }

// Row-major scale codes in 16-byte groups (a row's codes of 4 K tiles) are read whole -- 16 lanes'
// reads of 16 rows' groups are one pass over the banks, where 2-byte reads of 32 rows 16 bytes apart
// collide four ways -- and the K tile's dword (its 4 codes) picked: at compile time where the tile's
// place in its group (TQ) is known, else by a select on the run-time index.
struct RtTq {};  // a K tile's place in its group known at run time only
template <class TQ>
struct NextTq { using type = std::integral_constant<int, (TQ::value + 1) & 3>; };
template <>
struct NextTq<RtTq> { using type = RtTq; };
template <class TQ>
__device__ __forceinline__ uint32_t group_word(v4i q, int kt, TQ) {
  if constexpr (std::is_same_v<TQ, RtTq>) {
    const int t = kt & 3;  // wave-uniform
    return (uint32_t)(t & 2 ? (t & 1 ? q[3] : q[2]) : (t & 1 ? q[1] : q[0]));
  } else {
    return (uint32_t)q[TQ::value];
  }
}
// Byte-permute selector of half h's two codes in a dword of a K tile's four (e4m3x2_scale_f16x2_sel).
__device__ __forceinline__ uint32_t half_code_sel(int h) { return h ? 0x030C020Cu : 0x010C000Cu; }

// Scale-code copy plan SCM:
// 2: row-major scales with K % 256 == 0: 16 bytes per row for 4 K tiles (one copy per wave covers 64
//    rows, issued once per 4 K tiles into a two-slot ring).  Each row's codes are a separate piece of
//    memory, so the number of pieces copied, not their size, sets the cost: 4 tiles per piece.
// 1: dword-aligned scale rows otherwise (K-tile-major layout, where one copy reads 256 contiguous
//    bytes, or row-major with K % 64 == 0): 4 bytes per row and K tile, one copy per wave.
// 0: 2 bytes per row half (two copies per wave).
template <class CF, bool SHARED_A, Out O, bool BIAS, bool SILU, bool SPLIT, int SCM>
__global__ __launch_bounds__(THREADS, 1) void nvfp4_kernel(GemmArgs p) {
  select_batch(p);
  constexpr int BS = CF::BS, BP = CF::BP, TS = CF::TS, TP = CF::TP, NSC = CF::NSC;
  constexpr int RAW_DATA = CF::RAW_DATA, RAW_STAGE = CF::RAW_STAGE, DEC_STAGE = CF::DEC_STAGE;
  constexpr int BM = SHARED_A ? BS : BP, BN = SHARED_A ? BP : BS;
  constexpr bool SC4 = SCM >= 1;  // one copy per wave covers 64 rows' codes
  constexpr int NCOP = SCM == 2 ? COPIES - 2 : SCM == 1 ? COPIES - 1 : COPIES;  // copies per wave per K tile
  constexpr int SRING = CF::SRING;
  __shared__ __attribute__((aligned(16))) uint8_t lds[CF::LDS_BYTES];
  uint8_t* const raw = lds;
  uint8_t* const dec = lds + NR * RAW_STAGE;
  uint8_t* const sring = dec + 2 * DEC_STAGE;  // SCM 2: codes of K tiles 4g .. 4g+3 in slot g & 1

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn, split = 0;
  if constexpr (SPLIT) {
    // With a multiple of 8 tiles every split of tile t runs on XCD t % 8 (ids go to the XCDs
    // round-robin), and the finish kernel's blocks for tile t run there too (splitk.h).  Otherwise
    // consecutive ids take consecutive splits.
    const int T = p.tiles_m * p.tiles_n, b = (int)blockIdx.x;
    int t;
    if ((T & 7) == 0) {
      const int r = b >> 3;
      split = r % p.splits;
      t = (b & 7) + 8 * (r / p.splits);
    } else {
      split = b % p.splits;
      t = b / p.splits;
    }
    tm = t / p.tiles_n;
    tn = t - tm * p.tiles_n;
  } else {
    const int2 t = tile_of(blockIdx.x, p.tiles_m, p.tiles_n);
    tm = t.x;
    tn = t.y;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int K = p.K, KT = (K + BK - 1) / BK;
  // (split + 1) * KT < 2^29 (at most 16 splits, K < 2^31): 32-bit unsigned division
  const int kb = SPLIT ? (int)((uint32_t)split * (uint32_t)KT / (uint32_t)p.splits) : 0;
  const int ke = SPLIT ? (int)((uint32_t)(split + 1) * (uint32_t)KT / (uint32_t)p.splits) : KT;
  const uint32_t KH = (uint32_t)K >> 1, KS = (uint32_t)K >> 4;

  // Buffer resources of the shared and private operand rows of this tile (rows past M / N fall
  // outside the range and read as zeros).
  // row pitches (bytes) of the shared and private operands
  const uint32_t s_pitch = (uint32_t)(SHARED_A ? p.row_a : p.row_b), p_pitch = (uint32_t)(SHARED_A ? p.row_b : p.row_a);
  const uint8_t* s_q = SHARED_A ? p.A + (size_t)m0 * s_pitch : p.B + (size_t)n0 * s_pitch;
  // Scale codes: row-major [rows][KS], or K-tile-major (the 4 codes of K tile kt of row r at
  // (kt * rows + r) * 4): per-lane offsets from the tile's first row plus kt * (4 or 4 * rows).
  const bool ktile = p.scale_ktile != 0;
  const int s_all = SHARED_A ? p.M : p.N, p_all = SHARED_A ? p.N : p.M;  // operand rows
  const int s_first = SHARED_A ? m0 : n0, p_first = SHARED_A ? n0 : m0;
  const uint32_t s_rowb = ktile ? 4u : KS, s_ktb = ktile ? 4u * (uint32_t)s_all : 4u;
  const uint32_t p_rowb = ktile ? 4u : KS, p_ktb = ktile ? 4u * (uint32_t)p_all : 4u;
  const uint8_t* s_s = (SHARED_A ? p.sA : p.sB) + (size_t)s_first * s_rowb;
  const uint8_t* p_q = SHARED_A ? p.B + (size_t)n0 * p_pitch : p.A + (size_t)m0 * p_pitch;
  const uint8_t* p_s = (SHARED_A ? p.sB : p.sA) + (size_t)p_first * p_rowb;
  const int s_rows = SHARED_A ? min(BS, p.M - m0) : min(BS, p.N - n0);
  const int p_rows = SHARED_A ? min(BP, p.N - n0) : min(BP, p.M - m0);
  const __amdgpu_buffer_rsrc_t rs_q =
      __builtin_amdgcn_make_buffer_rsrc((void*)s_q, (short)0, (int)((s_rows - 1) * s_pitch + KH), (int)kRsrcWord3);
  // (K-tile-major: the range ends at the array's end; rows past the operand's last row read other
  // rows' codes, which only reach outputs that are never stored)
  const uint32_t groups = (KS + 3) >> 2;
  const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
      (void*)s_s, (short)0, (int)(ktile ? groups * 4u * (uint32_t)s_all - 4u * (uint32_t)s_first : s_rows * KS), (int)kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rp_q =
      __builtin_amdgcn_make_buffer_rsrc((void*)p_q, (short)0, (int)((p_rows - 1) * p_pitch + KH), (int)kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rp_s = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p_s, (short)0, (int)(ktile ? groups * 4u * (uint32_t)p_all - 4u * (uint32_t)p_first : p_rows * KS), (int)kRsrcWord3);

  // Wave roles: shared rows WSH_ROWS wsh .. +WSH_ROWS and private rows WP_ROWS wp .. +WP_ROWS; the
  // wave computes those outputs.
  const int wsh = CF::ALL_SHARED ? 0 : wave & 1, wp = CF::ALL_SHARED ? wave : wave >> 1;
  constexpr int WSH_ROWS = CF::WSH_ROWS, WP_ROWS = CF::WP_ROWS;

  // Copy plan.  A K tile needs ROWS/32 data copies of 32 rows x 32 bytes (lane l: row 32q + l/2,
  // half (l & 1) ^ ((R >> 3) & 1), 16 bytes at 1 KiB * q + 16 l; q < NSC shared, the rest private)
  // and as many scale copies (lane l: the 2 codes of that row's half l & 1 into the 4-byte slot at
  // 256 q + 4 l = 8R + 4 (l & 1)).  BS = 256: wave w issues shared copy w and private copy 8 + w.
  // BS = 128: wave w issues copy q2 = w + (w & 4) (shared copies 0..3 for w < 4; for w >= 4 a
  // repeat of its own private copy, which writes the same bytes to the same place) and private copy
  // 4 + w.  Either way the same copies in every wave, without selected LDS addresses (which would
  // make the compiler drain all copies before LDS reads).  (SCM 2 instead copies the codes of 4 K
  // tiles at once, 16 bytes per row, after the data of every fourth tile.)
  const int qp = NSC + wave, qs = NSC == 8 ? wave : wave + (wave & 4);
  const bool has_shared = qs < NSC;
  auto copy_off = [&](int q, bool data, uint32_t& off, int& half) {
    const int R = 32 * q + (lane >> 1);
    const int row = q < NSC ? R : R - BS;  // row within its operand's tile rows
    half = data ? (lane & 1) ^ ((R >> 3) & 1) : (lane & 1);
    off = data ? (uint32_t)row * (q < NSC ? s_pitch : p_pitch) + 16u * half
               : (uint32_t)row * (q < NSC ? s_rowb : p_rowb) + 2u * half;
  };
  uint32_t o_pd, o_ps, o_sd, o_ss;
  int h_unused;
  copy_off(qp, true, o_pd, h_unused);
  copy_off(qp, false, o_ps, h_unused);
  copy_off(qs, true, o_sd, h_unused);
  copy_off(qs, false, o_ss, h_unused);
  // SC4: wave w copies the codes of stage rows 64 c4 .. 64 c4 + 63 (4 bytes each) into RAW_DATA +
  // 256 c4; with 384 rows (BS = 128) waves 6 and 7 repeat copies 4 and 5 (same bytes, same place).
  constexpr int SC4_COPIES = CF::ROWS / 64;
  static_assert(SC4_COPIES <= 8 && 2 * SC4_COPIES >= 8 && BS % 64 == 0, "one 64-row scale copy per wave");
  const int c4 = wave < SC4_COPIES ? wave : wave - (8 - SC4_COPIES);
  const bool c4_shared = 64 * c4 < BS;  // wave-uniform
  const uint32_t o_s4 = (uint32_t)(64 * c4 + lane - (c4_shared ? 0 : BS)) * (c4_shared ? s_rowb : p_rowb);
  const __amdgpu_buffer_rsrc_t r4_s = c4_shared ? rs_s : rp_s;
  const uint32_t ktb4 = c4_shared ? s_ktb : p_ktb;
  const __amdgpu_buffer_rsrc_t r2_q = has_shared ? rs_q : rp_q;
  const __amdgpu_buffer_rsrc_t r2_s = has_shared ? rs_s : rp_s;
  const uint32_t ktb2 = has_shared ? s_ktb : p_ktb;
  // Copy offsets are loop-invariant (so the compiler's wait bookkeeping stays exact).  The missing
  // half of a final half tile (K % 64 == 32) is still copied -- the next row's first bytes, or zeros
  // past the range for the last row -- and the decode gives it scale code 0, i.e. zero elements.
  // Ring positions are K tile numbers mod NR; the steady-state loop starts at a multiple of NR, so that,
  // unrolled by the ring size, it sees every stage and decoded-buffer offset as a constant (immediate
  // LDS offsets).
  static_assert((NR & (NR - 1)) == 0 && NR == 4, "ring size a power of two; SCM 2 groups 4 K tiles");
  auto ring = [&](int kt) -> uint32_t { return (uint32_t)kt & (NR - 1); };
  // SCM 2: the codes of K tiles 4g .. 4g+3 (16 bytes per row at byte 16 g of the row; past K: other
  // rows' codes or zeros, never used), into slot g & 1.
  auto copy_scales = [&](int g) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r4_s, (lds_void*)(sring + (g & 1) * SRING + 1024 * c4), 16, o_s4, (uint32_t)g * 16u, 0, 0);
  };
  // SCALES (SCM 2): also the scale group that starts at K tile kt, issued after the tile's data.
  auto copy_tile = [&](int kt, bool scales) {
    const int kq = kt;
    kt = min(kt, ke - 1);  // past the last tile re-read it (never consumed): uniform load counts
    uint8_t* st = raw + ring(kt) * RAW_STAGE;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r2_q, (lds_void*)(st + 1024 * qs), 16, o_sd, (uint32_t)kt * 32u, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rp_q, (lds_void*)(st + 1024 * qp), 16, o_pd, (uint32_t)kt * 32u, 0, 0);
    if constexpr (SCM == 2) {
      if (scales) copy_scales(kq >> 2);
    } else if constexpr (SC4) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r4_s, (lds_void*)(st + RAW_DATA + 256 * c4), 4, o_s4, (uint32_t)kt * ktb4, 0, 0);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r2_s, (lds_void*)(st + RAW_DATA + 256 * qs), 2, o_ss, (uint32_t)kt * ktb2, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rp_s, (lds_void*)(st + RAW_DATA + 256 * qp), 2, o_ps, (uint32_t)kt * p_ktb, 0, 0);
    }
  };
  // Scale codes of half h of K tile kt, or 0 when that half lies past K.
  // CHECK: the tile may be the split's last one (prologue and drain loops); the steady-state loop
  // never reaches it and skips the test.
  auto half_scales = [&](uint32_t codes, int kt, int h, auto check) -> uint32_t {
    if constexpr (decltype(check)::value) return kt * BK + 32 * h < K ? codes : 0u;
    return codes;
  };
  using Checked = std::integral_constant<bool, true>;
  using Unchecked = std::integral_constant<bool, false>;

  // Shared decode.  BS = 128: thread t takes shared row t/4, quarter t&3 (half (t&3)/2, 8 bytes = one
  // scale block) and writes its two decoded pieces 4h + 2 sub + {0, 1}.  BS = 256: thread t takes
  // shared row t/2, half t&1 (16 bytes = two scale blocks) and writes pieces 4h + {0, 1, 2, 3}.
  constexpr int SD_PIECES = BS / 64;  // decoded 16-byte pieces per thread per K tile
  const int sd_row = BS == 256 ? tid >> 1 : tid >> 2;
  const int sd_h = BS == 256 ? tid & 1 : (tid >> 1) & 1, sd_sub = BS == 256 ? 0 : tid & 1;
  const uint32_t sd_raw = (uint32_t)(32 * sd_row + 16 * (sd_h ^ ((sd_row >> 3) & 1)));
  // The two codes of row R, half h of K tile kt: SCM 0: a zero-extended 4-byte slot at 8R + 4h of the
  // tile's raw stage; SCM 1: bytes 2h, 2h+1 of the row's 4-byte slot at 4R (read as 2 bytes: the same
  // value); SCM 2: bytes 4 (kt % 4) + 2h, +1 of the row's 16 bytes in the scale ring.  row_off: the
  // part that does not depend on kt.
  auto scale_row_off = [&](int R, int h) -> uint32_t {
    if constexpr (SCM == 2) return (uint32_t)(16 * R + 2 * h);
    return (uint32_t)(RAW_DATA + (SC4 ? 4 * R + 2 * h : 8 * R + 4 * h));
  };
  auto scale_at = [&](int kt, uint32_t row_off) -> const uint8_t* {
    if constexpr (SCM == 2) return sring + ((kt >> 2) & 1) * SRING + row_off + 4 * (kt & 3);
    return raw + ring(kt) * RAW_STAGE + row_off;
  };
  const uint32_t sd_scale = scale_row_off(sd_row, sd_h);
  auto scale_pair = [&](const uint8_t* at) -> uint32_t {
    if constexpr (SC4) return (uint32_t)*(const uint16_t*)at;
    return *(const uint32_t*)at;
  };
  uint32_t sd_out[SD_PIECES];
#pragma unroll
  for (int d = 0; d < SD_PIECES; ++d)
    sd_out[d] = (uint32_t)(128 * sd_row + (((4 * sd_h + 2 * sd_sub + d) ^ dec_row_swizzle(sd_row)) << 4));
  // The fp16 scale pair of row R, half h of K tile kt (TQ: kt % 4, when known at compile time).
  auto scale_f16x2 = [&](int kt, int R, int h, uint32_t row_off, auto check, auto tq) -> uint32_t {
    if constexpr (SCM == 2) {  // K % 256 == 0: no half tile
      const v4i g = *(const v4i*)(sring + ((kt >> 2) & 1) * SRING + 16 * R);
      return e4m3x2_scale_f16x2_sel(group_word(g, kt, tq), half_code_sel(h));
    } else {
      return e4m3x2_scale_f16x2(half_scales(scale_pair(scale_at(kt, row_off)), kt, h, check));
    }
  };
  auto decode_shared = [&](int kt, auto check, auto tq) {
    const uint8_t* st = raw + ring(kt) * RAW_STAGE;
    uint8_t* out = dec + (ring(kt) & 1) * DEC_STAGE;
    const v4i q4 = *(const v4i*)(st + sd_raw);  // the row's half
    const uint32_t s = scale_f16x2(kt, sd_row, sd_h, sd_scale, check, tq);
    if constexpr (BS == 256) {
      const uint32_t s0 = f16x2_splat_lo(s), s1 = f16x2_splat_hi(s);
      *(v4i*)(out + sd_out[0]) = e2m1x8_scaled_f16x8((uint32_t)q4[0], s0);
      *(v4i*)(out + sd_out[1]) = e2m1x8_scaled_f16x8((uint32_t)q4[1], s0);
      *(v4i*)(out + sd_out[2]) = e2m1x8_scaled_f16x8((uint32_t)q4[2], s1);
      *(v4i*)(out + sd_out[3]) = e2m1x8_scaled_f16x8((uint32_t)q4[3], s1);
    } else {  // 8 of the half's 16 bytes
      const uint2 q = sd_sub ? make_uint2((uint32_t)q4[2], (uint32_t)q4[3]) : make_uint2((uint32_t)q4[0], (uint32_t)q4[1]);
      const uint32_t s2 = sd_sub ? f16x2_splat_hi(s) : f16x2_splat_lo(s);
      *(v4i*)(out + sd_out[0]) = e2m1x8_scaled_f16x8(q.x, s2);
      *(v4i*)(out + sd_out[1]) = e2m1x8_scaled_f16x8(q.y, s2);
    }
  };

  // Fragment addressing.  Private block j: stage row BS + WP_ROWS wp + 32j + r, the lane's half hl.
  const int r32 = lane & 31, hl = lane >> 5;
  uint32_t pf_raw[TP], pf_scale[TP];
#pragma unroll
  for (int j = 0; j < TP; ++j) {
    const int R = BS + WP_ROWS * wp + 32 * j + r32;
    pf_raw[j] = (uint32_t)(32 * R + 16 * (hl ^ ((R >> 3) & 1)));
    pf_scale[j] = scale_row_off(R, hl);
  }
  // Shared block i, slice s: decoded row WSH_ROWS wsh + 32i + r, piece 4 hl + s.
  const uint32_t sf_row = (uint32_t)(128 * (WSH_ROWS * wsh + r32));
  const int sf_sw = dec_row_swizzle(r32);  // that of row WSH_ROWS wsh + 32i + r: a multiple of 16 plus r
  uint32_t sf_piece[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) sf_piece[s] = (uint32_t)(((4 * hl + s) ^ sf_sw) << 4);

  v16f acc[TS][TP];
#pragma unroll
  for (int i = 0; i < TS; ++i)
#pragma unroll
    for (int j = 0; j < TP; ++j) acc[i][j] = v16f{};

  // One K tile: tile kt's private rows are decoded into registers slice by slice, one slice ahead of
  // the MFMAs that use them; tile kt+1's shared rows go to the other decoded buffer.
  auto step = [&](int kt, auto check, auto tq) {
    const uint8_t* st = raw + ring(kt) * RAW_STAGE;
    const uint8_t* dst = dec + (ring(kt) & 1) * DEC_STAGE;
    v4i pq[TP];
    uint32_t ps[TP][2];
#pragma unroll
    for (int j = 0; j < TP; ++j) {
      pq[j] = *(const v4i*)(st + pf_raw[j]);
      const uint32_t s = scale_f16x2(kt, BS + WP_ROWS * wp + 32 * j + r32, hl, pf_scale[j], check, tq);
      ps[j][0] = f16x2_splat_lo(s);
      ps[j][1] = f16x2_splat_hi(s);
    }
    v4i pf[2][TP], sf[2][TS];
#pragma unroll
    for (int j = 0; j < TP; ++j) pf[0][j] = e2m1x8_scaled_f16x8((uint32_t)pq[j][0], ps[j][0]);
#pragma unroll
    for (int i = 0; i < TS; ++i) sf[0][i] = *(const v4i*)(dst + sf_row + 32 * 128 * i + sf_piece[0]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = s & 1, n = c ^ 1;
      if (s < 3) {
#pragma unroll
        for (int i = 0; i < TS; ++i) sf[n][i] = *(const v4i*)(dst + sf_row + 32 * 128 * i + sf_piece[s + 1]);
#pragma unroll
        for (int j = 0; j < TP; ++j) pf[n][j] = e2m1x8_scaled_f16x8((uint32_t)pq[j][s + 1], ps[j][(s + 1) >> 1]);
      }
#pragma unroll
      for (int i = 0; i < TS; ++i)
#pragma unroll
        for (int j = 0; j < TP; ++j)
          acc[i][j] = SHARED_A ? mfma_f16(sf[c][i], pf[c][j], acc[i][j]) : mfma_f16(pf[c][j], sf[c][i], acc[i][j]);
      // tile kt+1's shared rows, decoded behind the first slice's MFMAs rather than ahead of them
      // (4096^3: -3%); past the last tile: stale bytes into a buffer nobody reads
      if (s == 0) decode_shared(kt + 1, check, typename NextTq<decltype(tq)>::type{});
    }
  };

  // Copy waits: at most N + 1 of the wave's copies in flight when EXTRA (a scale group issued after
  // the data copies the wait leaves in flight), else N.
  auto wait_copies_x = [&](auto n, bool extra) {
    constexpr int N = decltype(n)::value;
    if constexpr (SCM == 2) {
      if (extra) {
        wait_copies<N + 1>();
        return;
      }
    }
    wait_copies<N>();
  };
  using IC0 = std::integral_constant<int, 0>;
  using ICN = std::integral_constant<int, NCOP>;
  auto starts_group = [&](int kt) { return SCM == 2 && (kt & 3) == 0; };

  // Prologue: copies of tiles kb .. kb+DIST-1 (clamped), with the scale group of tile kb first (SCM
  // 2) and any group that starts at kb+1 .. kb+DIST-1; tile kb's shared rows decoded.
  static_assert(DIST == 3, "prologue waits");
  if constexpr (SCM == 2) copy_scales(kb >> 2);
#pragma unroll
  for (int i = 0; i < DIST; ++i) copy_tile(kb + i, i > 0 && starts_group(kb + i));
  // tile kb (and its codes) landed: tiles kb+1, kb+2 and their groups may stay in flight
  wait_copies_x(std::integral_constant<int, 2 * NCOP>{}, starts_group(kb + 1) || starts_group(kb + 2));
  lds_barrier();  // every wave's copies of tile kb have landed
  decode_shared(kb, Checked{}, RtTq{});
  wait_copies_x(ICN{}, starts_group(kb + 2));
  lds_barrier();  // tile kb decoded, tile kb+1 landed
  // Steady state: step kt issues tile kt+DIST's copies, computes tile kt and decodes tile kt+1's
  // shared rows; before the barrier that ends it, the wave's copies of tile kt+2 (and its scale
  // group) must have landed: tile kt+3's copies, and its group if it starts one, may stay in flight.
  // Raw stages in use: kt .. kt+DIST: NR = DIST + 1.
  auto single = [&](int kt) {
    copy_tile(kt + DIST, starts_group(kt + DIST));
    step(kt, Unchecked{}, RtTq{});
    wait_copies_x(ICN{}, starts_group(kt + DIST));
    lds_barrier();
  };
  int kt = kb;
#pragma unroll 1
  for (; (kt & (NR - 1)) != 0 && kt + DIST < ke; ++kt) single(kt);  // up to a multiple of NR
  auto unrolled = [&](auto cc) {  // step kt + c with kt == 0 (mod NR): the tile's place in its group is c
    constexpr int c = decltype(cc)::value;
    copy_tile(kt + c + DIST, SCM == 2 && ((c + DIST) & 3) == 0);
    step(kt + c, Unchecked{}, cc);
    wait_copies_x(ICN{}, SCM == 2 && ((c + DIST) & 3) == 0);
    lds_barrier();
  };
  static_assert(NR == 4, "one scale group per unrolled iteration");
#pragma unroll 1
  for (; kt + NR - 1 + DIST < ke; kt += NR) {
    unrolled(std::integral_constant<int, 0>{});
    unrolled(std::integral_constant<int, 1>{});
    unrolled(std::integral_constant<int, 2>{});
    unrolled(std::integral_constant<int, 3>{});
  }
#pragma unroll 1
  for (; kt + DIST < ke; ++kt) single(kt);
  // Last DIST tiles: nothing left to copy.  Leaves no copy in flight past the end of the kernel.
#pragma unroll 1
  for (; kt < ke; ++kt) {
    step(kt, Checked{}, RtTq{});
    wait_copies<0>();
    lds_barrier();
  }
  (void)IC0{};

  // Epilogue, staged through LDS (free now: the last barrier has passed and no copy is in flight).
  // The wave's block -- SHARED_A: rows m0 + WSH_ROWS wsh + .., columns n0 + WP_ROWS wp + ..; otherwise
  // rows m0 + WP_ROWS wp + .., columns n0 + WSH_ROWS wsh + .. -- goes out in passes of 32 rows:
  // accumulator element e of block (i, j) is row 32 mi + 8*(e/4) + 4*hl + e%4, column 32 ni + r32
  // (mi, ni = i, j for SHARED_A, else j, i).  Rows are EPI_STRIDE floats apart (EPI_STRIDE = 8 mod
  // 16: the two rows a store instruction touches start 32 banks apart); each lane then reads 4
  // consecutive columns and the wave stores whole rows.
  constexpr int EPI_STRIDE = CF::EPI_STRIDE;
  constexpr int PASSES = SHARED_A ? TS : TP, ECOLS = 32 * (SHARED_A ? TP : TS);
  constexpr int LPR = ECOLS / 4, RPI = 64 / LPR;  // lanes per row (4 columns each), rows per read
  float* stage = (float*)lds + wave * (32 * EPI_STRIDE);
  const int mw = m0 + (SHARED_A ? WSH_ROWS * wsh : WP_ROWS * wp), nw = n0 + (SHARED_A ? WP_ROWS * wp : WSH_ROWS * wsh);
  const float alpha = load_alpha(p) * kRescale;
  auto write_out = [&](auto through) {
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
#pragma unroll
      for (int i = 0; i < TS; ++i)
#pragma unroll
        for (int j = 0; j < TP; ++j) {
          const int mi = SHARED_A ? i : j, ni = SHARED_A ? j : i;
          if (mi != pass) continue;
#pragma unroll
          for (int e = 0; e < 16; ++e)
            stage[(8 * (e >> 2) + 4 * hl + (e & 3)) * EPI_STRIDE + 32 * ni + r32] = acc[i][j][e];
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int c4 = 4 * (lane % LPR);
      const int n = nw + c4;
#pragma unroll
      for (int it = 0; it < 32 / RPI; ++it) {
        const int row = RPI * it + lane / LPR;
        const int m = mw + 32 * pass + row;
        const v4f v = *(const v4f*)(stage + row * EPI_STRIDE + c4);
        if (m >= p.M || n >= p.N) continue;  // N % 16 == 0: a lane's 4 columns are all in or all out
        if constexpr (SPLIT) {
          store_partials<decltype(through)::value>(p.ws + (size_t)split * p.M * p.N, (uint32_t)p.M * (uint32_t)p.N * 4u,
                                                   (uint32_t)m * (uint32_t)p.N + (uint32_t)n, v);
        } else {
          v4f b = {0.f, 0.f, 0.f, 0.f};
          if constexpr (BIAS) b = v4f{p.bias[n], p.bias[n + 1], p.bias[n + 2], p.bias[n + 3]};
          uint2 o;
          o.x = epi_pack2<SILU, O>(v[0], v[1], alpha, b[0], b[1]);
          o.y = epi_pack2<SILU, O>(v[2], v[3], alpha, b[2], b[3]);
          *(uint2*)((uint16_t*)p.D + (size_t)m * p.ldd + n) = o;
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next pass overwrites
    }
  };
  if constexpr (SPLIT) {
    if (p.ws_through)
      write_out(std::true_type{});
    else
      write_out(std::false_type{});
  } else {
    write_out(std::false_type{});
  }
}

// Warp-specialised variant of the 128-row-shared-side kernel, for K % 256 == 0 (either scale
// layout).  Waves 4..7 move data: they copy every row global -> LDS two K tiles at a time (64 bytes
// per row and copy: half the row pieces of single-tile copies) and decode the 128 shared rows of the
// next K tile into a double-buffered fp16 tile.  Waves 0..3 (one per SIMD) compute: wave w
// owns all 128 shared rows and private rows 64w .. 64w+63 (4 x 2 accumulators), reads the shared
// fragments from the decoded tile and decodes its own private rows from the packed bytes into MFMA
// operands, as nvfp4_kernel does.  Against eight waves that each take all shared rows and 32
// private rows, the LDS carries about a third less per K tile (each shared fragment is read by 4
// waves, not 8), which is what bounds these kernels; each private row is still decoded once.
namespace wsk {
constexpr int BS = 128, BP = 256, ROWS = BS + BP;
constexpr int PAIR = ROWS * 64;                      // packed bytes of a K-tile pair (24 KiB)
constexpr int NP = 4;                                // pair stages
constexpr int SRING = ROWS * 16;                     // scale codes of 4 K tiles
constexpr int DEC = BS * 128;                        // a decoded K tile of the shared rows
constexpr int TS = 4, TP = 2;                        // a compute wave's 32 x 32 blocks
constexpr int EPI_STRIDE = 32 * TS + 8;              // floats; as nvfp4_kernel's staging
constexpr int MAIN_LDS = NP * PAIR + 2 * SRING + 2 * DEC;
constexpr int EPI_LDS = 4 * 32 * EPI_STRIDE * 4;
constexpr int LDS_BYTES = MAIN_LDS > EPI_LDS ? MAIN_LDS : EPI_LDS;
static_assert(LDS_BYTES <= 160 * 1024, "LDS");
}  // namespace wsk

template <bool SHARED_A, Out O, bool BIAS, bool SILU, bool SPLIT, bool KTILE>
__global__ __launch_bounds__(THREADS, 1) void nvfp4_ws_kernel(GemmArgs p) {
  select_batch(p);
  using namespace wsk;
  constexpr int BM = SHARED_A ? BS : BP, BN = SHARED_A ? BP : BS;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  uint8_t* const raw = lds;                  // pair P in stage P & 3
  uint8_t* const sring = lds + NP * PAIR;    // scale group g in slot g & 1
  uint8_t* const dec = sring + 2 * SRING;    // shared rows of K tile t in buffer t & 1

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn, split = 0;
  if constexpr (SPLIT) {  // as nvfp4_kernel: a tile's splits on one XCD when the tiles are a multiple of 8
    const int T = p.tiles_m * p.tiles_n, b = (int)blockIdx.x;
    int t;
    if ((T & 7) == 0) {
      const int r = b >> 3;
      split = r % p.splits;
      t = (b & 7) + 8 * (r / p.splits);
    } else {
      split = b % p.splits;
      t = b / p.splits;
    }
    tm = t / p.tiles_n;
    tn = t - tm * p.tiles_n;
  } else {
    const int2 t = tile_of(blockIdx.x, p.tiles_m, p.tiles_n);
    tm = t.x;
    tn = t.y;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  // K % 256 == 0: K tiles come in scale groups of 4, and a split takes whole groups (at least one:
  // the host never splits K into more parts than it has groups)
  const int K = p.K, KG = K / (4 * BK);
  // (split + 1) * KG < 2^27: 32-bit unsigned division (64-bit took ~400 scalar instructions)
  const int kb = SPLIT ? 4 * (int)((uint32_t)split * (uint32_t)KG / (uint32_t)p.splits) : 0;
  const int ke = SPLIT ? 4 * (int)((uint32_t)(split + 1) * (uint32_t)KG / (uint32_t)p.splits) : 4 * KG;
  const uint32_t KH = (uint32_t)K >> 1, KS = (uint32_t)K >> 4;
  const int r32 = lane & 31, hl = lane >> 5;
  // Packed bytes of K tile t, row R (0 .. 383, shared rows first), half h: 16 bytes at
  // 64R + 16 ((2 (t & 1) + h) ^ ((R >> 2) & 3)) of pair stage (t >> 1) & 3 (the swizzle puts the 16
  // rows that 16 consecutive lanes read on distinct banks).  Scale codes, in scale slot (t >> 2) & 1:
  // row-major codes at 16R (a row's 16 codes of the 4-tile group, read whole: 16 lanes' 16-byte
  // reads of 16 rows are one pass over the banks, where 2-byte reads of 32 rows 16 bytes apart
  // collide four ways), K-tile-major codes as the layout has them, [tile][row] -- private rows'
  // 1 KiB per K tile at 1024 (t & 3), shared rows' 512 bytes at 4096 + 512 (t & 3), 4 bytes per row.
  // Either way a tile's four codes of a row are one dword ("code word"); half h's two are bytes 2h,
  // 2h + 1 of it, picked by a byte permute.
  auto raw_at = [&](int kt, int R, int h) -> const uint8_t* {
    return raw + ((kt >> 1) & (NP - 1)) * PAIR + 64 * R + 16 * ((2 * (kt & 1) + h) ^ ((R >> 2) & 3));
  };
  using CodeRead = std::conditional_t<KTILE, uint32_t, v4i>;  // what one read of a row's codes gets
  auto read_codes = [&](int kt, int R) -> CodeRead {
    const uint8_t* slot = sring + ((kt >> 2) & 1) * SRING;
    if constexpr (KTILE)
      return *(const uint32_t*)(slot + (R < BS ? 4096 + 512 * (kt & 3) + 4 * R : 1024 * (kt & 3) + 4 * (R - BS)));
    else
      return *(const v4i*)(slot + 16 * R);
  };
  auto code_word = [](const CodeRead& c, auto tq) -> uint32_t {  // tq: the tile's index in its group
    if constexpr (KTILE)
      return c;
    else
      return (uint32_t)c[decltype(tq)::value];
  };
  const uint32_t code_sel = half_code_sel(hl);  // this lane's half's two codes
  // Decoded shared rows: 16-byte piece j of row R at 128R + ((j ^ dec_row_swizzle(R)) << 4).

  if (wave >= 4) {
    // ---- data waves: copies and the shared rows' decode ------------------------------------------
    const int pw = wave - 4;
    const uint32_t s_pitch = (uint32_t)(SHARED_A ? p.row_a : p.row_b), p_pitch = (uint32_t)(SHARED_A ? p.row_b : p.row_a);
    const uint8_t* s_q = SHARED_A ? p.A + (size_t)m0 * s_pitch : p.B + (size_t)n0 * s_pitch;
    const uint8_t* p_q = SHARED_A ? p.B + (size_t)n0 * p_pitch : p.A + (size_t)m0 * p_pitch;
    const int s_first = SHARED_A ? m0 : n0, p_first = SHARED_A ? n0 : m0;
    // Scale codes: row-major [rows][KS], or K-tile-major (the 4 codes of K tile t of row r at
    // (t * rows + r) * 4; the range then ends at the array's end, and rows past the operand's last
    // row read other rows' codes, which only reach outputs that are never stored).
    const int s_all = SHARED_A ? p.M : p.N, p_all = SHARED_A ? p.N : p.M;  // operand rows
    const uint32_t s_rowb = KTILE ? 4u : KS, p_rowb = KTILE ? 4u : KS;
    const uint8_t* s_s = (SHARED_A ? p.sA : p.sB) + (size_t)s_first * s_rowb;
    const uint8_t* p_s = (SHARED_A ? p.sB : p.sA) + (size_t)p_first * p_rowb;
    const int s_rows = SHARED_A ? min(BS, p.M - m0) : min(BS, p.N - n0);
    const int p_rows = SHARED_A ? min(BP, p.N - n0) : min(BP, p.M - m0);
    const __amdgpu_buffer_rsrc_t rs_q =
        __builtin_amdgcn_make_buffer_rsrc((void*)s_q, (short)0, (int)((s_rows - 1) * s_pitch + KH), (int)kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rp_q =
        __builtin_amdgcn_make_buffer_rsrc((void*)p_q, (short)0, (int)((p_rows - 1) * p_pitch + KH), (int)kRsrcWord3);
    const uint32_t ktiles = KS >> 2;  // K tiles of 64: one 4-byte K-tile-major entry per row each
    const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
        (void*)s_s, (short)0, (int)(KTILE ? ktiles * 4u * (uint32_t)s_all - 4u * (uint32_t)s_first : s_rows * KS), (int)kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rp_s = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p_s, (short)0, (int)(KTILE ? ktiles * 4u * (uint32_t)p_all - 4u * (uint32_t)p_first : p_rows * KS), (int)kRsrcWord3);

    // Pair P: 24 copies of 16 rows x 64 bytes (copy q: rows 16q + l/4, lane l's 16-byte piece
    // j = l & 3 at byte 64R + 16j, holding the row's piece j ^ ((R >> 2) & 3) of the pair); data wave
    // pw issues copies 6pw .. 6pw+5.  Scale codes of K tiles 4g .. 4g+3: copy c (of 6) moves rows
    // 64c .. 64c+63, 16 bytes each; data wave pw issues c = pw and c = pw + 4 (waves 2, 3 repeat
    // c = pw: same bytes, same place).  Rows past M / N read as zeros (outside the buffer ranges).
    // (Offsets computed at each use: an offset array used from these lambdas made the host
    // compilation drop the launch stub.)
    auto copy_pair = [&](int P) {
      uint8_t* st = raw + (P & (NP - 1)) * PAIR;
#pragma unroll
      for (int u = 0; u < 6; ++u) {
        const int q = 6 * pw + u, R = 16 * q + (lane >> 2);
        const bool sh = q < BS / 16;  // wave-uniform
        const uint32_t off = (uint32_t)(sh ? R : R - BS) * (sh ? s_pitch : p_pitch) + 16u * (uint32_t)((lane & 3) ^ ((R >> 2) & 3));
        const __amdgpu_buffer_rsrc_t rq = sh ? rs_q : rp_q;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(st + 1024 * q), 16, off, (uint32_t)P * 64u, 0, 0);
      }
    };
    // K-tile-major codes of group g: copy c < 4 moves the private rows' 1 KiB of K tile 4g + c
    // (lane l: rows 4l .. 4l+3), copy 4 + c' the shared rows' 512 bytes of K tiles 4g + 2c' and
    // 4g + 2c' + 1 (lanes 0..31 and 32..63), each into its place in the slot.
    auto copy_scales = [&](int g) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int c4 = c == 0 ? pw : (pw < 2 ? pw + 4 : pw);
        if constexpr (KTILE) {
          const bool sh = c4 >= 4;  // wave-uniform
          const uint32_t off = sh ? (uint32_t)(2 * (c4 - 4) + (lane >> 5)) * 4u * (uint32_t)s_all + 16u * (uint32_t)(lane & 31)
                                  : (uint32_t)c4 * 4u * (uint32_t)p_all + 16u * (uint32_t)lane;
          const __amdgpu_buffer_rsrc_t rq = sh ? rs_s : rp_s;
          const uint32_t gofs = (uint32_t)g * 16u * (uint32_t)(sh ? s_all : p_all);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(sring + (g & 1) * SRING + 1024 * c4), 16, off, gofs, 0, 0);
        } else {
          const bool sh = 64 * c4 < BS;
          const uint32_t off = (uint32_t)(64 * c4 + lane - (sh ? 0 : BS)) * KS;
          const __amdgpu_buffer_rsrc_t rq = sh ? rs_s : rp_s;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(sring + (g & 1) * SRING + 1024 * c4), 16, off, (uint32_t)g * 16u, 0, 0);
        }
      }
    };
    // Shared decode of K tile t into buffer t & 1: lane l takes shared row 32pw + (l & 31), half
    // l >> 5, and stores its 32 fp16 values as pieces 4h .. 4h+3 of the row.  tq: t & 3.
    const int sd_row = 32 * pw + r32, sd_swz = dec_row_swizzle(sd_row);
    auto decode_shared = [&](int kt, auto tq) {
      const v4i q4 = *(const v4i*)raw_at(kt, sd_row, hl);
      const uint32_t s = e4m3x2_scale_f16x2_sel(code_word(read_codes(kt, sd_row), tq), code_sel);
      const uint32_t s0 = f16x2_splat_lo(s), s1 = f16x2_splat_hi(s);
      v4i r[4];
      r[0] = e2m1x8_scaled_f16x8((uint32_t)q4[0], s0);
      r[1] = e2m1x8_scaled_f16x8((uint32_t)q4[1], s0);
      r[2] = e2m1x8_scaled_f16x8((uint32_t)q4[2], s1);
      r[3] = e2m1x8_scaled_f16x8((uint32_t)q4[3], s1);
      uint8_t* out = dec + (kt & 1) * DEC + 128 * sd_row;
#pragma unroll
      for (int d = 0; d < 4; ++d) *(v4i*)(out + (((4 * hl + d) ^ sd_swz) << 4)) = r[d];
    };
    // Schedule (kb, ke multiples of 4).  Step t decodes the shared rows of tile t + 1; the compute
    // waves read the packed private rows of tile t (and, ahead, t + 1).  Step 4q copies scale group
    // q + 1 and then pair 2q + 3, step 4q + 2 pair 2q + 4: a pair's stage was last read at the step
    // before, the group's slot (group q - 1) too.  Before the barrier ending step t, tile t + 2 (its
    // pair and group) must have landed: at steps 4q and 4q + 1 the last 14 of the wave's copies may
    // stay in flight (pair 2q + 2, group q + 1, pair 2q + 3), at steps 4q + 2 and 4q + 3 the last 12
    // (pairs 2q + 3, 2q + 4); near the split's end, where copies past it are skipped, none.
    auto step = [&](int kt, auto cc) {
      constexpr int C = decltype(cc)::value;  // kt & 3
      const bool full = (kt & ~3) + 8 < ke;   // every copy the counted waits assume was issued
      if constexpr (C == 0) {
        if (kt + 4 < ke) {
          copy_scales((kt >> 2) + 1);
          copy_pair((kt >> 1) + 3);
        }
      } else if constexpr (C == 2) {
        if (kt + 6 < ke) copy_pair((kt >> 1) + 3);
      }
      if (kt + 1 < ke) decode_shared(kt + 1, std::integral_constant<int, (C + 1) & 3>{});
      if (!full)
        wait_copies<0>();
      else if constexpr (C < 2)
        wait_copies<14>();
      else
        wait_copies<12>();
      __builtin_amdgcn_s_waitcnt(0xC07F);  // as lds_barrier's lgkmcnt(0), seen by the compiler's wait
      lds_barrier();                       // bookkeeping
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;
    // Prologue: the copies the schedule would have issued before step kb -- pair kb/2, scale group
    // kb/4, pairs kb/2 + 1 and kb/2 + 2 (past a 4-tile split's end: bytes never used) -- then tile kb
    // (pair kb/2, group kb/4) landed and decoded.
    copy_pair(kb >> 1);
    copy_scales(kb >> 2);
    copy_pair((kb >> 1) + 1);
    copy_pair((kb >> 1) + 2);
    wait_copies<12>();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    lds_barrier();  // (1) pair kb/2 and group kb/4 visible
    decode_shared(kb, std::integral_constant<int, 0>{});
    __builtin_amdgcn_s_waitcnt(0xC07F);
    lds_barrier();  // (2) tile kb's shared rows decoded
#pragma unroll 1
    for (int kt = kb; kt < ke; kt += 4) {
      step(kt, C0{});
      step(kt + 1, C1{});
      step(kt + 2, C2{});
      step(kt + 3, C3{});
    }
    return;  // the epilogue is the compute waves'
  }

  // ---- compute waves ----------------------------------------------------------------------------
  v16f acc[TS][TP];
#pragma unroll
  for (int i = 0; i < TS; ++i)
#pragma unroll
    for (int j = 0; j < TP; ++j) acc[i][j] = v16f{};
  // Shared block i, slice s: decoded row 32i + r, piece (4 hl + s) ^ f(r) (f(32i + r) = f(r)).  Private
  // block j: row BS + 64 wave + 32j + r, the lane's half hl, decoded slice by slice in registers.
  const int sw = dec_row_swizzle(r32);
  uint32_t piece[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) piece[s] = (uint32_t)(((4 * hl + s) ^ sw) << 4);
  const uint32_t sf_row = (uint32_t)(128 * r32);
  // Packed private rows of tile t in register set t & 1 (read a step ahead).
  v4i pq0[TP], pq1[TP];
  CodeRead pc0[TP], pc1[TP];
  auto read_private = [&](int kt, v4i* pq, CodeRead* pc) {
#pragma unroll
    for (int j = 0; j < TP; ++j) {
      const int R = BS + 64 * wave + 32 * j + r32;
      pq[j] = *(const v4i*)raw_at(kt, R, hl);
      pc[j] = read_codes(kt, R);
    }
  };
  // Scale codes of a tile as fp16 pairs, in register set t & 1 like its packed rows.  tq: t & 3.
  uint32_t ps0[TP][2], ps1[TP][2];
  auto prep_scales = [&](const CodeRead* pc, uint32_t (*ps)[2], auto tq) {
#pragma unroll
    for (int j = 0; j < TP; ++j) {
      const uint32_t s2 = e4m3x2_scale_f16x2_sel(code_word(pc[j], tq), code_sel);
      ps[j][0] = f16x2_splat_lo(s2);
      ps[j][1] = f16x2_splat_hi(s2);
    }
  };
  v4i sf[2][TS], pf[2][TP];
  auto load_shared = [&](int kt, int s, v4i* f) {
    const uint8_t* d = dec + (kt & 1) * DEC + sf_row;
#pragma unroll
    for (int i = 0; i < TS; ++i) f[i] = *(const v4i*)(d + 32 * 128 * i + piece[s]);
  };
  auto decode_private = [&](const v4i* pq, uint32_t (*ps)[2], int s, v4i* f) {
#pragma unroll
    for (int j = 0; j < TP; ++j) f[j] = e2m1x8_scaled_f16x8((uint32_t)pq[j][s], ps[j][s >> 1]);
  };
  auto mfmas = [&](const v4i* a, const v4i* b) {
#pragma unroll
    for (int i = 0; i < TS; ++i)
#pragma unroll
      for (int j = 0; j < TP; ++j)
        acc[i][j] = SHARED_A ? mfma_f16(a[i], b[j], acc[i][j]) : mfma_f16(b[j], a[i], acc[i][j]);
  };
  // Scheduling groups for one slice: an MFMA, the LDS reads (whose data is needed a slice later),
  // then the remaining MFMAs with the VALU work spread between them.
  auto slice_groups = [](auto nreads, auto nvalu) {
    constexpr int NRD = decltype(nreads)::value, NV = decltype(nvalu)::value;
    constexpr int PER = (NV + TS * TP - 2) / (TS * TP - 1);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
#pragma unroll
    for (int m = 1; m < TS * TP; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x002, PER, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };
  // One K tile.  On entry sf[0] and pf[0] hold slice 0's fragments and set t & 1 the tile's packed
  // private rows and scales.  Slice s's MFMAs run while slice s + 1's shared fragments are read and
  // its private ones decoded; the tile t + 1 packed private rows are read during slice 0 (visible
  // since the previous barrier) and their scales prepared during slice 2.  The barrier that ends
  // the step comes before slice 3's MFMAs, which hide the next tile's first shared reads and
  // private decode.  At the split's last tile those reads fetch bytes that are never used.
  using I4 = std::integral_constant<int, 4>;
  using I8 = std::integral_constant<int, 8>;
  using I16 = std::integral_constant<int, 16>;
  using I28 = std::integral_constant<int, 28>;
  auto compute = [&](int kt, auto par, auto tqn) {  // tqn: (kt + 1) & 3
    constexpr int P = decltype(par)::value;  // kt & 1
    const v4i* pq = P ? pq1 : pq0;
    uint32_t (*ps)[2] = P ? ps1 : ps0;
    v4i* pqn = P ? pq0 : pq1;
    CodeRead* pcn = P ? pc0 : pc1;
    uint32_t (*psn)[2] = P ? ps0 : ps1;
    // slice 0
    mfmas(sf[0], pf[0]);
    load_shared(kt, 1, sf[1]);
    read_private(kt + 1, pqn, pcn);
    decode_private(pq, ps, 1, pf[1]);
    slice_groups(I8{}, I16{});
    __builtin_amdgcn_sched_barrier(0);
    // slice 1
    mfmas(sf[1], pf[1]);
    load_shared(kt, 2, sf[0]);
    decode_private(pq, ps, 2, pf[0]);
    slice_groups(I4{}, I16{});
    __builtin_amdgcn_sched_barrier(0);
    // slice 2
    mfmas(sf[0], pf[0]);
    load_shared(kt, 3, sf[1]);
    decode_private(pq, ps, 3, pf[1]);
    prep_scales(pcn, psn, tqn);
    slice_groups(I4{}, I28{});
    __builtin_amdgcn_sched_barrier(0);
    // tile kt's reads done; tile kt + 1's shared rows decoded (the data waves' step kt ends here)
    __builtin_amdgcn_s_waitcnt(0xC07F);
    lds_barrier();
    // slice 3, with the next tile's slice 0 fragments
    mfmas(sf[1], pf[1]);
    load_shared(kt + 1, 0, sf[0]);
    decode_private(pqn, psn, 0, pf[0]);
    slice_groups(I4{}, I16{});
    __builtin_amdgcn_sched_barrier(0);
  };
  lds_barrier();  // (1)
  read_private(kb, pq0, pc0);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  lds_barrier();  // (2): tile kb's shared rows decoded
  using T0 = std::integral_constant<int, 0>;
  using T1 = std::integral_constant<int, 1>;
  using T2 = std::integral_constant<int, 2>;
  using T3 = std::integral_constant<int, 3>;
  load_shared(kb, 0, sf[0]);
  prep_scales(pc0, ps0, T0{});
  decode_private(pq0, ps0, 0, pf[0]);
#pragma unroll 1
  for (int kt = kb; kt < ke; kt += 4) {  // kb and ke are multiples of 4
    compute(kt, T0{}, T1{});
    compute(kt + 1, T1{}, T2{});
    compute(kt + 2, T0{}, T3{});
    compute(kt + 3, T1{}, T0{});
  }

  // Epilogue (as nvfp4_kernel's, TS x TP blocks): SHARED_A: rows m0 + .., columns n0 + 64 wave + ..;
  // otherwise rows m0 + 64 wave + .., columns n0 + ...
  constexpr int PASSES = SHARED_A ? TS : TP, ECOLS = 32 * (SHARED_A ? TP : TS);
  constexpr int LPR = ECOLS / 4, RPI = 64 / LPR;
  float* stage = (float*)lds + wave * (32 * EPI_STRIDE);
  const int mw = m0 + (SHARED_A ? 0 : 64 * wave), nw = n0 + (SHARED_A ? 64 * wave : 0);
  const float alpha = load_alpha(p) * kRescale;
  auto write_out = [&](auto through) {
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
#pragma unroll
      for (int i = 0; i < TS; ++i)
#pragma unroll
        for (int j = 0; j < TP; ++j) {
          const int mi = SHARED_A ? i : j, ni = SHARED_A ? j : i;
          if (mi != pass) continue;
#pragma unroll
          for (int e = 0; e < 16; ++e)
            stage[(8 * (e >> 2) + 4 * hl + (e & 3)) * EPI_STRIDE + 32 * ni + r32] = acc[i][j][e];
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int c4 = 4 * (lane % LPR);
      const int n = nw + c4;
#pragma unroll
      for (int it = 0; it < 32 / RPI; ++it) {
        const int row = RPI * it + lane / LPR;
        const int m = mw + 32 * pass + row;
        const v4f v = *(const v4f*)(stage + row * EPI_STRIDE + c4);
        if (m >= p.M || n >= p.N) continue;  // N % 16 == 0: a lane's 4 columns are all in or all out
        if constexpr (SPLIT) {
          store_partials<decltype(through)::value>(p.ws + (size_t)split * p.M * p.N, (uint32_t)p.M * (uint32_t)p.N * 4u,
                                                   (uint32_t)m * (uint32_t)p.N + (uint32_t)n, v);
        } else {
          v4f b = {0.f, 0.f, 0.f, 0.f};
          if constexpr (BIAS) b = v4f{p.bias[n], p.bias[n + 1], p.bias[n + 2], p.bias[n + 3]};
          uint2 o;
          o.x = epi_pack2<SILU, O>(v[0], v[1], alpha, b[0], b[1]);
          o.y = epi_pack2<SILU, O>(v[2], v[3], alpha, b[2], b[3]);
          *(uint2*)((uint16_t*)p.D + (size_t)m * p.ldd + n) = o;
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next pass overwrites
    }
  };
  if constexpr (SPLIT) {
    if (p.ws_through)
      write_out(std::true_type{});
    else
      write_out(std::false_type{});
  } else {
    write_out(std::false_type{});
  }
}

template <class CF, bool SHARED_A, Out O, bool BIAS, bool SILU>
hipError_t launch(const GemmArgs& args, dim3 grid, dim3 block, hipStream_t stream) {
  void* kargs[] = {(void*)&args};
  // scale copy plan (see nvfp4_kernel): 16-byte row pieces for row-major codes with K % 256 == 0,
  // 4-byte pieces for other dword-aligned rows, else 2-byte pieces
  const int scm = !args.scale_ktile && args.K % 256 == 0 ? 2 : (args.scale_ktile || args.K % 64 == 0) ? 1 : 0;
  const bool ws = CF::BS == 128 && args.K % 256 == 0;  // warp-specialised kernel, either scale layout
  auto pick = [&](auto split) -> const void* {
    constexpr bool SP = decltype(split)::value;
    if constexpr (CF::BS == 128)
      if (ws)
        return args.scale_ktile ? (const void*)&nvfp4_ws_kernel<SHARED_A, O, BIAS, SILU, SP, true>
                                : (const void*)&nvfp4_ws_kernel<SHARED_A, O, BIAS, SILU, SP, false>;
    return scm == 2 ? (const void*)&nvfp4_kernel<CF, SHARED_A, O, BIAS, SILU, SP, 2>
         : scm == 1 ? (const void*)&nvfp4_kernel<CF, SHARED_A, O, BIAS, SILU, SP, 1>
                    : (const void*)&nvfp4_kernel<CF, SHARED_A, O, BIAS, SILU, SP, 0>;
  };
  if (args.splits <= 1) return hipLaunchKernel(pick(std::false_type{}), grid, block, kargs, 0, stream);
  hipError_t e = hipLaunchKernel(pick(std::true_type{}), grid, block, kargs, 0, stream);
  if (e != hipSuccess) return e;
  // accumulators carry 2^-16; with a multiple of 8 tiles the finish kernel follows the GEMM's XCDs
  constexpr int TBM = SHARED_A ? CF::BS : CF::BP, TBN = SHARED_A ? CF::BP : CF::BS;
  if ((args.tiles_m * args.tiles_n) % 8 == 0) return launch_splitk_finish<O, BIAS, SILU, 16, TBM, TBN>(args, grid.z, stream);
  return launch_splitk_finish<O, BIAS, SILU, 16>(args, grid.z, stream);
}

#define BSG_NVR(CF, SA, NAME, O, B, S, MAXS)                                                          \
  { NAME, &launch<CF, SA, O, B, S>, SA ? CF::BS : CF::BP, SA ? CF::BP : CF::BS, BK, THREADS, (uint32_t)CF::LDS_BYTES, \
    true, MAXS, kSplitKtileUs, kSplitPartialUsPerMib, kSplitFixedUs }
#define BSG_NVR_TABLE(CF, SA, NAME, MAXS)                                                                          \
  {                                                                                                                 \
    BSG_NVR(CF, SA, NAME, Out::BF16, false, false, MAXS), BSG_NVR(CF, SA, NAME, Out::BF16, false, true, MAXS),      \
        BSG_NVR(CF, SA, NAME, Out::BF16, true, false, MAXS), BSG_NVR(CF, SA, NAME, Out::BF16, true, true, MAXS),    \
        BSG_NVR(CF, SA, NAME, Out::F16, false, false, MAXS), BSG_NVR(CF, SA, NAME, Out::F16, false, true, MAXS),    \
        BSG_NVR(CF, SA, NAME, Out::F16, true, false, MAXS), BSG_NVR(CF, SA, NAME, Out::F16, true, true, MAXS),      \
  }
// Split-K cost model (see choose_splits): fitted to split sweeps of small-M shapes (M 128..256,
// N 4096..8192, K 4096..8192) on MI355X with streaming partial stores and 4-byte scale copies.
constexpr float kSplitKtileUs = 0.54f, kSplitPartialUsPerMib = 0.22f, kSplitFixedUs = 2.4f;
constexpr int kMaxSplits = 16;
static_assert(kMaxSplits <= kMaxFinishSplits, "the finish kernel sums at most kMaxFinishSplits partials");
const KernelVariant kSharedA[8] = BSG_NVR_TABLE(Cfg128, true, "nvfp4_128x256_sharedA", kMaxSplits);
const KernelVariant kSharedB[8] = BSG_NVR_TABLE(Cfg128, false, "nvfp4_256x128_sharedB", kMaxSplits);
// 256 x 256 tiles are chosen only when they give every CU a workgroup: never split
const KernelVariant kSharedB256[8] = BSG_NVR_TABLE(Cfg256, false, "nvfp4_256x256_sharedB", 1);
#undef BSG_NVR_TABLE
#undef BSG_NVR

}  // namespace nvr

// One 128-row tile of A (small M): A is the shared side.  Otherwise B is: 256 x 256 tiles (half the
// decode work per output of 256 x 128, twice the MFMAs per barrier) once they give every CU a
// workgroup, 256 x 128 tiles (split K when still too few) below that.
const KernelVariant* nvfp4_variants(int64_t M, int64_t N, int64_t /*K*/, int64_t batch) {
  if (M <= nvr::Cfg128::BS) return nvr::kSharedA;
  const int64_t tiles256 = ((M + 255) / 256) * ((N + 255) / 256) * batch;
  return tiles256 >= 256 ? nvr::kSharedB256 : nvr::kSharedB;
}

}  // namespace bsg
