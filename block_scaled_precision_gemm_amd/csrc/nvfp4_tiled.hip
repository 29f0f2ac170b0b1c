// NVFP4 block-scaled GEMM, LDS-tiled, for gfx950.
//
// D = epi(alpha * A x B^T (+ bias)): A [M][K/2] and B [N][K/2] packed E2M1 (element 2t in the low
// nibble of byte t), one E4M3 scale per 16 K elements, a global fp32 alpha (the operation of
// runNvfp4Gemm<T, kEnableSilu, kEnableBias> on the CUTLASS issue #3003 page).
//
// CDNA4's scaled MFMAs take power-of-two (E8M0) scales per 32 elements, which cannot carry an E4M3
// scale per 16 elements exactly.  The operands are therefore dequantised once per workgroup into
// fp16 and contracted on v_mfma_f32_32x32x16_f16:
// * each element becomes the fp16 number q * s * 2^-7 (exact, see codec.h), so each MFMA product is
//   the exact dequantised product times 2^-14, accumulated in fp32; the epilogue multiplies by
//   alpha * 2^14 (an exact power-of-two rescaling of alpha);
// * decoding happens once per workgroup and K tile: the 256 threads each take 16-byte chunks of
//   packed rows (32 elements, two scale blocks), decode them in registers and store 64 bytes of fp16
//   into a double-buffered LDS tile that all four waves read their MFMA fragments from.
//
// * Workgroup tile BM x BN (128 x 128 or 128 x 256), K tile 64, 4 waves as 2 x 2, each wave
//   (BM/2) x (BN/2) of D as TM x TN accumulators of 32 x 32.
// * Per K tile: the packed bytes of tile k+3 are loaded into registers, tile k's fragments are read
//   from LDS and fed to the MFMAs, and tile k+1 (loaded two tiles earlier) is decoded into the other
//   LDS buffer in between; one barrier per tile.
// * LDS rows are 128 bytes (64 fp16) = 8 pieces of 16 bytes; piece p of row R is stored at
//   p ^ f(R), f(R) = (R & 7) ^ ((R >> 3) & 1): both the decode stores (16 rows x one piece per
//   16 lanes) and the fragment reads (16 rows x one piece) hit distinct banks.
// * Split-K for small M x N: the grid holds tiles x S workgroups; split s covers K tiles
//   [s KT / S, (s+1) KT / S) and writes its raw fp32 accumulators to a plan-owned workspace
//   [S][M][N]; a second kernel sums the S partials in split order (deterministic), applies the
//   epilogue and writes D.  With S == 1 the epilogue runs in the GEMM kernel.
// * Any M >= 1, N % 16 == 0, K % 32 == 0: out-of-range rows are clamped to the last row for loading
//   and never stored; a final half K tile (K % 64 == 32) loads zeros for its missing half.
//
// v_mfma_f32_32x32x16_f16 register layout: A lane l (r = l % 32, h = l / 32) holds row r, K
// elements [8h, 8h+8) of the 16-element slice; B likewise for column r; accumulator element e of
// lane l: row 8*(e/4) + 4h + e%4, column r.
#include <type_traits>

#include "codec.h"
#include "common.h"
#include "epilogue.h"

namespace bsg {
namespace nvt {

constexpr int BK = 64;         // K elements per tile
constexpr int ROW_BYTES = 128; // fp16 bytes per LDS row per K tile
constexpr int THREADS = 256;
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)
constexpr uint32_t kOutOfRange = 0x80000000u;  // a buffer offset past any operand's size (< 2^31)

template <int BM_, int BN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int R = BM + BN;              // rows decoded per K tile
  static constexpr int CPT = 2 * R / THREADS;    // 16-byte chunks per thread per K tile
  static constexpr int TM = BM / 64, TN = BN / 64;
  static constexpr int STAGE = R * ROW_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static_assert(2 * R % THREADS == 0 && R % 64 == 0 && BM % 64 == 0, "chunk split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ v16f mfma_f16(v4i a, v4i b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}

// Wait for this wave's LDS accesses, then meet the other waves.  Outstanding global loads (the
// prefetch of the next tiles) stay in flight.
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

template <class C, Out O, bool BIAS, bool SILU, bool SPLIT>
__global__ __launch_bounds__(THREADS, 1) void nvfp4_tiled_kernel(GemmArgs p) {
  constexpr int BM = C::BM, BN = C::BN, R = C::R, CPT = C::CPT, TM = C::TM, TN = C::TN;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn, split = 0;
  if constexpr (SPLIT) {
    split = (int)blockIdx.x % p.splits;
    const int t = (int)blockIdx.x / p.splits;
    tm = t / p.tiles_n;
    tn = t - tm * p.tiles_n;
  } else {
    const int2 t = tile_of(blockIdx.x, p.tiles_m, p.tiles_n);
    tm = t.x;
    tn = t.y;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int K = p.K, KT = (K + BK - 1) / BK;
  const int kb = SPLIT ? (int)((int64_t)split * KT / p.splits) : 0;
  const int ke = SPLIT ? (int)((int64_t)(split + 1) * KT / p.splits) : KT;
  const size_t KH = (size_t)(K >> 1), KS = (size_t)(K >> 4);

  // This thread's chunks: chunk c = tid + 256 i is half (c >= R) of row (c mod R); rows [0, BM) are
  // A rows m0.., rows [BM, R) are B rows n0...  Half and operand are uniform across a wave, so each
  // chunk's buffer resource and K-tile offset are scalar; the lane keeps one 32-bit row offset.
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t bytes_a = (uint32_t)p.M * (uint32_t)KH, bytes_b = (uint32_t)p.N * (uint32_t)KH;
  __amdgpu_buffer_rsrc_t rq[CPT], rs[CPT];
  uint32_t vq[CPT], vs[CPT];
  int chalf[CPT];
  uint32_t woff[CPT][4];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c0 = 64 * wv + THREADS * i;  // the wave's first chunk
    const int h = c0 >= R ? 1 : 0;
    const bool is_a = c0 - h * R < BM;
    const int row = c0 - h * R + lane;
    const int g = is_a ? min(m0 + row, p.M - 1) : min(n0 + row - BM, p.N - 1);
    rq[i] = __builtin_amdgcn_make_buffer_rsrc((void*)(is_a ? p.A : p.B), (short)0, (int)(is_a ? bytes_a : bytes_b),
                                              (int)kRsrcWord3);
    rs[i] = __builtin_amdgcn_make_buffer_rsrc((void*)(is_a ? p.sA : p.sB), (short)0,
                                              (int)((is_a ? bytes_a : bytes_b) >> 3), (int)kRsrcWord3);
    vq[i] = (uint32_t)g * (uint32_t)KH + 16u * h;
    vs[i] = (uint32_t)g * (uint32_t)KS + 2u * h;
    chalf[i] = h;
    const int sw = swz(row);
#pragma unroll
    for (int d = 0; d < 4; ++d) woff[i][d] = (uint32_t)(row * ROW_BYTES + (((4 * h + d) ^ sw) << 4));
  }

  struct Raw {
    v4i q[CPT];
    uint32_t sc[CPT];
  };
  // Loads of K tile min(kt, ke - 1): unconditional and branch-free, and nothing touches the loaded
  // registers before the decode, so the compiler's wait counts stay exact and the prefetch stays in
  // flight.  The missing half of a final half tile (K % 64 == 32) gets an offset past the buffer's
  // end, which the buffer range check turns into zero bytes: zero elements with scale code 0.
  auto load = [&](Raw& r, int kt) {
    kt = min(kt, ke - 1);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const bool ok = kt * BK + 32 * chalf[i] < K;  // K % 32 == 0: a chunk is wholly in or out
      r.q[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rq[i], ok ? vq[i] : kOutOfRange,
                                                                             kt * 32, 0));
      r.sc[i] = __builtin_amdgcn_raw_buffer_load_b16(rs[i], ok ? vs[i] : kOutOfRange, kt * 4, 0);
    }
  };

  // Fragment offsets within a stage: A rows wm*BM/2 + 32i + r, B rows BM + wn*BN/2 + 32j + r; piece
  // 2*slice + h.  f(row) depends on row & 15 only, i.e. on the lane.
  const int r32 = lane & 31, hl = lane >> 5, lsw = swz(lane & 15);
  const uint32_t a_row0 = (uint32_t)((wm * (BM / 2) + r32) * ROW_BYTES);
  const uint32_t b_row0 = (uint32_t)((BM + wn * (BN / 2) + r32) * ROW_BYTES);
  uint32_t poff[4];
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) poff[sl] = (uint32_t)(((2 * sl + hl) ^ lsw) << 4);

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v16f{};

  // Three register buffers: tile k's packed bytes sit in raw[(k - kb) % 3]; the loads of tile k+3
  // are issued while tile k is computed, two tiles before they are decoded.
  Raw raw[3];
  load(raw[0], kb);
  load(raw[1], kb + 1);
  load(raw[2], kb + 2);
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    v4i o[4];
    e2m1x32_scaled_f16(raw[0].q[i], raw[0].sc[i], o);
#pragma unroll
    for (int d = 0; d < 4; ++d) *(v4i*)(lds + woff[i][d]) = o[d];
  }
  lds_barrier();

  // One K tile (u = (kt - kb) % 6): compute tile kt from LDS stage u & 1 while decoding tile kt+1
  // (raw[(u+1) % 3]) into the other stage and loading tile kt+3 into raw[u % 3].  The step has no
  // branches.
  auto step = [&](auto Ut, int kt) {
    constexpr int u = decltype(Ut)::value;
    constexpr int ST = u & 1, RL = u % 3, RD = (u + 1) % 3;
    const uint8_t* st = lds + ST * C::STAGE;
    uint8_t* nx = lds + (ST ^ 1) * C::STAGE;
    load(raw[RL], kt + 3);
    uint32_t s0[CPT], s1[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const uint32_t s = e4m3x2_scale_f16x2(raw[RD].sc[i]);
      s0[i] = f16x2_splat_lo(s);
      s1[i] = f16x2_splat_hi(s);
    }
    v4i fa[2][TM], fb[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[0][i] = *(const v4i*)(st + a_row0 + i * 32 * ROW_BYTES + poff[0]);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[0][j] = *(const v4i*)(st + b_row0 + j * 32 * ROW_BYTES + poff[0]);
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const int cb = sl & 1, nb = cb ^ 1;
      if (sl < 3) {
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[nb][i] = *(const v4i*)(st + a_row0 + i * 32 * ROW_BYTES + poff[sl + 1]);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[nb][j] = *(const v4i*)(st + b_row0 + j * 32 * ROW_BYTES + poff[sl + 1]);
      }
      // dwords [sl*CPT, (sl+1)*CPT) of the CPT*4 packed dwords of tile kt+1.  Unconditional (no
      // branch for the register allocator to split the accumulators around): after the last tile
      // this decodes the clamped reload into a buffer nobody reads.
#pragma unroll
      for (int x = sl * CPT; x < (sl + 1) * CPT; ++x) {
        const int i = x >> 2, d = x & 3;
        const v4i o = e2m1x8_scaled_f16x8((uint32_t)raw[RD].q[i][d], d < 2 ? s0[i] : s1[i]);
        *(v4i*)(nx + woff[i][d]) = o;
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_f16(fa[cb][i], fb[cb][j], acc[i][j]);
    }
    lds_barrier();
  };

  // Whole groups of six tiles in a loop with a single exit (so the compiler's wait counts at the loop
  // header are the steady-state ones), then at most five remaining tiles.
  int kt = kb;
  for (; kt + 6 <= ke; kt += 6) {
    step(std::integral_constant<int, 0>{}, kt);
    step(std::integral_constant<int, 1>{}, kt + 1);
    step(std::integral_constant<int, 2>{}, kt + 2);
    step(std::integral_constant<int, 3>{}, kt + 3);
    step(std::integral_constant<int, 4>{}, kt + 4);
    step(std::integral_constant<int, 5>{}, kt + 5);
  }
  const int rem = ke - kt;
  if (rem > 0) step(std::integral_constant<int, 0>{}, kt);
  if (rem > 1) step(std::integral_constant<int, 1>{}, kt + 1);
  if (rem > 2) step(std::integral_constant<int, 2>{}, kt + 2);
  if (rem > 3) step(std::integral_constant<int, 3>{}, kt + 3);
  if (rem > 4) step(std::integral_constant<int, 4>{}, kt + 4);

  // Epilogue.  Lane holds column n = n0 + wn*BN/2 + 32j + r32 and rows m0 + wm*BM/2 + 32i +
  // 8*(e/4) + 4*hl + e%4.
  const int mw = m0 + wm * (BM / 2), nw = n0 + wn * (BN / 2);
  if constexpr (SPLIT) {
    float* ws = p.ws + (size_t)split * p.M * p.N;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = nw + 32 * j + r32;
      if (n >= p.N) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = mw + 32 * i + 8 * (e >> 2) + 4 * hl + (e & 3);
          if (m < p.M) ws[(size_t)m * p.N + n] = acc[i][j][e];
        }
    }
  } else {
    const float alpha = load_alpha(p) * 16384.0f;  // restores the 2^-14 of the fp16 operands
    uint16_t* D = (uint16_t*)p.D;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = nw + 32 * j + r32;
      if (n >= p.N) continue;
      const float bv = BIAS ? p.bias[n] : 0.0f;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = mw + 32 * i + 8 * (e >> 2) + 4 * hl + (e & 3);
          if (m < p.M) D[(size_t)m * p.N + n] = to_out_bits<O>(epi_value<SILU>(acc[i][j][e], alpha, bv));
        }
    }
  }
}

// Split-K finish: D[m][n] = epi(alpha * 2^14 * sum_s ws[s][m][n] (+ bias[n])), summed in split
// order.  One thread per 4 consecutive columns (N % 16 == 0).
template <Out O, bool BIAS, bool SILU>
__global__ __launch_bounds__(256) void nvfp4_splitk_finish_kernel(GemmArgs p) {
  const int nq = p.N >> 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)p.M * nq) return;
  const int m = (int)(idx / nq), n = (int)(idx - (int64_t)m * nq) * 4;
  const size_t plane = (size_t)p.M * p.N;
  const float* src = p.ws + (size_t)m * p.N + n;
  v4f s = *(const v4f*)src;
  for (int k = 1; k < p.splits; ++k) s += *(const v4f*)(src + k * plane);
  const float alpha = load_alpha(p) * 16384.0f;
  v4f b = {0.f, 0.f, 0.f, 0.f};
  if constexpr (BIAS) b = v4f{p.bias[n], p.bias[n + 1], p.bias[n + 2], p.bias[n + 3]};  // bias: 4-byte aligned
  uint32_t* D = (uint32_t*)((uint16_t*)p.D + (size_t)m * p.N + n);
  D[0] = pack2_out<O>(epi_value<SILU>(s[0], alpha, b[0]), epi_value<SILU>(s[1], alpha, b[1]));
  D[1] = pack2_out<O>(epi_value<SILU>(s[2], alpha, b[2]), epi_value<SILU>(s[3], alpha, b[3]));
}

template <class C, Out O, bool BIAS, bool SILU>
hipError_t launch(const GemmArgs& args, dim3 grid, dim3 block, hipStream_t stream) {
  void* kargs[] = {(void*)&args};
  if (args.splits <= 1)
    return hipLaunchKernel((const void*)&nvfp4_tiled_kernel<C, O, BIAS, SILU, false>, grid, block, kargs, 0,
                           stream);
  hipError_t e = hipLaunchKernel((const void*)&nvfp4_tiled_kernel<C, O, BIAS, SILU, true>, grid, block, kargs, 0,
                                 stream);
  if (e != hipSuccess) return e;
  const int64_t threads = (int64_t)args.M * (args.N >> 2);
  return hipLaunchKernel((const void*)&nvfp4_splitk_finish_kernel<O, BIAS, SILU>,
                         dim3((unsigned)((threads + 255) / 256)), dim3(256), kargs, 0, stream);
}

using Cfg128 = Cfg<128, 128>;
using Cfg256 = Cfg<128, 256>;

#define BSG_NVT(C, NAME, O, B, S) \
  { NAME, &launch<C, O, B, S>, C::BM, C::BN, BK, THREADS, (uint32_t)C::LDS_BYTES, true, 16 }
#define BSG_NVT_TABLE(C, NAME)                                                              \
  {                                                                                          \
    BSG_NVT(C, NAME, Out::BF16, false, false), BSG_NVT(C, NAME, Out::BF16, false, true),    \
        BSG_NVT(C, NAME, Out::BF16, true, false), BSG_NVT(C, NAME, Out::BF16, true, true),  \
        BSG_NVT(C, NAME, Out::F16, false, false), BSG_NVT(C, NAME, Out::F16, false, true),  \
        BSG_NVT(C, NAME, Out::F16, true, false), BSG_NVT(C, NAME, Out::F16, true, true),    \
  }
const KernelVariant k128x128[8] = BSG_NVT_TABLE(Cfg128, "nvfp4_tiled_128x128");
const KernelVariant k128x256[8] = BSG_NVT_TABLE(Cfg256, "nvfp4_tiled_128x256");
#undef BSG_NVT_TABLE
#undef BSG_NVT

}  // namespace nvt

// Small M (one 128-row tile): the wider tile halves the A decode per output; otherwise 128 x 128.
const KernelVariant* nvfp4_tiled_variants(int64_t M, int64_t /*N*/) {
  return M <= 128 ? nvt::k128x256 : nvt::k128x128;
}

}  // namespace bsg
