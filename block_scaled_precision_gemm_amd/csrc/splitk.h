// Split-K finish kernel shared by the kernels that split K over workgroups.
//
// A split plan's GEMM kernel writes fp32 partial sums ws[z][s][m][n] (batch z, split s) of its K range
// into the plan's workspace; this kernel adds the S partials of each element in split order (a fixed
// order, so results are deterministic), applies the epilogue of epilogue.h (alpha, bias, SiLU, one
// rounding) and writes D.  RESCALE multiplies alpha for kernels whose accumulators carry a known
// power-of-two factor (the NVFP4 fp16 route: 2^-16).  One thread per 4 consecutive columns
// (N % 16 == 0); grid.z = batch.
//
// DEPTH: the partial loads a thread keeps in flight.  0 issues all S before the first sum: one
// memory round trip instead of S.  That pays while one partial plane (batch x M x N x 4 bytes, what
// all threads read per round trip) is smaller than latency x bandwidth (~4 MiB: 0.8 us at ~5 TB/s),
// where a plane-by-plane pass waits on latency (measured: 1-2 MiB planes 5-11% faster, 4 MiB planes
// 1% slower).  From 4 MiB planes go by one or two at a time: two for partials the GEMM left in the
// L2s (256x4096x4096: 2.0-2.6% faster per call than one; three or four at a time slower again),
// one for partials stored through the L2 (GemmArgs::ws_through; two: +0.6-1.8% at S = 4).
//
// TBM x TBN (0 x 0: rows in order): the GEMM kernel put every split of tile t on XCD t % 8
// (workgroups go to the 8 XCDs round-robin by id), and block b sums part of a tile t with
// t % 8 == b % 8, i.e. on the XCD that wrote those partials; TileMap turns t into the tile's
// (row, column) as the GEMM kernel numbered it.  Measured with the NVFP4 split kernels
// (256x4096x4096: 6-12% faster per call than splits and finish blocks spread over all XCDs);
// plain instead of streaming partial stores and loads were slower either way.
#pragma once

#include "common.h"
#include "epilogue.h"

namespace bsg {

// The largest split factor of any split-capable kernel (KernelVariant::max_splits).
constexpr int kMaxFinishSplits = 16;

// Store four partial sums at float `off` of a split's partial plane (`plane_bytes` long; a split
// plan's plane is far below 2^31 bytes).  Streaming stores by default: with the finish kernel's
// blocks on the XCD that wrote a tile's partials, a plan whose partials fit the L2s is summed from
// them.  THROUGH (GemmArgs::ws_through, set at plan time when the partials come to at least one
// L2's size per XCD): device-scope stores, which write through the L2 to memory.  Kernels choose
// the form once, outside their store loops (a per-store branch made the compiler wait for each
// staging read before its store).  Measured per call against streaming stores (interleaved,
// outputs bit-identical): 4 MiB of partials per XCD 3.3% faster, 3 MiB 0.5%, 2 MiB 3.3% slower.
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
constexpr int kCachePolicySc1 = 16;  // buffer store cache-policy bits: sc1 (device scope)
template <bool THROUGH>
__device__ __forceinline__ void store_partials(float* plane, uint32_t plane_bytes, uint32_t off, v4f v) {
  if constexpr (THROUGH) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)plane, (short)0, (int)plane_bytes, (int)0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, (int)(off * 4u), 0, kCachePolicySc1);
  } else {
    __builtin_nontemporal_store(v, (v4f*)(plane + off));
  }
}

// Tile t of a row-major tile grid.
struct RowMajorTiles {
  __device__ static int2 of(int t, int /*tiles_m*/, int tiles_n) {
    const int tm = t / tiles_n;
    return make_int2(tm, t - tm * tiles_n);
  }
};

template <Out O, bool BIAS, bool SILU, int RESCALE_LOG2, int DEPTH, int TBM = 0, int TBN = 0,
          class TileMap = RowMajorTiles>
__global__ __launch_bounds__(256) void splitk_finish_kernel(GemmArgs p) {
  select_batch(p);
  constexpr bool AFFINE = TBM > 0;
  int m, n;
  if constexpr (AFFINE) {
    constexpr int BPT = TBM * TBN / 4 / 256, TPR = TBN / 4;  // blocks per tile, threads per tile row
    static_assert(BPT * 256 * 4 == TBM * TBN && TBN % 4 == 0, "whole blocks per tile");
    const int b = (int)blockIdx.x, k = b >> 3;
    const int t = (b & 7) + 8 * (k / BPT), ti = (k % BPT) * 256 + (int)threadIdx.x;
    const int2 tt = TileMap::of(t, p.tiles_m, p.tiles_n);
    m = tt.x * TBM + ti / TPR;
    n = tt.y * TBN + (ti % TPR) * 4;
    if (m >= p.M || n >= p.N) return;  // ragged tiles (N % 16 == 0: 4 columns all in or all out)
  } else {
    const int nq = p.N >> 2;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)p.M * nq) return;
    m = (int)(idx / nq);
    n = (int)(idx - (int64_t)m * nq) * 4;
  }
  const size_t plane = (size_t)p.M * p.N;
  const float* src = p.ws + (size_t)m * p.N + n;
  // streaming loads: every partial is read exactly once; sums in split order either way
  auto ld = [&](int k) -> v4f { return __builtin_nontemporal_load((const v4f*)(src + k * plane)); };
  v4f s;
  static_assert(DEPTH >= 0 && DEPTH <= 2, "load depth");
  if constexpr (DEPTH == 0) {
    v4f part[kMaxFinishSplits];
#pragma unroll
    for (int k = 0; k < kMaxFinishSplits; ++k)
      if (k < p.splits) part[k] = ld(k);
    s = part[0];
#pragma unroll
    for (int k = 1; k < kMaxFinishSplits; ++k)
      if (k < p.splits) s += part[k];
  } else {
    s = ld(0);
    int k = 1;
    if constexpr (DEPTH == 2) {
      for (; k + 1 < p.splits; k += 2) {
        const v4f x = ld(k), y = ld(k + 1);
        s += x;
        s += y;
      }
    }
    for (; k < p.splits; ++k) s += ld(k);
  }
  const float alpha = load_alpha(p) * (float)(1u << RESCALE_LOG2);
  v4f b = {0.f, 0.f, 0.f, 0.f};
  if constexpr (BIAS) b = v4f{p.bias[n], p.bias[n + 1], p.bias[n + 2], p.bias[n + 3]};  // bias: 4-byte aligned
  uint32_t* D = (uint32_t*)((uint16_t*)p.D + (size_t)m * p.ldd + n);
  D[0] = epi_pack2<SILU, O>(s[0], s[1], alpha, b[0], b[1]);
  D[1] = epi_pack2<SILU, O>(s[2], s[3], alpha, b[2], b[3]);
}

// Enqueue the finish kernel of a split plan (grid.z of the GEMM launch = batch).  TBM x TBN > 0: the
// GEMM kept each tile's splits on one XCD (tiles a multiple of 8, tiles of TBM x TBN).
template <Out O, bool BIAS, bool SILU, int RESCALE_LOG2, int TBM = 0, int TBN = 0, class TileMap = RowMajorTiles>
hipError_t launch_splitk_finish(const GemmArgs& args, unsigned batch, hipStream_t stream) {
  if (args.splits < 1 || args.splits > kMaxFinishSplits) return hipErrorInvalidValue;
  void* kargs[] = {(void*)&args};
  const int64_t threads = (int64_t)args.M * (args.N >> 2);
  const int depth = 16.0 * (double)threads * (double)batch < 4.0 * 1024 * 1024 ? 0  // one plane < 4 MiB
                    : args.ws_through                                             ? 1
                                                                                  : 2;
  auto pick = [&](auto tbm) -> const void* {
    constexpr int BM = decltype(tbm)::value, BN = BM > 0 ? TBN : 0;
    return depth == 0   ? (const void*)&splitk_finish_kernel<O, BIAS, SILU, RESCALE_LOG2, 0, BM, BN, TileMap>
           : depth == 1 ? (const void*)&splitk_finish_kernel<O, BIAS, SILU, RESCALE_LOG2, 1, BM, BN, TileMap>
                        : (const void*)&splitk_finish_kernel<O, BIAS, SILU, RESCALE_LOG2, 2, BM, BN, TileMap>;
  };
  if constexpr (TBM > 0) {
    const unsigned blocks = (unsigned)(args.tiles_m * args.tiles_n) * (unsigned)(TBM * TBN / 4 / 256);
    return hipLaunchKernel(pick(std::integral_constant<int, TBM>{}), dim3(blocks, 1, batch), dim3(256), kargs, 0, stream);
  } else {
    return hipLaunchKernel(pick(std::integral_constant<int, 0>{}), dim3((unsigned)((threads + 255) / 256), 1, batch),
                           dim3(256), kargs, 0, stream);
  }
}

}  // namespace bsg
