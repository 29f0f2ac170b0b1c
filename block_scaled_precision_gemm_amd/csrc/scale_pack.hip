// Conversion of scale codes from row-major [rows][KB] to the K-tile-major layout that kernels read
// with one contiguous run per K tile: code 4g + c of row r at byte (g * rows + r) * 4 + c, the codes
// past KB in the last group written as 0.  A utility for callers that opt in to that layout (the
// role of the MXFP8 page's swizzled scale layout); the GEMM kernels read either layout directly.
#include "bsg.h"
#include "common.h"

namespace bsg {
void set_error(const char* fmt, ...);
}

namespace {

// One thread per output dword; threads of consecutive rows write consecutive dwords.
__global__ void pack_scales_kernel(const uint8_t* src, uint32_t* dst, int64_t rows, int64_t kb, int64_t n_words) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_words) return;
  const int64_t g = t / rows, r = t - g * rows;
  const uint8_t* s = src + r * kb + 4 * g;
  const int64_t left = kb - 4 * g;  // >= 1
  uint32_t w = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (c < left) w |= (uint32_t)s[c] << (8 * c);
  dst[t] = w;
}

}  // namespace

extern "C" int64_t bsg_scales_ktile_bytes(int64_t rows, int64_t codes_per_row) {
  if (rows < 1 || codes_per_row < 1) return 0;
  return (codes_per_row + 3) / 4 * rows * 4;
}

extern "C" bsg_status bsg_pack_scales(const void* src, void* dst, int64_t rows, int64_t codes_per_row, void* stream) {
  if (!src || !dst) {
    bsg::set_error("bsg_pack_scales: null pointer");
    return BSG_ERR_NULL;
  }
  if (rows < 1 || codes_per_row < 1 || bsg_scales_ktile_bytes(rows, codes_per_row) >= ((int64_t)1 << 31)) {
    bsg::set_error("bsg_pack_scales: rows and codes_per_row must be >= 1 and the result < 2^31 bytes (got %lld, %lld)",
                   (long long)rows, (long long)codes_per_row);
    return BSG_ERR_SHAPE;
  }
  if ((uintptr_t)dst & 3u) {
    bsg::set_error("bsg_pack_scales: dst must be 4-byte aligned");
    return BSG_ERR_ALIGN;
  }
  const int64_t n_words = bsg_scales_ktile_bytes(rows, codes_per_row) / 4;
  void* args[] = {(void*)&src, (void*)&dst, (void*)&rows, (void*)&codes_per_row, (void*)&n_words};
  const hipError_t e = hipLaunchKernel((const void*)&pack_scales_kernel, dim3((unsigned)((n_words + 255) / 256)),
                                       dim3(256), args, 0, (hipStream_t)stream);
  if (e != hipSuccess) {
    bsg::set_error("bsg_pack_scales: launch failed: %s", hipGetErrorString(e));
    return BSG_ERR_HIP;
  }
  return BSG_OK;
}
