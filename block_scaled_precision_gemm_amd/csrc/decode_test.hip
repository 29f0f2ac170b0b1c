// Launcher of the NVFP4 device dequantisation (codec.h), for a bit-exact test against a CPU decoding
// of every code.  Not on the GEMM path; it runs the very routine the GEMM kernels use.
#include "bsg_testing.h"
#include "codec.h"
#include "common.h"

namespace bsg {
void set_error(const char* fmt, ...);
}

namespace {

// One 16-byte chunk (32 elements, two scale blocks) per thread: q * s * 2^-8 as fp16.
__global__ void decode_nvfp4_f16_kernel(const uint8_t* packed, const uint8_t* scales, uint16_t* out,
                                        int64_t n_chunks) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_chunks) return;
  const bsg::v4i q = *(const bsg::v4i*)(packed + 16 * t);
  const uint32_t sc = (uint32_t)scales[2 * t] | ((uint32_t)scales[2 * t + 1] << 8);
  bsg::v4i r[4];
  bsg::e2m1x32_scaled_f16(q, sc, r);
  bsg::v4i* o = (bsg::v4i*)(out + 32 * t);
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = r[i];
}

bsg_status launch_status(hipError_t e) {
  if (e != hipSuccess) {
    bsg::set_error("kernel launch failed: %s", hipGetErrorString(e));
    return BSG_ERR_HIP;
  }
  return BSG_OK;
}

}  // namespace

extern "C" bsg_status bsg_test_decode_nvfp4_f16(const uint8_t* packed, const uint8_t* scale_codes, uint16_t* out_f16,
                                                int64_t n_elements, void* stream) {
  if (n_elements < 0 || n_elements % 32 != 0) {
    bsg::set_error("n_elements must be a non-negative multiple of 32 (got %lld)", (long long)n_elements);
    return BSG_ERR_SHAPE;
  }
  if (n_elements == 0) return BSG_OK;
  if (!packed || !scale_codes || !out_f16) {
    bsg::set_error("null pointer");
    return BSG_ERR_NULL;
  }
  if (((uintptr_t)packed | (uintptr_t)out_f16) & 15u) {
    bsg::set_error("packed and out_f16 must be 16-byte aligned");
    return BSG_ERR_ALIGN;
  }
  const int64_t n_chunks = n_elements / 32;
  const dim3 grid((unsigned)((n_chunks + 255) / 256));
  hipLaunchKernelGGL(decode_nvfp4_f16_kernel, grid, dim3(256), 0, (hipStream_t)stream, packed, scale_codes,
                     out_f16, n_chunks);
  return launch_status(hipGetLastError());
}
