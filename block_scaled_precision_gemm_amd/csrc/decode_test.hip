// Element-wise launchers of the device decoders (codec.h), for bit-exact tests against a CPU
// decoding of every code.  Not on the GEMM path; they run the very functions the GEMM kernels use.
#include "bsg_testing.h"
#include "codec.h"
#include "common.h"

namespace bsg {
void set_error(const char* fmt, ...);
}

namespace {

__global__ void decode_e4m3_kernel(const uint8_t* codes, float* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = bsg::e4m3_to_f32(codes[i]);
}

// One dword (8 elements, inside one 16-element block) per thread, decoded with the GEMM kernels'
// own routine.
__global__ void decode_nvfp4_kernel(const uint32_t* packed, const uint8_t* scales, uint16_t* out, int64_t n_words) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_words) return;
  const bsg::v4i v = bsg::e2m1x8_scaled_bf16x8(packed[t], bsg::e4m3_to_f32(scales[t >> 1]));
  ((bsg::v4i*)out)[t] = v;
}

// fp16 route: one 16-byte chunk (32 elements, two scale blocks) per thread, q * s * 2^-7 as fp16,
// through the same routine the tiled NVFP4 kernels use.
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
  if (e == hipSuccess) return BSG_OK;
  bsg::set_error("kernel launch failed: %s", hipGetErrorString(e));
  return BSG_ERR_HIP;
}

}  // namespace

extern "C" bsg_status bsg_test_decode_e4m3(const uint8_t* codes, float* out, int64_t n, void* stream) {
  if (n < 0) { bsg::set_error("n < 0"); return BSG_ERR_SHAPE; }
  if (n == 0) return BSG_OK;
  if (!codes || !out) { bsg::set_error("null pointer"); return BSG_ERR_NULL; }
  const dim3 grid((unsigned)((n + 255) / 256));
  hipLaunchKernelGGL(decode_e4m3_kernel, grid, dim3(256), 0, (hipStream_t)stream, codes, out, n);
  return launch_status(hipGetLastError());
}

extern "C" bsg_status bsg_test_decode_nvfp4(const uint8_t* packed, const uint8_t* scale_codes, uint16_t* out_bf16,
                                            int64_t n_elements, void* stream) {
  if (n_elements < 0 || n_elements % 16 != 0) {
    bsg::set_error("n_elements must be a non-negative multiple of 16 (got %lld)", (long long)n_elements);
    return BSG_ERR_SHAPE;
  }
  if (n_elements == 0) return BSG_OK;
  if (!packed || !scale_codes || !out_bf16) { bsg::set_error("null pointer"); return BSG_ERR_NULL; }
  if ((uintptr_t)packed & 3u) { bsg::set_error("packed must be 4-byte aligned"); return BSG_ERR_ALIGN; }
  const int64_t n_words = n_elements / 8;
  const dim3 grid((unsigned)((n_words + 255) / 256));
  hipLaunchKernelGGL(decode_nvfp4_kernel, grid, dim3(256), 0, (hipStream_t)stream, (const uint32_t*)packed,
                     scale_codes, out_bf16, n_words);
  return launch_status(hipGetLastError());
}

extern "C" bsg_status bsg_test_decode_nvfp4_f16(const uint8_t* packed, const uint8_t* scale_codes, uint16_t* out_f16,
                                                int64_t n_elements, void* stream) {
  if (n_elements < 0 || n_elements % 32 != 0) {
    bsg::set_error("n_elements must be a non-negative multiple of 32 (got %lld)", (long long)n_elements);
    return BSG_ERR_SHAPE;
  }
  if (n_elements == 0) return BSG_OK;
  if (!packed || !scale_codes || !out_f16) { bsg::set_error("null pointer"); return BSG_ERR_NULL; }
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
