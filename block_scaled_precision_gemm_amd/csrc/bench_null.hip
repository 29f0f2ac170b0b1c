// Back-to-back launches of an empty kernel: the per-launch floor (host submission and the GPU's
// dispatch period between dependent kernels on one stream) that every bsg_run call also pays, the
// launch cost the "Kernel Launch Overhead" glossary page describes.
#include <hip/hip_runtime.h>

#include <chrono>

#include "bsg_bench.h"

namespace bsg {
void set_error(const char* fmt, ...);
}

namespace {
__global__ __launch_bounds__(64) void bsg_null_kernel() {}
}  // namespace

extern "C" bsg_status bsg_bench_null_loop(int n, void* stream, double* wall_us, double* submit_us) {
  if (!wall_us) {
    bsg::set_error("null wall_us");
    return BSG_ERR_NULL;
  }
  if (n < 1) {
    bsg::set_error("need n >= 1");
    return BSG_ERR_SHAPE;
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    bsg::set_error("hipStreamSynchronize: %s", hipGetErrorString(e));
    return BSG_ERR_HIP;
  }
  const auto t0 = std::chrono::steady_clock::now();
  for (int i = 0; i < n; ++i) {
    e = hipLaunchKernel((const void*)&bsg_null_kernel, dim3(1), dim3(64), nullptr, 0, s);
    if (e != hipSuccess) {
      bsg::set_error("hipLaunchKernel: %s", hipGetErrorString(e));
      return BSG_ERR_HIP;
    }
  }
  const auto ts = std::chrono::steady_clock::now();
  e = hipStreamSynchronize(s);
  const auto t1 = std::chrono::steady_clock::now();
  if (e != hipSuccess) {
    bsg::set_error("hipStreamSynchronize: %s", hipGetErrorString(e));
    return BSG_ERR_HIP;
  }
  *wall_us = std::chrono::duration<double, std::micro>(t1 - t0).count();
  if (submit_us) *submit_us = std::chrono::duration<double, std::micro>(ts - t0).count();
  return BSG_OK;
}
