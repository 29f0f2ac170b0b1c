// Native call loop over bsg_run, direct or replayed from HIP graphs, timed with steady_clock.
// It uses only the public entry point bsg_run, so it measures exactly what a C/C++ caller pays.
#include <hip/hip_runtime.h>

#include <chrono>
#include <vector>

#include "bsg_bench.h"

namespace bsg {
void set_error(const char* fmt, ...);
}

namespace {

bsg_status hip_fail(const char* what, hipError_t e) {
  bsg::set_error("%s: %s", what, hipGetErrorString(e));
  return BSG_ERR_HIP;
}

}  // namespace

extern "C" bsg_status bsg_bench_loop(bsg_plan plan, int n_sets, const void* const* A, const void* const* B,
                                     const void* const* sA, const void* const* sB, const float* const* bias,
                                     const float* alpha, void* const* D, int calls_per_set, int mode, void* stream,
                                     double* wall_us, double* submit_us) {
  if (!plan || !A || !B || !sA || !sB || !alpha || !D || !wall_us) {
    bsg::set_error("null argument");
    return BSG_ERR_NULL;
  }
  if (n_sets < 1 || calls_per_set < 1 || (mode != 0 && mode != 1)) {
    bsg::set_error("need n_sets >= 1, calls_per_set >= 1, mode 0 or 1");
    return BSG_ERR_SHAPE;
  }
  hipStream_t s = (hipStream_t)stream;
  const float* no_bias = nullptr;
  auto bias_of = [&](int i) { return bias ? bias[i] : no_bias; };
  hipError_t e;

  if (mode == 0) {
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail("hipStreamSynchronize", e);
    const auto t0 = std::chrono::steady_clock::now();
    for (int i = 0; i < n_sets; ++i)
      for (int c = 0; c < calls_per_set; ++c) {
        const bsg_status st = bsg_run(plan, A[i], B[i], sA[i], sB[i], bias_of(i), alpha[i], D[i], stream);
        if (st != BSG_OK) return st;
      }
    const auto ts = std::chrono::steady_clock::now();
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail("hipStreamSynchronize", e);
    const auto t1 = std::chrono::steady_clock::now();
    *wall_us = std::chrono::duration<double, std::micro>(t1 - t0).count();
    if (submit_us) *submit_us = std::chrono::duration<double, std::micro>(ts - t0).count();
    return BSG_OK;
  }

  if (!stream) {
    bsg::set_error("graph mode needs a non-null stream");
    return BSG_ERR_NULL;
  }
  std::vector<hipGraphExec_t> execs(n_sets, nullptr);
  bsg_status result = BSG_OK;
  for (int i = 0; i < n_sets && result == BSG_OK; ++i) {
    hipGraph_t g = nullptr;
    if ((e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal)) != hipSuccess) {
      result = hip_fail("hipStreamBeginCapture", e);
      break;
    }
    bsg_status st = BSG_OK;
    for (int c = 0; c < calls_per_set && st == BSG_OK; ++c)
      st = bsg_run(plan, A[i], B[i], sA[i], sB[i], bias_of(i), alpha[i], D[i], stream);
    e = hipStreamEndCapture(s, &g);
    if (st != BSG_OK) {
      result = st;
    } else if (e != hipSuccess) {
      result = hip_fail("hipStreamEndCapture", e);
    } else if ((e = hipGraphInstantiate(&execs[i], g, nullptr, nullptr, 0)) != hipSuccess) {
      result = hip_fail("hipGraphInstantiate", e);
    }
    if (g) hipGraphDestroy(g);
  }
  if (result == BSG_OK) {
    // one untimed replay of each graph (first-launch upload), then the timed loop
    for (int i = 0; i < n_sets && result == BSG_OK; ++i)
      if ((e = hipGraphLaunch(execs[i], s)) != hipSuccess) result = hip_fail("hipGraphLaunch", e);
    if (result == BSG_OK && (e = hipStreamSynchronize(s)) != hipSuccess) result = hip_fail("hipStreamSynchronize", e);
  }
  if (result == BSG_OK) {
    const auto t0 = std::chrono::steady_clock::now();
    for (int i = 0; i < n_sets && result == BSG_OK; ++i)
      if ((e = hipGraphLaunch(execs[i], s)) != hipSuccess) result = hip_fail("hipGraphLaunch", e);
    const auto ts = std::chrono::steady_clock::now();
    if ((e = hipStreamSynchronize(s)) != hipSuccess && result == BSG_OK) result = hip_fail("hipStreamSynchronize", e);
    const auto t1 = std::chrono::steady_clock::now();
    *wall_us = std::chrono::duration<double, std::micro>(t1 - t0).count();
    if (submit_us) *submit_us = std::chrono::duration<double, std::micro>(ts - t0).count();
  }
  for (hipGraphExec_t x : execs)
    if (x) hipGraphExecDestroy(x);
  return result;
}
