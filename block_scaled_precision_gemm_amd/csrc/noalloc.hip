// bsg_run_noalloc: one GEMM call that allocates nothing, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// It builds the plan bsg_plan_create would build, in a stack object, and points its split-K
// workspace at `scratch`, a file-scope device array of kScratchBytes: each GPU the library runs on
// holds its own copy from the module's load until the process ends.  Host code never uses the
// array's name as an address (in host code it is a host-side stand-in): the device address is
// looked up once per device with hipGetSymbolAddress, with that device current, and cached.
//
// Every call on one GPU shares that GPU's array.  The split-K kernels write every partial they read
// back within the same call, so nothing in it has to start at zero, and no clearing is needed; but
// calls that overlap on one GPU (different streams without ordering) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "bsg.h"
#include "plan.h"

namespace {

constexpr size_t kScratchBytes = 32u << 20;  // BSG_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == BSG_NOALLOC_SCRATCH_BYTES, "header and array agree");

static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The device address of `scratch` on `dev`, looked up with `dev` current (the caller's current
// device is restored).
bsg_status scratch_for(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) {
    bsg::set_error("device ordinal %d out of range", dev);
    return BSG_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) cur = -1;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) {
      bsg::set_error("hipSetDevice(%d) failed", dev);
      return BSG_ERR_HIP;
    }
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) {
      bsg::set_error("hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return BSG_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BSG_OK;
}

}  // namespace

extern "C" bsg_status bsg_run_noalloc(const bsg_problem* problem, const void* A, const void* B, const void* sA,
                                      const void* sB, const float* bias, float alpha, void* D, void* stream) {
  bsg_plan_s plan;  // on the stack: no host allocation either
  bsg_status st = bsg::build_plan(problem, &plan);
  if (st != BSG_OK) return st;
  if (plan.workspace_bytes > kScratchBytes) {
    bsg::set_error("this problem's split-K workspace is %llu bytes, above the %zu-byte scratch of "
                   "bsg_run_noalloc; use bsg_plan_create / bsg_run",
                   (unsigned long long)plan.workspace_bytes, kScratchBytes);
    return BSG_ERR_UNSUPPORTED;
  }
  if (plan.workspace_bytes > 0) {
    void* ws = nullptr;
    st = scratch_for(plan.device, &ws);
    if (st != BSG_OK) return st;
    plan.args.ws = (float*)ws;
  }
  return bsg::launch_plan(&plan, A, B, sA, sB, bias, alpha, nullptr, D, stream);
}
