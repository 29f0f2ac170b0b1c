// The plan behind the opaque bsg_plan handle, and the plan steps shared by the entry points
// (bsg_plan_create / bsg_run in api.cpp, bsg_run_noalloc in noalloc.hip).  Library-internal.
#pragma once

#include <hip/hip_runtime.h>

#include "bsg.h"
#include "common.h"

struct bsg_plan_s {
  uint32_t magic;
  bsg_problem problem;
  bsg::GemmArgs args;  // template: shapes and tile counts; pointers patched per call
  bsg::LaunchFn launch;
  dim3 grid, block;
  uint32_t lds_bytes;
  bool needs_bias;
  int device;
  char variant[64];
  int tile_m, tile_n, tile_k;
  void* workspace;          // device memory owned by the plan (split-K partials), or null
  uint64_t workspace_bytes; // bytes of split-K partials the variant needs (0: no split)
  int log_level;            // BSG_LOG at plan creation: 1 logs the plan, 2 also every run
};

namespace bsg {

// Validate `problem`, choose the variant and fill *plan (caller-owned storage); allocates nothing.
// plan->workspace_bytes is the split-K workspace the plan needs; plan->args.ws is left null.
bsg_status build_plan(const bsg_problem* problem, bsg_plan_s* plan);

// The per-call checks (O(1)) and the launch(es) of a built plan on `stream`.
bsg_status launch_plan(const bsg_plan_s* plan, const void* A, const void* B, const void* sA, const void* sB,
                       const float* bias, float alpha, const float* alpha_dev, void* D, void* stream);

void set_error(const char* fmt, ...);

}  // namespace bsg
