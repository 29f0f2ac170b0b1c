// C ABI of the block-scaled GEMM: plan creation (all per-problem host work, once) and the
// per-call run entry point (O(1) checks + one kernel launch).
//
// The CUTLASS issue #3003 page measures a 91 us kernel inside a 625 us loop iteration, the rest
// being host work redone on every call by runNvfp4Gemm (argument construction, workspace
// allocation, can_implement, initialize with tensor-map encoding).  Here that work is split:
// bsg_plan_create does validation (the rules of validateInputsMxFp8ScaledMm on the nvFuser PR #5736
// page: K and N multiples of 16, matching K) plus variant choice and launch-shape computation;
// bsg_run only patches pointers into a copy of the prebuilt argument block and launches.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stddef.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>

#include "bsg.h"
#include "common.h"
#include "plan.h"

namespace bsg {

namespace {
thread_local char g_last_error[512] = "";
constexpr uint32_t kPlanMagic = 0x42534731u;  // "BSG1"
}  // namespace

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

}  // namespace bsg

namespace {

using bsg::set_error;

// Environment switches, read at plan creation only (never on the per-call path):
//   BSG_LOG=1              one line per plan on stderr (problem, variant, grid, split factor, workspace);
//   BSG_LOG=2              also one line per run of such a plan;
//   BSG_FORCE_ARCH=<name>  the architecture check sees <name> instead of the device's own: any name
//                          but gfx950 makes plan creation fail with BSG_ERR_DEVICE (a way to exercise
//                          that path without other hardware); gfx950 leaves the real check in place.
int env_log_level() {
  const char* s = getenv("BSG_LOG");
  return s ? atoi(s) : 0;
}

// Per-device result of the architecture check, computed once.
std::mutex g_dev_mutex;
signed char g_dev_ok[64];  // 0 unknown, 1 gfx950, -1 not
int g_dev_cus[64];         // compute units of a checked device
int g_dev_l2[64];          // L2 bytes of one XCD of a checked device

// BSG_FORCE_ARCH naming another architecture: refuse before any device query.
bsg_status check_forced_arch() {
  const char* forced = getenv("BSG_FORCE_ARCH");
  if (forced && *forced && strncmp(forced, "gfx950", 6) != 0) {
    set_error("BSG_FORCE_ARCH=%s: this library is built for gfx950 (MI355X) only", forced);
    return BSG_ERR_DEVICE;
  }
  return BSG_OK;
}

bsg_status check_device(int dev) {
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count <= 0) {
    set_error("no HIP device available (%s)", e == hipSuccess ? "count 0" : hipGetErrorString(e));
    return BSG_ERR_DEVICE;
  }
  if (dev < 0 || dev >= count || dev >= 64) {
    set_error("device ordinal %d out of range (%d devices)", dev, count);
    return BSG_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      set_error("hipGetDeviceProperties(%d): %s", dev, hipGetErrorString(e));
      return BSG_ERR_HIP;
    }
    g_dev_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_dev_cus[dev] = prop.multiProcessorCount;
    g_dev_l2[dev] = prop.l2CacheSize;
    if (g_dev_ok[dev] < 0) {
      set_error("device %d is %s; this library is built for gfx950 (MI355X) only", dev, prop.gcnArchName);
      return BSG_ERR_DEVICE;
    }
  }
  if (g_dev_ok[dev] < 0) {
    set_error("device %d is not gfx950", dev);
    return BSG_ERR_DEVICE;
  }
  return BSG_OK;
}

// Split-K factor for a kernel that supports it.  Candidates run from 1 to the largest factor that
// keeps the grid within one workgroup per compute unit (ceil(cus / tiles)), at least 4 K tiles per
// split and the kernel's maximum; the choice minimises the kernel's cost model
//   ktile_us * ceil(k_tiles / S) + (S > 1 ? split_fixed_us + partial_us_per_mib * S * plane_mib : 0),
// plane_mib = the fp32 partials of one split (batch x M x N x 4 bytes) in MiB.  A shorter loop per
// workgroup pays for itself only while it outweighs the partial traffic and the second launch.
int choose_splits(const bsg::KernelVariant& v, int64_t tiles, int64_t K, double plane_bytes, int cus) {
  if (v.max_splits <= 1 || tiles >= cus) return 1;
  const int64_t k_tiles = (K + v.tile_k - 1) / v.tile_k;
  int64_t s_max = (cus + tiles - 1) / tiles;
  if (s_max > k_tiles / 4) s_max = k_tiles / 4;
  if (s_max > v.max_splits) s_max = v.max_splits;
  const double plane_mib = plane_bytes / (1024.0 * 1024.0);
  int best = 1;
  double best_us = v.ktile_us * (double)k_tiles;
  for (int64_t s = 2; s <= s_max; ++s) {
    const double us = v.ktile_us * (double)((k_tiles + s - 1) / s) + v.split_fixed_us +
                      v.partial_us_per_mib * (double)s * plane_mib;
    if (us < best_us) best_us = us, best = (int)s;
  }
  return best;
}

// hipMalloc / hipFree on `dev`, restoring the caller's current device.
bsg_status device_alloc(int dev, size_t bytes, void** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) cur = -1;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) {
    set_error("hipSetDevice(%d) failed", dev);
    return BSG_ERR_HIP;
  }
  const hipError_t e = hipMalloc(out, bytes);
  if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess) {
    *out = nullptr;
    set_error("hipMalloc(%zu) of the split-K workspace failed: %s", bytes, hipGetErrorString(e));
    return BSG_ERR_HIP;
  }
  return BSG_OK;
}

void device_free(int dev, void* p) {
  if (!p) return;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) cur = -1;
  if (cur != dev) (void)hipSetDevice(dev);
  (void)hipFree(p);
  if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
}

static_assert(offsetof(bsg_problem, batch) == 44 && offsetof(bsg_problem, stride_a) == BSG_PROBLEM_V1_SIZE,
              "the batch fields extend the ABI-1 layout (batch sits in its tail padding)");
static_assert(offsetof(bsg_problem, lda) == BSG_PROBLEM_V2_SIZE && sizeof(bsg_problem) == BSG_PROBLEM_V2_SIZE + 24,
              "the leading dimensions extend the ABI-2 layout");

// Copy the caller's problem into `out`, reading only the bytes its struct_size covers: an ABI-1
// problem (no batch fields) becomes a single problem; ABI-1 and ABI-2 problems are packed (no
// leading dimensions).
bsg_status normalize(const bsg_problem* in, bsg_problem* out) {
  memset(out, 0, sizeof(*out));
  if (in->struct_size == sizeof(bsg_problem)) {
    *out = *in;
  } else if (in->struct_size == BSG_PROBLEM_V2_SIZE) {
    memcpy(out, in, BSG_PROBLEM_V2_SIZE);
  } else if (in->struct_size == BSG_PROBLEM_V1_SIZE) {
    memcpy(out, in, offsetof(bsg_problem, batch));
  } else {
    set_error("bsg_problem.struct_size is %u, expected %zu (or %u / %u for ABI 1 / 2)", in->struct_size,
              sizeof(bsg_problem), BSG_PROBLEM_V1_SIZE, BSG_PROBLEM_V2_SIZE);
    return BSG_ERR_ABI;
  }
  out->struct_size = sizeof(bsg_problem);
  if (out->batch == 0) out->batch = 1;
  if (out->batch == 1) out->stride_a = out->stride_b = out->stride_sa = out->stride_sb = out->stride_bias =
      out->stride_d = 0;
  if (out->lda == 0) out->lda = out->K;
  if (out->ldb == 0) out->ldb = out->K;
  if (out->ldd == 0) out->ldd = out->N;
  return BSG_OK;
}

bsg_status validate(const bsg_problem* p) {
  if (p->format != BSG_FMT_MXFP8 && p->format != BSG_FMT_NVFP4) {
    set_error("unknown format %d", p->format);
    return BSG_ERR_ABI;
  }
  if (p->out_dtype != BSG_OUT_BF16 && p->out_dtype != BSG_OUT_F16) {
    set_error("unsupported output dtype %d (BF16 or F16 only)", p->out_dtype);
    return BSG_ERR_ABI;
  }
  if (p->flags & ~(uint32_t)(BSG_EPI_BIAS | BSG_EPI_SILU | BSG_SCALES_KTILE)) {
    set_error("unknown flag bits 0x%x", p->flags);
    return BSG_ERR_ABI;
  }
  const int64_t lim = (int64_t)1 << 30;
  if (p->M < 1 || p->N < 1 || p->K < 1 || p->M > lim || p->N > lim || p->K > lim) {
    set_error("M, N, K must be in [1, 2^30] (got %lld, %lld, %lld)", (long long)p->M, (long long)p->N,
              (long long)p->K);
    return BSG_ERR_SHAPE;
  }
  if (p->N % 16 != 0) {
    set_error("N must be a multiple of 16 (got %lld)", (long long)p->N);
    return BSG_ERR_SHAPE;
  }
  const int blk = p->format == BSG_FMT_MXFP8 ? 32 : 16;
  if (p->K % blk != 0) {
    set_error("K must be a multiple of the scale block %d (got %lld)", blk, (long long)p->K);
    return BSG_ERR_SHAPE;
  }
  if (p->K % 32 != 0) {
    set_error("NVFP4 K %% 32 == 16 is not covered by a compiled kernel (K = %lld): packed rows would be only 8-byte "
              "aligned; pad K to a multiple of 32 with zero elements", (long long)p->K);
    return BSG_ERR_UNSUPPORTED;
  }
  if (p->lda < p->K || p->ldb < p->K || p->ldd < p->N || p->lda > lim || p->ldb > lim || p->ldd > lim) {
    set_error("leading dimensions must be in [K, 2^30] for A and B and [N, 2^30] for D (got %lld, %lld, %lld)",
              (long long)p->lda, (long long)p->ldb, (long long)p->ldd);
    return BSG_ERR_SHAPE;
  }
  const int64_t ld_mult = p->format == BSG_FMT_MXFP8 ? 16 : 32;  // 16-byte rows
  if (p->lda % ld_mult || p->ldb % ld_mult || p->ldd % 8) {
    set_error("leading dimensions must keep rows 16-byte aligned: lda, ldb multiples of %lld, ldd of 8",
              (long long)ld_mult);
    return BSG_ERR_ALIGN;
  }
  // element offsets (rows times pitch) must fit the kernels' 32-bit tile arithmetic
  if ((p->M * p->lda) >> 31 || (p->N * p->ldb) >> 31 || (p->M * p->ldd) >> 31) {
    set_error("operand or output spans >= 2^31 elements; not covered");
    return BSG_ERR_UNSUPPORTED;
  }
  if (p->batch < 1 || p->batch > 65535) {
    set_error("batch must be in [1, 65535] (got %d)", p->batch);
    return p->batch < 1 ? BSG_ERR_SHAPE : BSG_ERR_UNSUPPORTED;
  }
  if (p->stride_a < 0 || p->stride_b < 0 || p->stride_sa < 0 || p->stride_sb < 0 || p->stride_bias < 0 ||
      p->stride_d < 0) {
    set_error("batch strides must be >= 0");
    return BSG_ERR_SHAPE;
  }
  if (((p->stride_a | p->stride_b | p->stride_d) & 15) || ((p->stride_sa | p->stride_sb | p->stride_bias) & 3)) {
    set_error("batch strides of A, B and D must be multiples of 16 bytes, of sA, sB and bias of 4");
    return BSG_ERR_ALIGN;
  }
  return BSG_OK;
}

}  // namespace

extern "C" {

int bsg_abi_version(void) { return BSG_ABI_VERSION; }

const char* bsg_last_error(void) { return bsg::g_last_error; }

const char* bsg_status_string(bsg_status s) {
  switch (s) {
    case BSG_OK: return "BSG_OK";
    case BSG_ERR_NULL: return "BSG_ERR_NULL";
    case BSG_ERR_SHAPE: return "BSG_ERR_SHAPE";
    case BSG_ERR_UNSUPPORTED: return "BSG_ERR_UNSUPPORTED";
    case BSG_ERR_ALIGN: return "BSG_ERR_ALIGN";
    case BSG_ERR_DEVICE: return "BSG_ERR_DEVICE";
    case BSG_ERR_HIP: return "BSG_ERR_HIP";
    case BSG_ERR_ALLOC: return "BSG_ERR_ALLOC";
    case BSG_ERR_ABI: return "BSG_ERR_ABI";
    default: break;
  }
  return "BSG_ERR_UNKNOWN";
}

}  // extern "C"

namespace bsg {

// Everything bsg_plan_create does except allocating: validation, variant choice, launch shape and the
// argument template, written into *plan (caller-owned storage).  The split-K workspace size is
// plan->workspace_bytes; plan->args.ws is left null for the caller to point at a workspace.
bsg_status build_plan(const bsg_problem* problem, bsg_plan_s* plan) {
  if (!problem || !plan) {
    set_error("null problem or plan");
    return BSG_ERR_NULL;
  }
  bsg_problem prob;
  bsg_status st = normalize(problem, &prob);
  if (st != BSG_OK) return st;
  problem = &prob;
  st = validate(problem);
  if (st != BSG_OK) return st;
  st = check_forced_arch();
  if (st != BSG_OK) return st;
  int dev = problem->device;
  if (dev < 0) {
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
      set_error("no current HIP device: %s", hipGetErrorString(e));
      return BSG_ERR_DEVICE;
    }
  }
  st = check_device(dev);
  if (st != BSG_OK) return st;

  const bool bias = problem->flags & BSG_EPI_BIAS, silu = problem->flags & BSG_EPI_SILU;
  const bsg::Out out = problem->out_dtype == BSG_OUT_F16 ? bsg::Out::F16 : bsg::Out::BF16;
  const bsg::KernelVariant* table = problem->format == BSG_FMT_MXFP8
                                        ? bsg::mxfp8_variants(problem->M, problem->N, problem->K, problem->batch,
                                                              problem->lda == problem->K && problem->ldb == problem->K)
                                        : bsg::nvfp4_variants(problem->M, problem->N, problem->K, problem->batch);
  if (!table) {
    set_error("no kernel variant covers M=%lld N=%lld K=%lld", (long long)problem->M, (long long)problem->N,
              (long long)problem->K);
    return BSG_ERR_UNSUPPORTED;
  }
  const bsg::KernelVariant& v = table[bsg::variant_index(out, bias, silu)];

  memset((void*)plan, 0, sizeof(*plan));
  plan->magic = bsg::kPlanMagic;
  plan->problem = *problem;
  plan->problem.device = dev;
  plan->device = dev;
  plan->needs_bias = bias;
  plan->launch = v.launch;
  plan->tile_m = v.tile_m;
  plan->tile_n = v.tile_n;
  plan->tile_k = v.tile_k;
  plan->lds_bytes = v.lds_bytes;
  snprintf(plan->variant, sizeof(plan->variant), "%s_%s%s%s", v.name, out == bsg::Out::F16 ? "f16" : "bf16",
           bias ? "_bias" : "", silu ? "_silu" : "");
  bsg::GemmArgs& a = plan->args;
  a.M = (int)problem->M;
  a.N = (int)problem->N;
  a.K = (int)problem->K;
  a.tiles_m = (int)((problem->M + v.tile_m - 1) / v.tile_m);
  a.tiles_n = (int)((problem->N + v.tile_n - 1) / v.tile_n);
  a.scale_ktile = (problem->flags & BSG_SCALES_KTILE) ? 1 : 0;
  a.splits = choose_splits(v, (int64_t)a.tiles_m * a.tiles_n * problem->batch, problem->K,
                           4.0 * (double)problem->batch * (double)problem->M * (double)problem->N, g_dev_cus[dev]);
  a.stride_a = problem->stride_a;
  a.stride_b = problem->stride_b;
  a.stride_sa = problem->stride_sa;
  a.stride_sb = problem->stride_sb;
  a.stride_bias = problem->stride_bias;
  a.stride_d = problem->stride_d;
  const int64_t elem_den = problem->format == BSG_FMT_MXFP8 ? 1 : 2;  // elements per byte
  a.row_a = (int)(problem->lda / elem_den);
  a.row_b = (int)(problem->ldb / elem_den);
  a.ldd = (int)problem->ldd;
  if (a.splits > 1)
    plan->workspace_bytes =
        (uint64_t)problem->batch * a.splits * (uint64_t)problem->M * (uint64_t)problem->N * sizeof(float);
  // NVFP4 partials of at least one L2 per XCD (8 XCDs) are stored through the L2 (splitk.h,
  // store_partials); the MXFP8 tiled kernel always streams its partials.
  a.ws_through = problem->format == BSG_FMT_NVFP4 && a.splits > 1 && g_dev_l2[dev] > 0 &&
                 plan->workspace_bytes >= 8ull * (uint64_t)g_dev_l2[dev];
  plan->grid = v.linear_grid ? dim3((unsigned)(a.tiles_m * a.tiles_n * a.splits), 1, (unsigned)problem->batch)
                             : dim3((unsigned)a.tiles_n, (unsigned)a.tiles_m, (unsigned)problem->batch);
  plan->block = dim3((unsigned)v.block_threads, 1, 1);
  // A persistent kernel takes at most one workgroup per CU; a multiple of 8 keeps each workgroup's
  // tiles on one XCD (workgroups go to the XCDs round-robin).
  if (v.persistent && g_dev_cus[dev] > 0 && g_dev_cus[dev] % 8 == 0 && plan->grid.x > (unsigned)g_dev_cus[dev])
    plan->grid.x = (unsigned)g_dev_cus[dev];
  plan->log_level = env_log_level();
  if (plan->log_level >= 1)
    fprintf(stderr,
            "bsg: plan %s M=%lld N=%lld K=%lld batch=%lld -> %s tile %dx%dx%d grid (%u,%u,%u) block %u splits %d%s "
            "workspace %llu B on device %d\n",
            problem->format == BSG_FMT_MXFP8 ? "mxfp8" : "nvfp4", (long long)problem->M, (long long)problem->N,
            (long long)problem->K, (long long)problem->batch, plan->variant, plan->tile_m, plan->tile_n,
            plan->tile_k, plan->grid.x, plan->grid.y, plan->grid.z, plan->block.x, a.splits,
            a.ws_through ? " (partials through L2)" : "", (unsigned long long)plan->workspace_bytes, dev);
  return BSG_OK;
}

bsg_status launch_plan(const bsg_plan_s* plan, const void* A, const void* B, const void* sA, const void* sB,
                       const float* bias, float alpha, const float* alpha_dev, void* D, void* stream) {
  if (!plan || plan->magic != bsg::kPlanMagic) {
    set_error("invalid plan");
    return BSG_ERR_NULL;
  }
  if (!A || !B || !sA || !sB || !D || (plan->needs_bias && !bias)) {
    set_error("null operand pointer (A=%p B=%p sA=%p sB=%p D=%p bias=%p)", A, B, sA, sB, D, (const void*)bias);
    return BSG_ERR_NULL;
  }
  if (plan->workspace_bytes > 0 && !plan->args.ws) {
    set_error("plan has no split-K workspace");
    return BSG_ERR_NULL;
  }
  const uintptr_t bias_bits = plan->needs_bias ? (uintptr_t)bias : 0;
  if ((((uintptr_t)A | (uintptr_t)B | (uintptr_t)D) & 15u) || (((uintptr_t)sA | (uintptr_t)sB | bias_bits) & 3u)) {
    set_error("A, B and D must be 16-byte aligned and sA, sB, bias 4-byte aligned (A=%p B=%p D=%p sA=%p sB=%p "
              "bias=%p)", A, B, D, sA, sB, (const void*)bias);
    return BSG_ERR_ALIGN;
  }
  bsg::GemmArgs a = plan->args;
  a.A = (const uint8_t*)A;
  a.B = (const uint8_t*)B;
  a.sA = (const uint8_t*)sA;
  a.sB = (const uint8_t*)sB;
  a.bias = plan->needs_bias ? bias : nullptr;
  a.alpha = alpha;
  a.alpha_ptr = alpha_dev;
  a.D = D;
  if (plan->log_level >= 2)
    fprintf(stderr, "bsg: run %s A=%p B=%p sA=%p sB=%p bias=%p alpha=%g alpha_dev=%p D=%p stream=%p\n",
            plan->variant, A, B, sA, sB, (const void*)bias, (double)alpha, (const void*)alpha_dev, D, stream);
  const hipError_t e = plan->launch(a, plan->grid, plan->block, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_error("kernel launch failed: %s", hipGetErrorString(e));
    return BSG_ERR_HIP;
  }
  return BSG_OK;
}

}  // namespace bsg

extern "C" {

bsg_status bsg_plan_create(const bsg_problem* problem, bsg_plan* out_plan) {
  if (!problem || !out_plan) {
    set_error("null problem or out_plan");
    return BSG_ERR_NULL;
  }
  *out_plan = nullptr;
  bsg_plan_s* plan = new (std::nothrow) bsg_plan_s();
  if (!plan) {
    set_error("out of host memory");
    return BSG_ERR_ALLOC;
  }
  bsg_status st = bsg::build_plan(problem, plan);
  if (st == BSG_OK && plan->workspace_bytes > 0) {
    st = device_alloc(plan->device, (size_t)plan->workspace_bytes, &plan->workspace);
    plan->args.ws = (float*)plan->workspace;
  }
  if (st != BSG_OK) {
    delete plan;
    return st;
  }
  *out_plan = plan;
  return BSG_OK;
}

bsg_status bsg_run(bsg_plan plan, const void* A, const void* B, const void* sA, const void* sB, const float* bias,
                   float alpha, void* D, void* stream) {
  return bsg::launch_plan(plan, A, B, sA, sB, bias, alpha, nullptr, D, stream);
}

bsg_status bsg_run_alpha_ptr(bsg_plan plan, const void* A, const void* B, const void* sA, const void* sB,
                             const float* bias, const float* alpha_dev, void* D, void* stream) {
  if (!alpha_dev) {
    set_error("null alpha_dev");
    return BSG_ERR_NULL;
  }
  return bsg::launch_plan(plan, A, B, sA, sB, bias, 0.0f, alpha_dev, D, stream);
}

bsg_status bsg_plan_destroy(bsg_plan plan) {
  if (!plan) return BSG_OK;
  if (plan->magic != bsg::kPlanMagic) {
    set_error("invalid plan");
    return BSG_ERR_NULL;
  }
  plan->magic = 0;
  device_free(plan->device, plan->workspace);  // hipFree waits for work still using it
  delete plan;
  return BSG_OK;
}

bsg_status bsg_plan_query(bsg_plan plan, bsg_plan_info* info) {
  if (!plan || plan->magic != bsg::kPlanMagic || !info) {
    set_error("invalid plan or null info");
    return BSG_ERR_NULL;
  }
  if (info->struct_size != sizeof(bsg_plan_info)) {
    set_error("bsg_plan_info.struct_size is %u, expected %zu", info->struct_size, sizeof(bsg_plan_info));
    return BSG_ERR_ABI;
  }
  memset(info->variant, 0, sizeof(info->variant));
  snprintf(info->variant, sizeof(info->variant), "%s", plan->variant);
  info->tile_m = plan->tile_m;
  info->tile_n = plan->tile_n;
  info->tile_k = plan->tile_k;
  info->grid_x = plan->grid.x;
  info->grid_y = plan->grid.y;
  info->grid_z = plan->grid.z;
  info->block_x = plan->block.x;
  info->lds_bytes = plan->lds_bytes;
  info->workspace_bytes = plan->workspace_bytes;
  return BSG_OK;
}

}  // extern "C"
