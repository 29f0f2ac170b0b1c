/*
 * bsg.h -- block-scaled GEMM for AMD MI355X (gfx950), C ABI.
 *
 * Computes, on one GPU,
 *
 *     D[m][n] = epi( alpha * sum_k a[m][k] * b[n][k] + bias[n] )
 *
 * where a and b are the dequantised operands, epi is SiLU or the identity,
 * accumulation is fp32 and D is written as BF16 or FP16.  This is the
 * operation of the nvFuser PR #5736 page ("Add Cutlass MxFp8 Block Scale
 * Matrix Multiplication": mxfp8_scaled_mm, "compute C = alpha * A @ B",
 * A RowMajor, B ColumnMajor i.e. stored N x K, fp32 accumulator, FP16/BF16
 * output) and of the CUTLASS issue #3003 page (runNvfp4Gemm<T, kEnableSilu,
 * kEnableBias>(output, a, b, scales_a, scales_b, bias, float alpha, M, N, K,
 * stream)).
 *
 * Operand formats (element types as OCP Microscaling v1.0 defines them):
 *   BSG_FMT_MXFP8: A uint8[M][K] E4M3 codes, row-major; B uint8[N][K] E4M3,
 *                  K contiguous; sA uint8[M][K/32], sB uint8[N][K/32] E8M0
 *                  scale codes, one per 32 consecutive K elements, block b
 *                  covering k in [32b, 32b+32).
 *   BSG_FMT_NVFP4: A uint8[M][K/2], B uint8[N][K/2] packed E2M1, element 2t
 *                  in the low nibble of byte t; sA uint8[M][K/16],
 *                  sB uint8[N][K/16] E4M3 scale codes, one per 16 K elements.
 * Scale tensors are plain row-major [rows][K/block] (no padding, no swizzle)
 * by default.  With BSG_SCALES_KTILE they use the library's K-tile-major
 * layout instead (the role of the MXFP8 page's "swizzled" scale layout, which
 * the page names without defining): with KB = K/block codes per row and
 * G = ceil(KB/4) groups of 4 codes, code 4g + c of row r (0 <= c < 4) is byte
 * (g * rows + r) * 4 + c, so one K tile's codes for consecutive rows are
 * contiguous; codes past KB in the last group are padding (never used).  Size
 * G * rows * 4 bytes per operand; bsg_pack_scales converts.
 * bias: float[N] (fp32), broadcast over rows.  D: bf16/fp16 [M][N] row-major.
 * Shapes above are the packed case; with leading dimensions (bsg_problem.lda / ldb / ldd) the rows
 * of A, B and D sit lda, ldb and ldd elements apart instead.
 * All operand pointers are device pointers.
 *
 * Life cycle (the per-call work that the issue #3003 page measures as 534 of
 * 625 us per call -- argument building, workspace allocation, can_implement,
 * descriptor initialisation -- is done once, in bsg_plan_create):
 *   bsg_plan_create(problem)  once: validates, picks the kernel variant,
 *                             precomputes grid and kernel arguments, and
 *                             allocates the plan's device workspace if the
 *                             variant splits K (bsg_plan_info.workspace_bytes).
 *   bsg_run(plan, ...)        per call: O(1) pointer checks and one or two
 *                             kernel launches on the caller's stream (a
 *                             batched plan runs all its problems in them).  No
 *                             allocation, no synchronisation, no device query,
 *                             so it may be captured into a HIP graph.
 *   bsg_plan_destroy(plan)    frees the plan and its workspace.
 *
 * Ownership: the caller owns every operand buffer, D and the stream; the
 * library owns the plan and its workspace.  A plan is immutable after
 * creation.  Concurrent bsg_run calls on one plan are safe when the plan has
 * no workspace; a plan with a workspace (workspace_bytes > 0) keeps its split-K
 * partial sums there, so its calls must be ordered (one stream, or events):
 * overlapping calls on one such plan race.
 *
 * Errors: every function returns a bsg_status and never throws or aborts.
 * On failure nothing is launched and bsg_last_error() (thread-local) holds a
 * message.
 */
#ifndef BSG_H
#define BSG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSG_ABI_VERSION 3

typedef enum bsg_status {
  BSG_OK = 0,
  BSG_ERR_NULL = 1,        /* a required pointer is NULL */
  BSG_ERR_SHAPE = 2,       /* M, N or K out of range or not a multiple the format needs */
  BSG_ERR_UNSUPPORTED = 3, /* valid request that no compiled kernel variant covers */
  BSG_ERR_ALIGN = 4,       /* an operand pointer is not 16-byte aligned */
  BSG_ERR_DEVICE = 5,      /* no device, or the device is not gfx950 */
  BSG_ERR_HIP = 6,         /* a HIP runtime call failed (message holds hipGetErrorString) */
  BSG_ERR_ALLOC = 7,       /* host allocation of the plan failed */
  BSG_ERR_ABI = 8,         /* struct_size mismatch or bad enum value */
  /* Not statuses.  These two give each enum of this header the whole int32 range, so that any int a
   * C caller stores in one (an unknown status code, a bad format) is a value the library may read. */
  BSG_STATUS_RANGE_MIN_ = -2147483647 - 1,
  BSG_STATUS_RANGE_MAX_ = 2147483647
} bsg_status;

typedef enum bsg_format {
  BSG_FMT_MXFP8 = 1, /* E4M3 elements, E8M0 scale per 32 K */
  BSG_FMT_NVFP4 = 2, /* packed E2M1 elements, E4M3 scale per 16 K, global fp32 alpha */
  BSG_FMT_RANGE_MIN_ = -2147483647 - 1,
  BSG_FMT_RANGE_MAX_ = 2147483647
} bsg_format;

typedef enum bsg_out_dtype {
  BSG_OUT_BF16 = 1,
  BSG_OUT_F16 = 2,
  BSG_OUT_RANGE_MIN_ = -2147483647 - 1,
  BSG_OUT_RANGE_MAX_ = 2147483647
} bsg_out_dtype;

/* problem flags: epilogue (kEnableBias / kEnableSilu of runNvfp4Gemm) and scale layout */
enum {
  BSG_EPI_BIAS = 1u << 0,    /* add bias[n] after alpha */
  BSG_EPI_SILU = 1u << 1,    /* y = x / (1 + exp(-x)) on x = alpha*acc (+ bias) */
  BSG_SCALES_KTILE = 1u << 2 /* sA and sB in the K-tile-major layout described above */
};

typedef struct bsg_problem {
  uint32_t struct_size; /* = sizeof(bsg_problem), or the ABI-1 / ABI-2 size below; else BSG_ERR_ABI */
  int32_t format;       /* bsg_format */
  int32_t out_dtype;    /* bsg_out_dtype */
  uint32_t flags;       /* BSG_EPI_*, BSG_SCALES_KTILE */
  int64_t M, N, K;      /* M >= 1; N >= 16, N % 16 == 0; K >= 32, K % 32 == 0 (MXFP8) or K % 16 == 0 (NVFP4).
                         * NVFP4 with K % 32 == 16 is a valid shape that no compiled kernel covers
                         * (BSG_ERR_UNSUPPORTED): a packed row is then K/2 == 8 (mod 16) bytes long, so
                         * rows after the first are only 8-byte aligned, and every kernel moves
                         * operand rows in 16-byte pieces (the 32-element FP4 alignment that the
                         * CUTLASS kernels of the issue #3003 page also require).  Pad K to a multiple
                         * of 32 with zero elements (zero scale codes) to run such a problem. */
  int32_t device;       /* HIP device ordinal; -1 = the current device at create time */
  /* Batched GEMM (ABI 2): `batch` independent problems of the same shape in one launch.  Problem z
   * (0 <= z < batch) reads A + z*stride_a, B + z*stride_b, sA + z*stride_sa, sB + z*stride_sb and
   * bias + z*stride_bias (bytes), and writes D + z*stride_d.  A stride of 0 makes every problem use
   * the same operand (e.g. shared weights B, or one bias vector); strides must be >= 0, multiples
   * of 16 for A, B and D and of 4 for sA, sB and bias, and distinct problems' D must not overlap
   * (not checked).  batch 0 is read as 1; strides are ignored when batch is 1. */
  int32_t batch;
  int64_t stride_a, stride_b, stride_sa, stride_sb, stride_bias, stride_d;
  /* Leading dimensions (ABI 3), in elements; 0 = packed (lda = ldb = K, ldd = N).  Row m of A starts
   * lda elements after row m - 1 (NVFP4: lda / 2 bytes), row n of B ldb elements after row n - 1,
   * row m of D ldd elements after row m - 1; the gaps are never read or written.  Each must be at
   * least its packed value and keep every row 16-byte aligned: lda, ldb multiples of 16 (MXFP8) or
   * 32 (NVFP4), ldd a multiple of 8.  Scales stay packed, in either scale layout.  Leading
   * dimensions apply to every problem of a batch (batch strides are separate).  Strided A or B is
   * served by the tiled kernels (the large-shape MXFP8 kernel takes packed A and B). */
  int64_t lda, ldb, ldd;
} bsg_problem;

/* sizeof(bsg_problem) of ABI 1 (no batch or leading-dimension fields) and of ABI 2 (no leading-
 * dimension fields): still accepted, with the missing fields read as 0. */
#define BSG_PROBLEM_V1_SIZE 48u
#define BSG_PROBLEM_V2_SIZE 96u

typedef struct bsg_plan_s* bsg_plan; /* opaque, library-owned */

typedef struct bsg_plan_info {
  uint32_t struct_size; /* = sizeof(bsg_plan_info), set by the caller */
  char variant[64];     /* kernel variant name */
  int32_t tile_m, tile_n, tile_k;
  uint32_t grid_x, grid_y, grid_z, block_x;
  uint32_t lds_bytes;
  uint64_t workspace_bytes; /* device workspace the plan owns (0: none); grid_x includes the split-K factor,
                               grid_z is the batch count */
} bsg_plan_info;

/* Validate `problem`, choose the kernel variant for (format, out dtype, epilogue, M bucket) and
 * precompute everything a call needs.  On success *out_plan is a new plan.  Errors: BSG_ERR_NULL,
 * BSG_ERR_ABI, BSG_ERR_SHAPE, BSG_ERR_UNSUPPORTED, BSG_ERR_DEVICE, BSG_ERR_HIP, BSG_ERR_ALLOC.
 * Environment, read here (never by bsg_run): BSG_LOG=1 writes one line per plan to stderr (problem,
 * variant, tile, grid, split factor and partial-store form, workspace); BSG_LOG=2 also one line per
 * run of that plan.
 * BSG_FORCE_ARCH=<name> makes the architecture check see <name>: any name but gfx950 fails with
 * BSG_ERR_DEVICE (checked before the device is queried, so it works without a GPU); gfx950 keeps
 * the check of the real device. */
bsg_status bsg_plan_create(const bsg_problem* problem, bsg_plan* out_plan);

/* Enqueue D = epi(alpha * A x B^T (+ bias)) on `stream` (a hipStream_t; NULL = the null stream).
 * A, B, sA, sB, D: device pointers laid out as described at the top of this file; A, B and D must be
 * 16-byte aligned, sA and sB 4-byte aligned.  bias: device float[N], 4-byte aligned, required iff the plan has
 * BSG_EPI_BIAS (ignored otherwise).
 * alpha: host fp32 value.  Returns after enqueueing (asynchronous).  Errors: BSG_ERR_NULL,
 * BSG_ERR_ALIGN, BSG_ERR_HIP (launch failure). */
bsg_status bsg_run(bsg_plan plan, const void* A, const void* B, const void* sA, const void* sB,
                   const float* bias, float alpha, void* D, void* stream);

/* Same as bsg_run, with alpha read by the kernel from device memory (the alpha_ptr form of the
 * MXFP8 page's epilogue arguments).  alpha_dev: device pointer to one fp32. */
bsg_status bsg_run_alpha_ptr(bsg_plan plan, const void* A, const void* B, const void* sA, const void* sB,
                             const float* bias, const float* alpha_dev, void* D, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): one call of the GEMM described by `problem`, with the arguments
 * and results of bsg_plan_create followed by bsg_run, that allocates nothing -- no device memory, no
 * host memory.  The plan is built on the stack on every call (the full validation of
 * bsg_plan_create, so this costs more host time per call than bsg_run on a cached plan).  A problem
 * whose variant splits K keeps its fp32 partials in a library-owned device array of
 * BSG_NOALLOC_SCRATCH_BYTES that each GPU holds from its first use by this library until the process
 * ends; a problem that would need more is refused with BSG_ERR_UNSUPPORTED and nothing is launched
 * (bsg_plan_create / bsg_run serve it).  Every call on a GPU shares that GPU's array: calls that
 * overlap on one GPU (streams not ordered with each other) race on it and must not be issued.  The
 * array's device address is looked up on the first call on each device; make that first call
 * outside graph capture.  Errors: those of bsg_plan_create and bsg_run. */
#define BSG_NOALLOC_SCRATCH_BYTES (32u << 20)
bsg_status bsg_run_noalloc(const bsg_problem* problem, const void* A, const void* B, const void* sA, const void* sB,
                           const float* bias, float alpha, void* D, void* stream);

/* Free a plan.  NULL is accepted.  A plan without workspace is host memory only, and kernels already
 * enqueued with it are unaffected (their arguments were copied at launch).  A plan's workspace is
 * released with hipFree, which waits for the device's outstanding work first. */
bsg_status bsg_plan_destroy(bsg_plan plan);

/* Describe the chosen variant.  info->struct_size must be sizeof(bsg_plan_info). */
bsg_status bsg_plan_query(bsg_plan plan, bsg_plan_info* info);

/* Convert one operand's scale codes from row-major [rows][codes_per_row] (src) to the K-tile-major
 * layout of BSG_SCALES_KTILE (dst, bsg_scales_ktile_bytes(rows, codes_per_row) bytes; padding codes
 * are written as 0), enqueued on `stream` (NULL = the null stream).  src and dst: device pointers to
 * distinct buffers, dst 4-byte aligned.  For a batch of operands, call once per operand or treat
 * them as one operand of batch * rows rows only when each operand's rows are contiguous (the
 * K-tile-major layout interleaves rows per group, so per-operand calls are the general form).
 * Errors: BSG_ERR_NULL, BSG_ERR_SHAPE (rows or codes_per_row < 1, or the result would exceed 2^31
 * bytes), BSG_ERR_ALIGN, BSG_ERR_HIP (launch failure). */
bsg_status bsg_pack_scales(const void* src, void* dst, int64_t rows, int64_t codes_per_row, void* stream);

/* Bytes of one operand's scales in the K-tile-major layout: ceil(codes_per_row / 4) * rows * 4
 * (0 if an argument is < 1). */
int64_t bsg_scales_ktile_bytes(int64_t rows, int64_t codes_per_row);

/* Static text for a status code. */
const char* bsg_status_string(bsg_status s);

/* Message of the last failing call on this thread ("" if none). */
const char* bsg_last_error(void);

/* BSG_ABI_VERSION of the built library. */
int bsg_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSG_H */
