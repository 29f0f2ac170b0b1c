/* Drives the C ABI's host-side paths that need no GPU -- validation of every bsg_problem field,
 * the ABI-1 / ABI-2 struct sizes, status strings, the last-error text, invalid plan handles and the
 * forced-architecture refusal -- so that an AddressSanitizer / UndefinedBehaviorSanitizer build of
 * the plan code can check them.  Exits non-zero on the first unexpected status. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bsg.h"

static int failures = 0;

static void expect(const char* what, bsg_status got, bsg_status want) {
  const char* msg = bsg_last_error();
  if (got != want) {
    printf("FAIL %s: got %s want %s (%s)\n", what, bsg_status_string(got), bsg_status_string(want), msg);
    ++failures;
  } else if (!msg || strlen(msg) >= 512) {
    printf("FAIL %s: bad last-error text\n", what);
    ++failures;
  }
}

static bsg_problem base(void) {
  bsg_problem p;
  memset(&p, 0, sizeof(p));
  p.struct_size = sizeof(p);
  p.format = BSG_FMT_MXFP8;
  p.out_dtype = BSG_OUT_BF16;
  p.M = 256;
  p.N = 256;
  p.K = 256;
  p.device = -1;
  return p;
}

static bsg_status create(bsg_problem p) {
  bsg_plan plan = (bsg_plan)0x1;
  bsg_status st = bsg_plan_create(&p, &plan);
  if (plan != NULL) {
    printf("FAIL plan handle not cleared on error\n");
    ++failures;
  }
  return st;
}

int main(void) {
  bsg_problem p;
  int code;
  if (bsg_abi_version() < 3) { printf("FAIL abi version\n"); return 1; }
  for (code = -1; code <= 12; ++code) {
    const char* s = bsg_status_string((bsg_status)code);
    if (!s || !*s) { printf("FAIL status string %d\n", code); ++failures; }
  }
  expect("null problem", bsg_plan_create(NULL, NULL), BSG_ERR_NULL);
  p = base(); p.struct_size = 8;            expect("struct_size", create(p), BSG_ERR_ABI);
  p = base(); p.format = (bsg_format)3;     expect("format", create(p), BSG_ERR_ABI);
  p = base(); p.out_dtype = (bsg_out_dtype)0; expect("out dtype", create(p), BSG_ERR_ABI);
  p = base(); p.flags = 1u << 10;           expect("flags", create(p), BSG_ERR_ABI);
  p = base(); p.M = 0;                      expect("M", create(p), BSG_ERR_SHAPE);
  p = base(); p.N = 250;                    expect("N % 16", create(p), BSG_ERR_SHAPE);
  p = base(); p.K = 48;                     expect("K % 32", create(p), BSG_ERR_SHAPE);
  p = base(); p.M = (int64_t)1 << 40;       expect("huge M", create(p), BSG_ERR_SHAPE);
  p = base(); p.format = BSG_FMT_NVFP4; p.K = 40; expect("nvfp4 K % 16", create(p), BSG_ERR_SHAPE);
  p = base(); p.format = BSG_FMT_NVFP4; p.K = 48; expect("nvfp4 K % 32 == 16", create(p), BSG_ERR_UNSUPPORTED);
  p = base(); p.batch = -1;                 expect("batch", create(p), BSG_ERR_SHAPE);
  p = base(); p.batch = 2; p.stride_a = 8;  expect("stride_a", create(p), BSG_ERR_ALIGN);
  p = base(); p.batch = 2; p.stride_bias = 6; expect("stride_bias", create(p), BSG_ERR_ALIGN);
  p = base(); p.lda = 128;                  expect("lda", create(p), BSG_ERR_SHAPE);
  p = base(); p.ldd = 260;                  expect("ldd", create(p), BSG_ERR_ALIGN);
  /* ABI-1 / ABI-2 sizes: the fields past them are not read; a valid problem then fails at the
   * forced architecture (set by the caller), before any device query */
  p = base(); p.struct_size = BSG_PROBLEM_V1_SIZE; p.batch = 7; expect("abi1", create(p), BSG_ERR_DEVICE);
  p = base(); p.struct_size = BSG_PROBLEM_V2_SIZE; p.lda = 8; expect("abi2", create(p), BSG_ERR_DEVICE);
  p = base(); p.flags = BSG_EPI_BIAS | BSG_EPI_SILU | BSG_SCALES_KTILE; expect("valid", create(p), BSG_ERR_DEVICE);
  if (!strstr(bsg_last_error(), "BSG_FORCE_ARCH")) { printf("FAIL forced-arch message\n"); ++failures; }
  /* invalid handles: null, and a zeroed block that is not a plan */
  {
    static unsigned char fake[4096];
    bsg_plan_info info;
    memset(&info, 0, sizeof(info));
    info.struct_size = sizeof(info);
    expect("run null plan", bsg_run(NULL, fake, fake, fake, fake, NULL, 1.0f, fake, NULL), BSG_ERR_NULL);
    expect("run fake plan", bsg_run((bsg_plan)fake, fake, fake, fake, fake, NULL, 1.0f, fake, NULL), BSG_ERR_NULL);
    expect("alpha_ptr null", bsg_run_alpha_ptr((bsg_plan)fake, fake, fake, fake, fake, NULL, NULL, fake, NULL),
           BSG_ERR_NULL);
    expect("query null", bsg_plan_query(NULL, &info), BSG_ERR_NULL);
    expect("query fake", bsg_plan_query((bsg_plan)fake, &info), BSG_ERR_NULL);
    expect("destroy null", bsg_plan_destroy(NULL), BSG_OK);
    expect("destroy fake", bsg_plan_destroy((bsg_plan)fake), BSG_ERR_NULL);
  }
  printf("%s: %d failures\n", failures ? "FAIL" : "ok", failures);
  return failures != 0;
}
