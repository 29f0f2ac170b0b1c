/*
 * bsg_bench.h -- native call loop for measuring per-call host overhead of bsg_run.
 *
 * The CUTLASS issue #3003 page compares a 91 us GEMM kernel with a 625 us loop
 * iteration: per-call host work dominated.  This entry point drives bsg_run from C++
 * (so that no interpreter cost enters the measurement) over several input sets:
 * for set s = 0..n_sets-1, calls_per_set back-to-back calls on `stream`; one
 * hipStreamSynchronize at the end.  The host wall time of the whole loop, from the
 * first enqueue to the end of the final synchronisation, is written to *wall_us.
 *
 * mode 0: direct calls.  mode 1: for each set, the calls_per_set calls are captured
 * once into a HIP graph (outside the timed region) and the loop replays the graphs.
 * Arrays A..D hold n_sets device pointers each (bias may be NULL when the plan has
 * no bias); alpha holds n_sets host floats.  *submit_us (if not NULL) receives the host
 * time spent enqueueing alone (first call to the last call's return, before the
 * synchronisation).  Errors: as bsg_run, plus BSG_ERR_SHAPE for n_sets < 1 or
 * calls_per_set < 1, and BSG_ERR_HIP for capture failures.
 *
 * bsg_bench_null_loop: the same measurement for n launches of an empty kernel (one
 * workgroup of 64 threads) on `stream`: the floor that any per-call kernel launch pays
 * (host submission, and the GPU's back-to-back dispatch period).  *wall_us: first
 * enqueue to the end of the synchronisation; *submit_us (nullable): enqueueing alone.
 * Errors: BSG_ERR_NULL, BSG_ERR_SHAPE (n < 1), BSG_ERR_HIP.
 */
#ifndef BSG_BENCH_H
#define BSG_BENCH_H

#include "bsg.h"

#ifdef __cplusplus
extern "C" {
#endif

bsg_status bsg_bench_loop(bsg_plan plan, int n_sets, const void* const* A, const void* const* B,
                          const void* const* sA, const void* const* sB, const float* const* bias,
                          const float* alpha, void* const* D, int calls_per_set, int mode, void* stream,
                          double* wall_us, double* submit_us);

bsg_status bsg_bench_null_loop(int n, void* stream, double* wall_us, double* submit_us);

#ifdef __cplusplus
}
#endif

#endif /* BSG_BENCH_H */
