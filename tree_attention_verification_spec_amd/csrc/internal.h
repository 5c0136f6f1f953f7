/*
 * Internal entry points of libspectree: exported for the benchmark and the tests, not part of
 * the public C ABI (include/spectree.h).
 */
#pragma once

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel timing.  When enabled, the library launches each kernel through hipExtLaunchKernel
 * with a start/stop HIP event pair that the kernel's own dispatch stamps on the launch stream,
 * so each pair brackets exactly one kernel execution; elapsed times accumulate per kernel name.
 * spec_prof_read() waits for the recorded events.  Timing must be off while a stream is being
 * captured into a graph.  It changes nothing in what the kernels compute. */
void spec_prof_enable(int on);
void spec_prof_reset(void);
/* Total milliseconds and launch count recorded for kernel `name` since the last reset.
 * Returns 0 on success, -1 if the name was never launched while enabled. */
int spec_prof_read(const char* name, double* total_ms, int64_t* launches);

/* Forces a launch-shape choice for the calls that follow (tests cover every shape the library
 * can pick).  `name` is one of "attn_cb" (1, 2), "attn_waves" (4, 8),
 * "attn_splits" (>= 1), "attn_lpt" (0, 1), "attn_prio" (0, 1), "attn_lazy" (0: move the softmax
 * reference max with every new row maximum; > 0: only when it grows by more than that many
 * log2 units), "verify_chunk" (4096, 8192,
 * 16384), "verify_store_w" (0, 1), "verify_rows_list" (0, 1), "res_rowblocks" (1, 2, 4),
 * "lm_rowblocks" (4, 8), "walk_parts" (1-16 workgroups per node of the
 * WALK chain), "walk_spin" (>= 1 polls of a node's counter before a workgroup of a split chain
 * stops waiting; a small value exercises the path on which workgroup 0 finishes alone); a
 * negative value removes the override.  Workspace queries made while
 * an override is set size the workspace for the forced shape.  Returns 0, or -1 for an unknown
 * name.  Not thread-safe with respect to calls in flight on other host threads. */
int spec_internal_tune(const char* name, int value);

#ifdef __cplusplus
}
#endif
