/*
 * ubep_testing.h -- controls of libubep.so for tests, tuning and timing; not
 * part of the dispatch / combine path declared in ubep.h.  They are the
 * library's only mutable host state besides the allocation-free layout's
 * per-GPU array: a process-wide cap on layout workgroups, and a per-thread
 * pending pair of timing events.  Production callers need neither.
 */
#ifndef UBEP_TESTING_H
#define UBEP_TESTING_H

#include "ubep.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Profiling aid: the next kernel that a ubep_* call launches from this host
 * thread records `start` when it begins and `stop` when it ends.  The events
 * are written by that kernel's own dispatch (hipExtLaunchKernel), so no marker
 * packet sits between kernels; hipEventElapsedTime(start, stop) is then the
 * kernel's duration.  Every entry point of ubep.h launches one kernel,
 * except ubep_layout_dispatch when it falls back to two launches and
 * ubep_layout_noalloc when it clears its array first (the first launch is
 * timed), and ubep_dispatch_combine_chunked with the LPT order (the
 * pipeline kernel is timed, not the order kernel before it).  The pair stays pending until a launch takes it, also across calls
 * that fail validation.  Both null: clear a pending pair; exactly one null:
 * UBEP_ERR_INVALID_ARG.  The events must have been created by the caller. */
ubep_status ubep_time_next_launch(hipEvent_t start, hipEvent_t stop);

/* Process-wide cap on the number of layout workgroups of later ubep_layout /
 * ubep_layout_dispatch calls (n >= 1), or 0 for the default (two per compute
 * unit, at most one per tile).  The layout still launches at least as many
 * workgroups as its per-workgroup tile limit needs, so every result is the
 * same; a small cap makes workgroups take several tiles (a tuning and
 * testing control).  n < 0: UBEP_ERR_INVALID_ARG. */
ubep_status ubep_set_layout_workers(int32_t n);

#ifdef __cplusplus
}
#endif

#endif /* UBEP_TESTING_H */
