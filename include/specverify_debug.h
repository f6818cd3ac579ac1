/*
 * libspecverify -- measurement hooks.  Not operations of the verify method:
 * these exist so that a benchmark can time one kernel inside a real call.
 * They live apart from specverify.h; a serving caller needs none of them.
 */
#ifndef SPECVERIFY_DEBUG_H
#define SPECVERIFY_DEBUG_H

#include "specverify.h"

#ifdef __cplusplus
extern "C" {
#endif

/* For the calling thread's next call of a verify entry point (or of
 * sv_debug_read_ceiling), hand `before` and `after` (hipEvent_t) to the launch
 * of the kernel that streams the call's rows, so that they take that kernel's
 * own start and end times (the timestamps of its dispatch, as a profiler's
 * kernel trace reports them) on the call's stream:
 *   sv_verify_sample / _philox / _noalloc   the row statistics (the partials
 *                                            of every row, or the lazy
 *                                            statistics); with a one-tile
 *                                            vocabulary, the one-wave round;
 *   sv_verify_greedy                         the row argmax;
 *   sv_verify_tree / _greedy / _pointmass    the walk;
 *   sv_ngram_draft                           the prompt-lookup kernel;
 *   sv_debug_read_ceiling                    the streaming read.
 * The hook then disarms, also when that call fails or has no requests.
 * NULL, NULL disarms it; giving one event only is SV_E_ARG.  The events must
 * stay valid until that call returns.  Host function; the armed events are
 * thread-local state of the library. */
sv_status sv_debug_time_kernel_once(void* before, void* after);

/* A pure streaming read of `bytes` bytes at `buf` (16-byte aligned, bytes a
 * multiple of 16) with the same 16-byte non-temporal loads as the row
 * statistics, each block folding its words into one 32-bit value written to
 * out[block] (out: at least sv_debug_read_blocks(bytes) uint32 values): the
 * practical HBM read ceiling the verify kernels are measured against. */
int64_t sv_debug_read_blocks(int64_t bytes);
sv_status sv_debug_read_ceiling(const void* buf, int64_t bytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_DEBUG_H */
