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

/* For the calling thread's next sv_verify_sample or sv_verify_sample_philox
 * call, record `before` (a hipEvent_t) on that call's stream right before the
 * kernel that streams the target rows and `after` right after it (every such
 * call with batch > 0 launches one: the one-kernel round, the partials of
 * every row, or the lazy statistics), so a caller can time that kernel inside
 * a real call.  The hook then disarms, also when that call fails or has no
 * requests.  NULL, NULL disarms it; giving one event only is SV_E_ARG.  The
 * events must stay valid until that call returns.  Host function; the armed
 * events are thread-local state of the library. */
sv_status sv_debug_time_statistics_once(void* before, void* after);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_DEBUG_H */
