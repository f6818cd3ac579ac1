// Internal entry points shared by the library's translation units (not part of
// the C ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

// The thread-local error text behind sv_last_error(); returns `s`.
sv_status set_error(sv_status s, const char* fmt, ...);

// Workspace bytes of a sampled chain call (sv_sample_workspace_bytes without
// its argument checks).
size_t sample_need(int64_t B, int64_t t_rows, int64_t V, int64_t k_max);

// sv_verify_sample with the caller's uniforms on the given workspace; `what`
// names the entry point in error texts.
sv_status verify_sample_on(const void* target_logits, int32_t t_dtype, int32_t t_rows, const void* draft_probs,
                           int32_t q_dtype, int32_t q_rows, int64_t vocab, const int32_t* t_row_start,
                           const int32_t* q_row_start, const int32_t* draft_ids, const int32_t* draft_len,
                           int32_t batch, int32_t k_max, float temperature, const float* uniforms,
                           const int32_t* max_new, int32_t eos_id, int32_t* out_tokens, int32_t* out_count,
                           int32_t* out_accepted, float* out_diag, float* out_resid, int32_t* dev_status,
                           void* workspace, size_t workspace_bytes, void* stream, const char* what);

}  // namespace sv
