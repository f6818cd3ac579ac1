// sv_verify_sample for callers that cannot allocate device memory (code under
// HIP graph capture, serving loops that must not call hipMalloc, harnesses
// that forbid it): the same kernels, with the workspace taken from a static
// device array of kScratchBytes that each GPU holds for the life of the
// process.  The array's address on each device is looked up once, on the
// first call on that device, with that device current; host code uses only
// that address, never the array's name (which on the host is a stand-in, not a
// device address).
//
// Every call on a device shares that device's array, and each call leaves it
// holding its own words: calls that may overlap on one device (different
// streams, or threads) race and must be serialised by the caller.  A call
// writes every word it later reads (the statistics kernel, or a fill kernel,
// zeroes the words it polls), so what an earlier call left there never
// matters.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.hpp"
#include "launch.hpp"
#include "specverify.h"

namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(8) << 20;  // 8 MiB per device

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call on
// that device.
sv_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return sv::set_error(SV_E_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return sv::set_error(SV_E_DEVICE, "device %d is beyond the %d devices the scratch table covers", dev,
                         kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return sv::set_error(SV_E_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SV_OK;
}

}  // namespace

extern "C" sv_status sv_verify_sample_noalloc(const void* target_logits, int32_t t_dtype, int32_t t_rows,
                                              const void* draft_probs, int32_t q_dtype, int32_t q_rows,
                                              int64_t vocab, const int32_t* t_row_start,
                                              const int32_t* q_row_start, const int32_t* draft_ids,
                                              const int32_t* draft_len, int32_t batch, int32_t k_max,
                                              float temperature, const float* uniforms,
                                              const int32_t* max_new, int32_t eos_id, int32_t* out_tokens,
                                              int32_t* out_count, int32_t* out_accepted, float* out_diag,
                                              float* out_resid, int32_t* dev_status, void* stream) {
  // sizes the scratch cannot hold are rejected before any device call
  if (batch > 0 && t_rows >= 0 && vocab >= 1 && vocab <= sv::kMaxSampleVocab && k_max >= 0 &&
      k_max < sv::kMaxChainRows) {
    const size_t need = sv::sample_need(batch, t_rows, vocab, k_max);
    if (need > kScratchBytes)
      return sv::set_error(SV_E_WORKSPACE,
                           "sv_verify_sample_noalloc: this call needs %zu bytes of scratch; the static scratch "
                           "holds %zu (call sv_verify_sample with a workspace instead)",
                           need, kScratchBytes);
  }
  void* ws = nullptr;
  if (batch > 0)
    if (const sv_status s = scratch_address(&ws)) return s;
  return sv::verify_sample_on(target_logits, t_dtype, t_rows, draft_probs, q_dtype, q_rows, vocab, t_row_start,
                              q_row_start, draft_ids, draft_len, batch, k_max, temperature, uniforms, max_new,
                              eos_id, out_tokens, out_count, out_accepted, out_diag, out_resid, dev_status, ws,
                              kScratchBytes, stream, "sv_verify_sample_noalloc");
}
