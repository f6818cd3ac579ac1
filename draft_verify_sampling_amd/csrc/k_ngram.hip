// History n-gram (prompt-lookup) drafter.
//
// Method ("第 13 篇：推理引擎一次猜几个字——草稿 + 验证", notes under section ③):
// the context's last `window` tokens are the key; an identical fragment earlier
// in the history is looked up and the tokens that followed it are proposed.
// Readings: the most recent occurrence that is followed by at least one token
// wins (start j <= n - window - 1); the proposal stops at the context end.
//
// One block per request.  Threads test candidate starts in rounds of 256,
// newest first; a round that finds a match ends the search (LDS max of the
// matching starts), so a match near the end of a long context costs one round.
#include "common.hpp"
#include "launch.hpp"

namespace sv {

__global__ __launch_bounds__(kBlock) void k_ngram(const int32_t* __restrict__ ctx,
                                                  const int32_t* __restrict__ ctx_len, int32_t stride,
                                                  int32_t window, int32_t k, int32_t* __restrict__ ids,
                                                  int32_t* __restrict__ lens, int32_t* status) {
  __shared__ int32_t s_key[kMaxWindow];
  __shared__ int s_best;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t* row = ctx + static_cast<int64_t>(b) * stride;
  const int n = ctx_len[b];
  int32_t* out = ids + static_cast<int64_t>(b) * k;
  if (n < 0 || n > stride) {
    for (int i = tid; i < k; i += kBlock) out[i] = -1;
    if (tid == 0) {
      lens[b] = 0;
      flag(status, kFlagBadRequest);
    }
    return;
  }
  if (tid == 0) s_best = -1;
  if (k > 0 && n >= window + 1) {
    for (int i = tid; i < window; i += kBlock) s_key[i] = row[n - window + i];
    __syncthreads();
    for (int start = n - window - 1; start >= 0; start -= kBlock) {
      const int j = start - tid;
      if (j >= 0) {
        bool match = true;
        for (int i = 0; i < window && match; ++i) match = row[j + i] == s_key[i];
        if (match) atomicMax(&s_best, j);
      }
      __syncthreads();
      const int found = s_best;
      __syncthreads();  // every thread has read s_best before the next round writes it
      if (found >= 0) break;
    }
  }
  __syncthreads();
  const int j = s_best;
  int len = 0;
  if (j >= 0) {
    len = n - (j + window);
    if (len > k) len = k;
  }
  for (int i = tid; i < k; i += kBlock) out[i] = i < len ? row[j + window + i] : -1;
  if (tid == 0) lens[b] = len;
}

hipError_t launch_ngram(const int32_t* ctx, const int32_t* ctx_len, int32_t B, int32_t stride,
                        int32_t window, int32_t k, int32_t* ids, int32_t* lens, int32_t* status,
                        hipStream_t stream) {
  hipLaunchKernelGGL(k_ngram, dim3(static_cast<uint32_t>(B)), dim3(kBlock), 0, stream, ctx, ctx_len,
                     stride, window, k, ids, lens, status);
  return hipGetLastError();
}

}  // namespace sv
