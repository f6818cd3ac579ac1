// History n-gram (prompt-lookup) drafter.
//
// Method ("第 13 篇：推理引擎一次猜几个字——草稿 + 验证", notes under section ③):
// the context's last `window` tokens are the key; an identical fragment earlier
// in the history is looked up and the tokens that followed it are proposed.
// Readings: the most recent occurrence that is followed by at least one token
// wins (start j <= n - window - 1); the proposal stops at the context end.
//
// One block per request.  The candidate starts are tested newest first in
// chunks of 4096: a chunk's tokens (plus the window's overlap) are staged in
// LDS with coalesced 16-byte loads, all issued at once; every thread tests its
// starts of the chunk from LDS (newest first, stopping at its first match),
// and the block's largest matching start ends the search; a match in the
// newest 4096 starts costs one load round.  A chunk also stages the up to k
// tokens after its newest window, so the proposal of a match comes from LDS
// too.
#include "common.hpp"
#include "launch.hpp"

namespace sv {

constexpr int kNgramChunk = 4096;
constexpr int kMaxNgramDraft = 1024;  // k <= 1024 (checked on the host)
constexpr int kNgramStage = kNgramChunk + kMaxWindow + kMaxNgramDraft;
constexpr int kStageVecs = (kNgramStage / 4 + kBlock - 1) / kBlock;  // 16-byte loads per thread

// dst[0, n) = src[0, n): the 16-byte-aligned middle with every thread's loads
// issued at once (one load round), the unaligned head and tail element-wise.
__device__ __forceinline__ void stage_tokens(int32_t* dst, const int32_t* src, int n) {
  const int mis = static_cast<int>((reinterpret_cast<uintptr_t>(src) >> 2) & 3);
  const int head = min(mis != 0 ? 4 - mis : 0, n);
  const int nv = (n - head) / 4;
  const int4* vs = reinterpret_cast<const int4*>(src + head);
  int4 w[kStageVecs];
#pragma unroll
  for (int u = 0; u < kStageVecs; ++u) {
    const int v = threadIdx.x + u * kBlock;
    if (v < nv) w[u] = vs[v];
  }
  const int tail = head + 4 * nv;
  const int32_t e = threadIdx.x < head ? src[threadIdx.x]
                                       : (threadIdx.x < head + n - tail ? src[tail + threadIdx.x - head] : 0);
#pragma unroll
  for (int u = 0; u < kStageVecs; ++u) {
    const int v = threadIdx.x + u * kBlock;
    if (v < nv) {
      int32_t* d = dst + head + 4 * v;
      d[0] = w[u].x;
      d[1] = w[u].y;
      d[2] = w[u].z;
      d[3] = w[u].w;
    }
  }
  if (threadIdx.x < head) dst[threadIdx.x] = e;
  else if (threadIdx.x < head + n - tail) dst[tail + threadIdx.x - head] = e;
}

__global__ __launch_bounds__(kBlock) void k_ngram(const int32_t* __restrict__ ctx,
                                                  const int32_t* __restrict__ ctx_len, int32_t stride,
                                                  int32_t window, int32_t k, int32_t* __restrict__ ids,
                                                  int32_t* __restrict__ lens, int32_t* status) {
  __shared__ int32_t s_tok[kNgramStage];
  __shared__ int s_lo, s_end;  // tokens [s_lo, s_end) of the last staged chunk
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
  if (tid == 0) {
    s_best = -1;
    s_lo = s_end = 0;
  }
  if (k > 0 && n >= window + 1) {
    for (int i = tid; i < window; i += kBlock) s_key[i] = row[n - window + i];
    // candidate starts j in [lo, hi], newest chunk first (j <= n - window - 1:
    // at least one token follows the match)
    for (int hi = n - window - 1; hi >= 0; hi -= kNgramChunk) {
      const int lo = hi - kNgramChunk + 1 > 0 ? hi - kNgramChunk + 1 : 0;
      // tokens [lo, hi + window + k) within the context: the windows of the
      // chunk's starts and what follows the newest of them
      const int end = hi + window + k < n ? hi + window + k : n;
      stage_tokens(s_tok, row + lo, end - lo);
      if (tid == 0) {
        s_lo = lo;
        s_end = end;
      }
      __syncthreads();
      // this thread's starts hi - tid, hi - tid - 256, ... newest first, four
      // at a time: their first tokens are read together and only a start
      // whose first token matches is compared in full
      const int32_t k0 = s_key[0];
      bool found_here = false;
      for (int j0 = hi - tid; j0 >= lo && !found_here; j0 -= 4 * kBlock) {
        int32_t f[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = j0 - u * kBlock;
          f[u] = j >= lo ? s_tok[j - lo] : ~k0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = j0 - u * kBlock;
          if (found_here || f[u] != k0) continue;
          bool match = true;
          for (int i = 1; i < window && match; ++i) match = s_tok[j - lo + i] == s_key[i];
          if (match) {
            atomicMax(&s_best, j);
            found_here = true;  // this thread's later starts are older
          }
        }
      }
      __syncthreads();
      const int found = s_best;
      __syncthreads();  // every thread has read s_best (and s_tok) before the next chunk
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
  // the proposal: from the staged chunk when it holds it (a match found in
  // the chunk), else from the context
  const int lo = s_lo, end = s_end;
  for (int i = tid; i < k; i += kBlock) {
    const int at = j + window + i;
    out[i] = i < len ? (at >= lo && at < end ? s_tok[at - lo] : row[at]) : -1;
  }
  if (tid == 0) lens[b] = len;
}

hipError_t launch_ngram(const int32_t* ctx, const int32_t* ctx_len, int32_t B, int32_t stride,
                        int32_t window, int32_t k, int32_t* ids, int32_t* lens, int32_t* status,
                        hipStream_t stream) {
  launch_timed(k_ngram, dim3(static_cast<uint32_t>(B)), dim3(kBlock), 0, stream, ctx, ctx_len,
               stride, window, k, ids, lens, status);
  return hipGetLastError();
}

}  // namespace sv
