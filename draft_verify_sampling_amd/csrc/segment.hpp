// Online-softmax pair of one 8192-element segment of a target row, the unit
// of the statistics stream (the temperature softmax's normaliser of
// "投机解码:为什么一个字都不改", figure "一次目标前向验 k 个草稿 token").  Every
// thread of a 256-thread block issues its 16-byte loads of the segment at once
// (coalesced; non-temporal when NT); segment 0 also takes the row's unaligned
// head elements and the last segment its tail.  Shared by both statistics
// kernels (every row, and the lazy chain statistics), so a row's pair is the
// same bits whichever kernel forms it.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace sv {

// Online-softmax pair of segment `seg` of a row, valid in thread 0.  `sh`
// holds 2 * (kBlock / 64) floats.
template <class D, bool NT>
__device__ __forceinline__ MS segment_ms(const void* base, int64_t V, int32_t seg, int32_t nseg, float c,
                                         float* sh) {
  constexpr int U = kSegElems / (kBlock * D::kPerVec);
  constexpr int kSegVecs = kSegElems / D::kPerVec;
  const int64_t head = head_elems<D>(base, V);
  const int64_t nvec = (V - head) / D::kPerVec;
  const uint4* vp = reinterpret_cast<const uint4*>(static_cast<const char*>(base) + head * D::kSize);

  MS acc{-INFINITY, 0.f};
  {
    const int64_t v0 = static_cast<int64_t>(seg) * kSegVecs + threadIdx.x;
    uint4 w[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t v = v0 + j * kBlock;
      w[j] = uint4{0u, 0u, 0u, 0u};
      if (v < nvec) {
        if (NT) {
          const uint32_t* q = reinterpret_cast<const uint32_t*>(vp + v);
          w[j] = uint4{__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1),
                       __builtin_nontemporal_load(q + 2), __builtin_nontemporal_load(q + 3)};
        } else {
          w[j] = vp[v];
        }
      }
    }
    float x[U * D::kPerVec];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      D::unpack(w[j], x + j * D::kPerVec);
      if (v0 + j * kBlock >= nvec) {
#pragma unroll
        for (int t = 0; t < D::kPerVec; ++t) x[j * D::kPerVec + t] = -INFINITY;
      }
    }
    ms_fold<U * D::kPerVec>(acc, x, c);
  }
  if (seg == 0) {
    for (int64_t i = threadIdx.x; i < head; i += kBlock) {
      float x = D::at(base, i);
      ms_fold<1>(acc, &x, c);
    }
  }
  if (seg == nseg - 1) {
    for (int64_t i = head + nvec * D::kPerVec + threadIdx.x; i < V; i += kBlock) {
      float x = D::at(base, i);
      ms_fold<1>(acc, &x, c);
    }
  }
  // block reduction: DPP within each wave, then the four wave results
  const MS r = wave_ms_dpp(acc);
  const int wid = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sh[2 * wid] = r.m;
    sh[2 * wid + 1] = r.s;
  }
  __syncthreads();
  MS t{sh[0], sh[1]};
  for (int w = 1; w < kBlock / kWave; ++w) t = ms_combine(t, MS{sh[2 * w], sh[2 * w + 1]});
  return t;
}


}  // namespace sv
