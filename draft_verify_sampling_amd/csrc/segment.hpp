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

// One thread's share of a segment: its 16-byte vectors, loaded at once.
template <class D>
struct SegShare {
  static constexpr int U = kSegElems / (kBlock * D::kPerVec);
  uint4 w[U];
};

// The row's aligned body: its unaligned head elements, the 16-byte vectors
// after them and their count.
template <class D>
struct RowBody {
  int64_t head, nvec;
  const uint4* vp;
  __device__ __forceinline__ RowBody(const void* base, int64_t V) {
    head = head_elems<D>(base, V);
    nvec = (V - head) / D::kPerVec;
    vp = reinterpret_cast<const uint4*>(static_cast<const char*>(base) + head * D::kSize);
  }
};

// Issue the thread's loads of segment `seg` (none past the row's vectors).
template <class D, bool NT>
__device__ __forceinline__ void segment_issue(const RowBody<D>& r, int32_t seg, SegShare<D>& sh) {
  constexpr int kSegVecs = kSegElems / D::kPerVec;
  const int64_t v0 = static_cast<int64_t>(seg) * kSegVecs + threadIdx.x;
#pragma unroll
  for (int j = 0; j < SegShare<D>::U; ++j) {
    const int64_t v = v0 + j * kBlock;
    sh.w[j] = uint4{0u, 0u, 0u, 0u};
    if (v < r.nvec) {
      if (NT) {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(r.vp + v);
        sh.w[j] = uint4{__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1),
                        __builtin_nontemporal_load(q + 2), __builtin_nontemporal_load(q + 3)};
      } else {
        sh.w[j] = r.vp[v];
      }
    }
  }
}

// The thread's pair over its loaded vectors, then (segment 0) the row's head
// elements and (last segment) its tail.
template <class D>
__device__ __forceinline__ MS segment_fold(const void* base, int64_t V, const RowBody<D>& r, int32_t seg,
                                           int32_t nseg, float c, const SegShare<D>& sh) {
  constexpr int U = SegShare<D>::U;
  constexpr int kSegVecs = kSegElems / D::kPerVec;
  const int64_t v0 = static_cast<int64_t>(seg) * kSegVecs + threadIdx.x;
  MS acc{-INFINITY, 0.f};
  {
    // only a segment that reaches past the row's vectors masks them (a
    // block-uniform test, so full segments carry no per-element select)
    const bool full = static_cast<int64_t>(seg + 1) * kSegVecs <= r.nvec;
    float x[U * D::kPerVec];
    if (full) {
#pragma unroll
      for (int j = 0; j < U; ++j) D::unpack(sh.w[j], x + j * D::kPerVec);
    } else {
#pragma unroll
      for (int j = 0; j < U; ++j) {
        D::unpack(sh.w[j], x + j * D::kPerVec);
        if (v0 + j * kBlock >= r.nvec) {
#pragma unroll
          for (int t = 0; t < D::kPerVec; ++t) x[j * D::kPerVec + t] = -INFINITY;
        }
      }
    }
    ms_fold<U * D::kPerVec>(acc, x, c);
  }
  if (seg == 0) {
    for (int64_t i = threadIdx.x; i < r.head; i += kBlock) {
      float x = D::at(base, i);
      ms_fold<1>(acc, &x, c);
    }
  }
  if (seg == nseg - 1) {
    for (int64_t i = r.head + r.nvec * D::kPerVec + threadIdx.x; i < V; i += kBlock) {
      float x = D::at(base, i);
      ms_fold<1>(acc, &x, c);
    }
  }
  return acc;
}

// Block reduction of kN threads' pairs at once: DPP within each wave, then
// the four wave results in order.  `sh` holds kN * 2 * (kBlock / 64) floats.
template <int kN>
__device__ __forceinline__ void block_ms(const MS (&acc)[kN], float* sh, MS (&out)[kN]) {
  constexpr int kW = kBlock / kWave;
  const int wid = threadIdx.x / kWave;
#pragma unroll
  for (int n = 0; n < kN; ++n) {
    const MS r = wave_ms_dpp(acc[n]);
    if ((threadIdx.x & (kWave - 1)) == 0) {
      sh[n * 2 * kW + 2 * wid] = r.m;
      sh[n * 2 * kW + 2 * wid + 1] = r.s;
    }
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < kN; ++n) {
    const float* q = sh + n * 2 * kW;
    MS t{q[0], q[1]};
    for (int w = 1; w < kW; ++w) t = ms_combine(t, MS{q[2 * w], q[2 * w + 1]});
    out[n] = t;
  }
}

// Online-softmax pair of segment `seg` of a row, valid in every thread.
// `sh` holds 2 * (kBlock / 64) floats.
template <class D, bool NT>
__device__ __forceinline__ MS segment_ms(const void* base, int64_t V, int32_t seg, int32_t nseg, float c,
                                         float* sh) {
  const RowBody<D> r(base, V);
  SegShare<D> w;
  segment_issue<D, NT>(r, seg, w);
  const MS acc[1] = {segment_fold<D>(base, V, r, seg, nseg, c, w)};
  MS out[1];
  block_ms<1>(acc, sh, out);
  return out[0];
}

// The pairs of segments seg .. seg + kN - 1 of a row (those past the row
// are empty), every segment's loads in flight at once; each is the same bits
// as segment_ms's.  `sh` holds kN * 2 * (kBlock / 64) floats.
template <class D, bool NT, int kN>
__device__ __forceinline__ void segment_ms_n(const void* base, int64_t V, int32_t seg, int32_t nseg, float c,
                                             float* sh, MS (&out)[kN]) {
  const RowBody<D> r(base, V);
  SegShare<D> w[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n) segment_issue<D, NT>(r, seg + n, w[n]);
  MS acc[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n) acc[n] = segment_fold<D>(base, V, r, seg + n, nseg, c, w[n]);
  block_ms<kN>(acc, sh, out);
}


}  // namespace sv
