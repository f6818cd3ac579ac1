// Row statistics of the temperature softmax, streamed from HBM.
//
// For every target row l (vocab elements) the verify step needs the softmax
// normaliser of l / T ("投机解码:为什么一个字都不改", figure "一次目标前向验 k 个
// 草稿 token": P = softmax(f / T) over the whole vocabulary).  This kernel reads
// each row exactly once and leaves, per (row, segment), the online-softmax pair
// (m = max l, s = sum 2^((l - m) log2(e) / T)); consumers combine the nseg
// pairs of a row.  The pair is kept in the scaled domain: m = max(l) * log2(e) / T
// (rounded once), s = sum 2^(l * log2(e) / T - m).
//
// Layout: grid = rows * nseg blocks of 256 threads, nseg = ceil(V / 8192);
// block (row, seg) reads the seg-th 8192-element chunk of the row's
// 16-byte-aligned body with coalesced 16-byte non-temporal loads, all of a
// thread's loads in flight at once; segment 0 also takes the unaligned head
// elements and the last segment the tail.
#include "common.hpp"
#include "launch.hpp"

namespace sv {

// One 8192-element chunk per block: every thread issues its U 16-byte loads
// at once (lanes past the row's end read nothing and fold -inf), so each
// block has its whole chunk in flight; NT selects non-temporal loads.
//
// `clear` (optional, n16 16-byte words) is zeroed on the side, for the exchange
// words of the walk that follows this kernel on the stream.
template <class D, bool NT>
__global__ __launch_bounds__(kBlock) void k_row_stats(const void* __restrict__ rows, int64_t V,
                                                      int32_t nseg, float c,
                                                      float2* __restrict__ partial,
                                                      uint4* __restrict__ clear, int64_t n16) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n16;
       i += static_cast<int64_t>(gridDim.x) * kBlock)
    clear[i] = uint4{0u, 0u, 0u, 0u};
  constexpr int U = kSegElems / (kBlock * D::kPerVec);
  constexpr int kSegVecs = kSegElems / D::kPerVec;
  __shared__ float sh[2 * (kBlock / kWave)];
  const int64_t row = blockIdx.x / nseg;
  const int32_t seg = blockIdx.x - static_cast<int32_t>(row) * nseg;
  const void* base = row_ptr<D>(rows, row, V);
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
  if (threadIdx.x == 0) {
    MS t{sh[0], sh[1]};
    for (int w = 1; w < kBlock / kWave; ++w) t = ms_combine(t, MS{sh[2 * w], sh[2 * w + 1]});
    partial[blockIdx.x] = make_float2(t.m, t.s);
  }
}

hipError_t launch_row_stats(int dtype, const void* rows, int64_t n_rows, int64_t V, int32_t nseg,
                            float c, float2* partial, hipStream_t stream, uint64_t* clear,
                            int64_t clear_words) {
  const dim3 grid(static_cast<uint32_t>(n_rows * nseg)), block(kBlock);
  uint4* c16 = reinterpret_cast<uint4*>(clear);
  const int64_t n16 = clear != nullptr ? (clear_words + 1) / 2 : 0;
  if (dtype == kDtypeBF16)
    hipLaunchKernelGGL((k_row_stats<BF16, true>), grid, block, 0, stream, rows, V, nseg, c, partial, c16, n16);
  else
    hipLaunchKernelGGL((k_row_stats<F32, true>), grid, block, 0, stream, rows, V, nseg, c, partial, c16, n16);
  return hipGetLastError();
}

}  // namespace sv
