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
// Layout: grid = rows * nseg blocks of 256 threads; block (row, seg) streams
// the seg-th slice of the row's 16-byte-aligned body with coalesced 16-byte
// loads, U vectors in flight per thread; segment 0 also takes the unaligned
// head elements and the last segment the tail.
#include "common.hpp"
#include "launch.hpp"

namespace sv {

template <class D, int U>
__global__ __launch_bounds__(kBlock) void k_row_stats(const void* __restrict__ rows, int64_t V,
                                                      int32_t nseg, float c,
                                                      float2* __restrict__ partial) {
  __shared__ float sh[2 * (kBlock / kWave)];
  const int64_t row = blockIdx.x / nseg;
  const int32_t seg = blockIdx.x - static_cast<int32_t>(row) * nseg;
  const void* base = row_ptr<D>(rows, row, V);
  const int64_t head = head_elems<D>(base, V);
  const int64_t nvec = (V - head) / D::kPerVec;
  const int64_t v0 = nvec * seg / nseg, v1 = nvec * (seg + 1) / nseg;
  const uint4* vp = reinterpret_cast<const uint4*>(static_cast<const char*>(base) + head * D::kSize);

  MS acc{-INFINITY, 0.f};
  int64_t v = v0 + threadIdx.x;
  for (; v + (U - 1) * kBlock < v1; v += U * kBlock) {
    uint4 w[U];
#pragma unroll
    for (int j = 0; j < U; ++j) w[j] = vp[v + j * kBlock];
    float x[U * D::kPerVec];
#pragma unroll
    for (int j = 0; j < U; ++j) D::unpack(w[j], x + j * D::kPerVec);
    ms_fold<U * D::kPerVec>(acc, x, c);
  }
  for (; v < v1; v += kBlock) {
    float x[D::kPerVec];
    D::unpack(vp[v], x);
    ms_fold<D::kPerVec>(acc, x, c);
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
  const MS r = block_ms(acc, sh);
  if (threadIdx.x == 0) partial[blockIdx.x] = make_float2(r.m, r.s);
}

hipError_t launch_row_stats(int dtype, const void* rows, int64_t n_rows, int64_t V, int32_t nseg,
                            float c, float2* partial, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(n_rows * nseg)), block(kBlock);
  if (dtype == kDtypeBF16)
    hipLaunchKernelGGL((k_row_stats<BF16, 4>), grid, block, 0, stream, rows, V, nseg, c, partial);
  else
    hipLaunchKernelGGL((k_row_stats<F32, 4>), grid, block, 0, stream, rows, V, nseg, c, partial);
  return hipGetLastError();
}

}  // namespace sv
