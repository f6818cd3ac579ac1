// Greedy (T = 0) chain verify.
//
// Method ("第 13 篇：推理引擎一次猜几个字——草稿 + 验证", section ③ and its notes;
// "Speculative decoding explained", four-case table): the target's pick at each
// drafted position is the argmax of its row; drafts are compared left to right,
// the round stops at the first difference, the drafts before it are kept and the
// target's own pick is appended (after a full match: the pick of the row after
// the last draft, unless the request's budget is used up).
//
// Two kernels.  k_row_argmax: grid = rows * nseg blocks; each block streams a
// slice of one row with 16-byte loads and leaves one 64-bit key per slice,
// (order-preserving bits of the value) << 32 | ~index, so that one unsigned max
// picks the largest value and, among equal values, the lowest index; a slice
// holding a NaN leaves the key 0xFFFF...F instead.  k_greedy_resolve: one block
// per request merges the keys of its k_b + 1 rows (thread i ends with row i's
// argmax) and runs the prefix compare.
#include "common.hpp"
#include "launch.hpp"

namespace sv {

namespace {

constexpr uint64_t kNanKey = ~0ull;

__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7fffffffu) == 0u) b = 0u;  // -0 and +0 compare equal
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

struct Best {
  float v;
  int64_t i;
  bool nan;
};

__device__ __forceinline__ void best_update(Best& s, float v, int64_t i) {
  s.nan |= (v != v);
  if (v > s.v || (v == s.v && i < s.i)) {
    s.v = v;
    s.i = i;
  }
}

__device__ __forceinline__ uint64_t best_key(const Best& s) {
  if (s.nan) return kNanKey;
  return (static_cast<uint64_t>(order_bits(s.v)) << 32) |
         static_cast<uint64_t>(~static_cast<uint32_t>(s.i));
}


}  // namespace

template <class D, int U>
__global__ __launch_bounds__(kBlock) void k_row_argmax(const void* __restrict__ rows, int64_t V,
                                                       int32_t nseg, uint64_t* __restrict__ keys) {
  __shared__ uint64_t sh[kBlock / kWave];
  const int64_t row = blockIdx.x / nseg;
  const int32_t seg = blockIdx.x - static_cast<int32_t>(row) * nseg;
  const void* base = row_ptr<D>(rows, row, V);
  const int64_t head = head_elems<D>(base, V);
  const int64_t nvec = (V - head) / D::kPerVec;
  const int64_t v0 = nvec * seg / nseg, v1 = nvec * (seg + 1) / nseg;
  const uint4* vp = reinterpret_cast<const uint4*>(static_cast<const char*>(base) + head * D::kSize);

  // sentinel index INT32_MAX: loses every tie against a real element
  Best best{-INFINITY, 0x7fffffff, false};
  // chunks of U * kBlock vectors; a chunk's loads are all issued before any
  // is used (non-temporal: the rows are read once), so a slice of up to
  // U * kBlock vectors costs one load round.  A chunk's largest value first
  // (fmaxf skips NaN, which only sets the flag), then the first element
  // holding it, the lowest id, since a thread's elements ascend.
  for (int64_t c0 = v0 + threadIdx.x; c0 < v1; c0 += U * kBlock) {
    uint4 w[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t v = c0 + j * kBlock;
      w[j] = uint4{0u, 0u, 0u, 0u};
      if (v < v1) {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(vp + v);
        w[j] = uint4{__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1),
                     __builtin_nontemporal_load(q + 2), __builtin_nontemporal_load(q + 3)};
      }
    }
    float x[U][D::kPerVec];
    float m = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      D::unpack(w[j], x[j]);
      if (c0 + j * kBlock < v1) {
#pragma unroll
        for (int t = 0; t < D::kPerVec; ++t) {
          m = fmaxf(m, x[j][t]);
          nan |= x[j][t] != x[j][t];
        }
      }
    }
    int32_t at = 0x7fffffff;
#pragma unroll
    for (int j = U - 1; j >= 0; --j) {
      if (c0 + j * kBlock < v1) {
        const int32_t e = static_cast<int32_t>(head + (c0 + j * kBlock) * D::kPerVec);
#pragma unroll
        for (int t = D::kPerVec - 1; t >= 0; --t) at = x[j][t] == m ? e + t : at;
      }
    }
    best.nan |= nan;
    if (m > best.v || (m == best.v && at < best.i)) {
      best.v = m;
      best.i = at;
    }
  }
  if (seg == 0)
    for (int64_t i = threadIdx.x; i < head; i += kBlock) best_update(best, D::at(base, i), i);
  if (seg == nseg - 1)
    for (int64_t i = head + nvec * D::kPerVec + threadIdx.x; i < V; i += kBlock)
      best_update(best, D::at(base, i), i);

  uint64_t key = wave_max_u64(best_key(best));
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  if (lane == 0) sh[wid] = key;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t r = sh[0];
    for (int w = 1; w < kBlock / kWave; ++w) r = sh[w] > r ? sh[w] : r;
    keys[blockIdx.x] = r;
  }
}

// One block per request; thread i holds draft i and, after the key merge,
// row i's argmax.  Two dependent load rounds: the request (its row start,
// draft count, budget and drafts), then the keys of its rows.
static_assert(kMaxChainRows <= kBlock, "one chain row per thread");
__global__ __launch_bounds__(kBlock) void k_greedy_resolve(GreedyArgs a) {
  __shared__ unsigned long long s_best[kMaxChainRows];
  __shared__ int s_bits, s_m, s_eos, s_pick;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int ustride = a.k_max + 1;
  int32_t* out = a.out_tok + static_cast<int64_t>(b) * ustride;
  const int k = a.dlen[b];
  const int ts = a.t_rs[b];
  const int budget = a.max_new != nullptr ? a.max_new[b] : 0;
  const int x = tid < a.k_max ? a.ids[static_cast<int64_t>(b) * a.k_max + tid] : -1;
  if (tid == 0) {
    s_bits = 0;
    s_m = k;
    s_eos = kMaxChainRows;
  }
  s_best[tid] = 0;
  const bool bad_req = k < 0 || k > a.k_max || ts < 0 || static_cast<int64_t>(ts) + k >= a.t_rows;
  __syncthreads();
  if (!bad_req) {
    if (tid < k && (x < 0 || x >= a.V)) atomicOr(&s_bits, kFlagBadToken);
    const int64_t n = static_cast<int64_t>(k + 1) * a.nseg;
    const uint64_t* kk = a.keys + static_cast<int64_t>(ts) * a.nseg;
    for (int64_t j = tid; j < n; j += kBlock) atomicMax(&s_best[j / a.nseg], static_cast<unsigned long long>(kk[j]));
  }
  __syncthreads();
  int bits = bad_req ? kFlagBadRequest : s_bits;
  if (!bits) {
    // every row of the request must be NaN-free; the drafts are kept up to
    // the first one that differs from its row's argmax
    if (tid == 0 && a.max_new != nullptr && k > budget) flag(a.status, kFlagOverBudget);
    const uint64_t best = s_best[tid];
    if (tid <= k && best == kNanKey) atomicOr(&s_bits, kFlagNonfinite);
    const int am = static_cast<int>(~static_cast<uint32_t>(best));
    if (tid < k && x != am) atomicMin(&s_m, tid);
    __syncthreads();
    bits = s_bits;
    if (!bits) {
      const int m = s_m;
      if (tid == m) s_pick = am;
      if (tid < m && a.eos >= 0 && x == a.eos) atomicMin(&s_eos, tid);
      __syncthreads();
      // the kept drafts up to the first EOS among them; the target's pick
      // after them unless an EOS ended the round; then the budget
      int cnt = s_eos < m ? s_eos + 1 : m + 1;
      if (a.max_new != nullptr) cnt = min(cnt, max(budget, 0));
      if (tid < ustride) out[tid] = tid < cnt ? (tid < m ? x : s_pick) : -1;
      if (tid == 0) {
        a.out_cnt[b] = cnt;
        a.out_acc[b] = m;
      }
      return;
    }
  }
  if (tid < ustride) out[tid] = -1;
  if (tid == 0) {
    a.out_cnt[b] = 0;
    a.out_acc[b] = 0;
    flag(a.status, bits);
  }
}

hipError_t launch_row_argmax(int dtype, const void* rows, int64_t n_rows, int64_t V, int32_t nseg,
                             uint64_t* keys, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(n_rows * nseg)), block(kBlock);
  if (dtype == kDtypeBF16)
    launch_timed((k_row_argmax<BF16, 4>), grid, block, 0, stream, rows, V, nseg, keys);
  else
    launch_timed((k_row_argmax<F32, 4>), grid, block, 0, stream, rows, V, nseg, keys);
  return hipGetLastError();
}

hipError_t launch_greedy_resolve(const GreedyArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(a.B)), block(kBlock);
  hipLaunchKernelGGL(k_greedy_resolve, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace sv
