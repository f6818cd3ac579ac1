// Speculative-sampling chain verify: accept scan, residual and inverse-CDF draw.
//
// Method ("投机解码:为什么一个字都不改", sections "改进:接受概率 min(1, p/q),
// 拒绝时从残差重采" and "一轮能出几个 token"): draft x_i is kept with
// probability min(1, p_i(x_i) / q_i(x_i)) -- with the uniform u_i, kept iff
// u_i q_i(x_i) < p_i(x_i); the first draft that is not kept ends the round and
// is replaced by a draw from norm(max(0, p_m - q_m)); when all k drafts are
// kept one more token is drawn from p_k.
//
// Runs after the row-statistics kernel has left the softmax partials of every
// target row.  Grid: batch * chunks blocks; block (b, ch) owns tiles
// [ch * tpb, ch * tpb + tpb) of request b's draw row.  Every block of a
// request first repeats the request's small preamble (row normalisers from the
// partials, p and q at the drafted tokens, the accept scan), so all of them
// agree on the break position m without talking to each other.  Each block then
// streams its tiles of target row m (and draft row m when m < k), writing per
// tile the float64 sums of the draw weights r, of p, and of q.  The last block
// of the request to arrive (agent-scope counter, cleared by the row-statistics
// kernel at the start of the call)
// scans the tile sums, finds the tile holding u_k * total, rescans that one
// tile with a block prefix sum and picks the smallest id whose running weight
// exceeds it.  Only the break row's draft row is read from HBM: the accept
// test needs just q_i(x_i).
#include "common.hpp"
#include "launch.hpp"

namespace sv {

namespace {

__device__ void write_invalid(const SampleArgs& a, int b, int bits) {
  const int ustride = a.k_max + 1;
  for (int i = threadIdx.x; i < ustride; i += blockDim.x) a.out_tok[static_cast<int64_t>(b) * ustride + i] = -1;
  if (threadIdx.x == 0) {
    a.out_cnt[b] = 0;
    a.out_acc[b] = 0;
    if (a.resid) a.resid[b] = 0.f;
    flag(a.status, bits);
  }
}

// Draw weights of 16 consecutive elements starting at e: residual
// max(0, p - q) (resid) or p itself; p = 2^((l - M) c) / S.
template <class DT, class DQ>
__device__ __forceinline__ void draw_weights(const void* trow, const void* qrow, int64_t V, int64_t e,
                                             float c, float Mc, float invS, bool resid, float* w,
                                             float* p, float* q) {
  float l[kPerThreadTile];
  load_run<DT, kPerThreadTile>(trow, V, e, l, -INFINITY);
  if (resid) {
    load_run<DQ, kPerThreadTile>(qrow, V, e, q, 0.f);
  } else {
#pragma unroll
    for (int j = 0; j < kPerThreadTile; ++j) q[j] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < kPerThreadTile; ++j) {
    p[j] = ex2(fmaf(l[j], c, -Mc)) * invS;
    w[j] = resid ? fmaxf(p[j] - q[j], 0.f) : p[j];
  }
}

template <int n>
__device__ __forceinline__ float pairwise(const float* x) {
  float t[n];
#pragma unroll
  for (int j = 0; j < n; ++j) t[j] = x[j];
#pragma unroll
  for (int w = 1; w < n; w *= 2) {
#pragma unroll
    for (int j = 0; j + w < n; j += 2 * w) t[j] += t[j + w];
  }
  return t[0];
}

}  // namespace

template <class DT, class DQ>
__global__ __launch_bounds__(kBlock) void k_sample_resolve(SampleArgs a) {
  constexpr int kWaves = kBlock / kWave;
  __shared__ float s_m[kMaxChainRows], s_S[kMaxChainRows], s_p[kMaxChainRows], s_q[kMaxChainRows];
  __shared__ double s_tile[kSampleTilesPerBlock][kWaves][3];
  __shared__ double s_red[3 * kWaves];
  __shared__ int s_int[4];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int b = blockIdx.x / a.chunks;
  const int ch = blockIdx.x - b * a.chunks;
  const int ustride = a.k_max + 1;
  const int k = a.dlen[b];
  const int ts = a.t_rs[b];
  const int qs = a.q_rs[b];

  // ---- request checks (identical in every block of the request) ----
  const bool bad = k < 0 || k > a.k_max || ts < 0 || static_cast<int64_t>(ts) + k >= a.t_rows ||
                   (k > 0 && (qs < 0 || static_cast<int64_t>(qs) + k > a.q_rows));
  if (bad) {
    if (ch == 0) write_invalid(a, b, kFlagBadRequest);
    return;
  }
  if (tid == 0) {
    s_int[0] = k;
    s_int[1] = 0;
  }
  __syncthreads();
  int x = 0;
  if (tid < k) {
    x = a.ids[static_cast<int64_t>(b) * a.k_max + tid];
    if (x < 0 || x >= a.V) atomicOr(&s_int[1], kFlagBadToken);
  }
  __syncthreads();
  if (s_int[1]) {
    if (ch == 0) write_invalid(a, b, s_int[1]);
    return;
  }

  // ---- row normalisers ----
  if (tid <= k) {
    const float2* pp = a.partial + static_cast<int64_t>(ts + tid) * a.nseg;
    MS r{-INFINITY, 0.f};
    for (int s = 0; s < a.nseg; ++s) {
      const float2 v = pp[s];
      r = ms_combine(r, MS{v.x, v.y});
    }
    s_m[tid] = r.m;
    s_S[tid] = r.s;
    if (!(r.s > 0.f && r.s < INFINITY)) atomicOr(&s_int[1], kFlagNonfinite);
  }
  __syncthreads();
  if (s_int[1]) {
    if (ch == 0) write_invalid(a, b, s_int[1]);
    return;
  }

  // ---- p, q at the drafted tokens; accept scan ----
  if (tid < k) {
    const float l = DT::at(row_ptr<DT>(a.tgt, ts + tid, a.V), x);
    const float p = ex2(fmaf(l, a.c, -s_m[tid])) * (1.f / s_S[tid]);
    const float q = DQ::at(row_ptr<DQ>(a.dq, qs + tid, a.V), x);
    s_p[tid] = p;
    s_q[tid] = q;
    const float uu = a.u[static_cast<int64_t>(b) * ustride + tid];
    if (!(uu * q < p)) atomicMin(&s_int[0], tid);
  }
  __syncthreads();
  const int m = s_int[0];

  if (ch == 0) {
    if (tid == 0 && a.max_new != nullptr && k > a.max_new[b]) flag(a.status, kFlagOverBudget);
    if (a.diag != nullptr && tid <= k) {
      float* d = a.diag + (static_cast<int64_t>(b) * ustride + tid) * 4;
      d[0] = s_m[tid] * kLn2;
      d[1] = s_S[tid];
      d[2] = tid < k ? s_p[tid] : 0.f;
      d[3] = tid < k ? s_q[tid] : 0.f;
    }
  }

  // ---- tile sums of the draw row ----
  const bool resid = m < k;
  const float Mc = s_m[m];
  const float invS = 1.f / s_S[m];
  const void* trow = row_ptr<DT>(a.tgt, ts + m, a.V);
  const void* qrow = resid ? row_ptr<DQ>(a.dq, qs + m, a.V) : nullptr;
  const int t0 = ch * a.tpb;
  const int t1 = min(t0 + a.tpb, a.ntiles);
  for (int t = t0; t < t1; ++t) {
    float w[kPerThreadTile], p[kPerThreadTile], q[kPerThreadTile];
    draw_weights<DT, DQ>(trow, qrow, a.V, static_cast<int64_t>(t) * kTile + tid * kPerThreadTile, a.c,
                         Mc, invS, resid, w, p, q);
    double v0 = wave_sum(static_cast<double>(pairwise<kPerThreadTile>(w)));
    double v1 = wave_sum(static_cast<double>(pairwise<kPerThreadTile>(p)));
    double v2 = wave_sum(static_cast<double>(pairwise<kPerThreadTile>(q)));
    if (lane == 0) {
      s_tile[t - t0][wid][0] = v0;
      s_tile[t - t0][wid][1] = v1;
      s_tile[t - t0][wid][2] = v2;
    }
  }
  __syncthreads();
  if (tid < (t1 - t0) * 3) {
    const int t = tid / 3, j = tid - 3 * (tid / 3);
    double s = 0.0;
    for (int wv = 0; wv < kWaves; ++wv) s += s_tile[t][wv][j];
    a.tiles[(static_cast<int64_t>(b) * a.ntiles + t0 + t) * 3 + j] = s;
  }

  // ---- last block of the request draws the token ----
  if (a.chunks > 1) {
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = atomicAdd(&a.counters[b], 1u);
      s_int[2] = (prev == static_cast<unsigned>(a.chunks - 1));
    }
    __syncthreads();
    if (!s_int[2]) return;
    __threadfence();
  } else {
    __syncthreads();
  }

  const double* T = a.tiles + static_cast<int64_t>(b) * a.ntiles * 3;
  double tot[3] = {0.0, 0.0, 0.0};
  for (int t = tid; t < a.ntiles; t += kBlock) {
    tot[0] += T[3 * t];
    tot[1] += T[3 * t + 1];
    tot[2] += T[3 * t + 2];
  }
  block_sum<3>(tot, s_red);
  int bits = 0;
  int which = 0;  // 0: weights are r; 1: weights are p
  if (resid) {
    if (isnan(tot[2]) || !isfinite(tot[0])) {
      write_invalid(a, b, kFlagNonfinite);
      return;
    }
    if (!(tot[0] > 0.0)) {
      bits = kFlagFallback;
      which = 1;
    }
  }
  const double total = tot[which];
  const double target = static_cast<double>(a.u[static_cast<int64_t>(b) * ustride + k]) * total;

  // first tile whose running sum exceeds the target (else the last tile with mass)
  if (tid == 0) {
    s_int[2] = a.ntiles;   // first crossing tile
    s_int[3] = -1;         // last tile with mass
  }
  __syncthreads();
  double carry = 0.0, tile_base = 0.0;
  for (int c0 = 0; c0 < a.ntiles; c0 += kBlock) {
    const int t = c0 + tid;
    const double wt = t < a.ntiles ? T[3 * t + which] : 0.0;
    double chunk_total;
    const double excl = carry + block_exclusive_scan(wt, &chunk_total, s_red);
    if (t < a.ntiles) {
      if (wt > 0.0 && excl + wt > target) atomicMin(&s_int[2], t);
      if (wt > 0.0) atomicMax(&s_int[3], t);
    }
    __syncthreads();
    const int hit = s_int[2];
    if (hit >= c0 && hit < c0 + kBlock) {
      if (t == hit) s_red[0] = excl;
      __syncthreads();
      tile_base = s_red[0];
      __syncthreads();
      break;
    }
    carry += chunk_total;
  }
  int tile = s_int[2];
  bool overshoot = false;
  if (tile >= a.ntiles) {
    tile = s_int[3];
    overshoot = true;
  }
  __syncthreads();
  if (tile < 0) {          // no mass anywhere (cannot happen with S > 0); defined output
    write_invalid(a, b, kFlagNonfinite);
    return;
  }

  // rescan the chosen tile: smallest id whose running weight exceeds target
  if (tid == 0) {
    s_int[2] = INT32_MAX;  // first crossing element
    s_int[3] = -1;         // last element with weight
  }
  __syncthreads();
  {
    float w[kPerThreadTile], p[kPerThreadTile], q[kPerThreadTile];
    const int64_t e0 = static_cast<int64_t>(tile) * kTile + tid * kPerThreadTile;
    draw_weights<DT, DQ>(trow, qrow, a.V, e0, a.c, Mc, invS, resid, w, p, q);
    double cum[kPerThreadTile];
    double run = 0.0;
#pragma unroll
    for (int j = 0; j < kPerThreadTile; ++j) {
      run += static_cast<double>(which ? p[j] : w[j]);
      cum[j] = run;
    }
    double tile_total;
    const double excl = block_exclusive_scan(run, &tile_total, s_red);
    int first = INT32_MAX, lastpos = -1;
#pragma unroll
    for (int j = kPerThreadTile - 1; j >= 0; --j) {
      const float wj = which ? p[j] : w[j];
      if (!overshoot && wj > 0.f && tile_base + excl + cum[j] > target)
        first = static_cast<int>(e0 - static_cast<int64_t>(tile) * kTile) + j;
      if (wj > 0.f && lastpos < 0) lastpos = static_cast<int>(e0 - static_cast<int64_t>(tile) * kTile) + j;
    }
    if (first != INT32_MAX) atomicMin(&s_int[2], first);
    if (lastpos >= 0) atomicMax(&s_int[3], lastpos);
  }
  __syncthreads();
  int pick = s_int[2] != INT32_MAX ? s_int[2] : s_int[3];
  const int y = static_cast<int>(static_cast<int64_t>(tile) * kTile + pick);

  if (tid == 0) {
    int32_t* out = a.out_tok + static_cast<int64_t>(b) * ustride;
    int cnt = 0;
    bool stop = false;
    for (int i = 0; i < m && !stop; ++i) {
      const int32_t tok = a.ids[static_cast<int64_t>(b) * a.k_max + i];
      out[cnt++] = tok;
      if (a.eos >= 0 && tok == a.eos) stop = true;
    }
    if (!stop) out[cnt++] = y;
    if (a.max_new != nullptr) {
      const int budget = a.max_new[b] > 0 ? a.max_new[b] : 0;
      if (cnt > budget) cnt = budget;
    }
    for (int i = cnt; i < ustride; ++i) out[i] = -1;
    a.out_cnt[b] = cnt;
    a.out_acc[b] = m;
    if (a.resid) a.resid[b] = static_cast<float>(total);
    flag(a.status, bits);
  }
}

hipError_t launch_sample_resolve(int t_dtype, int q_dtype, const SampleArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(a.B) * a.chunks)), block(kBlock);
  if (t_dtype == kDtypeBF16 && q_dtype == kDtypeBF16)
    hipLaunchKernelGGL((k_sample_resolve<BF16, BF16>), grid, block, 0, stream, a);
  else if (t_dtype == kDtypeBF16)
    hipLaunchKernelGGL((k_sample_resolve<BF16, F32>), grid, block, 0, stream, a);
  else if (q_dtype == kDtypeBF16)
    hipLaunchKernelGGL((k_sample_resolve<F32, BF16>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((k_sample_resolve<F32, F32>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace sv
