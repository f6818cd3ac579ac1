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
// target row.  Two kernels, with no communication between blocks of one grid:
//
// k_sample_tiles: grid = batch * ntiles blocks, one 4096-element tile each.
//   Every block repeats the request's small preamble (row normalisers from
//   the partials, p and q at the drafted tokens, the accept scan), so all of
//   a request's blocks agree on the break position m.  The block then reads
//   its tile of target row m (and of draft row m when m < k) and writes the
//   float64 sums of the draw weights r, of p and of q for that tile.  Tile 0
//   also writes the request's record (status bits, m, row scale) and the
//   diagnostics.  When the vocabulary fits one tile the block draws the token
//   itself and no second kernel runs.
// k_sample_draw: one block per request.  Scans the tile sums, finds the tile
//   holding u_k * total, rescans that tile with a block prefix sum and picks
//   the smallest id whose running weight exceeds it; writes the tokens.
//
// Only the break row's draft row is read from HBM: the accept test needs just
// q_i(x_i) from the other draft rows.
#include "common.hpp"
#include "launch.hpp"

namespace sv {

namespace {

constexpr int kMaxPartialsInLds = 1024;

struct Pre {
  int bits;     // status bits; INVALID ones end the request
  int k, m;
  int ts, qs;
  float Mc;     // scaled-domain max of the draw row
  float invS;   // 1 / normaliser of the draw row
};

struct SampleShared {
  float m[kMaxChainRows], S[kMaxChainRows], p[kMaxChainRows], q[kMaxChainRows];
  float2 part[kMaxPartialsInLds];
  double red[3 * (kBlock / kWave)];
  int i[4];
};

constexpr int kInvalid = kFlagBadRequest | kFlagBadToken | kFlagNonfinite;

// The request's preamble; identical in every block that runs it.
template <class DT, class DQ>
__device__ Pre preamble(const SampleArgs& a, int b, bool write_diag, SampleShared& sh) {
  const int tid = threadIdx.x;
  const int ustride = a.k_max + 1;
  Pre r{};
  r.k = a.dlen[b];
  r.ts = a.t_rs[b];
  r.qs = a.q_rs[b];
  const int k = r.k;
  if (k < 0 || k > a.k_max || r.ts < 0 || static_cast<int64_t>(r.ts) + k >= a.t_rows ||
      (k > 0 && (r.qs < 0 || static_cast<int64_t>(r.qs) + k > a.q_rows))) {
    r.bits = kFlagBadRequest;
    return r;
  }
  if (tid == 0) {
    sh.i[0] = k;
    sh.i[1] = 0;
  }
  const int np = (k + 1) * a.nseg;
  const bool lds_parts = np <= kMaxPartialsInLds;
  if (lds_parts) {
    const float2* src = a.partial + static_cast<int64_t>(r.ts) * a.nseg;
    for (int i = tid; i < np; i += kBlock) sh.part[i] = src[i];
  }
  __syncthreads();
  int x = 0;
  if (tid < k) {
    x = a.ids[static_cast<int64_t>(b) * a.k_max + tid];
    if (x < 0 || x >= a.V) atomicOr(&sh.i[1], kFlagBadToken);
  }
  if (tid <= k) {
    const float2* pp = lds_parts ? sh.part + tid * a.nseg
                                 : a.partial + static_cast<int64_t>(r.ts + tid) * a.nseg;
    MS acc{-INFINITY, 0.f};
    for (int s = 0; s < a.nseg; ++s) acc = ms_combine(acc, MS{pp[s].x, pp[s].y});
    sh.m[tid] = acc.m;
    sh.S[tid] = acc.s;
    if (!(acc.s > 0.f && acc.s < INFINITY)) atomicOr(&sh.i[1], kFlagNonfinite);
  }
  __syncthreads();
  if (sh.i[1] & kFlagBadToken) {
    r.bits = kFlagBadToken;
    return r;
  }
  if (sh.i[1]) {
    r.bits = sh.i[1];
    return r;
  }
  if (tid < k) {
    const float l = DT::at(row_ptr<DT>(a.tgt, r.ts + tid, a.V), x);
    const float p = ex2(fmaf(l, a.c, -sh.m[tid])) * (1.f / sh.S[tid]);
    const float q = DQ::at(row_ptr<DQ>(a.dq, r.qs + tid, a.V), x);
    sh.p[tid] = p;
    sh.q[tid] = q;
    const float uu = a.u[static_cast<int64_t>(b) * ustride + tid];
    if (!(uu * q < p)) atomicMin(&sh.i[0], tid);
  }
  __syncthreads();
  r.m = sh.i[0];
  if (write_diag && a.diag != nullptr && tid <= k) {
    float* d = a.diag + (static_cast<int64_t>(b) * ustride + tid) * 4;
    d[0] = sh.m[tid] * kLn2;
    d[1] = sh.S[tid];
    d[2] = tid < k ? sh.p[tid] : 0.f;
    d[3] = tid < k ? sh.q[tid] : 0.f;
  }
  if (a.max_new != nullptr && k > a.max_new[b]) r.bits |= kFlagOverBudget;
  r.Mc = sh.m[r.m];
  r.invS = 1.f / sh.S[r.m];
  return r;
}

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

// Draw weights of the 16 elements this thread owns starting at e: residual
// max(0, p - q) (resid) or p itself, and p and q.
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

// Sums (r, p, q) of one tile over the block; valid in every thread.
template <class DT, class DQ>
__device__ __forceinline__ void tile_sums(const SampleArgs& a, const void* trow, const void* qrow,
                                          const Pre& pr, int t, double* v, double* red) {
  float w[kPerThreadTile], p[kPerThreadTile], q[kPerThreadTile];
  draw_weights<DT, DQ>(trow, qrow, a.V, static_cast<int64_t>(t) * kTile + threadIdx.x * kPerThreadTile,
                       a.c, pr.Mc, pr.invS, pr.m < pr.k, w, p, q);
  v[0] = pairwise<kPerThreadTile>(w);
  v[1] = pairwise<kPerThreadTile>(p);
  v[2] = pairwise<kPerThreadTile>(q);
  block_sum<3>(v, red);
}

// Draw the last token from the tile sums T[ntiles][3] and write the outputs.
template <class DT, class DQ>
__device__ void draw_and_emit(const SampleArgs& a, int b, const Pre& pr, const double* T,
                              SampleShared& sh) {
  const int tid = threadIdx.x;
  const int ustride = a.k_max + 1;
  const bool resid = pr.m < pr.k;
  double tot[3] = {0.0, 0.0, 0.0};
  for (int t = tid; t < a.ntiles; t += kBlock) {
    tot[0] += T[3 * t];
    tot[1] += T[3 * t + 1];
    tot[2] += T[3 * t + 2];
  }
  block_sum<3>(tot, sh.red);
  int bits = pr.bits;
  int which = 0;  // 0: weights are r; 1: weights are p
  if (resid) {
    if (isnan(tot[2]) || !isfinite(tot[0])) {
      write_invalid(a, b, kFlagNonfinite | bits);
      return;
    }
    if (!(tot[0] > 0.0)) {
      bits |= kFlagFallback;
      which = 1;
    }
  }
  const double total = tot[which];
  const double target = static_cast<double>(a.u[static_cast<int64_t>(b) * ustride + pr.k]) * total;

  // first tile with mass whose running sum exceeds the target (else the last tile with mass)
  if (tid == 0) {
    sh.i[2] = a.ntiles;
    sh.i[3] = -1;
  }
  __syncthreads();
  double carry = 0.0, tile_base = 0.0;
  for (int c0 = 0; c0 < a.ntiles; c0 += kBlock) {
    const int t = c0 + tid;
    const double wt = t < a.ntiles ? T[3 * t + which] : 0.0;
    double chunk_total;
    const double excl = carry + block_exclusive_scan(wt, &chunk_total, sh.red);
    if (t < a.ntiles && wt > 0.0) {
      if (excl + wt > target) atomicMin(&sh.i[2], t);
      atomicMax(&sh.i[3], t);
    }
    __syncthreads();
    const int hit = sh.i[2];
    if (hit >= c0 && hit < c0 + kBlock) {
      if (t == hit) sh.red[0] = excl;
      __syncthreads();
      tile_base = sh.red[0];
      __syncthreads();
      break;
    }
    carry += chunk_total;
  }
  int tile = sh.i[2];
  const bool overshoot = tile >= a.ntiles;
  if (overshoot) tile = sh.i[3];
  __syncthreads();
  if (tile < 0) {  // no mass anywhere (cannot happen when S > 0); defined output
    write_invalid(a, b, kFlagNonfinite | bits);
    return;
  }

  // rescan the chosen tile: smallest id with positive weight whose running
  // weight exceeds the target (else the last id with weight)
  if (tid == 0) {
    sh.i[2] = INT32_MAX;
    sh.i[3] = -1;
  }
  __syncthreads();
  const void* trow = row_ptr<DT>(a.tgt, pr.ts + pr.m, a.V);
  const void* qrow = resid ? row_ptr<DQ>(a.dq, pr.qs + pr.m, a.V) : nullptr;
  {
    float w[kPerThreadTile], p[kPerThreadTile], q[kPerThreadTile];
    const int off = tid * kPerThreadTile;
    draw_weights<DT, DQ>(trow, qrow, a.V, static_cast<int64_t>(tile) * kTile + off, a.c, pr.Mc, pr.invS,
                         resid, w, p, q);
    if (which) {
#pragma unroll
      for (int j = 0; j < kPerThreadTile; ++j) w[j] = p[j];
    }
    double own = 0.0;
#pragma unroll
    for (int j = 0; j < kPerThreadTile; ++j) own += static_cast<double>(w[j]);
    double tile_total;
    double run = tile_base + block_exclusive_scan(own, &tile_total, sh.red);
    int first = INT32_MAX, lastpos = -1;
#pragma unroll
    for (int j = 0; j < kPerThreadTile; ++j) {
      run += static_cast<double>(w[j]);
      if (w[j] > 0.f) {
        if (first == INT32_MAX && !overshoot && run > target) first = off + j;
        lastpos = off + j;
      }
    }
    if (first != INT32_MAX) atomicMin(&sh.i[2], first);
    if (lastpos >= 0) atomicMax(&sh.i[3], lastpos);
  }
  __syncthreads();
  const int pick = sh.i[2] != INT32_MAX ? sh.i[2] : sh.i[3];
  const int y = static_cast<int>(static_cast<int64_t>(tile) * kTile + pick);

  if (tid == 0) {
    int32_t* out = a.out_tok + static_cast<int64_t>(b) * ustride;
    int cnt = 0;
    bool stop = false;
    for (int i = 0; i < pr.m && !stop; ++i) {
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
    a.out_acc[b] = pr.m;
    if (a.resid) a.resid[b] = static_cast<float>(total);
    flag(a.status, bits);
  }
}

}  // namespace

template <class DT, class DQ>
__global__ __launch_bounds__(kBlock) void k_sample_tiles(SampleArgs a) {
  __shared__ SampleShared sh;
  __shared__ double s_tile[3];
  const int b = blockIdx.x / a.ntiles;
  const int t = blockIdx.x - b * a.ntiles;
  const Pre pr = preamble<DT, DQ>(a, b, t == 0, sh);
  if (pr.bits & kInvalid) {
    if (a.ntiles == 1) {
      write_invalid(a, b, pr.bits);
    } else if (t == 0 && threadIdx.x == 0) {
      a.records[b] = make_int4(pr.bits, 0, 0, 0);
    }
    return;
  }
  const void* trow = row_ptr<DT>(a.tgt, pr.ts + pr.m, a.V);
  const void* qrow = pr.m < pr.k ? row_ptr<DQ>(a.dq, pr.qs + pr.m, a.V) : nullptr;
  double v[3];
  tile_sums<DT, DQ>(a, trow, qrow, pr, t, v, sh.red);
  if (a.ntiles == 1) {
    if (threadIdx.x == 0) {
      s_tile[0] = v[0];
      s_tile[1] = v[1];
      s_tile[2] = v[2];
    }
    __syncthreads();
    draw_and_emit<DT, DQ>(a, b, pr, s_tile, sh);
    return;
  }
  if (threadIdx.x == 0) {
    double* T = a.tiles + (static_cast<int64_t>(b) * a.ntiles + t) * 3;
    T[0] = v[0];
    T[1] = v[1];
    T[2] = v[2];
    if (t == 0)
      a.records[b] = make_int4(pr.bits, pr.m, __float_as_int(pr.Mc), __float_as_int(pr.invS));
  }
}

template <class DT, class DQ>
__global__ __launch_bounds__(kBlock) void k_sample_draw(SampleArgs a) {
  __shared__ SampleShared sh;
  const int b = blockIdx.x;
  const int4 rec = a.records[b];
  if (rec.x & kInvalid) {
    write_invalid(a, b, rec.x);
    return;
  }
  Pre pr{};
  pr.bits = rec.x;
  pr.m = rec.y;
  pr.Mc = __int_as_float(rec.z);
  pr.invS = __int_as_float(rec.w);
  pr.k = a.dlen[b];
  pr.ts = a.t_rs[b];
  pr.qs = a.q_rs[b];
  draw_and_emit<DT, DQ>(a, b, pr, a.tiles + static_cast<int64_t>(b) * a.ntiles * 3, sh);
}

template <class DT, class DQ>
static hipError_t launch_pair(const SampleArgs& a, hipStream_t stream) {
  const dim3 block(kBlock);
  hipLaunchKernelGGL((k_sample_tiles<DT, DQ>),
                     dim3(static_cast<uint32_t>(static_cast<int64_t>(a.B) * a.ntiles)), block, 0, stream, a);
  if (a.ntiles > 1)
    hipLaunchKernelGGL((k_sample_draw<DT, DQ>), dim3(static_cast<uint32_t>(a.B)), block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_sample_resolve(int t_dtype, int q_dtype, const SampleArgs& a, hipStream_t stream) {
  if (t_dtype == kDtypeBF16 && q_dtype == kDtypeBF16) return launch_pair<BF16, BF16>(a, stream);
  if (t_dtype == kDtypeBF16) return launch_pair<BF16, F32>(a, stream);
  if (q_dtype == kDtypeBF16) return launch_pair<F32, BF16>(a, stream);
  return launch_pair<F32, F32>(a, stream);
}

}  // namespace sv
