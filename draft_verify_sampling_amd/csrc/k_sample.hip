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
// k_sample_tiles: grid = batch * ceil(ntiles / 4) blocks, so the whole grid
//   is resident at once.  Every block repeats the request's small preamble
//   (row normalisers from the partials, p and q at the drafted tokens, the
//   accept scan), so all of a request's blocks agree on the break position m.
//   Then each of the block's four waves reads one 2048-element tile of target
//   row m (and of draft row m when m < k), all of its loads in flight at once,
//   and writes the float64 sums of the draw weights r, of p and of q for that
//   tile.  Block 0 of a request also writes the request's record (status bits,
//   m, row scale) and the diagnostics.
// k_sample_single replaces both when the vocabulary fits one tile: one block
//   per request runs the preamble, then one wave sums the tile and draws.
// k_sample_draw: one wave per request.  Scans the tile sums, finds the tile
//   holding u_k * total, rescans that tile with a wave prefix sum and picks
//   the smallest id whose running weight exceeds it; writes the tokens.
//
// Only the break row's draft row is read from HBM: the accept test needs just
// q_i(x_i) from the other draft rows.
#include "tiles.hpp"

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
  int32_t ids[kMaxChainRows];
  float2 part[kMaxPartialsInLds];
  double red[3 * (kBlock / kWave)];
  float ufinal;
  int i[4];
};


constexpr int kInvalid = kFlagBadRequest | kFlagBadToken | kFlagNonfinite;

// The request's preamble; identical in every block that runs it.  Two rounds
// of loads: (1) the request's row starts, draft count, drafted tokens and
// uniforms; (2) its rows' softmax partials and the target/draft values at the
// drafted tokens.
template <class DT, class DQ>
__device__ Pre preamble(const SampleArgs& a, int b, bool write_diag, SampleShared& sh) {
  const int tid = threadIdx.x;
  const int ustride = a.k_max + 1;
  Pre r{};
  // round 1
  r.k = a.dlen[b];
  r.ts = a.t_rs[b];
  r.qs = a.q_rs[b];
  const int x = tid < a.k_max ? a.ids[static_cast<int64_t>(b) * a.k_max + tid] : 0;
  const float uu = tid <= a.k_max ? a.u[static_cast<int64_t>(b) * ustride + tid] : 0.f;
  const int k = r.k;
  if (k < 0 || k > a.k_max || r.ts < 0 || static_cast<int64_t>(r.ts) + k >= a.t_rows ||
      (k > 0 && (r.qs < 0 || static_cast<int64_t>(r.qs) + k > a.q_rows))) {
    r.bits = kFlagBadRequest;
    return r;
  }
  const bool xin = tid < k && x >= 0 && x < a.V;
  // round 2
  const int np = (k + 1) * a.nseg;
  const bool lds_parts = np <= kMaxPartialsInLds;
  if (lds_parts) {
    const float2* src = a.partial + static_cast<int64_t>(r.ts) * a.nseg;
    for (int i = tid; i < np; i += kBlock) sh.part[i] = src[i];
  }
  const float lx = xin ? DT::at(row_ptr<DT>(a.tgt, r.ts + tid, a.V), x) : 0.f;
  const float qx = xin ? DQ::at(row_ptr<DQ>(a.dq, r.qs + tid, a.V), x) : 0.f;
  if (tid == 0) {
    sh.i[0] = k;
    sh.i[1] = 0;
  }
  if (tid < k) sh.ids[tid] = x;
  if (tid == k) sh.ufinal = uu;
  __syncthreads();
  if (tid < k && !xin) atomicOr(&sh.i[1], kFlagBadToken);
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
    const float p = ex2(fmaf(lx, a.c, -sh.m[tid])) * (1.f / sh.S[tid]);
    sh.p[tid] = p;
    sh.q[tid] = qx;
    if (!(uu * qx < p)) atomicMin(&sh.i[0], tid);
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

// Draw the last token from the tile sums T[ntiles][3] and write the outputs.
// Run by exactly one wave (64 lanes); ids[0..m) and ufinal are the request's
// drafted tokens and final uniform.  Lane l owns the contiguous tiles
// [l * tpl, (l + 1) * tpl), then the contiguous 32 elements [32 l, 32 l + 32)
// of the chosen tile; crossings are located with wave scans and ballots.
template <class DT, class DQ>
__device__ void wave_draw_emit(const SampleArgs& a, int b, const Pre& pr, const double* T,
                               const int32_t* ids, float ufinal) {
  const int lane = threadIdx.x & (kWave - 1);
  const int ustride = a.k_max + 1;
  const bool resid = pr.m < pr.k;
  int ta, tb;
  lane_tiles(a.ntiles, lane, ta, tb);
  double own[3] = {0.0, 0.0, 0.0};
  for (int t = ta; t < tb; ++t) {
    own[0] += T[3 * t];
    own[1] += T[3 * t + 1];
    own[2] += T[3 * t + 2];
  }
  const double tot_r = wave_total(own[0]), tot_p = wave_total(own[1]), tot_q = wave_total(own[2]);
  int bits = pr.bits;
  int which = 0;  // 0: weights are r; 1: weights are p
  if (resid) {
    if (isnan(tot_q) || !isfinite(tot_r)) {
      write_invalid(a, b, kFlagNonfinite | bits);
      return;
    }
    if (!(tot_r > 0.0)) {
      bits |= kFlagFallback;
      which = 1;
    }
  }
  const double total = which ? tot_p : tot_r;
  const double target = static_cast<double>(ufinal) * total;

  TileHit h;
  if (!wave_find_tile(T + which, 3, a.ntiles, which ? own[1] : own[0], target, h)) {
    // no mass anywhere (cannot happen when S > 0); defined output
    write_invalid(a, b, kFlagNonfinite | bits);
    return;
  }
  const DrawRow row{row_ptr<DT>(a.tgt, pr.ts + pr.m, a.V),
                    resid ? row_ptr<DQ>(a.dq, pr.qs + pr.m, a.V) : nullptr,
                    a.c, pr.Mc, pr.invS, 1.f, resid && !which};
  const int y = wave_pick_in_tile<DT, DQ>(row, a.V, h, target);

  if (lane == 0) {
    int32_t* out = a.out_tok + static_cast<int64_t>(b) * ustride;
    int cnt = 0;
    bool stop = false;
    for (int i = 0; i < pr.m && !stop; ++i) {
      const int32_t tok = ids[i];
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
  constexpr int kTilesPerBlock = kBlock / kWave;
  __shared__ SampleShared sh;
  const int bpr = (a.ntiles + kTilesPerBlock - 1) / kTilesPerBlock;  // blocks per request
  const int b = blockIdx.x / bpr;
  const int g = blockIdx.x - b * bpr;
  const Pre pr = preamble<DT, DQ>(a, b, g == 0, sh);
  if (pr.bits & kInvalid) {
    if (g == 0 && threadIdx.x == 0) a.records[b] = make_int4(pr.bits, 0, 0, 0);
    return;
  }
  if (g == 0 && threadIdx.x == 0)
    a.records[b] = make_int4(pr.bits, pr.m, __float_as_int(pr.Mc), __float_as_int(pr.invS));
  const int t = g * kTilesPerBlock + threadIdx.x / kWave;
  if (t >= a.ntiles) return;
  const void* trow = row_ptr<DT>(a.tgt, pr.ts + pr.m, a.V);
  const void* qrow = pr.m < pr.k ? row_ptr<DQ>(a.dq, pr.qs + pr.m, a.V) : nullptr;
  const DrawRow row{trow, qrow, a.c, pr.Mc, pr.invS, 1.f, pr.m < pr.k};
  double v[1][3];
  wave_tile_sums<DT, DQ, 1>(row, a.V, t, 0, v);
  if ((threadIdx.x & (kWave - 1)) == 0) {
    double* T = a.tiles + (static_cast<int64_t>(b) * a.ntiles + t) * 3;
    T[0] = v[0][0];
    T[1] = v[0][1];
    T[2] = v[0][2];
  }
}

// Vocabularies of one tile: one block per request runs the preamble, then its
// first wave sums the tile and draws.
template <class DT, class DQ>
__global__ __launch_bounds__(kBlock) void k_sample_single(SampleArgs a) {
  __shared__ SampleShared sh;
  __shared__ double s_tile[3];
  const int b = blockIdx.x;
  const Pre pr = preamble<DT, DQ>(a, b, true, sh);
  if (pr.bits & kInvalid) {
    write_invalid(a, b, pr.bits);
    return;
  }
  if (threadIdx.x >= kWave) return;
  const void* trow = row_ptr<DT>(a.tgt, pr.ts + pr.m, a.V);
  const void* qrow = pr.m < pr.k ? row_ptr<DQ>(a.dq, pr.qs + pr.m, a.V) : nullptr;
  const DrawRow row{trow, qrow, a.c, pr.Mc, pr.invS, 1.f, pr.m < pr.k};
  double v[1][3];
  wave_tile_sums<DT, DQ, 1>(row, a.V, 0, 0, v);
  if (threadIdx.x == 0) {
    s_tile[0] = v[0][0];
    s_tile[1] = v[0][1];
    s_tile[2] = v[0][2];
  }
  wave_draw_emit<DT, DQ>(a, b, pr, s_tile, sh.ids, sh.ufinal);
}

template <class DT, class DQ>
__global__ __launch_bounds__(kWave) void k_sample_draw(SampleArgs a) {
  __shared__ int32_t s_ids[kMaxChainRows];
  __shared__ float s_u[kMaxChainRows];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  // one round of loads: the record, the request's metadata, its drafted
  // tokens and uniforms (the tile sums follow inside the draw)
  const int4 rec = a.records[b];
  Pre pr{};
  pr.k = a.dlen[b];
  pr.ts = a.t_rs[b];
  pr.qs = a.q_rs[b];
  for (int i = lane; i < a.k_max; i += kWave) s_ids[i] = a.ids[static_cast<int64_t>(b) * a.k_max + i];
  for (int i = lane; i <= a.k_max; i += kWave) s_u[i] = a.u[static_cast<int64_t>(b) * (a.k_max + 1) + i];
  if (rec.x & kInvalid) {
    write_invalid(a, b, rec.x);
    return;
  }
  pr.bits = rec.x;
  pr.m = rec.y;
  pr.Mc = __int_as_float(rec.z);
  pr.invS = __int_as_float(rec.w);
  __syncthreads();
  wave_draw_emit<DT, DQ>(a, b, pr, a.tiles + static_cast<int64_t>(b) * a.ntiles * 3, s_ids, s_u[pr.k]);
}

template <class DT, class DQ>
static hipError_t launch_pair(const SampleArgs& a, hipStream_t stream) {
  const dim3 block(kBlock);
  if (a.ntiles == 1) {
    hipLaunchKernelGGL((k_sample_single<DT, DQ>), dim3(static_cast<uint32_t>(a.B)), block, 0, stream, a);
    return hipGetLastError();
  }
  const int64_t bpr = (a.ntiles + (kBlock / kWave) - 1) / (kBlock / kWave);
  hipLaunchKernelGGL((k_sample_tiles<DT, DQ>), dim3(static_cast<uint32_t>(a.B * bpr)), block, 0, stream, a);
  hipLaunchKernelGGL((k_sample_draw<DT, DQ>), dim3(static_cast<uint32_t>(a.B)), dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_sample_resolve(int t_dtype, int q_dtype, const SampleArgs& a, hipStream_t stream) {
  if (t_dtype == kDtypeBF16 && q_dtype == kDtypeBF16) return launch_pair<BF16, BF16>(a, stream);
  if (t_dtype == kDtypeBF16) return launch_pair<BF16, F32>(a, stream);
  if (q_dtype == kDtypeBF16) return launch_pair<F32, BF16>(a, stream);
  return launch_pair<F32, F32>(a, stream);
}

}  // namespace sv
