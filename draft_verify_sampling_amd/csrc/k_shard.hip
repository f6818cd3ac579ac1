// Sampled chain verify over a vocabulary split into column shards, as a
// vocabulary-parallel LM head leaves it: each device holds columns
// [bounds[g], bounds[g+1]) of every target and draft row.  Method as the
// chain verify ("投机解码:为什么一个字都不改", sections "改进" and
// "一轮能出几个 token"; P = softmax(f / T) over the whole vocabulary per the
// figure "一次目标前向验 k 个草稿 token"); only the data movement differs.
//
// Three steps per shard, with an exchange of a few bytes per row or request
// between them (an all-gather over the devices; on one device, arrays):
//   1. k_shard_fold + k_shard_gather: the shard's softmax pair of every
//      target row (from the statistics kernel's segment partials), and the
//      target logit and draft probability at every drafted token the shard
//      holds.
//   2. k_shard_residual: every shard combines all shards' pairs (shard
//      order), takes p(x_i) from the owning shard, runs the same accept scan,
//      and sums the weights of its own columns of the break row (residual
//      max(0, p - q), or p for the extra token) per 2048-id tile.
//   3. k_shard_draw: from all shards' totals, the shard whose columns hold
//      u times the total finds the tile and the id and writes the round's
//      outputs; shard 0 writes the outputs of invalid requests.
#include "tiles.hpp"

namespace sv {

namespace {

constexpr int kShardBlock = 1024;
constexpr int kShardWaves = kShardBlock / kWave;

__device__ __forceinline__ float lane_f(float v, int g) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), g));
}

__device__ __forceinline__ double lane_d(double v, int g) { return lane_value(v, g); }

// Scaled-domain pair of a row from the G shards' pairs, combined in shard
// order; valid in every lane of the calling wave.  Lane g loads shard g's pair
// (one load round), then the wave folds them in shard order.
__device__ __forceinline__ MS wave_shard_combine(const float* all_pairs, int G, int64_t t_rows, int64_t row) {
  const int lane = threadIdx.x & (kWave - 1);
  float pm = -INFINITY, ps = 0.f;
  if (lane < G) {
    const float* p = all_pairs + (static_cast<int64_t>(lane) * t_rows + row) * 2;
    pm = p[0];
    ps = p[1];
  }
  MS acc{-INFINITY, 0.f};
  for (int g = 0; g < G; ++g) acc = ms_combine(acc, MS{lane_f(pm, g), lane_f(ps, g)});
  return acc;
}

__device__ __forceinline__ int shard_of(const ShardBounds& sb, int64_t x) {
  int g = 0;
  for (int h = 1; h < sb.G; ++h)
    if (sb.b[h] <= x) g = h;
  return g;
}

// Emitted tokens of a round (drafts 0..m-1, then y), cut after the first EOS
// and at the request's budget; called by a whole wave (lane i writes slots i,
// i + 64, ...).
__device__ void emit_round(const ShardArgs& a, int b, int m, int y, float resid, int flags) {
  const int lane = threadIdx.x & (kWave - 1);
  const int width = a.k_max + 1;
  int32_t* out = a.out_tok + static_cast<int64_t>(b) * width;
  const int32_t* x = a.ids + static_cast<int64_t>(b) * a.k_max;
  int stop = m;  // the first EOS among the kept drafts, or m
  for (int i0 = 0; i0 < m && a.eos >= 0; i0 += kWave) {
    const int i = i0 + lane;
    const uint64_t hit = __ballot(i < m && x[i] == a.eos);
    if (hit != 0) {
      stop = i0 + __ffsll(static_cast<long long>(hit)) - 1;
      break;
    }
  }
  int cnt = stop < m ? stop + 1 : m + 1;
  if (a.max_new != nullptr) cnt = min(cnt, max(a.max_new[b], 0));
  for (int i = lane; i < width; i += kWave) out[i] = i < cnt ? (i < m ? x[i] : y) : -1;
  if (lane == 0) {
    a.out_cnt[b] = cnt;
    a.out_acc[b] = m;
    if (a.resid != nullptr) a.resid[b] = resid;
    flag(a.status, flags);
  }
}

// Outputs of an invalid request; called by a whole wave.
__device__ void emit_invalid(const ShardArgs& a, int b, int flags) {
  const int lane = threadIdx.x & (kWave - 1);
  const int width = a.k_max + 1;
  for (int i = lane; i < width; i += kWave) a.out_tok[static_cast<int64_t>(b) * width + i] = -1;
  if (lane == 0) {
    a.out_cnt[b] = 0;
    a.out_acc[b] = 0;
    if (a.resid != nullptr) a.resid[b] = 0.f;
    flag(a.status, flags);
  }
}

}  // namespace

// One wave per row: the shard's pair from its segment partials (canonical order).
__global__ __launch_bounds__(kBlock) void k_shard_fold(const float2* partial, int64_t rows, int32_t nseg,
                                                       float* pairs) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kBlock / kWave) + threadIdx.x / kWave;
  if (row >= rows) return;
  const float2* pp = partial + row * nseg;
  const MS acc = wave_combine_segments(nseg, [&](int s) { return MS{pp[s].x, pp[s].y}; });
  if ((threadIdx.x & (kWave - 1)) == 0) {
    pairs[row * 2] = acc.m;
    pairs[row * 2 + 1] = acc.s;
  }
}

// One thread per drafted token: its target logit and draft probability when the
// shard holds it (other entries are left as they are).
template <class DT, class DQ>
__global__ __launch_bounds__(kBlock) void k_shard_gather(ShardArgs a, float* at) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (t >= static_cast<int64_t>(a.B) * a.k_max) return;
  const int b = static_cast<int>(t / a.k_max), i = static_cast<int>(t % a.k_max);
  const int k = a.dlen[b];
  if (i >= k || k > a.k_max) return;
  const int ts = a.t_rs[b], qs = a.q_rs[b];
  if (ts < 0 || static_cast<int64_t>(ts) + k >= a.t_rows || qs < 0 || static_cast<int64_t>(qs) + k > a.q_rows)
    return;
  const int64_t x = a.ids[t];
  const int64_t c0 = a.sb.b[a.shard], vg = a.sb.b[a.shard + 1] - c0;
  if (x < c0 || x >= c0 + vg) return;
  at[t * 2] = DT::at(row_ptr<DT>(a.tgt, ts + i, vg), x - c0);
  at[t * 2 + 1] = DQ::at(row_ptr<DQ>(a.dq, qs + i, vg), x - c0);
}

// One block per request: decisions from all shards' pairs and gathered values,
// then the weight sums of this shard's columns of the break row.
template <class DT, class DQ>
__global__ __launch_bounds__(kShardBlock) void k_shard_residual(ShardArgs a) {
  __shared__ float s_m[kMaxChainRows], s_S[kMaxChainRows];
  __shared__ int s_bad, s_brk;
  __shared__ double s_red[kShardWaves][3];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int k = a.dlen[b];
  const int ts = a.t_rs[b], qs = a.q_rs[b];
  const int64_t c0 = a.sb.b[a.shard], vg = a.sb.b[a.shard + 1] - c0;
  int64_t* state = a.state + static_cast<int64_t>(b) * 2;
  double* mass = a.mass + static_cast<int64_t>(a.shard * a.B + b) * 3;
  if (k < 0 || k > a.k_max || ts < 0 || static_cast<int64_t>(ts) + k >= a.t_rows ||
      (k > 0 && (qs < 0 || static_cast<int64_t>(qs) + k > a.q_rows))) {
    if (tid == 0) {
      state[0] = -1;
      state[1] = kFlagBadRequest;
    }
    return;
  }
  if (tid == 0) {
    s_bad = 0;
    s_brk = k;
  }
  __syncthreads();
  // wave i: row i's pair over the shards and, for i < k, the accept test of
  // draft i (kept iff u_i q_i(x_i) < p_i(x_i); m = the first not kept); lane g
  // holds shard g's pair and gathered values, all loaded in one round
  for (int i = wid; i <= k; i += kShardWaves) {
    const int G = a.sb.G;
    float pm = -INFINITY, ps = 0.f, lv = 0.f, qv = 0.f;
    if (lane < G) {
      const float* pp = a.pairs + (static_cast<int64_t>(lane) * a.t_rows + ts + i) * 2;
      pm = pp[0];
      ps = pp[1];
      if (i < k) {
        const float* v = a.at + ((static_cast<int64_t>(lane) * a.B + b) * a.k_max + i) * 2;
        lv = v[0];
        qv = v[1];
      }
    }
    const int64_t x = i < k ? a.ids[static_cast<int64_t>(b) * a.k_max + i] : 0;
    const float u = i < k ? slot_uniform(a.u, a.seed, a.offset, b, a.k_max + 1, i) : 0.f;
    MS st{-INFINITY, 0.f};
    for (int g = 0; g < G; ++g) st = ms_combine(st, MS{lane_f(pm, g), lane_f(ps, g)});
    if (lane == 0) {
      s_m[i] = st.m;
      s_S[i] = st.s;
      if (i < k) {
        if (x < 0 || x >= a.V) {
          atomicOr(&s_bad, kFlagBadToken);
        } else {
          const int g = shard_of(a.sb, x);
          const float p = ex2(fmaf(lane_f(lv, g), a.c, -st.m)) * (1.f / st.s);
          if (!(u * lane_f(qv, g) < p)) atomicMin(&s_brk, i);
        }
      }
    }
  }
  __syncthreads();
  const int m = s_brk;
  int bad = s_bad;
  // rows 0..m are read: each must have a finite, positive normaliser
  if (!bad) {
    bool fin = true;
    for (int i = 0; i <= m; ++i) fin &= s_S[i] > 0.f && s_S[i] < INFINITY;
    if (!fin) bad = kFlagNonfinite;
  }
  if (bad) {
    if (tid == 0) {
      state[0] = -1;
      state[1] = bad;
    }
    return;
  }
  // this shard's weights of row m: residual against draft row m, or p (extra token)
  const bool resid = m < k;
  const DrawRow r{row_ptr<DT>(a.tgt, ts + m, vg), resid ? row_ptr<DQ>(a.dq, qs + m, vg) : nullptr, a.c,
                  s_m[m], 1.f / s_S[m], 1.f, resid};
  const int nt = static_cast<int>((vg + kSampleTile - 1) / kSampleTile);
  double* ts_out = a.tiles + static_cast<int64_t>(b) * a.tile_cap * 2;
  double w = 0.0, p = 0.0, q = 0.0;
  for (int t = wid; t < nt; t += kShardWaves) {
    double v[1][3];
    wave_tile_sums<DT, DQ, 1>(r, vg, t, 0, v);
    if (lane == 0) {
      ts_out[t * 2] = v[0][0];
      ts_out[t * 2 + 1] = v[0][1];
    }
    w += v[0][0];
    p += v[0][1];
    q += v[0][2];
  }
  if (lane == 0) {
    s_red[wid][0] = w;
    s_red[wid][1] = p;
    s_red[wid][2] = q;
  }
  __syncthreads();
  if (tid == 0) {
    double W = 0.0, P = 0.0, Q = 0.0;
    for (int h = 0; h < kShardWaves; ++h) {
      W += s_red[h][0];
      P += s_red[h][1];
      Q += s_red[h][2];
    }
    mass[0] = W;
    mass[1] = P;
    mass[2] = Q;
    state[0] = m;
    state[1] = 0;
  }
}

// One wave per request: the shard holding the target draws; outputs written once.
template <class DT, class DQ>
__global__ __launch_bounds__(kBlock) void k_shard_draw(ShardArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t b64 = static_cast<int64_t>(blockIdx.x) * (kBlock / kWave) + threadIdx.x / kWave;
  if (b64 >= a.B) return;
  const int b = static_cast<int>(b64);
  const int64_t* state = a.state + b64 * 2;
  const int G = a.sb.G;
  // one load round: the decision, the request, and (lane g) shard g's sums
  const int m = static_cast<int>(state[0]);
  const int bad = static_cast<int>(state[1]);
  const int k = a.dlen[b];
  const int ts = a.t_rs[b], qs = a.q_rs[b];
  const float u = k >= 0 && k <= a.k_max ? slot_uniform(a.u, a.seed, a.offset, b, a.k_max + 1, k) : 0.f;
  double mw = 0.0, mp = 0.0, mq = 0.0;
  if (lane < G) {
    const double* ms = a.mass + static_cast<int64_t>(lane * a.B + b) * 3;
    mw = ms[0];
    mp = ms[1];
    mq = ms[2];
  }
  // more drafts than the budget: reported for every request whose drafts were read
  const int extra = (a.max_new != nullptr && k > a.max_new[b]) ? kFlagOverBudget : 0;
  if (m < 0) {
    if (a.shard == 0) emit_invalid(a, b, bad | (bad == kFlagNonfinite ? extra : 0));
    return;
  }
  const bool resid = m < k;
  // totals over the shards, in shard order; the draft row's sum classes
  double W = 0.0, P = 0.0;
  bool qnan = false, qpinf = false, qninf = false;
  for (int g = 0; g < G; ++g) {
    W += lane_d(mw, g);
    P += lane_d(mp, g);
    const double q = lane_d(mq, g);
    qnan |= isnan(q);
    qpinf |= q == INFINITY;
    qninf |= q == -INFINITY;
  }
  if (resid && (qnan || (qpinf && qninf) || !isfinite(W))) {
    if (a.shard == 0) emit_invalid(a, b, kFlagNonfinite | extra);
    return;
  }
  int fallback = 0;
  bool use_p = !resid;
  double total = resid ? W : P;
  if (resid && !(W > 0.0)) {  // no residual mass: draw from p_m
    fallback = kFlagFallback;
    use_p = true;
    total = P;
  }
  const double target = static_cast<double>(u) * total;
  // the shard holding the target: the first with weight whose running sum exceeds it
  int gs = -1, glast = -1;
  double base = 0.0, run = 0.0, base_last = 0.0;
  for (int g = 0; g < G; ++g) {
    const double wg = use_p ? lane_d(mp, g) : lane_d(mw, g);
    if (wg > 0.0) {
      if (gs < 0 && run + wg > target) {
        gs = g;
        base = run;
      }
      glast = g;
      base_last = run;
    }
    run += wg;
  }
  if (gs < 0) {
    gs = glast;
    base = base_last;
  }
  if (gs < 0) {
    if (a.shard == 0) emit_invalid(a, b, kFlagNonfinite | fallback | extra);
    return;
  }
  if (gs != a.shard) return;
  const int64_t c0 = a.sb.b[a.shard], vg = a.sb.b[a.shard + 1] - c0;
  const int nt = static_cast<int>((vg + kSampleTile - 1) / kSampleTile);
  const double* tw = a.tiles + b64 * a.tile_cap * 2 + (use_p ? 1 : 0);
  int ta, tb;
  lane_tiles(nt, lane, ta, tb);
  double own = 0.0;
  for (int i = ta; i < tb; ++i) own += tw[i * 2];
  TileHit hit;
  if (!wave_find_tile(tw, 2, nt, own, target - base, hit)) {
    emit_invalid(a, b, kFlagNonfinite | fallback | extra);
    return;
  }
  hit.base += base;
  const MS st = wave_shard_combine(a.pairs, G, a.t_rows, ts + m);
  const DrawRow r{row_ptr<DT>(a.tgt, ts + m, vg), use_p ? nullptr : row_ptr<DQ>(a.dq, qs + m, vg), a.c, st.m,
                  1.f / st.s, 1.f, !use_p};
  const int y = wave_pick_in_tile<DT, DQ>(r, vg, hit, target);
  emit_round(a, b, m, static_cast<int>(c0 + y), static_cast<float>(total), fallback | extra);
}

// ---- host side ----

namespace {

template <class DT, class DQ>
void launch_stats_t(const ShardArgs& a, float* at, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(a.B) * a.k_max;
  if (n > 0)
    hipLaunchKernelGGL((k_shard_gather<DT, DQ>), dim3(static_cast<uint32_t>((n + kBlock - 1) / kBlock)),
                       dim3(kBlock), 0, stream, a, at);
}

template <class DT, class DQ>
void launch_res_t(const ShardArgs& a, int step, hipStream_t stream) {
  if (step == 2)
    hipLaunchKernelGGL((k_shard_residual<DT, DQ>), dim3(static_cast<uint32_t>(a.B)), dim3(kShardBlock), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((k_shard_draw<DT, DQ>),
                       dim3(static_cast<uint32_t>((a.B + kBlock / kWave - 1) / (kBlock / kWave))), dim3(kBlock), 0,
                       stream, a);
}

}  // namespace

hipError_t launch_shard_fold(const float2* partial, int64_t rows, int32_t nseg, float* pairs, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_shard_fold, dim3(static_cast<uint32_t>((rows + kBlock / kWave - 1) / (kBlock / kWave))),
                     dim3(kBlock), 0, stream, partial, rows, nseg, pairs);
  return hipGetLastError();
}

hipError_t launch_shard_step(int step, int t_dtype, int q_dtype, const ShardArgs& a, float* at, hipStream_t stream) {
  const bool tb = t_dtype == kDtypeBF16, qb = q_dtype == kDtypeBF16;
  if (step == 1) {
    if (tb && qb) launch_stats_t<BF16, BF16>(a, at, stream);
    else if (tb) launch_stats_t<BF16, F32>(a, at, stream);
    else if (qb) launch_stats_t<F32, BF16>(a, at, stream);
    else launch_stats_t<F32, F32>(a, at, stream);
  } else {
    if (tb && qb) launch_res_t<BF16, BF16>(a, step, stream);
    else if (tb) launch_res_t<BF16, F32>(a, step, stream);
    else if (qb) launch_res_t<F32, BF16>(a, step, stream);
    else launch_res_t<F32, F32>(a, step, stream);
  }
  return hipGetLastError();
}

}  // namespace sv
