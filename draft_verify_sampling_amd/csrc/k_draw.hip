// The last stage of a sampled chain round: the accept scan's outcome, the
// residual pass over the break row and the inverse-CDF draw.
//
// Method ("投机解码:为什么一个字都不改", sections "改进:接受概率 min(1, p/q),
// 拒绝时从残差重采" and "一轮能出几个 token"): with p_i = softmax(target row i / T),
// draft i is kept iff u_i q_i(x_i) < p_i(x_i); the round stops at the first
// draft that is not kept (m), and the last token is drawn from
// norm(max(0, p_m - q_m)), or from p_k when every draft is kept: the smallest
// id whose running weight exceeds u_k times the total.
//
// It runs after a statistics kernel that left either the softmax partials of
// every target row (k_row_stats) or, for rounds whose requests own their rows,
// the break row already decided with its softmax pair (k_chain_stats).  Grid:
// B x nblk blocks of 256 threads; block r of request b:
//   1. one wave finds the break row m and its pair: from the partials (the
//      rows' pairs combined in the canonical order, the drafts tested in
//      turn, stopping at the first not kept) or from the lazy statistics'
//      words.  Every block of the request takes the same decision, bit for
//      bit;
//   2. each wave sums tpw tiles of the block's run of 4 tpw tiles of the break
//      row: the weights max(0, p_m - q_m) (or p_k), p_m (for the zero-mass
//      fallback) and q_m (its NaN class), and stores each tile's sums (tpw is
//      chosen by the host so that every block of the grid is resident at
//      once, each paying the one-round prologue once);
//   3. the request's last block to finish (an atomic count) gathers the tile
//      sums, finds the tile holding u_k times the total, re-reads that tile,
//      picks the id and writes the request's outputs.
// No block waits for another block to run: the last one only waits for the
// visibility of words every other block stored before counting itself, so the
// kernel needs no particular residency.  Data moves between blocks inside
// 64-bit words with a valid bit (relaxed agent-scope atomics, no fences); the
// statistics kernel zeroes them before this kernel starts.
#include <algorithm>
#include <atomic>

#include "launch.hpp"
#include "tiles.hpp"
#include "timeline.hpp"
#include "words.hpp"

// Time line of each draw block (builds with -DSV_TIMELINE only): record =
// block index; slot 0 its start, 1 the break row known, 2 its tiles summed, 3
// its count returned; the request's last block: 4 the tile sums gathered, 5
// the tile found, 6 the id picked, 7 the outputs written.
SV_TIMELINE_ARRAY(sv_timeline_draw)

namespace sv {

namespace {

__device__ __forceinline__ bool request_ok(const ChainDrawArgs& a, int b, int& k, int& ts, int& qs) {
  k = a.dlen[b];
  ts = a.t_rs[b];
  qs = a.q_rs[b];
  return k >= 0 && k <= a.k_max && ts >= 0 && static_cast<int64_t>(ts) + k < a.t_rows &&
         (k == 0 || (qs >= 0 && static_cast<int64_t>(qs) + k <= a.q_rows));
}

// Outputs of an invalid request, written by one wave.
__device__ void draw_invalid(const ChainDrawArgs& a, int b, int bits) {
  const int lane = threadIdx.x & (kWave - 1);
  const int width = a.k_max + 1;
  for (int c = lane; c < width; c += kWave) a.out_tok[static_cast<int64_t>(b) * width + c] = -1;
  if (lane == 0) {
    a.out_cnt[b] = 0;
    a.out_acc[b] = 0;
    if (a.resid != nullptr) a.resid[b] = 0.f;
    flag(a.status, bits);
  }
}

struct BreakRow {
  int m;       // the row the last token is drawn from
  int bad;     // a drafted token is out of range
  float pm, ps;  // its softmax pair (scaled-domain max, normaliser); ps NaN: not available
};

constexpr int kPreRows = 8;  // rows whose partials one wave loads before deciding

// The break row of request b from the softmax partials of its rows (one wave).
// Row r's pair combines its segment pairs in the canonical order; the first
// row whose normaliser is not finite and positive, whose draft is not kept, or
// r = k ends the round.  Lane i holds draft i and its uniform (rows < 64) on
// entry; the partials of the first rows and the values at the drafted tokens
// are then loaded together, one round.
template <class DT, class DQ>
__device__ BreakRow break_from_partials(const ChainDrawArgs& a, int b, int k, int ts, int qs, int x, float u) {
  const int lane = threadIdx.x & (kWave - 1);
  const int R = a.k_max + 1;
  const bool one = a.nseg <= kWave;
  float2 pre[kPreRows];
#pragma unroll
  for (int r = 0; r < kPreRows; ++r) {
    pre[r] = make_float2(-INFINITY, 0.f);
    if (one && r <= k && lane < a.nseg) pre[r] = a.partial[(static_cast<int64_t>(ts) + r) * a.nseg + lane];
  }
  float lx = 0.f, qx = 0.f;
  BreakRow br{k, 0, 0.f, NAN};
  for (int r = 0; r <= k; ++r) {
    if ((r & (kWave - 1)) == 0) {
      // lane i: the two values at draft r + i (its token and uniform are
      // reloaded past the first 64 rows)
      const int i = r + lane;
      if (r > 0) {
        x = i < k ? a.ids[static_cast<int64_t>(b) * a.k_max + i] : -1;
        u = i <= k ? slot_uniform(a.u, a.seed, a.offset, b, R, i) : 0.f;
      }
      lx = qx = 0.f;
      if (i < k && x >= 0 && x < a.V) {
        lx = DT::at(row_ptr<DT>(a.tgt, ts + i, a.V), x);
        qx = DQ::at(row_ptr<DQ>(a.dq, qs + i, a.V), x);
      }
    }
    const float2* pp = a.partial + (static_cast<int64_t>(ts) + r) * a.nseg;
    MS row;
    if (one && r < kPreRows) {
      float2 v = pre[0];
#pragma unroll
      for (int q = 1; q < kPreRows; ++q) v = r == q ? pre[q] : v;
      row = wave_combine_segments(a.nseg, [&](int) { return MS{v.x, v.y}; });
    } else {
      row = wave_combine_segments(a.nseg, [&](int sg) {
        const float2 v = pp[sg];
        return MS{v.x, v.y};
      });
    }
    bool stop = !(row.s > 0.f && row.s < INFINITY) || r == k;
    if (!stop) {
      const int src = r & (kWave - 1);
      const float ur = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(u), src));
      const float lr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lx), src));
      const float qr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(qx), src));
      stop = !(ur * qr < ex2(fmaf(lr, a.c, -row.m)) * (1.f / row.s));
    }
    if (stop) {
      br.m = r;
      br.pm = row.m;
      br.ps = row.s;
      return br;
    }
  }
  return br;
}

// Wave 0 of the last block: the tile holding u_k W among the tile sums
// s_tw[0, ntiles) (mine: the lane's own sum over lane_tiles, in order).
// Returns 1, or 0 when no tile has weight (the outputs are then written).
__device__ __forceinline__ int last_block_pick_tile(const ChainDrawArgs& a, int b, int k, float u0,
                                                    const double* s_tw, double mine, double W, int bits,
                                                    TileHit& s_hit, double& s_target) {
  const int lane = threadIdx.x & (kWave - 1);
  // the last token's uniform: lane k of this wave loaded it at the start
  const float uk = k < kWave ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(u0), k))
                             : slot_uniform(a.u, a.seed, a.offset, b, a.k_max + 1, k);
  const double target = static_cast<double>(uk) * W;
  TileHit hit;
  if (!wave_find_tile(s_tw, 1, a.ntiles, mine, target, hit)) {
    draw_invalid(a, b, kFlagNonfinite | bits);
    return 0;
  }
  if (lane == 0) {
    s_hit = hit;
    s_target = target;
    SV_STAMP(sv_timeline_draw, blockIdx.x, 5);
  }
  return 1;
}

// The last block's wave 0: gathers the request's tile sums of the draw
// weights and the block classes, and totals them (W).  Returns 0 when the
// request's outputs are already written (invalid) or the gather timed out,
// 3 when the residual has no mass (the caller then sums p over the row, the
// zero-mass fallback), else 1 after finding the tile holding u_k W (s_hit,
// s_target).  s_tw[t]: the tile sums (the first ntiles doubles).
template <class DT, class DQ>
__device__ __forceinline__ int last_block_find(const ChainDrawArgs& a, int b, int k, int extra, float u0,
                                               bool resid, double* s_tw, int& bits, double& W,
                                               TileHit& s_hit, double& s_target) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t* tw = a.tile_w + static_cast<int64_t>(b) * a.ntiles;
  const uint64_t* bq = a.blk_q + static_cast<int64_t>(b) * a.nblk;
  int ta, tb;
  lane_tiles(a.ntiles, lane, ta, tb);
  constexpr int kBatch = 4;
  double wsum = 0.0;
  uint64_t cls = 0;
  bool ok = true;
  for (int t0 = ta, first = 1; ok && (t0 < tb || first); t0 += kBatch, first = 0) {
    uint64_t vw[kBatch], vq = kValid;
    int it = 0;
    for (; it < a.spin_limit; ++it) {
      bool mine = true;
      if (first) {
        for (int j = lane; j < a.nblk; j += kWave) {
          const uint64_t v = load_word(bq + j);
          mine = mine && (v & kValid) != 0;
          vq = j == lane ? v : (vq | v);
        }
      }
#pragma unroll
      for (int x = 0; x < kBatch; ++x) {
        vw[x] = kValid;
        if (t0 + x < tb) vw[x] = load_word(tw + t0 + x);
        mine = mine && (vw[x] & kValid);
      }
      if (__all(mine)) break;
      __builtin_amdgcn_s_sleep(1);
    }
    ok = it < a.spin_limit;
    if (first) cls = lane < a.nblk ? vq : 0ull;
#pragma unroll
    for (int x = 0; x < kBatch; ++x) {
      if (t0 + x < tb) {
        const double dw = dec_sum(vw[x]);
        s_tw[t0 + x] = dw;
        wsum += dw;
      }
    }
  }
  if (!__all(ok)) {
    if (lane == 0) flag(a.status, kFlagSyncTimeout);
    return 0;
  }
  if (lane == 0) SV_STAMP(sv_timeline_draw, blockIdx.x, 4);
  for (int sft = 32; sft >= 1; sft >>= 1)
    cls |= static_cast<uint64_t>(__shfl_xor(static_cast<long long>(cls), sft));
  W = wave_total(wsum);
  bits = extra;
  if (resid) {
    if (qclass_nan(cls) || !isfinite(W)) {
      draw_invalid(a, b, kFlagNonfinite | extra);
      return 0;
    }
    if (!(W > 0.0)) return 3;  // no residual mass: the row's p sums are needed
  }
  return last_block_pick_tile(a, b, k, u0, s_tw, wsum, W, bits, s_hit, s_target);
}

}  // namespace

// Dynamic LDS: the gathered tile sums, ntiles doubles.
template <class DT, class DQ>
__global__ __launch_bounds__(kBlock) void k_chain_draw(ChainDrawArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* s_tw = reinterpret_cast<double*>(smem);
  __shared__ BreakRow s_br;
  __shared__ uint64_t s_q[kDrawTiles];
  __shared__ int s_last;
  const int b = static_cast<int>(blockIdx.x / a.nblk);
  const int r = static_cast<int>(blockIdx.x - static_cast<int64_t>(b) * a.nblk);
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  if (threadIdx.x == 0) SV_STAMP(sv_timeline_draw, blockIdx.x, 0);
  // the first wave's draft tokens and uniforms are loaded with the request's
  // row starts and draft count (they depend on b alone)
  int x0 = -1;
  float u0 = 0.f;
  if (wid == 0) {
    if (lane < a.k_max) x0 = a.ids[static_cast<int64_t>(b) * a.k_max + lane];
    if (lane <= a.k_max) u0 = slot_uniform(a.u, a.seed, a.offset, b, a.k_max + 1, lane);
  }
  int k, ts, qs;
  if (!request_ok(a, b, k, ts, qs)) {
    if (r == 0 && wid == 0) draw_invalid(a, b, kFlagBadRequest);
    return;
  }
  const int extra = (a.max_new != nullptr && k > a.max_new[b]) ? kFlagOverBudget : 0;

  // 1. the break row and its pair; every drafted token in range?
  if (wid == 0) {
    bool bad = __ballot(lane < k && (x0 < 0 || x0 >= a.V)) != 0;
    for (int i0 = kWave; i0 < k; i0 += kWave) {
      const int i = i0 + lane;
      const int xi = i < k ? a.ids[static_cast<int64_t>(b) * a.k_max + i] : 0;
      bad |= __ballot(i < k && (xi < 0 || xi >= a.V)) != 0;
    }
    BreakRow br;
    if (a.partial != nullptr) {
      br = bad ? BreakRow{0, 0, 0.f, NAN} : break_from_partials<DT, DQ>(a, b, k, ts, qs, x0, u0);
    } else {
      // decided by the lazy statistics: the first row that stops the round
      // and that row's pair (absent if its statistics did not complete)
      const uint32_t sw = a.stop[b];
      br.m = sw != 0 ? kMaxChainRows - static_cast<int>(sw) : k;
      const uint64_t rw = a.row_words[static_cast<int64_t>(b) * (a.k_max + 1) + br.m];
      const MS p = dec_ms(rw);
      br.pm = p.m;
      br.ps = (rw & kValid) ? p.s : NAN;
    }
    br.bad = bad ? 1 : 0;
    if (lane == 0) s_br = br;
  }
  __syncthreads();
  if (threadIdx.x == 0) SV_STAMP(sv_timeline_draw, blockIdx.x, 1);
  const BreakRow br = s_br;
  if (br.bad) {
    if (r == 0 && wid == 0) draw_invalid(a, b, kFlagBadToken);
    return;
  }
  if (!(br.ps > 0.f && br.ps < INFINITY)) {
    if (r == 0 && wid == 0) draw_invalid(a, b, kFlagNonfinite | extra);
    return;
  }
  const int m = br.m;
  const bool resid = m < k;
  DrawRow row{row_ptr<DT>(a.tgt, ts + m, a.V), resid ? row_ptr<DQ>(a.dq, qs + m, a.V) : nullptr, a.c, br.pm,
              1.f / br.ps, 1.f, resid};

  // 2. the block's tiles, wave w taking tiles w, w + 4, ...: sums of
  // max(0, p - q) (or p) and of q
  double qsum = 0.0;
  const int t_first = r * kDrawTiles * a.tpw;
  for (int i = 0; i < a.tpw; ++i) {
    const int t = t_first + i * kDrawTiles + wid;
    if (t >= a.ntiles) break;
    double v[1][3];
    if (resid)
      wave_tile_sums<DT, DQ, 1, true, 0, false, false, true>(row, a.V, t, 0, v);
    else
      wave_tile_sums<DT, DQ, 1, false, 0, false, false>(row, a.V, t, 0, v);
    qsum += v[0][2];
    if (lane == 0) store_word(a.tile_w + static_cast<int64_t>(b) * a.ntiles + t, enc_sum(v[0][0]));
  }
  if (lane == 0) s_q[wid] = enc_qclass(qsum);
  __syncthreads();
  if (threadIdx.x == 0) {
    SV_STAMP(sv_timeline_draw, blockIdx.x, 2);
    uint64_t cls = 0;
    for (int w = 0; w < kDrawTiles; ++w) cls |= s_q[w];
    store_word(a.blk_q + static_cast<int64_t>(b) * a.nblk + r, cls);
    const uint32_t done = __hip_atomic_fetch_add(a.rcnt + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = done == static_cast<uint32_t>(a.nblk - 1);
    SV_STAMP(sv_timeline_draw, blockIdx.x, 3);
  }
  __syncthreads();
  if (!s_last) return;

  // 3. the request's last block: wave 0 gathers the tile sums and the classes
  // of the draft row's block sums (loads in flight a batch at a time, waiting
  // only for their visibility), totals them and finds the tile; the block's
  // four waves then pick the id in it.  When the residual has no mass the
  // four waves first sum p over the break row's tiles (the zero-mass
  // fallback draws from p_m).
  __shared__ PickLds s_pick;
  __shared__ TileHit s_hit;
  __shared__ double s_target;
  __shared__ int s_go;  // 0: done (invalid), 1: pick from the row's weights, 2: from p_m, 3: p sums needed
  int bits = extra;
  double W = 0.0;
  if (wid == 0) {
    const int go = last_block_find<DT, DQ>(a, b, k, extra, u0, resid, s_tw, bits, W, s_hit, s_target);
    if (lane == 0) s_go = go;
  }
  __syncthreads();
  if (s_go == 3) {
    DrawRow prow = row;
    prow.use_q = false;
    for (int t = wid; t < a.ntiles; t += kDrawTiles) {
      double v[1][3];
      wave_tile_sums<DT, DQ, 1, false, 0, false, false>(prow, a.V, t, 0, v);
      if (lane == 0) s_tw[t] = v[0][0];
    }
    __syncthreads();
    if (wid == 0) {
      int ta, tb;
      lane_tiles(a.ntiles, lane, ta, tb);
      double psum = 0.0;
      for (int t = ta; t < tb; ++t) psum += s_tw[t];
      bits |= kFlagFallback;
      W = wave_total(psum);
      const int go = last_block_pick_tile(a, b, k, u0, s_tw, psum, W, bits, s_hit, s_target);
      if (lane == 0) s_go = go == 1 ? 2 : 0;
    }
    __syncthreads();
  }
  const int go = s_go;
  if (go == 0) return;
  if (go == 2) row.use_q = false;  // the zero-mass fallback draws from p_m
  const int y = block_pick_in_tile<DT, DQ>(row, a.V, s_hit, s_target, s_pick);
  if (wid != 0) return;
  if (lane == 0) SV_STAMP(sv_timeline_draw, blockIdx.x, 6);
  // emission: drafts 0..m-1 then y, cut after the first end token and at the
  // budget (lane c of this wave holds draft c from the start, c < 64)
  const int width = a.k_max + 1;
  int32_t* out = a.out_tok + static_cast<int64_t>(b) * width;
  const int32_t* xs = a.ids + static_cast<int64_t>(b) * a.k_max;
  auto draft_at = [&](int c) { return c < kWave ? x0 : xs[c]; };  // c = c0 + lane
  int cnt = m + 1;
  for (int c0 = 0; c0 <= m; c0 += kWave) {  // the first end token among positions 0..m
    const int c = c0 + lane;
    const int tok = c < m ? draft_at(c) : y;
    const uint64_t hit_eos = a.eos >= 0 ? __ballot(c <= m && tok == a.eos) : 0ull;
    if (hit_eos) {
      cnt = c0 + __ffsll(static_cast<long long>(hit_eos));
      break;
    }
  }
  if (a.max_new != nullptr) {
    const int budget = a.max_new[b] > 0 ? a.max_new[b] : 0;
    cnt = cnt < budget ? cnt : budget;
  }
  for (int c = lane; c < width; c += kWave) out[c] = c < cnt ? (c < m ? draft_at(c) : y) : -1;
  if (lane == 0) {
    a.out_cnt[b] = cnt;
    a.out_acc[b] = m;
    if (a.resid != nullptr) a.resid[b] = static_cast<float>(W);
    flag(a.status, bits);
    SV_STAMP(sv_timeline_draw, blockIdx.x, 7);
  }
}

static_assert(kDrawTiles == kBlock / kWave, "one tile per wave and step");

namespace {
template <class DT, class DQ>
const void* draw_fn() {
  return reinterpret_cast<const void*>(&k_chain_draw<DT, DQ>);
}
}  // namespace

int draw_occupancy(int t_dtype, int q_dtype, size_t lds) {
  static std::atomic<int> cache[2][2][16];  // by dtypes and 4 KB of LDS
  const int tb = t_dtype == kDtypeBF16, qb = q_dtype == kDtypeBF16;
  const size_t bucket = std::min<size_t>(lds / 4096, 15);
  std::atomic<int>& slot = cache[tb][qb][bucket];
  if (const int n = slot.load(std::memory_order_relaxed)) return n;
  const void* fn = tb ? (qb ? draw_fn<BF16, BF16>() : draw_fn<BF16, F32>()) : (qb ? draw_fn<F32, BF16>() : draw_fn<F32, F32>());
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kBlock, (bucket + 1) * 4096) != hipSuccess || n < 1) n = 1;
  slot.store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_chain_draw(int t_dtype, int q_dtype, const ChainDrawArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(a.B) * a.nblk)), block(kBlock);
  const size_t lds = static_cast<size_t>(a.ntiles) * sizeof(double);
  const bool tb = t_dtype == kDtypeBF16, qb = q_dtype == kDtypeBF16;
  if (tb && qb)
    hipLaunchKernelGGL((k_chain_draw<BF16, BF16>), grid, block, lds, stream, a);
  else if (tb)
    hipLaunchKernelGGL((k_chain_draw<BF16, F32>), grid, block, lds, stream, a);
  else if (qb)
    hipLaunchKernelGGL((k_chain_draw<F32, BF16>), grid, block, lds, stream, a);
  else
    hipLaunchKernelGGL((k_chain_draw<F32, F32>), grid, block, lds, stream, a);
  return hipGetLastError();
}

}  // namespace sv
