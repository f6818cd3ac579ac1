// Speculative-sampling verify of draft trees as a walk, plus the one-wave
// chain round for one-tile vocabularies and the diagnostics kernels.
//
// Method ("投机解码:为什么一个字都不改", sections "改进:接受概率 min(1, p/q),
// 拒绝时从残差重采" and "一轮能出几个 token"; "Speculative Decoding II", EAGLE
// section, for trees verified by applying speculative sampling recursively as
// SpecInfer does):
//   cur = root, p = softmax(target row of cur / T), q = draft row of cur;
//   for each child c of cur in index order: keep iff u * q(x_c) < p(x_c);
//   kept -> emit x_c, descend, reload p and q; rejected -> p <- norm(max(0, p - q)).
//   With no child kept (or at a leaf) the last token is drawn from the current
//   p: the smallest id whose running mass exceeds u times the total.
//
// Repeated residual updates against one q stay in closed form: after j
// rejections the current distribution is max(0, p - c_j q) / R_j with
// c_0 = 0, R_0 = 1, c_{j+1} = c_j + R_j and R_{j+1} = sum max(0, p - c_{j+1} q),
// so every rejection costs one pass over the node's two rows that yields
// R_{j+1} and the per-tile sums the final inverse-CDF draw needs.  The
// node's first such pass also leaves p and q of the workgroup's slice in LDS
// (when the host finds room: 16 KB per tile), and its later passes read that
// copy instead of the rows: the same weights in the same order, so the same
// sums, without the loads or the exponentials.
//
// Statistics: the walk computes the statistics of a node when it arrives there
// (one pass over that row), so only the rows of its kept path are read.
//
// Work split: G workgroups of 512 threads per request, G chosen by the host
// from the occupancy of this kernel so that the whole grid is resident at
// once (G = resident workgroups / requests, at most 32).  Workgroup g owns a
// contiguous slice of the vocabulary's 2048-element tiles; each pass (softmax
// pair of a target row, or a residual / plain weight pass) covers only the
// slice.  The G partial results of a pass are exchanged
// through 64-bit words in the workspace: each workgroup stores its words with
// relaxed agent-scope atomic stores and reads the others' with relaxed
// agent-scope atomic loads until all carry their valid bit.  The data travels
// inside the atomic words, so no fence is needed.  The words start at zero:
// each workgroup zeroes its own words at its start, waits until those stores
// have completed, and then stores the call's ticket, and the request's first
// exchange polls the G tickets before any word, so no word left by an earlier
// call is read (under graph capture k_walk_clear zeroes them before the walk
// instead).  Every workgroup combines the G words in the same order, so all
// of them take the same decisions.  The wait is bounded: on expiry the
// workgroup sets the sync-timeout status bit and exits.  With G = 1 nothing is
// exchanged through memory.
//
// The last token is drawn by the workgroup whose slice holds u * R: one wave
// scans the slice's tile sums (kept in LDS) and rescans the chosen tile.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "tiles.hpp"
#include "timeline.hpp"
#include "words.hpp"

// Time line of each workgroup (builds with -DSV_TIMELINE only): record
// b * G + g; slot 0 the start, 1 the end of the prologue; for exchange n < 9
// the slots 2 + 6 n + (0 the pass starts, 1 its tile sums are in LDS, 2 the
// exchange starts, 3 wave 0 has seen every word, 4 the exchange's barrier is
// passed, 5 the words are folded); 60 the slice of the last draw is known, 61
// the drawing wave starts, 62 its tile is found, 63 the outputs are written.
// The readings go to LDS first and to the record at the workgroup's end.
SV_TIMELINE_ARRAY(sv_timeline_walk)
#ifdef SV_TIMELINE
__shared__ uint64_t sv_walk_tl[sv::kTimelineSlots];
#define WALK_TL(slot)                                                                 \
  do {                                                                                \
    if (threadIdx.x == 0 && (slot) < 60) sv_walk_tl[(slot)] = sv::timeline_now();     \
  } while (0)
#define WALK_TL_DRAW(slot)                                                            \
  do {                                                                                \
    if (threadIdx.x == 0) sv_walk_tl[(slot)] = sv::timeline_now();                     \
  } while (0)
#else
#define WALK_TL(slot) ((void)0)
#define WALK_TL_DRAW(slot) ((void)0)
#endif

namespace sv {

namespace {

constexpr int kWalkWaves = kWalkBlock / kWave;
constexpr int kXcds = 8;  // accelerator complex dies of an MI355X
constexpr int kMaxNodeGroups = kMaxTreeNodes / kWave;
static_assert(2 * kMaxWalkGroups <= kWave, "one wave reads every exchanged word");
static_assert(kMaxChainRows <= kWalkBlock, "one chain row per thread");

struct Walk {
  const WalkArgs* a;
  int b, g;
  int lo, hi;       // this workgroup's tiles [lo, hi)
  int nsync;        // exchanges so far (the same count in every workgroup)
  uint64_t* s_x;    // LDS [2][2 * kMaxWalkGroups]
  int* s_ok;        // LDS [2]
};

// Publish (w0, w1) and collect every workgroup's pair into the LDS words
// [2h], [2h + 1] of the current buffer.  Returns false when the bounded wait
// expired.  Ends with a block barrier.
__device__ __forceinline__ bool exchange(Walk& wk, uint64_t w0, uint64_t w1) {
  const WalkArgs& a = *wk.a;
  const int lane = threadIdx.x & (kWave - 1);
  const int buf = wk.nsync & 1;
  uint64_t* x = wk.s_x + buf * 2 * kMaxWalkGroups;
  WALK_TL(2 + 6 * wk.nsync + 2);
  if (a.G == 1) {
    if (threadIdx.x == 0) {
      x[0] = w0;
      x[1] = w1;
      wk.s_ok[buf] = 1;
    }
  } else if (wk.nsync >= a.max_sync) {  // more exchanges than a walk can need: never taken
    if (threadIdx.x == 0) wk.s_ok[buf] = 0;
  } else {
    uint64_t* row = a.slots + (static_cast<int64_t>(wk.b) * a.max_sync + wk.nsync) * 2 * a.G;
    if (threadIdx.x == 0) {
      store_word(row + 2 * wk.g, w0);
      store_word(row + 2 * wk.g + 1, w1);
    }
    if (threadIdx.x < kWave) {
      const int n = 2 * a.G;
      uint64_t v = 0;
      int done = 0;
      int it = 0;
      if (wk.nsync == 0 && a.arrive != nullptr) {
        // the tickets first: a workgroup's words are read only once its
        // zeroing of them has completed (the polls share one budget)
        const uint64_t* arr = a.arrive + static_cast<int64_t>(wk.b) * a.G;
        for (; it < a.spin_limit; ++it) {
          if (__all(lane >= a.G || load_word(arr + lane) == a.ticket)) break;
          __builtin_amdgcn_s_sleep(1);
        }
      }
      for (; it < a.spin_limit; ++it) {
        if (lane < n) v = load_word(row + lane);
        if (__all(lane >= n || (v & kValid) != 0)) {
          done = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (lane < n) x[lane] = v;
      if (lane == 0) wk.s_ok[buf] = done;
      WALK_TL(2 + 6 * wk.nsync + 3);
    }
  }
  __syncthreads();
  WALK_TL(2 + 6 * wk.nsync + 4);
  ++wk.nsync;
  return wk.s_ok[buf] != 0;
}

__device__ __forceinline__ const uint64_t* last_words(const Walk& wk) {
  return wk.s_x + ((wk.nsync - 1) & 1) * 2 * kMaxWalkGroups;
}

// Softmax pair of a target row over the slice, combined across the request.
template <class DT>
__device__ __forceinline__ bool row_stats(Walk& wk, const void* trow, MS* s_wms, MS& out) {
  const WalkArgs& a = *wk.a;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  MS acc{-INFINITY, 0.f};
  WALK_TL(2 + 6 * wk.nsync + 0);
  for (int t = wk.lo + wid; t < wk.hi; t += kWalkWaves) {
    MS v, unused;
    wave_tile_ms<DT, false>(trow, nullptr, a.V, a.c, t, v, unused);
    acc = ms_combine(acc, v);
  }
  if (lane == 0) s_wms[wid] = acc;
  __syncthreads();
  WALK_TL(2 + 6 * wk.nsync + 1);
  MS r = s_wms[0];
  for (int w = 1; w < kWalkWaves; ++w) r = ms_combine(r, s_wms[w]);
  if (!exchange(wk, enc_ms(r), kValid)) return false;
  const uint64_t* x = last_words(wk);
  MS m = dec_ms(x[0]);
  for (int h = 1; h < a.G; ++h) m = ms_combine(m, dec_ms(x[2 * h]));
  out = m;
  WALK_TL(2 + 6 * (wk.nsync - 1) + 5);
  return true;
}

// How a residual weight pass of the sampled tree walk uses the LDS copy of
// its slice's draw inputs: not at all, filling it (the node's first residual
// pass), or reading it instead of the rows (the node's later passes).
constexpr int kCacheNone = 0, kCacheFill = 1, kCacheUse = 2;

// One weight pass over the slice: per-tile weight sums into wt[] (slice-local
// index); then, across the request, the total W and the NaN-ness of the draft
// row's sum.  Every slice's total stays readable in the exchanged words until
// the next exchange.  With kCacheFill / kCacheUse, `cache` is the slice's LDS
// copy (tile i: p, then q) and *qcls the draft-sum class word of this
// workgroup's slice, stored by the fill and sent again by later passes (the
// draft row is the same, so is its class).
// kResid: a residual pass (r.use_q holds): the weights take the draft row
// without a per-element select.  (No pass reads the p sums, so none forms them.)
template <class DT, class DQ, bool kQ = true, int kCache = kCacheNone, bool kResid = false>
__device__ __forceinline__ bool weight_pass(Walk& wk, const DrawRow& r, double* wt, double* s_wq, double& W, bool& qnan,
                                            float4* cache = nullptr, uint64_t* qcls = nullptr) {
  const WalkArgs& a = *wk.a;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  using TC = TileCache<DT, DQ>;
  double qw = 0.0;
  WALK_TL(2 + 6 * wk.nsync + 0);
  for (int t = wk.lo + wid; t < wk.hi; t += kWalkWaves) {
    const int i = t - wk.lo;
    TC tc;
    if constexpr (kCache != kCacheNone) {
      tc.p = cache + static_cast<int64_t>(2 * i) * TC::kFloat4;
      tc.q = tc.p + TC::kFloat4;
    }
    if constexpr (kCache == kCacheUse) {
      const double s = wave_tile_wsum_cached<DT, DQ>(tc, r.coef);
      if (lane == 0) wt[i] = s;
    } else {
      double v[1][3];
      wave_tile_sums<DT, DQ, 1, kQ, 0, kCache == kCacheFill, false, kResid>(r, a.V, t, 0, v, tc);
      if (lane == 0) wt[i] = v[0][0];
      qw += v[0][2];
    }
  }
  if (lane == 0) s_wq[wid] = qw;
  __syncthreads();
  WALK_TL(2 + 6 * wk.nsync + 1);
  int ta, tb;
  lane_tiles(wk.hi - wk.lo, lane, ta, tb);
  double w = 0.0;
  for (int i = ta; i < tb; ++i) w += wt[i];
  w = wave_total(w);
  uint64_t w1;
  if constexpr (kCache == kCacheUse) {
    w1 = *qcls;
  } else {
    double q = s_wq[0];
    for (int i = 1; i < kWalkWaves; ++i) q += s_wq[i];
    w1 = enc_qclass(q);
    if constexpr (kCache == kCacheFill) *qcls = w1;
  }
  if (!exchange(wk, enc_sum(w), w1)) return false;
  const uint64_t* x = last_words(wk);
  double tot = 0.0;
  uint64_t cls = 0;
  for (int h = 0; h < a.G; ++h) {
    tot += dec_sum(x[2 * h]);
    cls |= x[2 * h + 1];
  }
  W = tot;
  qnan = qclass_nan(cls);
  WALK_TL(2 + 6 * (wk.nsync - 1) + 5);
  return true;
}

// Argmax of a target row over the slice, combined across the request (the
// largest value, the lowest id among equal values); nan: the row holds a NaN.
template <class DT>
__device__ __forceinline__ bool row_argmax(Walk& wk, const void* trow, uint64_t* s_key, uint32_t* s_knan, int& amax,
                           bool& nan) {
  const WalkArgs& a = *wk.a;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  ArgBest s{-INFINITY, 0x7fffffff, false};
  WALK_TL(2 + 6 * wk.nsync + 0);
  for (int t = wk.lo + wid; t < wk.hi; t += kWalkWaves) lane_tile_argmax<DT>(trow, a.V, t, s);
  const uint64_t key =
      wave_max_u64((static_cast<uint64_t>(order_bits(s.v)) << 32) | static_cast<uint32_t>(~s.i));
  const bool wnan = __ballot(s.nan) != 0;
  if (lane == 0) {
    s_key[wid] = key;
    s_knan[wid] = wnan ? 1u : 0u;
  }
  __syncthreads();
  WALK_TL(2 + 6 * wk.nsync + 1);
  uint64_t k = s_key[0];
  uint32_t n = s_knan[0];
  for (int w = 1; w < kWalkWaves; ++w) {
    k = s_key[w] > k ? s_key[w] : k;
    n |= s_knan[w];
  }
  if (!exchange(wk, kValid | (static_cast<uint64_t>(n) << 32) | (k >> 32), kValid | (k & 0xffffffffull)))
    return false;
  const uint64_t* x = last_words(wk);
  uint64_t best = 0;
  bool any_nan = false;
  for (int h = 0; h < a.G; ++h) {
    const uint64_t kk = ((x[2 * h] & 0xffffffffull) << 32) | (x[2 * h + 1] & 0xffffffffull);
    best = kk > best ? kk : best;
    any_nan |= ((x[2 * h] >> 32) & 1u) != 0;
  }
  amax = static_cast<int>(~static_cast<uint32_t>(best));
  nan = any_nan;
  WALK_TL(2 + 6 * (wk.nsync - 1) + 5);
  return true;
}

// The workgroup whose slice holds tile t.
__device__ __forceinline__ int tile_owner(int t, int ntiles, int G) {
  int h = 0;
  for (int g = 1; g < G; ++g)
    if (static_cast<int64_t>(g) * ntiles / G <= t) h = g;
  return h;
}

// Outputs of an invalid request: every token and path slot -1, counts 0,
// status bits.  Threads [first, first + stride, ...) write.
__device__ __forceinline__ void walk_invalid(const WalkArgs& a, int b, int bits, int first, int stride) {
  const int64_t o = static_cast<int64_t>(b) * a.N;
  for (int c = first; c < a.N; c += stride) {
    a.out_tok[o + c] = -1;
    a.out_path[o + c] = -1;
  }
  if (first == 0) {
    a.out_cnt[b] = 0;
    a.out_acc[b] = 0;
    flag(a.status, bits);
  }
}

}  // namespace

template <int kMode, class DT, class DQ>
__global__ __launch_bounds__(kWalkBlock) void k_walk(WalkArgs a) {
  constexpr bool kPoint = kMode == kWalkPoint;
  constexpr bool kGreedy = kMode == kWalkGreedy;
  constexpr bool kUseQ = kMode == kWalkTree;  // reads draft rows
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ uint64_t s_kids[2][kMaxNodeGroups];
  __shared__ uint64_t s_x[2][2 * kMaxWalkGroups];
  __shared__ MS s_wms[kWalkWaves];
  __shared__ double s_wq[kWalkWaves];
  __shared__ uint64_t s_key[kGreedy ? kWalkWaves : 1];  // greedy: per-wave argmax keys
  __shared__ uint32_t s_knan[kGreedy ? kWalkWaves : 1];
  __shared__ double s_tot[kPoint ? kMaxWalkGroups : 1];  // point mass: slice totals
  __shared__ double s_two[2];                            // point mass: one tile's sums
  __shared__ int s_ok[2];
  __shared__ int s_bad;
  __shared__ std::conditional_t<kGreedy, char, PickLds> s_pick;  // the last draw's pick
  __shared__ TileHit s_hit;
  __shared__ int s_pick_go;

  // dynamic LDS: tile sums [2][tile_cap] doubles, then node arrays [node_cap]
  double* s_wt0 = reinterpret_cast<double*>(smem);
  double* s_wt1 = s_wt0 + a.tile_cap;
  int32_t* s_par = reinterpret_cast<int32_t*>(s_wt1 + a.tile_cap);
  int32_t* s_tok = s_par + a.node_cap;
  int32_t* s_path = s_tok + a.node_cap;
  float* s_px = reinterpret_cast<float*>(s_path + a.node_cap);
  float* s_qx = s_px + a.node_cap;
  float* s_u = s_qx + a.node_cap;
  int32_t* s_ex = reinterpret_cast<int32_t*>(s_u + a.node_cap);  // point mass: ids removed at cur
  // sampled tree walk: the LDS copy of the slice's p and q (16 KB per tile)
  float4* s_cache = reinterpret_cast<float4*>(
      smem + ((reinterpret_cast<unsigned char*>(s_ex + a.node_cap) - smem + 15) & ~static_cast<intptr_t>(15)));

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  // Workgroups are dealt to the 8 XCDs in turn (workgroup i to XCD i % 8), so
  // with B a multiple of 8 the G workgroups of a request are taken from one
  // XCD: i -> XCD x = i % 8 and rank j = i / 8 there; request (j / G) * 8 + x,
  // workgroup j % G.  Their exchanges then stay within one L2.
  int wb = static_cast<int>(blockIdx.x) / a.G, wg = static_cast<int>(blockIdx.x) % a.G;
  if (a.B % kXcds == 0) {
    const int x = static_cast<int>(blockIdx.x) % kXcds, j = static_cast<int>(blockIdx.x) / kXcds;
    wb = (j / a.G) * kXcds + x;
    wg = j % a.G;
  }
  Walk wk{&a, wb, wg, 0, 0, 0, &s_x[0][0], s_ok};
  wk.lo = static_cast<int>(static_cast<int64_t>(wk.g) * a.ntiles / a.G);
  wk.hi = static_cast<int>(static_cast<int64_t>(wk.g + 1) * a.ntiles / a.G);
  const int b = wk.b;
  const int64_t V = a.V;
#ifdef SV_TIMELINE
  if (tid < kTimelineSlots) sv_walk_tl[tid] = 0;
#endif
  WALK_TL(0);

  // ---- the request: its tree and uniforms ----
  const int N = a.N;                                     // nodes
  const int64_t trow0 = static_cast<int64_t>(b) * a.N;   // node c: target / draft row trow0 + c
  const int64_t qrow0 = trow0;
  if (tid == 0) s_bad = 0;
  // the tree and the uniforms (the greedy walk has none); this workgroup's
  // exchange words are zeroed meanwhile
  if (a.arrive != nullptr) {
    uint64_t* own = a.slots + static_cast<int64_t>(b) * a.max_sync * 2 * a.G + 2 * wk.g;
    for (int j = tid; j < 2 * a.max_sync; j += kWalkBlock)
      store_word(own + static_cast<int64_t>(j >> 1) * 2 * a.G + (j & 1), 0ull);
  }
  __syncthreads();
  for (int c = tid; c < N; c += kWalkBlock) {
    const int par = a.parent[trow0 + c];
    const int tok = a.token[trow0 + c];
    int bad = 0;
    if (c == 0 ? par != -1 : (par < 0 || par >= c)) bad |= kFlagBadTree;
    if (c > 0 && (tok < 0 || tok >= V)) bad |= kFlagBadToken;
    if (bad) atomicOr(&s_bad, bad);
    s_par[c] = par;
    s_tok[c] = tok;
    s_u[c] = kGreedy ? 0.f : slot_uniform(a.u, a.seed, a.offset, b, N, c);
  }
  // every thread's zeroing stores have completed before the barrier, so
  // the ticket stored after it certifies them
  if (a.arrive != nullptr) asm volatile("s_waitcnt vmcnt(0)");
  __syncthreads();
  if (a.arrive != nullptr && tid == 0) store_word(a.arrive + static_cast<int64_t>(b) * a.G + wk.g, a.ticket);
  WALK_TL(1);
  if (const int bad = s_bad) {
    if (wk.g == 0) walk_invalid(a, b, (bad & kFlagBadTree) ? kFlagBadTree : bad, tid, kWalkBlock);
    return;
  }

  // ---- the walk ----
  constexpr int kNodesPerThread = kMaxTreeNodes / kWalkBlock;
  const int ngroups = (N + kWave - 1) / kWave;
  int n_emit = 0, fallback = 0, step = 0, npass = 0, tiles_buf = -1;
  int cur = 0;
  bool ok = true, synced = true;
  float coef = 0.f, R = 1.f;
  double Rd = 1.0;
  MS st{0.f, 0.f};
  int amax = 0;            // greedy: the argmax of cur's row
  int n_ex = 0;            // point mass: ids removed from cur's distribution (s_ex)
  bool have_pass = false;  // point mass: cur's tile sums are in s_wt0, slice totals in s_tot
  double Wrest = 1.0;      // point mass: mass of cur's distribution left after the removals
  bool cached = false;     // sampled: s_cache holds cur's p and q (from cur's first residual pass)
  uint64_t own_qcls = 0;   // sampled: this slice's draft-sum class word from that pass
  while (true) {
    // children of cur (one bit mask per 64 nodes, index order), and the target
    // logit / draft probability at their tokens, in flight during the pass
    for (int gi = wid; gi < ngroups; gi += kWalkWaves) {
      const int c = gi * kWave + lane;
      const uint64_t km = __ballot(c < N && c > 0 && s_par[c] == cur);
      if (lane == 0) s_kids[step & 1][gi] = km;
    }
    const void* trow = row_ptr<DT>(a.tgt, trow0 + cur, V);
    const void* qrow = kUseQ ? row_ptr<DQ>(a.dq, qrow0 + cur, V) : nullptr;
    if constexpr (kGreedy) {
      bool nan = false;
      if (!row_argmax<DT>(wk, trow, s_key, s_knan, amax, nan)) {
        synced = false;
        break;
      }
      ok = !nan;
      if (!ok) break;
    } else {
      float lx[kNodesPerThread], qv[kNodesPerThread];
#pragma unroll
      for (int j = 0; j < kNodesPerThread; ++j) {
        const int c = tid + j * kWalkBlock;
        lx[j] = qv[j] = 0.f;
        if (c < N && c > 0 && s_par[c] == cur) {
          lx[j] = DT::at(trow, s_tok[c]);
          if constexpr (kUseQ) qv[j] = DQ::at(qrow, s_tok[c]);
        }
      }
      if (!row_stats<DT>(wk, trow, s_wms, st)) {
        synced = false;
        break;
      }
      ok = st.s > 0.f && st.s < INFINITY;
      if (!ok) break;
      const float invS = 1.f / st.s;
#pragma unroll
      for (int j = 0; j < kNodesPerThread; ++j) {
        const int c = tid + j * kWalkBlock;
        if (c < N && c > 0 && s_par[c] == cur) {
          s_px[c] = ex2(fmaf(lx[j], a.c, -st.m)) * invS;
          s_qx[c] = qv[j];
        }
      }
    }
    const float invS = kGreedy ? 1.f : 1.f / st.s;
    __syncthreads();
    const DrawRow base{trow, qrow, a.c, st.m, invS, 0.f, false};
    int kept = -1;
    for (int gi = 0; gi < ngroups && kept < 0 && ok && synced; ++gi) {
      uint64_t m = s_kids[step & 1][gi];
      while (m != 0 && ok && synced) {
        const int ch = gi * kWave + __ffsll(static_cast<long long>(m)) - 1;
        m &= m - 1;
        if constexpr (kGreedy) {
          // the target's own pick: the first child carrying it is kept
          if (s_tok[ch] == amax) {
            kept = ch;
            break;
          }
        } else if constexpr (kPoint) {
          // candidate x tested as a draw from the point mass on x: kept iff
          // u < p'(x), p' = cur's distribution with the removed ids' mass
          // taken out and renormalised (u Wrest < p(x))
          const int x = s_tok[ch];
          bool gone = false;
          for (int i = 0; i < n_ex; ++i) gone |= s_ex[i] == x;
          const float p = gone ? 0.f : s_px[ch];
          if (static_cast<double>(s_u[ch - 1]) * Wrest < static_cast<double>(p)) {
            kept = ch;
            break;
          }
          if (gone) continue;  // removing it again changes nothing
          // rejected: x leaves the distribution.  The first time at this
          // node, one pass gives cur's tile sums and slice totals; after
          // that only x's tile changes, re-summed by every workgroup alike.
          if (!have_pass) {
            double W;
            bool qnan;
            if (!weight_pass<DT, DQ, false>(wk, base, s_wt0, s_wq, W, qnan)) {
              synced = false;
              break;
            }
            if (tid == 0) {
              const uint64_t* xw = last_words(wk);
              for (int h = 0; h < a.G; ++h) s_tot[h] = dec_sum(xw[2 * h]);
            }
            have_pass = true;
            tiles_buf = 0;
          }
          DrawRow rr = base;
          rr.excl = s_ex;
          rr.nexcl = n_ex;
          const int t = x / kSampleTile;
          if (wid == 0) {
            float with, without;
            lane_partial_excl<DT, DQ>(rr, V, t, x, with, without);
            if (lane == 0) {
              s_two[0] = with;
              s_two[1] = without;
            }
          }
          __syncthreads();
          const double d = s_two[0] - s_two[1];  // x's share of its tile's sum
          const int h = tile_owner(t, a.ntiles, a.G);
          double Wn = 0.0;
          for (int hh = 0; hh < a.G; ++hh) Wn += hh == h ? s_tot[hh] - d : s_tot[hh];
          __syncthreads();
          if (Wn > 0.0) {
            if (tid == 0) {
              s_tot[h] -= d;
              s_ex[n_ex] = x;
              if (wk.g == h) s_wt0[t - wk.lo] -= d;
            }
            ++n_ex;
            Wrest = Wn;
          } else {  // nothing left: keep the distribution as it was
            fallback = kFlagFallback;
          }
          __syncthreads();
        } else {
          const float p = s_px[ch], q = s_qx[ch];
          const float pc = coef == 0.f ? p : fmaxf(fmaf(-coef, q, p), 0.f) / R;
          if (s_u[ch - 1] * q < pc) {
            kept = ch;
            break;
          }
          // rejected: residual pass with the next coefficient
          DrawRow rr = base;
          rr.coef = coef + R;
          rr.use_q = true;
          const int nb = npass & 1;
          ++npass;
          double W;
          bool qnan;
          double* wt = nb ? s_wt1 : s_wt0;
          bool passed;
          if (a.cache == 0) {
            passed = weight_pass<DT, DQ, true, kCacheNone, true>(wk, rr, wt, s_wq, W, qnan);
          } else if (!cached) {
            passed = weight_pass<DT, DQ, true, kCacheFill, true>(wk, rr, wt, s_wq, W, qnan, s_cache, &own_qcls);
            cached = true;
          } else {
            passed = weight_pass<DT, DQ, true, kCacheUse, true>(wk, rr, wt, s_wq, W, qnan, s_cache, &own_qcls);
          }
          if (!passed) {
            synced = false;
          } else if (qnan || !isfinite(W)) {
            ok = false;
          } else if (W > 0.0) {
            coef = rr.coef;
            R = static_cast<float>(W);
            Rd = W;
            tiles_buf = nb;
          } else {  // no residual mass: keep the current distribution
            fallback = kFlagFallback;
            tiles_buf = -1;
          }
        }
      }
    }
    if (!ok || !synced || kept < 0) break;
    if (tid == 0) s_path[n_emit] = kept;
    ++n_emit;
    ++step;
    cur = kept;
    coef = 0.f;
    R = 1.f;
    Rd = 1.0;
    tiles_buf = -1;
    n_ex = 0;
    have_pass = false;
    Wrest = 1.0;
    cached = false;
  }
  if (!synced) {
    if (tid == 0) flag(a.status, kFlagSyncTimeout);
    return;
  }
  if (!ok) {
    if (wk.g == 0) walk_invalid(a, b, kFlagNonfinite | fallback, tid, kWalkBlock);
    return;
  }

  // ---- the last token: the greedy pick, or a draw from the current distribution ----
  int y = amax;
  if constexpr (!kGreedy) {
    DrawRow row{row_ptr<DT>(a.tgt, trow0 + cur, V), kUseQ ? row_ptr<DQ>(a.dq, qrow0 + cur, V) : nullptr,
                a.c, st.m, 1.f / st.s, coef, coef != 0.f};
    row.excl = s_ex;
    row.nexcl = kPoint ? n_ex : 0;
    if (tiles_buf < 0) {
      tiles_buf = npass & 1;
      bool qnan;
      if (!weight_pass<DT, DQ, kUseQ>(wk, row, tiles_buf ? s_wt1 : s_wt0, s_wq, Rd, qnan)) {
        if (tid == 0) flag(a.status, kFlagSyncTimeout);
        return;
      }
      if constexpr (kPoint) {
        if (tid == 0) {
          const uint64_t* xw = last_words(wk);
          for (int h = 0; h < a.G; ++h) s_tot[h] = dec_sum(xw[2 * h]);
        }
        __syncthreads();
      }
    }
    // slice h's weight: the words of the last exchange (the weight pass of the
    // current distribution), or the point-mass walk's updated totals
    const uint64_t* sw = last_words(wk);
    auto slice_w = [&](int h) { return kPoint ? s_tot[h] : dec_sum(sw[2 * h]); };
    if constexpr (kPoint) {
      Rd = 0.0;
      for (int h = 0; h < a.G; ++h) Rd += slice_w(h);
    }
    const double target = static_cast<double>(s_u[N - 1]) * Rd;
    // the slice holding the target: the first with weight whose running sum
    // exceeds it, else the last slice with weight
    int gs = -1, glast = -1;
    double base_s = 0.0, run = 0.0, base_last = 0.0;
    for (int h = 0; h < a.G; ++h) {
      const double w = slice_w(h);
      if (w > 0.0) {
        if (gs < 0 && run + w > target) {
          gs = h;
          base_s = run;
        }
        glast = h;
        base_last = run;
      }
      run += w;
    }
    if (gs < 0) {
      gs = glast;
      base_s = base_last;
    }
    if (gs < 0) {  // no mass anywhere: cannot happen with S > 0; defined output
      if (wk.g == 0) walk_invalid(a, b, kFlagNonfinite | fallback, tid, kWalkBlock);
      return;
    }
#ifdef SV_TIMELINE
    if (tid == 0) sv_walk_tl[60] = timeline_now();
    if (wk.g != gs) {  // the other workgroups' records (the drawing wave writes its own below)
      __syncthreads();
      if (tid < kTimelineSlots && static_cast<int64_t>(b) * a.G + wk.g < kTimelineRecords)
        sv_timeline_walk_records[(static_cast<int64_t>(b) * a.G + wk.g) * kTimelineSlots + tid] = sv_walk_tl[tid];
      return;
    }
#endif
    if (wk.g != gs) return;
    // the owning workgroup: wave 0 finds the tile, waves 0..3 pick the id
    WALK_TL_DRAW(61);
    if (wid == 0) {
      const double* wt = tiles_buf ? s_wt1 : s_wt0;
      const int nsl = wk.hi - wk.lo;
      int ta, tb;
      lane_tiles(nsl, lane, ta, tb);
      double own = 0.0;
      for (int i = ta; i < tb; ++i) own += wt[i];
      TileHit hit;
      const bool found = wave_find_tile(wt, 1, nsl, own, target - base_s, hit);
      if (!found) walk_invalid(a, b, kFlagNonfinite | fallback, lane, kWave);
      hit.tile += wk.lo;
      hit.base += base_s;
      if (lane == 0) {
        s_pick_go = found ? 1 : 0;
        s_hit = hit;
      }
    }
    __syncthreads();
    if (!s_pick_go) return;
    WALK_TL_DRAW(62);
    y = block_pick_in_tile<DT, DQ, kPoint>(row, V, s_hit, target, s_pick);
    if (wid != 0) return;
  } else {
#ifdef SV_TIMELINE
    if (wk.g != 0) {
      __syncthreads();
      if (tid < kTimelineSlots && static_cast<int64_t>(b) * a.G + wk.g < kTimelineRecords)
        sv_timeline_walk_records[(static_cast<int64_t>(b) * a.G + wk.g) * kTimelineSlots + tid] = sv_walk_tl[tid];
      return;
    }
#endif
    if (wk.g != 0 || wid != 0) return;
  }
  const int64_t o = static_cast<int64_t>(b) * N;
  for (int i = lane; i < N; i += kWave) {
    a.out_tok[o + i] = i < n_emit ? s_tok[s_path[i]] : (i == n_emit ? y : -1);
    a.out_path[o + i] = i < n_emit ? s_path[i] : -1;
  }
  if (lane == 0) {
    a.out_cnt[b] = n_emit + 1;
    a.out_acc[b] = n_emit;
    flag(a.status, fallback);
  }
#ifdef SV_TIMELINE
  WALK_TL_DRAW(63);
  if (static_cast<int64_t>(b) * a.G + wk.g < kTimelineRecords)
    sv_timeline_walk_records[(static_cast<int64_t>(b) * a.G + wk.g) * kTimelineSlots + lane] = sv_walk_tl[lane];
#endif
}

// Chains whose vocabulary is one tile (V <= 2048): one wave per request does
// the whole round with wave scans and ballots, no LDS and no barriers.  Lane
// i holds draft i and row i: softmax pair (one segment), p_i(x_i), q_i(x_i)
// and u_i.  Same decisions and draw as k_walk.
template <class DT, class DQ>
__global__ __launch_bounds__(kBlock) void k_walk_small(WalkArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t b = static_cast<int64_t>(blockIdx.x) * (kBlock / kWave) + threadIdx.x / kWave;
  if (b >= a.B) return;
  const int64_t V = a.V;
  const int width = a.k_max + 1;
  auto invalid = [&](int bits) {
    for (int i = lane; i < width; i += kWave) a.out_tok[b * width + i] = -1;
    if (lane == 0) {
      a.out_cnt[b] = 0;
      a.out_acc[b] = 0;
      if (a.resid != nullptr) a.resid[b] = 0.f;
      flag(a.status, bits);
    }
  };
  const int k = a.dlen[b];
  const int ts = a.t_rs[b], qs = a.q_rs[b];
  if (k < 0 || k > a.k_max || ts < 0 || static_cast<int64_t>(ts) + k >= a.t_rows ||
      (k > 0 && (qs < 0 || static_cast<int64_t>(qs) + k > a.q_rows))) {
    invalid(kFlagBadRequest);
    return;
  }
  const int extra = (a.max_new != nullptr && k > a.max_new[b]) ? kFlagOverBudget : 0;
  // rows are handled kWave at a time (k_max < 256); every drafted token is
  // checked, also those after the break
  int m = k;               // first draft not kept
  bool bad_tok = false, nonfinite = false;
  for (int i0 = kWave; i0 < k; i0 += kWave) {
    const int i = i0 + lane;
    const int x = i < k ? a.ids[b * a.k_max + i] : 0;
    if (__ballot(i < k && (x < 0 || x >= V))) bad_tok = true;
  }
  float Mm = 0.f, Sm = 1.f;
  for (int i0 = 0; i0 <= k; i0 += kWave) {
    const int i = i0 + lane;
    const bool row = i <= k, draft = i < k;
    const int x = draft ? a.ids[b * a.k_max + i] : 0;
    const bool xin = x >= 0 && x < V;
    if (__ballot(draft && !xin)) bad_tok = true;
    const float u = row ? slot_uniform(a.u, a.seed, a.offset, b, width, i) : 0.f;
    float2 ms = make_float2(-INFINITY, 0.f);
    float lx = 0.f, qx = 0.f;
    if (row) ms = a.partial[static_cast<int64_t>(ts + i) * a.nseg];
    if (draft && xin) {
      lx = DT::at(row_ptr<DT>(a.tgt, ts + i, V), x);
      qx = DQ::at(row_ptr<DQ>(a.dq, qs + i, V), x);
    }
    if (bad_tok) continue;
    const bool fin = ms.y > 0.f && ms.y < INFINITY;
    const float p = ex2(fmaf(lx, a.c, -ms.x)) * (1.f / ms.y);
    // stop at the first row that is not finite or whose draft is not kept
    const bool stop = row && (!fin || (draft && !(u * qx < p)) || i == k);
    const uint64_t st = __ballot(stop);
    if (st == 0) continue;
    const int j = __ffsll(static_cast<long long>(st)) - 1;
    const int ij = i0 + j;
    const int fin_j = __builtin_amdgcn_readlane(fin ? 1 : 0, j);
    if (!fin_j) {
      nonfinite = true;
    } else {
      m = ij;
      Mm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ms.x), j));
      Sm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ms.y), j));
    }
    break;
  }
  if (bad_tok) {
    invalid(kFlagBadToken);
    return;
  }
  if (nonfinite) {
    invalid(kFlagNonfinite | extra);
    return;
  }
  // the last token: residual max(0, p_m - q_m) after a rejection, else p_k
  const bool resid = m < k;
  DrawRow row{row_ptr<DT>(a.tgt, ts + m, V), resid ? row_ptr<DQ>(a.dq, qs + m, V) : nullptr, a.c, Mm,
              1.f / Sm, 1.f, resid};
  double v[1][3];
  wave_tile_sums<DT, DQ, 1>(row, V, 0, 0, v);
  int bits = extra;
  double total = v[0][0];
  if (resid) {
    if (isnan(v[0][2]) || !isfinite(v[0][0])) {
      invalid(kFlagNonfinite | extra);
      return;
    }
    if (!(v[0][0] > 0.0)) {  // no residual mass: draw from p_m
      bits |= kFlagFallback;
      row.use_q = false;
      total = v[0][1];
    }
  }
  const double target = static_cast<double>(slot_uniform(a.u, a.seed, a.offset, b, width, k)) * total;
  const TileHit h{0, 0.0, false};
  const int y = wave_pick_in_tile<DT, DQ>(row, V, h, target);
  if (lane == 0) {
    int32_t* out = a.out_tok + b * width;
    int cnt = 0;
    bool stop = false;
    for (int i = 0; i < m && !stop; ++i) {
      const int32_t tok = a.ids[b * a.k_max + i];
      out[cnt++] = tok;
      if (a.eos >= 0 && tok == a.eos) stop = true;
    }
    if (!stop) out[cnt++] = y;
    if (a.max_new != nullptr) {
      const int budget = a.max_new[b] > 0 ? a.max_new[b] : 0;
      if (cnt > budget) cnt = budget;
    }
    for (int i = cnt; i < width; ++i) out[i] = -1;
    a.out_cnt[b] = cnt;
    a.out_acc[b] = m;
    if (a.resid != nullptr) a.resid[b] = static_cast<float>(total);
    flag(a.status, bits);
  }
}

// Zero the exchange words before the walk.
__global__ __launch_bounds__(kBlock) void k_walk_clear(uint4* w, int64_t n16) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n16;
       i += static_cast<int64_t>(gridDim.x) * kBlock)
    w[i] = uint4{0u, 0u, 0u, 0u};
}

hipError_t launch_clear(void* p, size_t bytes, hipStream_t stream) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  if (n16 <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n16 + kBlock - 1) / kBlock, 2048);
  hipLaunchKernelGGL(k_walk_clear, dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), 0, stream,
                     static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

// The Philox uniforms of [B, slots] slots, one thread per slot.
__global__ __launch_bounds__(kBlock) void k_philox_fill(uint64_t seed, uint64_t offset, int32_t slots,
                                                        int64_t n, float* u) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (t >= n) return;
  u[t] = philox_uniform(seed, offset, t / slots, static_cast<int>(t % slots));
}

hipError_t launch_philox_fill(uint64_t seed, uint64_t offset, int32_t B, int32_t slots, float* u,
                              hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(B) * slots;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_philox_fill, dim3(static_cast<uint32_t>((n + kBlock - 1) / kBlock)), dim3(kBlock), 0,
                     stream, seed, offset, slots, n, u);
  return hipGetLastError();
}

// ---- diagnostics (only when asked for), from the softmax partials of every row ----

// Tree: (M_c, S_c, p_parent(x_c), q_parent(x_c)), p being the parent's softmax
// before any residual update.  One block per request, one node per thread.
template <class DT, class DQ>
__global__ __launch_bounds__(kMaxTreeNodes) void k_tree_diag(WalkArgs a) {
  __shared__ float s_m[kMaxTreeNodes], s_S[kMaxTreeNodes];
  const int b = blockIdx.x, c = threadIdx.x;
  const int64_t row0 = static_cast<int64_t>(b) * a.N;
  const bool mine = c < a.N;
  int par = -1, tok = 0;
  float lx = 0.f, qx = 0.f;
  if (mine) {
    par = a.parent[row0 + c];
    tok = a.token[row0 + c];
  }
  const bool edge = mine && c > 0 && par >= 0 && par < c && tok >= 0 && tok < a.V;
  if (edge) {
    lx = DT::at(row_ptr<DT>(a.tgt, row0 + par, a.V), tok);
    qx = DQ::at(row_ptr<DQ>(a.dq, row0 + par, a.V), tok);
  }
  MS st{-INFINITY, 0.f};
  if (mine) {
    const float2* pp = a.partial + (row0 + c) * a.nseg;
#pragma unroll 8
    for (int s = 0; s < a.nseg; ++s) {
      const float2 v = pp[s];
      st = ms_combine(st, MS{v.x, v.y});
    }
    s_m[c] = st.m;
    s_S[c] = st.s;
  }
  __syncthreads();
  if (mine) {
    float* d = a.diag + (row0 + c) * 4;
    d[0] = st.m * kLn2;
    d[1] = st.s;
    d[2] = edge ? ex2(fmaf(lx, a.c, -s_m[par])) * (1.f / s_S[par]) : 0.f;
    d[3] = edge ? qx : 0.f;
  }
}

// Chain: (M_i, S_i, p_i(x_i), q_i(x_i)) for i <= k_b (p, q = 0 at i = k_b),
// for requests whose rows and tokens are in range.  One block per request,
// one position per thread.
template <class DT, class DQ>
__global__ __launch_bounds__(kWalkBlock) void k_chain_diag(WalkArgs a) {
  __shared__ int s_bad;
  const int b = blockIdx.x, i = threadIdx.x;
  const int k = a.dlen[b], ts = a.t_rs[b], qs = a.q_rs[b];
  if (k < 0 || k > a.k_max || ts < 0 || static_cast<int64_t>(ts) + k >= a.t_rows ||
      (k > 0 && (qs < 0 || static_cast<int64_t>(qs) + k > a.q_rows)))
    return;
  if (i == 0) s_bad = 0;
  __syncthreads();
  const int x = i < k ? a.ids[static_cast<int64_t>(b) * a.k_max + i] : 0;
  if (i < k && (x < 0 || x >= a.V)) atomicOr(&s_bad, 1);
  __syncthreads();
  if (s_bad || i > k) return;
  const float2* pp = a.partial + (static_cast<int64_t>(ts) + i) * a.nseg;
  MS st{-INFINITY, 0.f};
  for (int s = 0; s < a.nseg; ++s) {
    const float2 v = pp[s];
    st = ms_combine(st, MS{v.x, v.y});
  }
  float* d = a.diag + (static_cast<int64_t>(b) * (a.k_max + 1) + i) * 4;
  d[0] = st.m * kLn2;
  d[1] = st.s;
  d[2] = i < k ? ex2(fmaf(DT::at(row_ptr<DT>(a.tgt, ts + i, a.V), x), a.c, -st.m)) * (1.f / st.s) : 0.f;
  d[3] = i < k ? DQ::at(row_ptr<DQ>(a.dq, qs + i, a.V), x) : 0.f;
}

// ---- host side ----

namespace {

template <int kMode, class DT, class DQ>
const void* walk_fn() {
  return reinterpret_cast<const void*>(&k_walk<kMode, DT, DQ>);
}

// The point-mass and greedy walks read no draft rows: one instantiation per
// target dtype (DQ = DT, unused).
const void* pick_walk(int mode, int t_dtype, int q_dtype) {
  const bool tb = t_dtype == kDtypeBF16, qb = q_dtype == kDtypeBF16;
  switch (mode) {
    case kWalkTree:
      if (tb && qb) return walk_fn<kWalkTree, BF16, BF16>();
      if (tb) return walk_fn<kWalkTree, BF16, F32>();
      if (qb) return walk_fn<kWalkTree, F32, BF16>();
      return walk_fn<kWalkTree, F32, F32>();
    case kWalkPoint:
      return tb ? walk_fn<kWalkPoint, BF16, BF16>() : walk_fn<kWalkPoint, F32, F32>();
    default:
      return tb ? walk_fn<kWalkGreedy, BF16, BF16>() : walk_fn<kWalkGreedy, F32, F32>();
  }
}

template <int kMode, class DT, class DQ>
void launch_t(const WalkArgs& a, size_t lds, bool clear_slots, hipStream_t stream) {
  if constexpr (kMode == kWalkTree) {
    if (a.diag != nullptr)
      hipLaunchKernelGGL((k_tree_diag<DT, DQ>), dim3(static_cast<uint32_t>(a.B)), dim3(kMaxTreeNodes), 0, stream, a);
  }
  if (a.G > 1 && clear_slots) {
    const int64_t n16 = (static_cast<int64_t>(a.B) * a.max_sync * 2 * a.G + 1) / 2;
    const int64_t blocks = std::min<int64_t>((n16 + kBlock - 1) / kBlock, 2048);
    hipLaunchKernelGGL(k_walk_clear, dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), 0, stream,
                       reinterpret_cast<uint4*>(a.slots), n16);
  }
  launch_timed(k_walk<kMode, DT, DQ>, dim3(static_cast<uint32_t>(static_cast<int64_t>(a.B) * a.G)), dim3(kWalkBlock),
               lds, stream, a);
}

template <int kMode>
void launch_mode(int t_dtype, int q_dtype, const WalkArgs& a, size_t lds, bool clear_slots,
                 hipStream_t stream) {
  const bool tb = t_dtype == kDtypeBF16, qb = q_dtype == kDtypeBF16;
  if constexpr (kMode == kWalkPoint || kMode == kWalkGreedy) {
    if (tb) launch_t<kMode, BF16, BF16>(a, lds, clear_slots, stream);
    else launch_t<kMode, F32, F32>(a, lds, clear_slots, stream);
  } else {
    if (tb && qb) launch_t<kMode, BF16, BF16>(a, lds, clear_slots, stream);
    else if (tb) launch_t<kMode, BF16, F32>(a, lds, clear_slots, stream);
    else if (qb) launch_t<kMode, F32, BF16>(a, lds, clear_slots, stream);
    else launch_t<kMode, F32, F32>(a, lds, clear_slots, stream);
  }
}

}  // namespace

size_t walk_lds_bytes(int node_cap, int tile_cap, bool with_cache) {
  const size_t base = static_cast<size_t>(tile_cap) * 2 * sizeof(double) + static_cast<size_t>(node_cap) * 7 * 4;
  if (!with_cache) return base;
  return ((base + 15) & ~static_cast<size_t>(15)) + static_cast<size_t>(tile_cap) * 2 * kSampleTile * sizeof(float);
}

int walk_occupancy(int mode, int t_dtype, int q_dtype, size_t lds) {
  static std::mutex mu;
  // by mode, dtypes and LDS rounded up to 8 KB (up to 168 KB); n + 1 once known
  static int cache[4][2][2][21] = {};
  const size_t bucket = std::min<size_t>((lds + 8191) / 8192, 21) - (lds == 0 ? 0 : 1);
  const size_t lds_key = (bucket + 1) * 8192;
  const int m = mode < 0 || mode > 3 ? 0 : mode;
  std::lock_guard<std::mutex> lock(mu);
  int& slot = cache[m][t_dtype == kDtypeBF16][q_dtype == kDtypeBF16][bucket];
  if (slot == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, pick_walk(m, t_dtype, q_dtype), kWalkBlock,
                                                     lds_key) != hipSuccess)
      n = 0;
    slot = (n < 0 ? 0 : n) + 1;
  }
  return slot - 1;
}

hipError_t launch_chain_diag(int t_dtype, int q_dtype, const WalkArgs& a, hipStream_t stream) {
  const bool tb = t_dtype == kDtypeBF16, qb = q_dtype == kDtypeBF16;
  const dim3 grid(static_cast<uint32_t>(a.B)), block(kWalkBlock);
  if (tb && qb)
    hipLaunchKernelGGL((k_chain_diag<BF16, BF16>), grid, block, 0, stream, a);
  else if (tb)
    hipLaunchKernelGGL((k_chain_diag<BF16, F32>), grid, block, 0, stream, a);
  else if (qb)
    hipLaunchKernelGGL((k_chain_diag<F32, BF16>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((k_chain_diag<F32, F32>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_walk_small(int t_dtype, int q_dtype, const WalkArgs& a, hipStream_t stream) {
  const bool tb = t_dtype == kDtypeBF16, qb = q_dtype == kDtypeBF16;
  const int64_t blocks = (static_cast<int64_t>(a.B) + kBlock / kWave - 1) / (kBlock / kWave);
  const dim3 grid(static_cast<uint32_t>(blocks)), block(kBlock);
  if (a.diag != nullptr) {
    const hipError_t e = launch_chain_diag(t_dtype, q_dtype, a, stream);
    if (e != hipSuccess) return e;
  }
  if (tb && qb)
    launch_timed((k_walk_small<BF16, BF16>), grid, block, 0, stream, a);
  else if (tb)
    launch_timed((k_walk_small<BF16, F32>), grid, block, 0, stream, a);
  else if (qb)
    launch_timed((k_walk_small<F32, BF16>), grid, block, 0, stream, a);
  else
    launch_timed((k_walk_small<F32, F32>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_walk(int mode, int t_dtype, int q_dtype, const WalkArgs& a, size_t lds,
                       bool clear_slots, hipStream_t stream) {
  switch (mode) {
    case kWalkTree: launch_mode<kWalkTree>(t_dtype, q_dtype, a, lds, clear_slots, stream); break;
    case kWalkPoint: launch_mode<kWalkPoint>(t_dtype, q_dtype, a, lds, clear_slots, stream); break;
    default: launch_mode<kWalkGreedy>(t_dtype, q_dtype, a, lds, clear_slots, stream); break;
  }
  return hipGetLastError();
}

}  // namespace sv
