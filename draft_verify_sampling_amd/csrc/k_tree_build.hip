// EAGLE-2 dynamic draft tree, built on the device.
//
// Method ("Speculative Decoding II", EAGLE-2 section, "Context-Aware Dynamic
// Draft Tree", and its worked example): a node's value is the product of the
// draft's confidences on its path (the root's is 1); each round expands the
// best nodes of the newest layer by value, each proposing the top-k tokens of
// the draft's distribution at that node; afterwards the whole tree is
// reranked by value and the best nodes are kept (ties to the shallower node,
// which keeps the kept set connected), then flattened breadth-first for the
// target's one forward with each node seeing itself and its ancestors.
//
// Candidates of request b live in caller-owned arrays [B, max_cand] (index =
// creation order, 0 = the root): token, parent, depth, confidence, value.
//
// k_topk_partial: one block per (row, segment) of the expanded nodes' draft
//   rows; every thread keeps the K best (value, id) keys of its elements in
//   registers (key = order-preserving bits of the clamped value << 32 | ~id,
//   so one unsigned compare ranks larger values first and lower ids first
//   among equals), only for elements at or above a threshold taken from the
//   threads' maxima; each wave then extracts its k best keys and one wave the
//   block's k best of those.
// k_tree_round: one block per request: merges each expanded row's segment
//   keys into its k children, appends them (parent value times confidence,
//   in fp64), and ranks the appended candidates for the next frontier.
// k_tree_finalize: one block per request (one thread per candidate): rank by
//   (-value, depth, creation order), keep the best, flatten depth by depth by
//   (parent's flat index, -confidence, token, creation order), write the flat
//   arrays and the ancestor mask.  The pairwise counts (rank; rank among kept
//   siblings) are split over all threads of the block; a node's flat index is
//   the first index of its parent's kept children plus its sibling rank, and
//   those first indices come from one wave's scan per depth.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace sv {

namespace {

// A stored draft probability as a confidence: clamped into [0, 1], NaN -> 0.
__device__ __forceinline__ float conf_of(float p) {
  return p == p ? fminf(fmaxf(p, 0.f), 1.f) : 0.f;
}

// Key of a confidence (non-negative, so its bits order like the value) and id.
__device__ __forceinline__ uint64_t conf_key(float c, int64_t id) {
  return (static_cast<uint64_t>(__float_as_uint(c) | 0x80000000u) << 32) |
         static_cast<uint32_t>(~static_cast<uint32_t>(id));
}

__device__ __forceinline__ float key_conf(uint64_t k) {
  return __uint_as_float(static_cast<uint32_t>(k >> 32) & 0x7fffffffu);
}

__device__ __forceinline__ int32_t key_id(uint64_t k) {
  return static_cast<int32_t>(~static_cast<uint32_t>(k));
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t min_u64(uint64_t a, uint64_t b) { return a < b ? a : b; }

__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f<0x111, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x112, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x114, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x118, 0xf>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x142, 0xa>(v, -INFINITY));
  v = fmaxf(v, dpp_f<0x143, 0xc>(v, -INFINITY));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

// Inclusive prefix sum of an int over the wave's lanes (DPP row shifts and
// row broadcasts, no LDS round trip).
template <int ctrl, int row_mask>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, ctrl, row_mask, 0xf, false);
}
__device__ __forceinline__ int wave_incl_scan_i(int x) {
  x += dpp_i<0x111, 0xf>(x);  // row_shr:1
  x += dpp_i<0x112, 0xf>(x);  // row_shr:2
  x += dpp_i<0x114, 0xf>(x);  // row_shr:4
  x += dpp_i<0x118, 0xf>(x);  // row_shr:8
  x += dpp_i<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_i<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// Insert key into the descending list top[0..K) (the smallest falls off).
template <int K>
__device__ __forceinline__ void list_insert(uint64_t (&top)[K], uint64_t key) {
  if (key <= top[K - 1]) return;
  uint64_t x = key;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const uint64_t hi = max_u64(top[j], x);
    x = min_u64(top[j], x);
    top[j] = hi;
  }
}


}  // namespace

// The k largest lane values of a wave, in rounds of a wave max (one copy of
// the maximum leaves per round); returns the r-th largest in round r's lane
// 0 through `emit(r, value)`.
template <class Emit>
__device__ __forceinline__ void wave_k_largest(float v, int k, Emit emit) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int r = 0; r < k; ++r) {
    const float w = wave_max_f32(v);
    const uint64_t at = __ballot(v == w);
    if (lane == __ffsll(static_cast<long long>(at)) - 1) v = -2.f;
    emit(r, w);
  }
}

// The k-th largest of one value per thread over the block (k <= 16; values
// >= -1): each wave's k largest, then the k-th largest of those (kWaves * k
// <= 64 values, one wave).  Valid in every thread.
__device__ __forceinline__ float block_kth_largest(float m, int k, float* s_tk) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  constexpr int kWaves = kBlock / kWave;
  static_assert(kWaves * kMaxTreeTop <= kWave, "one wave holds every wave's k largest");
  wave_k_largest(m, k, [&](int r, float w) {
    if (lane == 0) s_tk[wid * k + r] = w;
  });
  __syncthreads();
  if (wid == 0) {
    const float v = lane < kWaves * k ? s_tk[lane] : -2.f;
    wave_k_largest(v, k, [&](int r, float w) {
      if (lane == 0 && r == k - 1) s_tk[kWave] = w;
    });
  }
  __syncthreads();
  return s_tk[kWave];
}

template <class D, int K>
__global__ __launch_bounds__(kBlock) void k_topk_partial(const void* __restrict__ rows, int64_t V, int32_t nseg,
                                                         int32_t k, uint64_t* __restrict__ keys) {
  __shared__ uint64_t s_w[kBlock / kWave * kMaxTreeTop];
  __shared__ float s_tk[kWave + 1];
  const int64_t row = blockIdx.x / nseg;
  const int32_t seg = blockIdx.x - static_cast<int32_t>(row) * nseg;
  const void* base = row_ptr<D>(rows, row, V);
  const int64_t head = head_elems<D>(base, V);
  const int64_t nvec = (V - head) / D::kPerVec;
  const int64_t v0 = nvec * seg / nseg, v1 = nvec * (seg + 1) / nseg;
  const uint4* vp = reinterpret_cast<const uint4*>(static_cast<const char*>(base) + head * D::kSize);
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;

  uint64_t top[K];
#pragma unroll
  for (int j = 0; j < K; ++j) top[j] = 0;  // below every real key
  // Chunks of U vectors per thread, all loads in flight.  After the first
  // chunk the block knows a threshold T: the k-th largest of its threads'
  // largest confidences, so at least k of its elements have a confidence
  // >= T and no element below T can be among its k best.  Only elements at
  // or above T form keys.  Confidences are clamped raw values, and clamping
  // commutes with the maximum (fmaxf skips NaN, whose confidence 0 is the
  // floor anyway), so the thread maximum is taken on the raw values; with
  // T > 0 an element passes iff its raw value is >= T (NaN fails), with T <= 0
  // every element passes.
  constexpr int U = 8;
  const int64_t nchunk = (v1 - v0 + U * kBlock - 1) / (U * kBlock);
  float T = -1.f;
  for (int64_t ch = 0; ch < nchunk; ++ch) {
    const int64_t v = v0 + ch * U * kBlock + threadIdx.x;
    uint4 w[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t vv = v + j * kBlock;
      w[j] = vv < v1 ? vp[vv] : uint4{0u, 0u, 0u, 0u};
    }
    // each vector's largest raw value, and the thread's
    float vm[U];
    float m = -1.f;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      vm[j] = -INFINITY;
      if (v + j * kBlock < v1) {
        float x[D::kPerVec];
        D::unpack(w[j], x);
#pragma unroll
        for (int t = 0; t < D::kPerVec; ++t) vm[j] = fmaxf(vm[j], x[t]);
        m = fmaxf(m, vm[j]);
      }
    }
    if (ch == 0) {
      // the thread's largest confidence; -1 for a thread with no elements
      const float mc = v < v1 ? fminf(fmaxf(m, 0.f), 1.f) : -1.f;
      T = block_kth_largest(mc, k, s_tk);
    }
    const bool every = !(T > 0.f);
    // a wave none of whose threads reached T has no key in this chunk; in the
    // others only vectors whose largest value reached T are opened
    if (!every && !__any(m >= T)) continue;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t vv = v + j * kBlock;
      if (vv >= v1) break;
      if (!every && !(vm[j] >= T)) continue;
      float x[D::kPerVec];
      D::unpack(w[j], x);
#pragma unroll
      for (int t = 0; t < D::kPerVec; ++t)
        if (every || x[t] >= T) list_insert<K>(top, conf_key(conf_of(x[t]), head + vv * D::kPerVec + t));
    }
  }
  if (seg == 0)
    for (int64_t i = threadIdx.x; i < head; i += kBlock) list_insert<K>(top, conf_key(conf_of(D::at(base, i)), i));
  if (seg == nseg - 1)
    for (int64_t i = head + nvec * D::kPerVec + threadIdx.x; i < V; i += kBlock)
      list_insert<K>(top, conf_key(conf_of(D::at(base, i)), i));

  // the block's k best: each wave's k best (k rounds of a wave max over its
  // threads' list heads), then the k best of those in wave 0
  if (__any(top[0] != 0)) {
    for (int r = 0; r < k; ++r) {
      const uint64_t m = wave_max_u64(top[0]);
      if (top[0] == m && m != 0) {  // keys are distinct: one owner
#pragma unroll
        for (int j = 0; j + 1 < K; ++j) top[j] = top[j + 1];
        top[K - 1] = 0;
      }
      if (lane == 0) s_w[wid * k + r] = m;
    }
  } else if (lane < k) {
    s_w[wid * k + lane] = 0;  // a wave without keys
  }
  __syncthreads();
  if (wid == 0) {
    static_assert(kBlock / kWave * kMaxTreeTop <= kWave, "one lane per wave key");
    uint64_t x = lane < kBlock / kWave * k ? s_w[lane] : 0;
    uint64_t* out = keys + static_cast<int64_t>(blockIdx.x) * k;
    for (int r = 0; r < k; ++r) {
      const uint64_t m = wave_max_u64(x);
      if (x == m) x = 0;
      if (lane == 0) out[r] = m;
    }
  }
}

__global__ __launch_bounds__(kBlock) void k_tree_round(TreeRoundArgs a) {
  static_assert(kMaxTreeExpand <= kWave, "one wave checks the expanded nodes");
  __shared__ int s_base, s_bad, s_nv;
  __shared__ int s_node[kMaxTreeExpand], s_slot[kMaxTreeExpand];
  __shared__ double s_v[kMaxTreeExpand * kMaxTreeTop];  // the appended candidates' values
  __shared__ int s_d[kMaxTreeExpand * kMaxTreeTop];     // ... and depths
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wid = tid / kWave;
  const int64_t c0 = static_cast<int64_t>(b) * a.max_cand;
  const int k = a.top;
  const int nk = a.nseg * k;  // keys of an expanded row: <= 64 segments x 16 keys, 16 per lane
  constexpr int kPerLane = 64 * kMaxTreeTop / kWave;
  const int used = (nk + kWave - 1) / kWave;  // registers of kv holding keys
  uint64_t kv[kPerLane];
  auto load_keys = [&](int e) {
    const uint64_t* keys = a.keys + (static_cast<int64_t>(b) * a.n_exp + e) * nk;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const int idx = lane + j * kWave;
      kv[j] = j < used && idx < nk ? keys[idx] : 0;
    }
  };
  // wave w's first expanded row's keys: their address depends on the request
  // only, so they load with the round below
  if (wid < a.n_exp) load_keys(wid);

  // the expanded nodes of this request, one lane each (the first round: the
  // root, created here), checked against the request's candidate count
  if (wid == 0) {
    int cnt = a.first ? 1 : a.count[b];
    const int n = lane >= a.n_exp ? -1 : (a.first ? (lane == 0 ? 0 : -1) : a.exp[static_cast<int64_t>(b) * a.n_exp + lane]);
    if (a.first && lane == 0) {
      a.token[c0] = -1;
      a.parent[c0] = -1;
      a.depth[c0] = 0;
      a.conf[c0] = 1.f;
      a.value[c0] = 1.0;
    }
    const bool cnt_ok = cnt >= 1 && cnt <= a.max_cand;
    if (!cnt_ok) cnt = 0;
    const bool valid = lane < a.n_exp && n >= 0 && n < cnt;
    const bool wrong = lane < a.n_exp && (n >= cnt || n < -1);
    const uint64_t vm = __ballot(valid);
    const uint64_t wm = __ballot(wrong);
    const int nv = __popcll(vm);
    if (lane < a.n_exp) {
      s_node[lane] = valid ? n : -1;
      s_slot[lane] = __popcll(vm & ((1ull << lane) - 1));
    }
    if (lane == 0) {
      int bad = (!cnt_ok || wm != 0) ? kFlagBadRequest : 0;
      if (!bad && cnt + nv * k > a.max_cand) bad = kFlagBadRequest;  // no room: nothing appended
      s_bad = bad;
      s_base = cnt;
      s_nv = nv;
    }
  }
  __syncthreads();
  const int bad = s_bad, base = s_base;
  if (bad) {  // nothing appended; the next frontier is empty
    for (int j = tid; j < a.expand_next; j += kBlock) a.next[static_cast<int64_t>(b) * a.expand_next + j] = -1;
    if (tid == 0) {
      a.count[b] = base;
      flag(a.status, bad);
    }
    return;
  }
  // slot of expanded row e among the appended groups
  // (rows with no node contribute no children; the order is the order given)
  for (int e = wid; e < a.n_exp; e += kBlock / kWave) {
    const int node = s_node[e];
    if (node < 0) continue;
    const int slot = s_slot[e];
    if (e != wid) load_keys(e);
    const double pv = a.value[c0 + node];
    const int pd = a.depth[c0 + node];
    uint64_t thr = ~0ull;
    for (int r = 0; r < k; ++r) {  // r-th best key of the row: the largest below the previous one
      uint64_t m = 0;
#pragma unroll
      for (int j = 0; j < kPerLane; ++j)
        if (j < used) m = kv[j] < thr ? max_u64(m, kv[j]) : m;
      m = wave_max_u64(m);
      thr = m;
      if (lane == 0) {
        const int slot_r = slot * k + r;
        const int64_t ci = c0 + base + slot_r;
        const float c = key_conf(m);
        const double v = pv * static_cast<double>(c);
        a.token[ci] = key_id(m);
        a.parent[ci] = node;
        a.depth[ci] = pd + 1;
        a.conf[ci] = c;
        a.value[ci] = v;
        s_v[slot_r] = v;
        s_d[slot_r] = pd + 1;
      }
    }
  }
  __syncthreads();
  const int n_app = s_nv * k;
  // the next frontier: the best expand_next of the appended candidates.  A
  // candidate's rank is counted by one 16-lane DPP row, each lane over a
  // sixteenth of the others, and summed along the row.
  constexpr int kRow = 16;
  const int chunk = (n_app + kRow - 1) / kRow;
  for (int i0 = 0; i0 < n_app; i0 += kBlock / kRow) {
    const int i = i0 + tid / kRow, part = tid % kRow;
    int r = 0;
    if (i < n_app) {
      const double vi = s_v[i];
      const int di = s_d[i];
      const int j1 = min(n_app, (part + 1) * chunk);
      for (int j = part * chunk; j < j1; ++j) {
        const double vj = s_v[j];
        const int dj = s_d[j];
        r += (vj > vi) | ((vj == vi) & ((dj < di) | ((dj == di) & (j < i))));
      }
    }
    r += dpp_i<0x111, 0xf>(r);  // row_shr:1
    r += dpp_i<0x112, 0xf>(r);  // row_shr:2
    r += dpp_i<0x114, 0xf>(r);  // row_shr:4
    r += dpp_i<0x118, 0xf>(r);  // row_shr:8: the row's last lane holds the sum
    if (i < n_app && part == kRow - 1 && r < a.expand_next)
      a.next[static_cast<int64_t>(b) * a.expand_next + r] = base + i;
  }
  for (int j = n_app + tid; j < a.expand_next; j += kBlock) a.next[static_cast<int64_t>(b) * a.expand_next + j] = -1;
  if (tid == 0) a.count[b] = base + n_app;
}

// Pairwise counts split over the block: candidate c (1 <= c < M) is handled
// by P = kMaxTreeCand / (M - 1) threads, each over a contiguous part of
// j = 1 .. M - 1; `count(c, j0, j1)` returns how many j in [j0, j1) come
// before c, and the parts are added into s_cnt[c] (zeroed by the caller).
template <class Count>
__device__ __forceinline__ void split_count(int M, int* s_cnt, Count count) {
  const int nc = M - 1;
  if (nc <= 0) return;
  const int P = max(1, kMaxTreeCand / nc);
  const int ci = static_cast<int>(threadIdx.x) / P, part = static_cast<int>(threadIdx.x) - ci * P;
  if (ci >= nc) return;
  const int chunk = (nc + P - 1) / P;
  const int j0 = 1 + part * chunk, j1 = min(M, j0 + chunk);
  if (j0 >= j1) return;
  const int r = count(1 + ci, j0, j1);
  if (r != 0) atomicAdd(&s_cnt[1 + ci], r);
}

__global__ __launch_bounds__(kMaxTreeCand) void k_tree_finalize(TreeFinalArgs a) {
  __shared__ double s_val[kMaxTreeCand];
  __shared__ float s_conf[kMaxTreeCand];
  __shared__ int s_dep[kMaxTreeCand], s_par[kMaxTreeCand], s_tok[kMaxTreeCand], s_flat[kMaxTreeCand];
  __shared__ int s_of[kMaxTreeCand];    // candidate at each flat index
  __shared__ int s_rank[kMaxTreeCand];  // candidates ranked before (value, depth, creation order)
  __shared__ int s_sib[kMaxTreeCand];   // kept siblings placed before (confidence, token, creation order)
  __shared__ int s_nk[kMaxTreeCand];    // kept children
  __shared__ int s_cst[kMaxTreeCand];   // flat index of the first kept child
  __shared__ int s_dcnt[kMaxTreeCand];  // kept candidates per depth
  __shared__ unsigned char s_kept[kMaxTreeCand];
  const int b = blockIdx.x, i = threadIdx.x;
  const int lane = i & (kWave - 1), wid = i / kWave;
  const int64_t c0 = static_cast<int64_t>(b) * a.max_cand;
  const int M = a.count[b];
  const int N = a.n_nodes;
  const int64_t o = static_cast<int64_t>(b) * N;
  if (M < 1 || M > a.max_cand) {
    for (int f = i; f < N; f += kMaxTreeCand) {
      a.out_parent[o + f] = a.out_token[o + f] = a.out_depth[o + f] = a.out_cand[o + f] = -1;
    }
    if (a.out_mask != nullptr)
      for (int64_t x = i; x < static_cast<int64_t>(N) * N; x += kMaxTreeCand) a.out_mask[o * N + x] = 0;
    if (i == 0) flag(a.status, kFlagBadRequest);
    return;
  }
  if (i < M) {
    s_val[i] = a.value[c0 + i];
    s_conf[i] = a.conf[c0 + i];
    s_dep[i] = a.depth[c0 + i];
    s_par[i] = a.parent[c0 + i];
    s_tok[i] = a.token[c0 + i];
  }
  s_rank[i] = s_sib[i] = s_nk[i] = s_dcnt[i] = 0;
  s_of[i] = s_flat[i] = -1;
  s_cst[i] = -2 * kMaxTreeCand;  // no place until the node's own place is known
  __syncthreads();
  // kept: the root and the best N - 1 others by (-value, depth, creation
  // order)
  split_count(M, s_rank, [&](int c, int j0, int j1) {
    const double vc = s_val[c];
    const int dc = s_dep[c];
    int r = 0;
    for (int j = j0; j < j1; ++j) {
      const double vj = s_val[j];
      const int dj = s_dep[j];
      r += (vj > vc) | ((vj == vc) & ((dj < dc) | ((dj == dc) & (j < c))));
    }
    return r;
  });
  __syncthreads();
  const bool kept = i == 0 || (i < M && s_rank[i] < N - 1);
  s_kept[i] = kept ? 1 : 0;
  if (kept && i > 0) {  // (a parent precedes its children)
    const int p = s_par[i], d = s_dep[i];
    if (p >= 0 && p < i) atomicAdd(&s_nk[p], 1);
    if (d >= 1 && d < kMaxTreeCand) atomicAdd(&s_dcnt[d], 1);
  }
  __syncthreads();
  // breadth-first order: a depth's nodes by (parent's flat index,
  // -confidence, token, creation order), so a node's place is the first
  // place of its parent's children plus its rank among its kept siblings
  split_count(M, s_sib, [&](int c, int j0, int j1) {
    if (!s_kept[c]) return 0;
    const int pc = s_par[c], tc = s_tok[c];
    const float cc = s_conf[c];
    int r = 0;
    for (int j = j0; j < j1; ++j) {
      const float cj = s_conf[j];
      const int tj = s_tok[j];
      r += (s_kept[j] != 0) & (s_par[j] == pc) &
           ((cj > cc) | ((cj == cc) & ((tj < tc) | ((tj == tc) & (j < c)))));
    }
    return r;
  });
  if (i == 0) {
    s_flat[0] = 0;
    s_of[0] = 0;
    s_cst[0] = 1;
  }
  __syncthreads();
  const int n = M < N ? M : N;  // kept nodes
  int off = 1;  // flat index of depth d's first node
  // the kept set is connected, so its depths run 1, 2, ... without a gap
  for (int d = 1; d < n; ++d) {
    const int cnt = s_dcnt[d];
    if (cnt == 0) break;
    if (kept && i > 0 && s_dep[i] == d && s_par[i] >= 0 && s_par[i] < i) {
      const int f = s_cst[s_par[i]] + s_sib[i];
      if (f > 0 && f < n) {
        s_flat[i] = f;
        s_of[f] = i;
      }
    }
    __syncthreads();
    // first child places of depth d's nodes: after depth d, in their order
    if (wid == 0) {
      int carry = off + cnt;
      for (int f0 = off; f0 < off + cnt; f0 += kWave) {
        const int f = f0 + lane;
        const int q = f < off + cnt ? s_of[f] : -1;
        const int v = q >= 0 ? s_nk[q] : 0;
        const int x = wave_incl_scan_i(v);
        if (q >= 0) s_cst[q] = carry + x - v;
        carry += __builtin_amdgcn_readlane(x, kWave - 1);
      }
    }
    __syncthreads();
    off += cnt;
  }
  for (int f = i; f < N; f += kMaxTreeCand) {
    const int ci = f < n ? s_of[f] : -1;
    if (ci >= 0) {
      a.out_parent[o + f] = ci == 0 ? -1 : s_flat[s_par[ci]];
      a.out_token[o + f] = s_tok[ci];
      a.out_depth[o + f] = s_dep[ci];
      a.out_cand[o + f] = ci;
    } else {
      a.out_parent[o + f] = a.out_token[o + f] = a.out_depth[o + f] = a.out_cand[o + f] = -1;
    }
  }
  if (a.out_mask != nullptr) {
    // row f: ones at f and its ancestors
    for (int f = i; f < N; f += kMaxTreeCand) {
      uint8_t* row = a.out_mask + (o + f) * N;
      for (int j = 0; j < N; ++j) row[j] = 0;
      if (f < n) {
        int g = f;
        for (int step = 0; step < n && g >= 0 && g < n; ++step) {
          row[g] = 1;
          const int cg = s_of[g];
          g = cg <= 0 ? -1 : s_flat[s_par[cg]];
        }
      }
    }
  }
}

hipError_t launch_tree_expand(int dtype, const void* rows, int64_t n_rows, int64_t V, const TreeRoundArgs& a,
                              hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(n_rows * a.nseg));
  const bool bf = dtype == kDtypeBF16;
#define SV_TOPK(KK)                                                                                   \
  if (bf) hipLaunchKernelGGL((k_topk_partial<BF16, KK>), grid, dim3(kBlock), 0, stream, rows, V, a.nseg, \
                             a.top, a.keys);                                                          \
  else hipLaunchKernelGGL((k_topk_partial<F32, KK>), grid, dim3(kBlock), 0, stream, rows, V, a.nseg,     \
                          a.top, a.keys);
  if (n_rows > 0) {
    if (a.top <= 4) {
      SV_TOPK(4)
    } else if (a.top <= 8) {
      SV_TOPK(8)
    } else {
      SV_TOPK(16)
    }
  }
#undef SV_TOPK
  hipLaunchKernelGGL(k_tree_round, dim3(static_cast<uint32_t>(a.B)), dim3(kBlock), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_tree_finalize(const TreeFinalArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(k_tree_finalize, dim3(static_cast<uint32_t>(a.B)), dim3(kMaxTreeCand), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sv
