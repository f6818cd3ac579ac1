// Tree verify (EAGLE / SpecInfer style): recursive speculative sampling over a
// flattened draft tree.
//
// Method ("Speculative Decoding II", EAGLE section: every node of the draft
// tree is verified by applying speculative sampling recursively, keeping a
// candidate or adjusting the distribution, as SpecInfer does; the EAGLE-2
// worked example gives the breadth-first flattened layout):
//   cur = root, p = softmax(target row / T), q = draft row of cur;
//   for each child c of cur in index order: keep iff u * q(x_c) < p(x_c);
//   kept -> emit x_c, descend, reload p and q; rejected -> p <- norm(max(0, p - q)).
//   With no child kept, draw the last token from the current p.
//
// Repeated residual updates against one q stay in closed form: after j
// rejections the current distribution is max(0, p - c_j q) / R_j with
// c_0 = 0, R_0 = 1, c_{j+1} = c_j + R_j and R_{j+1} = sum max(0, p - c_{j+1} q),
// so every rejection costs one pass over the node's two rows that yields
// R_{j+1} and the per-tile sums the final inverse-CDF draw needs.
//
// Only the nodes the walk visits need their softmax statistics: the walk
// computes them itself (one pass over the visited node's target row), so rows
// of nodes it never reaches are never read.
//
// Work split: G workgroups of 1024 threads per request, G chosen by the host
// so that every workgroup of the grid can be resident at once.  Workgroup g
// owns a contiguous slice of the vocabulary's 2048-element tiles; each pass
// (softmax statistics of a visited row, or a residual / plain weight pass)
// covers only the slice, and the G partial results are exchanged through
// 64-bit words in the workspace: each workgroup stores its words with relaxed
// agent-scope atomic stores and reads the others' with relaxed agent-scope
// atomic loads until all carry their valid bit.  The data travels inside the
// atomic words, so no fence is needed; k_tree_clear zeroes the words before
// the walk.  Every workgroup combines the G words in the same order, so all of
// them take the same decisions.  The spin is bounded: on expiry the workgroup
// sets the sync-timeout status bit and exits.  With G = 1 nothing is
// exchanged through memory.
//
// The last token is drawn by the workgroup whose slice holds u * R: one wave
// scans the slice's tile sums (kept in LDS) and rescans the chosen tile.
#include <algorithm>

#include "tiles.hpp"

namespace sv {

namespace {

constexpr int kTreeBlock = 1024;
constexpr int kTreeWaves = kTreeBlock / kWave;
static_assert(kTreeBlock >= kMaxTreeNodes, "one node per thread");
static_assert(2 * kMaxTreeGroups <= kWave, "one wave reads every exchanged word");

constexpr uint64_t kValid = 1ull << 63;

// ---- exchanged words (bit 63 set = written in this call) ----
__device__ __forceinline__ uint64_t enc_ms(MS v) {
  return (static_cast<uint64_t>(__float_as_uint(v.s) | 0x80000000u) << 32) | __float_as_uint(v.m);
}
__device__ __forceinline__ MS dec_ms(uint64_t w) {
  return MS{__uint_as_float(static_cast<uint32_t>(w)),
            __uint_as_float(static_cast<uint32_t>(w >> 32) & 0x7fffffffu)};
}
// A sum of non-negative terms (or NaN): its sign bit carries the valid bit.
__device__ __forceinline__ uint64_t enc_sum(double x) {
  if (isnan(x)) return 0xfff8000000000001ull;
  return static_cast<uint64_t>(__double_as_longlong(x)) | kValid;
}
__device__ __forceinline__ double dec_sum(uint64_t w) {
  return __longlong_as_double(static_cast<long long>(w & ~kValid));
}
// Class of a slice's draft-row sum: NaN, +inf, -inf.  The row's total is NaN
// iff some slice is NaN or the slices hold both infinities.
__device__ __forceinline__ uint64_t enc_qclass(double q) {
  return kValid | (isnan(q) ? 1u : 0u) | (q == INFINITY ? 2u : 0u) | (q == -INFINITY ? 4u : 0u);
}

struct Walk {
  const TreeArgs* a;
  int b, g;
  int lo, hi;       // this workgroup's tiles [lo, hi)
  int nsync;        // exchanges so far (the same count in every workgroup)
  uint64_t* s_x;    // LDS [2][2 * kMaxTreeGroups]
  int* s_ok;        // LDS [2]
};

// Publish (w0, w1) and collect every workgroup's pair into the LDS words
// [2h], [2h + 1] of the current buffer.  Returns false when the bounded spin
// expired.  Ends with a block barrier.
__device__ bool exchange(Walk& wk, uint64_t w0, uint64_t w1) {
  const TreeArgs& a = *wk.a;
  const int lane = threadIdx.x & (kWave - 1);
  const int buf = wk.nsync & 1;
  uint64_t* x = wk.s_x + buf * 2 * kMaxTreeGroups;
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
      __hip_atomic_store(row + 2 * wk.g, w0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(row + 2 * wk.g + 1, w1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (threadIdx.x < kWave) {
      const int n = 2 * a.G;
      uint64_t v = 0;
      int done = 0;
      for (int it = 0; it < a.spin_limit; ++it) {
        if (lane < n) v = __hip_atomic_load(row + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__all(lane >= n || (v & kValid) != 0)) {
          done = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (lane < n) x[lane] = v;
      if (lane == 0) wk.s_ok[buf] = done;
    }
  }
  ++wk.nsync;
  __syncthreads();
  return wk.s_ok[buf] != 0;
}

__device__ __forceinline__ const uint64_t* last_words(const Walk& wk) {
  return wk.s_x + ((wk.nsync - 1) & 1) * 2 * kMaxTreeGroups;
}

// Softmax pair of a target row over the slice, combined across the request.
template <class DT>
__device__ bool row_stats(Walk& wk, const void* trow, MS* s_wms, MS& out) {
  const TreeArgs& a = *wk.a;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  MS acc{-INFINITY, 0.f};
  for (int t = wk.lo + wid; t < wk.hi; t += kTreeWaves) acc = ms_combine(acc, wave_tile_ms<DT>(trow, a.V, a.c, t));
  if (lane == 0) s_wms[wid] = acc;
  __syncthreads();
  MS r = s_wms[0];
  for (int w = 1; w < kTreeWaves; ++w) r = ms_combine(r, s_wms[w]);
  if (!exchange(wk, enc_ms(r), kValid)) return false;
  const uint64_t* x = last_words(wk);
  MS m = dec_ms(x[0]);
  for (int h = 1; h < a.G; ++h) m = ms_combine(m, dec_ms(x[2 * h]));
  out = m;
  return true;
}

// One weight pass over the slice: per-tile sums of the weights and of q into
// wt[] / qt[] (slice-local index); then, across the request, the total W and
// the NaN-ness of the draft row's sum.  Every slice's total stays readable in
// the exchanged words until the next exchange.
template <class DT, class DQ>
__device__ bool weight_pass(Walk& wk, const DrawRow& r, double* wt, double* qt, double& W, bool& qnan) {
  const TreeArgs& a = *wk.a;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const int lo = wk.lo, hi = wk.hi;
  for (int t = lo + wid; t < hi; t += kTreeWaves) {
    double v[1][3];
    wave_tile_sums<DT, DQ, 1>(r, a.V, t, 0, v);
    if (lane == 0) {
      wt[t - lo] = v[0][0];
      qt[t - lo] = v[0][2];
    }
  }
  __syncthreads();
  int ta, tb;
  lane_tiles(hi - lo, lane, ta, tb);
  double w = 0.0, q = 0.0;
  for (int i = ta; i < tb; ++i) {
    w += wt[i];
    q += qt[i];
  }
  w = wave_total(w);
  q = wave_total(q);
  if (!exchange(wk, enc_sum(w), enc_qclass(q))) return false;
  const uint64_t* x = last_words(wk);
  double tot = 0.0;
  uint64_t cls = 0;
  for (int h = 0; h < a.G; ++h) {
    tot += dec_sum(x[2 * h]);
    cls |= x[2 * h + 1];
  }
  W = tot;
  qnan = (cls & 1u) || ((cls & 2u) && (cls & 4u));
  return true;
}

// Invalid request: every output slot -1, counts 0, status bits.  Threads
// [first, first + stride, ...) write.
__device__ void tree_invalid(const TreeArgs& a, int b, int bits, int first, int stride) {
  const int64_t row0 = static_cast<int64_t>(b) * a.N;
  for (int c = first; c < a.N; c += stride) {
    a.out_tok[row0 + c] = -1;
    a.out_path[row0 + c] = -1;
  }
  if (first == 0) {
    a.out_cnt[b] = 0;
    a.out_acc[b] = 0;
    flag(a.status, bits);
  }
}

}  // namespace

template <class DT, class DQ>
__global__ __launch_bounds__(kTreeBlock) void k_tree_walk(TreeArgs a) {
  __shared__ int32_t s_par[kMaxTreeNodes], s_tok[kMaxTreeNodes], s_path[kMaxTreeNodes];
  __shared__ float s_px[kMaxTreeNodes], s_qx[kMaxTreeNodes], s_u[kMaxTreeNodes];
  __shared__ double s_wt[2][kMaxTreeTiles], s_qt[2][kMaxTreeTiles];
  __shared__ uint64_t s_x[2][2 * kMaxTreeGroups];
  __shared__ uint64_t s_kids[2][kTreeWaves];
  __shared__ MS s_wms[kTreeWaves];
  __shared__ int s_ok[2];
  __shared__ int s_bad;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  Walk wk{&a, static_cast<int>(blockIdx.x) / a.G, static_cast<int>(blockIdx.x) % a.G, 0, 0, 0,
          &s_x[0][0], s_ok};
  wk.lo = static_cast<int>(static_cast<int64_t>(wk.g) * a.ntiles / a.G);
  wk.hi = static_cast<int>(static_cast<int64_t>(wk.g + 1) * a.ntiles / a.G);
  const int b = wk.b;
  const int N = a.N;
  const int64_t V = a.V;
  const int64_t row0 = static_cast<int64_t>(b) * N;
  const int c = tid;  // this thread's node
  const bool mine = c < N;

  // ---- the tree and the uniforms ----
  int par = -1, tok = 0;
  float uu = 0.f;
  if (mine) {
    par = a.parent[row0 + c];
    tok = a.token[row0 + c];
    uu = a.u[row0 + c];
  }
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (mine) {
    int bad = 0;
    if (c == 0 ? par != -1 : (par < 0 || par >= c)) bad |= kFlagBadTree;
    if (c > 0 && (tok < 0 || tok >= V)) bad |= kFlagBadToken;
    if (bad) atomicOr(&s_bad, bad);
    s_par[c] = par;
    s_tok[c] = tok;
    s_u[c] = uu;
  }
  __syncthreads();
  if (const int bad = s_bad) {
    if (wk.g == 0) tree_invalid(a, b, (bad & kFlagBadTree) ? kFlagBadTree : bad, tid, kTreeBlock);
    return;
  }

  // ---- the walk ----
  int n_emit = 0, fallback = 0, step = 0, npass = 0, tiles_buf = -1;
  int cur = 0;
  bool ok = true, synced = true;
  float coef = 0.f, R = 1.f;
  double Rd = 1.0;
  MS st{0.f, 0.f};
  while (true) {
    // children of cur (one bit mask per wave, index order), and the target
    // logit / draft probability at their tokens, in flight during the pass
    const bool kid = mine && par == cur;
    const uint64_t km = __ballot(kid);
    if (lane == 0) s_kids[step & 1][wid] = km;
    const void* trow = row_ptr<DT>(a.tgt, row0 + cur, V);
    const void* qrow = row_ptr<DQ>(a.dq, row0 + cur, V);
    float lx = 0.f, qv = 0.f;
    if (kid) {
      lx = DT::at(trow, tok);
      qv = DQ::at(qrow, tok);
    }
    if (!row_stats<DT>(wk, trow, s_wms, st)) {
      synced = false;
      break;
    }
    ok = st.s > 0.f && st.s < INFINITY;
    if (!ok) break;
    const float invS = 1.f / st.s;
    if (kid) {
      s_px[c] = ex2(fmaf(lx, a.c, -st.m)) * invS;
      s_qx[c] = qv;
    }
    __syncthreads();
    const DrawRow base{trow, qrow, a.c, st.m, invS, 0.f, false};
    int kept = -1;
    for (int w = 0; w < kTreeWaves && kept < 0 && ok && synced; ++w) {
      uint64_t m = s_kids[step & 1][w];
      while (m != 0 && ok && synced) {
        const int ch = w * kWave + __ffsll(static_cast<long long>(m)) - 1;
        m &= m - 1;
        const float p = s_px[ch], q = s_qx[ch];
        const float pc = coef == 0.f ? p : fmaxf(p - coef * q, 0.f) / R;
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
        if (!weight_pass<DT, DQ>(wk, rr, s_wt[nb], s_qt[nb], W, qnan)) {
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
    if (!ok || !synced || kept < 0) break;
    if (tid == 0) s_path[n_emit] = kept;
    ++n_emit;
    ++step;
    cur = kept;
    coef = 0.f;
    R = 1.f;
    Rd = 1.0;
    tiles_buf = -1;
  }
  if (!synced) {
    if (tid == 0) flag(a.status, kFlagSyncTimeout);
    return;
  }
  if (!ok) {
    if (wk.g == 0) tree_invalid(a, b, kFlagNonfinite | fallback, tid, kTreeBlock);
    return;
  }

  // ---- the last token, from the current distribution ----
  const DrawRow row{row_ptr<DT>(a.tgt, row0 + cur, V), row_ptr<DQ>(a.dq, row0 + cur, V), a.c,
                    st.m, 1.f / st.s, coef, coef != 0.f};
  if (tiles_buf < 0) {
    tiles_buf = npass & 1;
    bool qnan;
    if (!weight_pass<DT, DQ>(wk, row, s_wt[tiles_buf], s_qt[tiles_buf], Rd, qnan)) {
      if (tid == 0) flag(a.status, kFlagSyncTimeout);
      return;
    }
  }
  const double target = static_cast<double>(s_u[N - 1]) * Rd;
  // the slice holding the target: the first with weight whose running sum
  // exceeds it, else the last slice with weight (the slice totals are the
  // words of the last exchange, the weight pass of the current distribution)
  const uint64_t* sw = last_words(wk);
  int gs = -1, glast = -1;
  double base_s = 0.0, run = 0.0, base_last = 0.0;
  for (int h = 0; h < a.G; ++h) {
    const double w = dec_sum(sw[2 * h]);
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
    if (wk.g == 0) tree_invalid(a, b, kFlagNonfinite | fallback, tid, kTreeBlock);
    return;
  }
  if (wk.g != gs || wid != 0) return;
  const double* wt = s_wt[tiles_buf];
  const int nsl = wk.hi - wk.lo;
  int ta, tb;
  lane_tiles(nsl, lane, ta, tb);
  double own = 0.0;
  for (int i = ta; i < tb; ++i) own += wt[i];
  TileHit h;
  if (!wave_find_tile(wt, 1, nsl, own, target - base_s, h)) {
    tree_invalid(a, b, kFlagNonfinite | fallback, lane, kWave);
    return;
  }
  h.tile += wk.lo;
  h.base += base_s;
  const int y = wave_pick_in_tile<DT, DQ>(row, V, h, target);
  for (int i = lane; i < N; i += kWave) {
    a.out_tok[row0 + i] = i < n_emit ? s_tok[s_path[i]] : (i == n_emit ? y : -1);
    a.out_path[row0 + i] = i < n_emit ? s_path[i] : -1;
  }
  if (lane == 0) {
    a.out_cnt[b] = n_emit + 1;
    a.out_acc[b] = n_emit;
    flag(a.status, fallback);
  }
}

// Zero the exchange words before the walk.
__global__ __launch_bounds__(kBlock) void k_tree_clear(uint64_t* w, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kBlock)
    w[i] = 0;
}

// Per-node diagnostics from the softmax partials of every row: (M_c, S_c,
// p_parent(x_c), q_parent(x_c)), p being the parent's softmax before any
// residual update.  One block per request, one node per thread.
template <class DT, class DQ>
__global__ __launch_bounds__(kTreeBlock) void k_tree_diag(TreeArgs a) {
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

template <class DT, class DQ>
static void launch_tree_t(const TreeArgs& a, hipStream_t stream) {
  if (a.diag != nullptr)
    hipLaunchKernelGGL((k_tree_diag<DT, DQ>), dim3(static_cast<uint32_t>(a.B)), dim3(kTreeBlock), 0, stream, a);
  if (a.G > 1) {
    const int64_t n = static_cast<int64_t>(a.B) * a.max_sync * 2 * a.G;
    const int64_t blocks = std::min<int64_t>((n + kBlock - 1) / kBlock, 1024);
    hipLaunchKernelGGL(k_tree_clear, dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), 0, stream, a.slots, n);
  }
  hipLaunchKernelGGL((k_tree_walk<DT, DQ>), dim3(static_cast<uint32_t>(a.B * a.G)), dim3(kTreeBlock), 0,
                     stream, a);
}

hipError_t launch_tree_walk(int t_dtype, int q_dtype, const TreeArgs& a, hipStream_t stream) {
  if (t_dtype == kDtypeBF16 && q_dtype == kDtypeBF16)
    launch_tree_t<BF16, BF16>(a, stream);
  else if (t_dtype == kDtypeBF16)
    launch_tree_t<BF16, F32>(a, stream);
  else if (q_dtype == kDtypeBF16)
    launch_tree_t<F32, BF16>(a, stream);
  else
    launch_tree_t<F32, F32>(a, stream);
  return hipGetLastError();
}

}  // namespace sv
