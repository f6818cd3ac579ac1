// Tree verify (EAGLE / SpecInfer style): recursive speculative sampling over a
// flattened draft tree.
//
// Method ("Speculative Decoding II", EAGLE section: every node of the draft
// tree is verified by applying speculative sampling recursively, keeping a
// candidate or adjusting the distribution, as SpecInfer does; the EAGLE-2
// worked example gives the breadth-first flattened layout):
//   cur = root, p = softmax(target row / T), q = draft row of cur;
//   for each child c of cur in order: keep iff u * q(x_c) < p(x_c); kept ->
//   emit x_c, descend, reload p and q; rejected -> p <- norm(max(0, p - q)).
//   With no child kept, draw the last token from the current p.
//
// Repeated residual updates against one q stay in closed form: after j
// rejections the current distribution is max(0, p - c_j q) / R_j with
// c_0 = 0, R_0 = 1, c_{j+1} = c_j + R_j and R_{j+1} = sum max(0, p - c_{j+1} q),
// so every rejection costs one fused pass over the node's two rows that yields
// R_{j+1} and, per 4096-element tile, the sums the final inverse-CDF draw needs.
//
// One block per request; the walk's state is uniform across the block.  Node
// ids, parents, sibling lists and per-node softmax statistics (combined from the
// row-statistics kernel's partials) live in LDS.
#include "common.hpp"
#include "launch.hpp"

namespace sv {

namespace {

template <int n>
__device__ __forceinline__ float pairwise_t(const float* x) {
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

// Weights of 16 elements at e: p (coef == 0) or max(0, p - coef q).
template <class DT, class DQ>
__device__ __forceinline__ void tree_weights(const void* trow, const void* qrow, int64_t V, int64_t e,
                                             float c, float Mc, float invS, float coef, float* w,
                                             float* q) {
  float l[kPerThreadTile];
  load_run<DT, kPerThreadTile>(trow, V, e, l, -INFINITY);
  if (coef != 0.f) {
    load_run<DQ, kPerThreadTile>(qrow, V, e, q, 0.f);
  } else {
#pragma unroll
    for (int j = 0; j < kPerThreadTile; ++j) q[j] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < kPerThreadTile; ++j) {
    const float p = ex2(fmaf(l[j], c, -Mc)) * invS;
    w[j] = coef != 0.f ? fmaxf(p - coef * q[j], 0.f) : p;
  }
}

}  // namespace

template <class DT, class DQ>
__global__ __launch_bounds__(kBlock) void k_tree_walk(TreeArgs a) {
  constexpr int kWaves = kBlock / kWave;
  __shared__ int32_t s_par[kMaxTreeNodes], s_tok[kMaxTreeNodes];
  __shared__ int32_t s_first[kMaxTreeNodes], s_next[kMaxTreeNodes];
  __shared__ int32_t s_emit[kMaxTreeNodes], s_path[kMaxTreeNodes];
  __shared__ float s_m[kMaxTreeNodes], s_S[kMaxTreeNodes];
  __shared__ double s_wt[kMaxTreeTiles][kWaves];
  __shared__ double s_red[3 * kWaves];
  __shared__ int32_t s_kids[kMaxTreeNodes];
  __shared__ float s_kp[kMaxTreeNodes], s_kq[kMaxTreeNodes];
  __shared__ int s_int[4];

  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int N = a.N;
  const int64_t V = a.V;
  const int64_t row0 = static_cast<int64_t>(b) * N;

  if (tid == 0) s_int[0] = 0;
  for (int c = tid; c < N; c += kBlock) {
    s_par[c] = a.parent[row0 + c];
    s_tok[c] = a.token[row0 + c];
    s_first[c] = -1;
    s_next[c] = -1;
  }
  __syncthreads();
  for (int c = tid; c < N; c += kBlock) {
    const int pc = s_par[c];
    if (c == 0 ? pc != -1 : (pc < 0 || pc >= c)) atomicOr(&s_int[0], kFlagBadTree);
    if (c > 0 && (s_tok[c] < 0 || s_tok[c] >= V)) atomicOr(&s_int[0], kFlagBadToken);
  }
  __syncthreads();
  int bits = s_int[0];
  bits = (bits & kFlagBadTree) ? kFlagBadTree : bits;
  int32_t* out = a.out_tok + row0;
  int32_t* path = a.out_path + row0;
  if (bits) {
    for (int c = tid; c < N; c += kBlock) {
      out[c] = -1;
      path[c] = -1;
    }
    if (tid == 0) {
      a.out_cnt[b] = 0;
      a.out_acc[b] = 0;
      flag(a.status, bits);
    }
    return;
  }

  // per-node softmax statistics
  for (int c = tid; c < N; c += kBlock) {
    const float2* pp = a.partial + (row0 + c) * a.nseg;
    MS r{-INFINITY, 0.f};
    for (int s = 0; s < a.nseg; ++s) {
      const float2 v = pp[s];
      r = ms_combine(r, MS{v.x, v.y});
    }
    s_m[c] = r.m;
    s_S[c] = r.s;
  }
  __syncthreads();
  if (a.diag != nullptr) {
    for (int c = tid; c < N; c += kBlock) {
      float* d = a.diag + (row0 + c) * 4;
      d[0] = s_m[c] * kLn2;
      d[1] = s_S[c];
      float pv = 0.f, qv = 0.f;
      if (c > 0) {
        const int pr = s_par[c];
        const float l = DT::at(row_ptr<DT>(a.tgt, row0 + pr, V), s_tok[c]);
        pv = ex2(fmaf(l, a.c, -s_m[pr])) * (1.f / s_S[pr]);
        qv = DQ::at(row_ptr<DQ>(a.dq, row0 + pr, V), s_tok[c]);
      }
      d[2] = pv;
      d[3] = qv;
    }
  }
  if (tid == 0) {
    for (int c = N - 1; c >= 1; --c) {
      s_next[c] = s_first[s_par[c]];
      s_first[s_par[c]] = c;
    }
  }
  __syncthreads();

  // ---- the walk ----
  int cur = 0, n_emit = 0, fallback = 0;
  bool ok = s_S[0] > 0.f && s_S[0] < INFINITY;
  float coef = 0.f, R = 1.f;
  bool have_tiles = false;
  while (ok) {
    // children of cur, and p(x), q(x) at their tokens under cur's rows
    if (tid == 0) {
      int nk = 0;
      for (int c = s_first[cur]; c != -1; c = s_next[c]) s_kids[nk++] = c;
      s_int[1] = nk;
    }
    __syncthreads();
    const int nk = s_int[1];
    const void* trow = row_ptr<DT>(a.tgt, row0 + cur, V);
    const void* qrow = row_ptr<DQ>(a.dq, row0 + cur, V);
    const float Mc = s_m[cur];
    const float invS = 1.f / s_S[cur];
    for (int j = tid; j < nk; j += kBlock) {
      const int x = s_tok[s_kids[j]];
      s_kp[j] = ex2(fmaf(DT::at(trow, x), a.c, -Mc)) * invS;
      s_kq[j] = DQ::at(qrow, x);
    }
    __syncthreads();
    int kept = -1;
    for (int j = 0; j < nk && ok; ++j) {
      const float p = s_kp[j], q = s_kq[j];
      const float pc = coef == 0.f ? p : fmaxf(p - coef * q, 0.f) / R;
      const float u = a.u[row0 + s_kids[j] - 1];
      if (u * q < pc) {
        kept = s_kids[j];
        break;
      }
      // rejected: residual pass with the next coefficient
      const float coefn = coef + R;
      float qacc = 0.f;
      for (int t = 0; t < a.ntiles; ++t) {
        float w[kPerThreadTile], qq[kPerThreadTile];
        tree_weights<DT, DQ>(trow, qrow, V, static_cast<int64_t>(t) * kTile + tid * kPerThreadTile,
                             a.c, Mc, invS, coefn, w, qq);
        const double ws = wave_sum(static_cast<double>(pairwise_t<kPerThreadTile>(w)));
        qacc += pairwise_t<kPerThreadTile>(qq);
        if (lane == 0) s_wt[t][wid] = ws;
      }
      const int qnan = __syncthreads_or(isnan(qacc));
      double Rn = 0.0;
      for (int t = 0; t < a.ntiles; ++t)
        for (int wv = 0; wv < kWaves; ++wv) Rn += s_wt[t][wv];
      if (qnan || !isfinite(Rn)) {
        ok = false;
        break;
      }
      if (Rn > 0.0) {
        coef = coefn;
        R = static_cast<float>(Rn);
        have_tiles = true;
      } else {
        fallback = kFlagFallback;
        have_tiles = false;
      }
      __syncthreads();
    }
    if (!ok || kept < 0) break;
    if (tid == 0) {
      s_emit[n_emit] = s_tok[kept];
      s_path[n_emit] = kept;
    }
    ++n_emit;
    cur = kept;
    coef = 0.f;
    R = 1.f;
    have_tiles = false;
    ok = s_S[cur] > 0.f && s_S[cur] < INFINITY;
    __syncthreads();
  }
  if (!ok) {
    for (int c = tid; c < N; c += kBlock) {
      out[c] = -1;
      path[c] = -1;
    }
    if (tid == 0) {
      a.out_cnt[b] = 0;
      a.out_acc[b] = 0;
      flag(a.status, kFlagNonfinite | fallback);
    }
    return;
  }

  // ---- final draw from the current distribution ----
  const void* trow = row_ptr<DT>(a.tgt, row0 + cur, V);
  const void* qrow = row_ptr<DQ>(a.dq, row0 + cur, V);
  const float Mc = s_m[cur];
  const float invS = 1.f / s_S[cur];
  if (!have_tiles) {
    for (int t = 0; t < a.ntiles; ++t) {
      float w[kPerThreadTile], qq[kPerThreadTile];
      tree_weights<DT, DQ>(trow, qrow, V, static_cast<int64_t>(t) * kTile + tid * kPerThreadTile, a.c,
                           Mc, invS, coef, w, qq);
      const double ws = wave_sum(static_cast<double>(pairwise_t<kPerThreadTile>(w)));
      if (lane == 0) s_wt[t][wid] = ws;
    }
  }
  __syncthreads();
  // tile sums (ntiles <= 256 = block size): one scan finds the crossing tile
  const double wt = [&] {
    double s = 0.0;
    if (tid < a.ntiles)
      for (int wv = 0; wv < kWaves; ++wv) s += s_wt[tid][wv];
    return s;
  }();
  double total;
  const double excl = block_exclusive_scan(wt, &total, s_red);
  const double target = static_cast<double>(a.u[row0 + N - 1]) * total;
  if (tid == 0) {
    s_int[2] = a.ntiles;
    s_int[3] = -1;
  }
  __syncthreads();
  if (tid < a.ntiles) {
    if (wt > 0.0 && excl + wt > target) atomicMin(&s_int[2], tid);
    if (wt > 0.0) atomicMax(&s_int[3], tid);
  }
  __syncthreads();
  int tile = s_int[2];
  const bool overshoot = tile >= a.ntiles;
  if (overshoot) tile = s_int[3];
  if (tile >= 0 && tile == tid) s_red[3 * kWaves - 1] = excl;
  __syncthreads();
  const double tile_base = s_red[3 * kWaves - 1];
  __syncthreads();
  if (tid == 0) {
    s_int[2] = INT32_MAX;
    s_int[3] = -1;
  }
  __syncthreads();
  if (tile >= 0) {
    float w[kPerThreadTile], qq[kPerThreadTile];
    const int off = tid * kPerThreadTile;
    tree_weights<DT, DQ>(trow, qrow, V, static_cast<int64_t>(tile) * kTile + off, a.c, Mc, invS, coef,
                         w, qq);
    double cum[kPerThreadTile];
    double run = 0.0;
#pragma unroll
    for (int j = 0; j < kPerThreadTile; ++j) {
      run += static_cast<double>(w[j]);
      cum[j] = run;
    }
    double tt;
    const double ex = block_exclusive_scan(run, &tt, s_red);
    int first = INT32_MAX, lastpos = -1;
#pragma unroll
    for (int j = kPerThreadTile - 1; j >= 0; --j) {
      if (!overshoot && w[j] > 0.f && tile_base + ex + cum[j] > target) first = off + j;
      if (w[j] > 0.f && lastpos < 0) lastpos = off + j;
    }
    if (first != INT32_MAX) atomicMin(&s_int[2], first);
    if (lastpos >= 0) atomicMax(&s_int[3], lastpos);
  }
  __syncthreads();
  const int pick = s_int[2] != INT32_MAX ? s_int[2] : s_int[3];
  if (tile < 0 || pick < 0) {  // no mass at all: cannot happen with S > 0; defined output
    for (int c = tid; c < N; c += kBlock) {
      out[c] = -1;
      path[c] = -1;
    }
    if (tid == 0) {
      a.out_cnt[b] = 0;
      a.out_acc[b] = 0;
      flag(a.status, kFlagNonfinite | fallback);
    }
    return;
  }
  const int y = static_cast<int>(static_cast<int64_t>(tile) * kTile + pick);
  for (int c = tid; c < N; c += kBlock) {
    out[c] = c < n_emit ? s_emit[c] : (c == n_emit ? y : -1);
    path[c] = c < n_emit ? s_path[c] : -1;
  }
  if (tid == 0) {
    a.out_cnt[b] = n_emit + 1;
    a.out_acc[b] = n_emit;
    flag(a.status, fallback);
  }
}

hipError_t launch_tree_walk(int t_dtype, int q_dtype, const TreeArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(a.B)), block(kBlock);
  if (t_dtype == kDtypeBF16 && q_dtype == kDtypeBF16)
    hipLaunchKernelGGL((k_tree_walk<BF16, BF16>), grid, block, 0, stream, a);
  else if (t_dtype == kDtypeBF16)
    hipLaunchKernelGGL((k_tree_walk<BF16, F32>), grid, block, 0, stream, a);
  else if (q_dtype == kDtypeBF16)
    hipLaunchKernelGGL((k_tree_walk<F32, BF16>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((k_tree_walk<F32, F32>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace sv
