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
// One 1024-thread block per request (one node per thread for the set-up).
// The prologue takes two rounds of loads: the tree and the uniforms, then
// every node's softmax partials together with p_parent(x_c) and q_parent(x_c)
// at every node's token, so the walk itself reads no scattered values.  The
// walk's decisions are uniform across the block; each rejection is a pass in
// which all 16 waves stream their own tiles of the two rows (two tiles in
// flight per wave for bf16 rows) and leave per-tile sums in LDS (two buffers,
// one barrier per pass).  The last token is drawn by one wave from the tile
// sums.
#include "tiles.hpp"

namespace sv {

namespace {

constexpr int kTreeBlock = 1024;
constexpr int kTreeWaves = kTreeBlock / kWave;
static_assert(kTreeBlock >= kMaxTreeNodes, "one node per thread");

// One residual (or plain) pass over row r: per-tile sums of the weights and
// of q into wt[] / qt[], then the row totals W and Q, identical in every wave
// (each wave adds the tile sums in the same order).
template <class DT, class DQ>
__device__ __forceinline__ void block_pass(const DrawRow& r, int64_t V, int ntiles, double* wt, double* qt,
                                           double& W, double& Q) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  // two tiles in flight per wave for 2-byte rows; one 4-byte tile moves as many bytes
  constexpr bool kPairs = DT::kSize == 2 && DQ::kSize == 2;
  int t = wid;
  for (; kPairs && t + kTreeWaves < ntiles; t += 2 * kTreeWaves) {
    double v[2][3];
    wave_tile_sums<DT, DQ, 2>(r, V, t, kTreeWaves, v);
    if (lane == 0) {
      wt[t] = v[0][0];
      qt[t] = v[0][2];
      wt[t + kTreeWaves] = v[1][0];
      qt[t + kTreeWaves] = v[1][2];
    }
  }
  for (; t < ntiles; t += kTreeWaves) {
    double v[1][3];
    wave_tile_sums<DT, DQ, 1>(r, V, t, 0, v);
    if (lane == 0) {
      wt[t] = v[0][0];
      qt[t] = v[0][2];
    }
  }
  __syncthreads();
  int ta, tb;
  lane_tiles(ntiles, lane, ta, tb);
  double w = 0.0, q = 0.0;
  for (int i = ta; i < tb; ++i) {
    w += wt[i];
    q += qt[i];
  }
  W = wave_total(w);
  Q = wave_total(q);
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
  __shared__ float s_m[kMaxTreeNodes], s_S[kMaxTreeNodes];
  __shared__ float s_px[kMaxTreeNodes], s_qx[kMaxTreeNodes], s_u[kMaxTreeNodes];
  __shared__ double s_wt[2][kMaxTreeTiles], s_qt[2][kMaxTreeTiles];
  __shared__ uint64_t s_kids[2][kTreeWaves];
  __shared__ int s_bad;

  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int N = a.N;
  const int64_t V = a.V;
  const int64_t row0 = static_cast<int64_t>(b) * N;
  const int c = tid;  // this thread's node
  const bool mine = c < N;

  // ---- round 1: the tree and the uniforms ----
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
    tree_invalid(a, b, (bad & kFlagBadTree) ? kFlagBadTree : bad, tid, kTreeBlock);
    return;
  }

  // ---- round 2: node statistics, and the parent's p and q at each token ----
  float lx = 0.f, qx = 0.f;
  if (mine && c > 0) {
    lx = DT::at(row_ptr<DT>(a.tgt, row0 + par, V), tok);
    qx = DQ::at(row_ptr<DQ>(a.dq, row0 + par, V), tok);
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
    const float px = c > 0 ? ex2(fmaf(lx, a.c, -s_m[par])) * (1.f / s_S[par]) : 0.f;
    s_px[c] = px;
    s_qx[c] = qx;
    if (a.diag != nullptr) {
      float* d = a.diag + (row0 + c) * 4;
      d[0] = st.m * kLn2;
      d[1] = st.s;
      d[2] = px;
      d[3] = qx;
    }
  }
  __syncthreads();

  // ---- the walk ----
  int cur = 0, n_emit = 0, fallback = 0, step = 0, npass = 0, tiles_buf = -1;
  bool ok = s_S[0] > 0.f && s_S[0] < INFINITY;
  float coef = 0.f, R = 1.f;
  double Rd = 1.0;
  while (ok) {
    // children of cur, one bit mask per wave, in index order
    const uint64_t km = __ballot(mine && par == cur);
    if (lane == 0) s_kids[step & 1][wid] = km;
    __syncthreads();
    const DrawRow base{row_ptr<DT>(a.tgt, row0 + cur, V), row_ptr<DQ>(a.dq, row0 + cur, V), a.c,
                       s_m[cur], 1.f / s_S[cur], 0.f, false};
    int kept = -1;
    for (int w = 0; w < kTreeWaves && kept < 0 && ok; ++w) {
      uint64_t m = s_kids[step & 1][w];
      while (m != 0 && ok) {
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
        double W, Q;
        block_pass<DT, DQ>(rr, V, a.ntiles, s_wt[nb], s_qt[nb], W, Q);
        if (isnan(Q) || !isfinite(W)) {
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
    if (!ok || kept < 0) break;
    if (tid == 0) s_path[n_emit] = kept;
    ++n_emit;
    ++step;
    cur = kept;
    coef = 0.f;
    R = 1.f;
    Rd = 1.0;
    tiles_buf = -1;
    ok = s_S[cur] > 0.f && s_S[cur] < INFINITY;
  }
  if (!ok) {
    tree_invalid(a, b, kFlagNonfinite | fallback, tid, kTreeBlock);
    return;
  }

  // ---- the last token, from the current distribution ----
  const DrawRow row{row_ptr<DT>(a.tgt, row0 + cur, V), row_ptr<DQ>(a.dq, row0 + cur, V), a.c,
                    s_m[cur], 1.f / s_S[cur], coef, coef != 0.f};
  if (tiles_buf < 0) {
    tiles_buf = npass & 1;
    double Q;
    block_pass<DT, DQ>(row, V, a.ntiles, s_wt[tiles_buf], s_qt[tiles_buf], Rd, Q);
  }
  if (wid != 0) return;
  const double* wt = s_wt[tiles_buf];
  int ta, tb;
  lane_tiles(a.ntiles, lane, ta, tb);
  double own = 0.0;
  for (int i = ta; i < tb; ++i) own += wt[i];
  const double target = static_cast<double>(s_u[N - 1]) * Rd;
  TileHit h;
  if (!wave_find_tile(wt, 1, a.ntiles, own, target, h)) {  // no mass: cannot happen with S > 0
    tree_invalid(a, b, kFlagNonfinite | fallback, lane, kWave);
    return;
  }
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

hipError_t launch_tree_walk(int t_dtype, int q_dtype, const TreeArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(a.B)), block(kTreeBlock);
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
