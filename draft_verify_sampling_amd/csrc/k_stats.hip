// Row statistics of the temperature softmax, streamed from HBM.
//
// For every target row l (vocab elements) the verify step needs the softmax
// normaliser of l / T ("投机解码:为什么一个字都不改", figure "一次目标前向验 k 个
// 草稿 token": P = softmax(f / T) over the whole vocabulary).  A block reads one
// 8192-element segment of a row and forms its online-softmax pair
// (m = max l, s = sum 2^((l - m) log2(e) / T)); consumers combine the nseg
// pairs of a row.  The pair is kept in the scaled domain: m = max(l) * log2(e) / T
// (rounded once), s = sum 2^(l * log2(e) / T - m).
//
// k_row_stats: grid = rows * nseg blocks of 256 threads; every row, every
// segment.
//
// k_chain_stats: the chain verify's lazy variant.  A round reads target rows
// 0..m only (m = the first draft that is not kept, "改进" section), so blocks
// are ordered row-major over the requests -- all rows 0 first, then all rows
// 1, ... -- and the last block to finish a (request, row) combines the row's
// pairs and decides that row's draft at once (kept iff u q(x) < p(x)).  A
// block whose request has already stopped at an earlier row does nothing.
// Blocks never wait for a decision: a block that starts before the decision
// it could use computes its segment anyway, which is only wasted bandwidth.
// The draw (k_chain_draw) then takes the break row and its pair from the
// words this kernel leaves.
#include "common.hpp"
#include "launch.hpp"
#include "segment.hpp"
#include "timeline.hpp"
#include "words.hpp"

// Time lines (builds with -DSV_TIMELINE only), record = block index.
// k_row_stats: slot 0 the block's start, 1 its pair written.
// k_chain_stats: slot 0 the block's start, 1 it is to load its segment (a
// block of a row that is not needed has slot 0 only), 2 its word stored and
// its count returned, 3 the row decided (the row's last block).
SV_TIMELINE_ARRAY(sv_timeline_stats)
SV_TIMELINE_ARRAY_SIZED(sv_timeline_lazy, 65536, 4)

namespace sv {

// `clear` (optional, n16 16-byte words) is zeroed on the side, for the exchange
// words of the kernel that follows this one on the stream (the chain draw, or
// a tree walk asked for diagnostics).
template <class D, bool NT>
__global__ __launch_bounds__(kBlock) void k_row_stats(const void* __restrict__ rows, int64_t V,
                                                      int32_t nseg, float c,
                                                      float2* __restrict__ partial,
                                                      uint4* __restrict__ clear, int64_t n16) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n16;
       i += static_cast<int64_t>(gridDim.x) * kBlock)
    clear[i] = uint4{0u, 0u, 0u, 0u};
  __shared__ float sh[2 * (kBlock / kWave)];
  if (threadIdx.x == 0) SV_STAMP(sv_timeline_stats, blockIdx.x, 0);
  const int64_t row = blockIdx.x / nseg;
  const int32_t seg = blockIdx.x - static_cast<int32_t>(row) * nseg;
  const MS t = segment_ms<D, NT>(row_ptr<D>(rows, row, V), V, seg, nseg, c, sh);
  if (threadIdx.x == 0) {
    partial[blockIdx.x] = make_float2(t.m, t.s);
    SV_STAMP(sv_timeline_stats, blockIdx.x, 1);
  }
}

hipError_t launch_row_stats(int dtype, const void* rows, int64_t n_rows, int64_t V, int32_t nseg,
                            float c, float2* partial, hipStream_t stream, uint64_t* clear,
                            int64_t clear_words) {
  const dim3 grid(static_cast<uint32_t>(n_rows * nseg)), block(kBlock);
  uint4* c16 = reinterpret_cast<uint4*>(clear);
  const int64_t n16 = clear != nullptr ? (clear_words + 1) / 2 : 0;
  if (dtype == kDtypeBF16)
    launch_timed((k_row_stats<BF16, true>), grid, block, 0, stream, rows, V, nseg, c, partial, c16, n16);
  else
    launch_timed((k_row_stats<F32, true>), grid, block, 0, stream, rows, V, nseg, c, partial, c16, n16);
  return hipGetLastError();
}

// ---- the HBM read ceiling (a measurement tool) ----

// Every thread issues its 16-byte non-temporal loads of a 64 KiB chunk at once
// (as the statistics blocks do for a segment) and folds the words with xor;
// one value per block is written so the loads cannot be dropped.
__global__ __launch_bounds__(kBlock) void k_read_ceiling(const uint4* __restrict__ buf, int64_t n16,
                                                         uint32_t* __restrict__ out) {
  constexpr int U = 4 * kSegElems / 8 / kBlock;  // 16-byte vectors per thread
  const int64_t v0 = static_cast<int64_t>(blockIdx.x) * (U * kBlock) + threadIdx.x;
  uint4 w[U];
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int64_t v = v0 + j * kBlock;
    w[j] = uint4{0u, 0u, 0u, 0u};
    if (v < n16) {
      const uint32_t* q = reinterpret_cast<const uint32_t*>(buf + v);
      w[j] = uint4{__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1),
                   __builtin_nontemporal_load(q + 2), __builtin_nontemporal_load(q + 3)};
    }
  }
  uint32_t x = 0;
#pragma unroll
  for (int j = 0; j < U; ++j) x ^= w[j].x ^ w[j].y ^ w[j].z ^ w[j].w;
  __shared__ uint32_t sh[kBlock / kWave];
  for (int o = 32; o >= 1; o >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), o));
  if ((threadIdx.x & (kWave - 1)) == 0) sh[threadIdx.x / kWave] = x;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = sh[0] ^ sh[1] ^ sh[2] ^ sh[3];
}

hipError_t launch_read_ceiling(const void* buf, int64_t bytes, uint32_t* out, hipStream_t stream) {
  const int64_t blocks = read_blocks(bytes);
  launch_timed(k_read_ceiling, dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), 0, stream,
                     static_cast<const uint4*>(buf), bytes / 16, out);
  return hipGetLastError();
}

// ---- the lazy statistics of the chain verify ----


// Whether request b's metadata is usable (the draw reports the others);
// k, ts, qs: its draft count and row starts.
__device__ __forceinline__ bool chain_request_ok(const ChainStatsArgs& a, int b, int& k, int& ts, int& qs) {
  k = a.dlen[b];
  ts = a.t_rs[b];
  qs = a.q_rs[b];
  return !(k > a.k_max || k < 0 || ts < 0 || static_cast<int64_t>(ts) + k >= a.t_rows ||
           (k > 0 && (qs < 0 || static_cast<int64_t>(qs) + k > a.q_rows)));
}

// Segments seg .. seg + kN - 1 of target row i of request b (those before
// nseg; a usable request, i <= k): their pairs go out as words and count on
// the row's counter, and the row's last segment combines the row's pairs in
// segment order and decides the row (the stop word keeps the earliest row
// that stops).  Every thread of the block calls it; it returns in every
// thread, wave 0 of the deciding block last.  sh: kN * 8 floats.
template <class DT, class DQ, int kN = 1>
__device__ __forceinline__ void chain_segment(const ChainStatsArgs& a, int i, int b, int seg, int k, int ts, int qs,
                                              float* sh, uint64_t* s_w, int& s_last, int64_t rec) {
  static_assert(kN >= 1 && kN <= 4, "one to four segments");
  const int R = a.k_max + 1;
  // thread 0 fetches what the decision needs together with the segments
  int x = -1;
  float lx = 0.f, qx = 0.f, u = 0.f;
  if (threadIdx.x == 0 && i < k) {
    x = a.ids[static_cast<int64_t>(b) * a.k_max + i];
    u = slot_uniform(a.u, a.seed, a.offset, b, R, i);
    if (x >= 0 && x < a.V) {
      lx = DT::at(row_ptr<DT>(a.tgt, ts + i, a.V), x);
      qx = DQ::at(row_ptr<DQ>(a.dq, qs + i, a.V), x);
    }
  }
  // Rows decided one by one (kN = 1) are read with ordinary loads: most
  // rounds break at them, and the draw's re-read of the break row then finds
  // it in the last-level cache.  The later rows (read speculatively, kN > 1)
  // are mostly not break rows and stream non-temporally.
  MS t[kN];
  if constexpr (kN == 1)
    t[0] = segment_ms<DT, false>(row_ptr<DT>(a.tgt, ts + i, a.V), a.V, seg, a.nseg, a.c, sh);
  else
    segment_ms_n<DT, true, kN>(row_ptr<DT>(a.tgt, ts + i, a.V), a.V, seg, a.nseg, a.c, sh, t);
  const int n = min(kN, a.nseg - seg);
  uint64_t* words = a.seg_words + (static_cast<int64_t>(b) * R + i) * a.nseg;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int j = 0; j < kN; ++j)
      if (j < n) store_word(words + seg + j, enc_ms(t[j]));
    const uint32_t done = __hip_atomic_fetch_add(a.count + static_cast<int64_t>(b) * R + i, static_cast<uint32_t>(n),
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = done + n == static_cast<uint32_t>(a.nseg);
    SV_STAMP(sv_timeline_lazy, rec, 2);
  }
  __syncthreads();
  if (!s_last || threadIdx.x >= kWave) return;

  // The last segment of row i: every segment has added its count, so every
  // pair word is written; read them (waiting only for their visibility),
  // combine in segment order and decide the row's draft.
  const int lane = threadIdx.x;
  int ok = 1;
  for (int s0 = 0; s0 < a.nseg; s0 += kWave) {
    const int s = s0 + lane;
    uint64_t v = 0;
    int done = 0;
    for (int it = 0; it < a.spin_limit; ++it) {
      if (s < a.nseg) v = load_word(words + s);
      if (__all(s >= a.nseg || (v & kValid) != 0)) {
        done = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    ok &= done;
    if (s < a.nseg) s_w[s] = v;
  }
  // the canonical combine of the segment pairs (the draw combines the
  // partials of every row the same way)
  const MS row = wave_combine_segments(a.nseg, [&](int s) { return dec_ms(s_w[s]); });
  if (lane != 0) return;
  bool stop_here;
  if (!ok) {
    flag(a.status, kFlagSyncTimeout);
    stop_here = true;
  } else {
    store_word(a.row_words + static_cast<int64_t>(b) * R + i, enc_ms(row));
    stop_here = !(row.s > 0.f && row.s < INFINITY);
    if (!stop_here && i < k) {
      if (x < 0 || x >= a.V) {
        stop_here = true;  // the draw reports the token
      } else {
        const float p = ex2(fmaf(lx, a.c, -row.m)) * (1.f / row.s);
        stop_here = !(u * qx < p);
      }
    }
  }
  if (stop_here)
    __hip_atomic_fetch_max(a.stop + b, static_cast<uint32_t>(kMaxChainRows - i), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  SV_STAMP(sv_timeline_lazy, rec, 3);
}

// Rows 0 .. a.row_hi - 1, one block per segment, row-major over requests (all
// requests' row 0 first), so that a row's blocks mostly start after the
// previous row's decision and skip their loads when the round has stopped.
template <class DT, class DQ>
__global__ __launch_bounds__(kBlock) void k_chain_stats(ChainStatsArgs a) {
  __shared__ float sh[2 * (kBlock / kWave)];
  __shared__ uint64_t s_w[kMaxChainSegs];
  __shared__ int s_last;
  const int64_t per_row = static_cast<int64_t>(a.B) * a.nseg;
  const int i = static_cast<int>(blockIdx.x / per_row);
  const int64_t rem = blockIdx.x - static_cast<int64_t>(i) * per_row;
  const int b = static_cast<int>(rem / a.nseg);
  const int seg = static_cast<int>(rem - static_cast<int64_t>(b) * a.nseg);
  if (threadIdx.x == 0) SV_STAMP(sv_timeline_lazy, blockIdx.x, 0);
  // one round: the request's metadata and, past row 0, whether its round has
  // already stopped at an earlier row
  int k, ts, qs;
  const bool ok = chain_request_ok(a, b, k, ts, qs);
  const uint32_t sv = i > 0 ? __hip_atomic_load(a.stop + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
  if (!ok || i > k) return;  // a request the draw reports as invalid, or no such row
  // Row i is not needed.  The stop word can change while the block's waves
  // read it, so some waves may leave and the rest form a partial pair; that
  // happens only once an earlier row has stopped the round, so row i's pair
  // and decision are never used (the stop word keeps the earliest row).
  if (sv > static_cast<uint32_t>(kMaxChainRows - i)) return;
  if (threadIdx.x == 0) SV_STAMP(sv_timeline_lazy, blockIdx.x, 1);
  chain_segment<DT, DQ>(a, i, b, seg, k, ts, qs, sh, s_w, s_last, blockIdx.x);
}

// Rows a.row_lo .. k_b of every usable request whose round has not stopped
// before row a.row_lo, all at once: the grid's blocks take the items
// (request, row, kTailSegs consecutive segments), request-major, in turn.  Rows are decided
// independently (a later row's decision may go unused); the stop word keeps
// the earliest row that stops, so the outcome is the one of deciding them in
// order.  Each block first lays out the items itself: the requests' row
// counts and their exclusive scan, with their row starts, in LDS (B <=
// kMaxTailRequests).  Stop words set during this kernel come from rows >=
// a.row_lo, so every block sees the same requests running.
template <class DT, class DQ>
__global__ __launch_bounds__(kBlock) void k_chain_stats_tail(ChainStatsArgs a) {
  __shared__ float sh[kTailSegs * 2 * (kBlock / kWave)];
  __shared__ uint64_t s_w[kMaxChainSegs];
  __shared__ int s_last;
  __shared__ int32_t s_first[kMaxTailRequests + 1];  // first row slot of each request
  __shared__ int2 s_rs[kMaxTailRequests];            // its target and draft row starts
  __shared__ int32_t s_wsum[kBlock / kWave];
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const uint32_t running = static_cast<uint32_t>(kMaxChainRows - a.row_lo);  // stop words up to this
  // each thread counts the rows of its requests b = per t .. per (t + 1) - 1
  const int per = (a.B + kBlock - 1) / kBlock;
  const int b0 = min(a.B, static_cast<int>(threadIdx.x) * per), b1 = min(a.B, b0 + per);
  int mine = 0;
  for (int b = b0; b < b1; ++b) {
    int k, ts, qs;
    const bool ok = chain_request_ok(a, b, k, ts, qs);
    const uint32_t sv = __hip_atomic_load(a.stop + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int n = (ok && sv <= running && k >= a.row_lo) ? k - a.row_lo + 1 : 0;
    s_first[b] = n;
    s_rs[b] = int2{ts, qs};
    mine += n;
  }
  // block-wide exclusive scan of the threads' counts
  int incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) s_wsum[wid] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wid; ++w) base += s_wsum[w];
  int run = base + incl - mine;
  for (int b = b0; b < b1; ++b) {
    const int n = s_first[b];
    s_first[b] = run;
    run += n;
  }
  if (threadIdx.x == kBlock - 1) s_first[a.B] = run;
  __syncthreads();
  const int npair = (a.nseg + kTailSegs - 1) / kTailSegs;
  const int64_t total = static_cast<int64_t>(s_first[a.B]) * npair;
  // time-line records of the items follow those of the row-major kernel
  const int64_t rec0 = static_cast<int64_t>(a.row_hi) * a.B * a.nseg;
  (void)rec0;
  for (int64_t it = blockIdx.x; it < total; it += gridDim.x) {
    if (threadIdx.x == 0) SV_STAMP(sv_timeline_lazy, rec0 + it, 0);
    const int slot = static_cast<int>(it / npair);
    const int seg = kTailSegs * static_cast<int>(it - static_cast<int64_t>(slot) * npair);
    // the request owning row slot `slot`: the last b with s_first[b] <= slot
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_first[mid] <= slot) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int i = a.row_lo + (slot - s_first[b]);
    const int k = a.row_lo + (s_first[b + 1] - s_first[b]) - 1;  // rows row_lo .. k
    const int2 rs = s_rs[b];
    if (threadIdx.x == 0) SV_STAMP(sv_timeline_lazy, rec0 + it, 1);
    chain_segment<DT, DQ, kTailSegs>(a, i, b, seg, k, rs.x, rs.y, sh, s_w, s_last, rec0 + it);
  }
}

hipError_t launch_chain_stats(int t_dtype, int q_dtype, const ChainStatsArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(a.row_hi) * a.B * a.nseg)), block(kBlock);
  const bool tb = t_dtype == kDtypeBF16, qb = q_dtype == kDtypeBF16;
  if (tb && qb)
    launch_timed((k_chain_stats<BF16, BF16>), grid, block, 0, stream, a);
  else if (tb)
    launch_timed((k_chain_stats<BF16, F32>), grid, block, 0, stream, a);
  else if (qb)
    launch_timed((k_chain_stats<F32, BF16>), grid, block, 0, stream, a);
  else
    launch_timed((k_chain_stats<F32, F32>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_chain_stats_tail(int t_dtype, int q_dtype, const ChainStatsArgs& a, int64_t blocks,
                                   hipStream_t stream) {
  if (a.B > kMaxTailRequests || blocks < 1) return hipErrorInvalidValue;
  const dim3 grid(static_cast<uint32_t>(blocks)), block(kBlock);
  const bool tb = t_dtype == kDtypeBF16, qb = q_dtype == kDtypeBF16;
  if (tb && qb)
    launch_timed((k_chain_stats_tail<BF16, BF16>), grid, block, 0, stream, a);
  else if (tb)
    launch_timed((k_chain_stats_tail<BF16, F32>), grid, block, 0, stream, a);
  else if (qb)
    launch_timed((k_chain_stats_tail<F32, BF16>), grid, block, 0, stream, a);
  else
    launch_timed((k_chain_stats_tail<F32, F32>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace sv
