// Host-side launchers of the verify kernels and the workspace layout.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stddef.h>
#include <stdint.h>

namespace sv {

// The measurement hook: HIP events that the next launch_timed on this thread
// hands to the kernel launch itself, so that they take the kernel's own start
// and end times; that launch disarms it.
struct TimedEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local TimedEvents g_timed;

template <class F, class... A>
inline void launch_timed(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream, A... args) {
  if (g_timed.start != nullptr) {
    const TimedEvents ev = g_timed;
    g_timed = TimedEvents{};
    hipExtLaunchKernelGGL(kernel, grid, block, static_cast<uint32_t>(lds), stream, ev.start, ev.stop, 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
  }
}

constexpr int kDtypeF32 = 0;
constexpr int kDtypeBF16 = 1;
constexpr int kMaxChainRows = 256;     // k_max + 1 rows per request at most
constexpr int kMaxTreeNodes = 1024;
constexpr int kMaxWindow = 64;
constexpr float kLog2e = 1.4426950408889634f;

// Segments per row of the softmax-statistics kernel: one 8192-element chunk
// per block (for any row alignment the 16-byte-aligned body of a row needs at
// most this many chunks; the unaligned head and tail ride on the first and
// last segment).
constexpr int64_t kSegElems = 8192;
inline int32_t row_segments(int64_t /*rows*/, int64_t V) {
  const int64_t n = (V + kSegElems - 1) / kSegElems;
  return static_cast<int32_t>(n < 1 ? 1 : n);
}

// Segments per row of the argmax kernel: about 32 Ki elements per block, and at
// least ~1024 blocks in total when rows are few.
inline int32_t argmax_segments(int64_t rows, int64_t V) {
  int64_t nseg = (V + 32767) / 32768;
  if (rows > 0 && rows * nseg < 1024) {
    const int64_t want = (1024 + rows - 1) / rows;
    const int64_t cap = (V + 2047) / 2048;
    nseg = want < cap ? want : cap;
  }
  if (nseg < 1) nseg = 1;
  if (nseg > 64) nseg = 64;
  return static_cast<int32_t>(nseg);
}

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// The inverse-CDF unit of the sampled verify: one wave sums one tile.
constexpr int kSampleTile = 2048;
inline int64_t sample_tiles(int64_t V) { return (V + kSampleTile - 1) / kSampleTile; }
constexpr int64_t kMaxSampleVocab = 4194304;   // 2048 tiles: their sums fit in LDS

// The tree walk: G workgroups of kWalkBlock threads per request, each owning
// a slice of the tiles, exchanging 64-bit words.
constexpr int kWalkBlock = 512;
constexpr int kMaxWalkGroups = 32;
constexpr int64_t kMaxCoopBlocks = 2048;       // B * G never exceeds this
constexpr int kSpinLimit = 1 << 20;            // polls of one exchange before giving up

// G for a call: as many as keep every workgroup of the grid resident
// (occupancy per CU times the CU count), at most one per tile and 32.
inline int32_t walk_groups(int64_t B, int64_t V, int64_t resident) {
  if (resident > kMaxCoopBlocks) resident = kMaxCoopBlocks;
  int64_t g = B > 0 ? resident / B : 1;
  const int64_t nt = sample_tiles(V);
  if (g > kMaxWalkGroups) g = kMaxWalkGroups;
  if (g > nt) g = nt;
  return static_cast<int32_t>(g < 1 ? 1 : g);
}

// Upper bound of G over devices (the workspace query knows no device).
inline int64_t walk_groups_bound(int64_t B) {
  int64_t g = B > 0 ? kMaxCoopBlocks / B : 1;
  if (g > kMaxWalkGroups) g = kMaxWalkGroups;
  return g < 1 ? 1 : g;
}

// Exchanges of one walk over n nodes: one per visited node (its softmax pair)
// and one per weight pass (each rejected child, and the last distribution):
// the visited nodes and the rejected children are distinct nodes, so n + 1.
inline int64_t walk_max_sync(int64_t n_nodes) { return n_nodes + 1; }

// Workspace of the tree verify, carved per call: softmax partials of every
// row (diagnostics only), then the walk's exchange words [B, max_sync, 2 G]
// and tickets [B, G].  A walk's workgroups zero their own exchange words and
// then store the call's ticket (or a fill kernel zeroes them first).
struct WalkLayout {
  size_t partial_off, slots_off, arrive_off, end;
};

inline WalkLayout walk_layout(int64_t B, int64_t rows, int64_t V, int64_t G, int64_t max_sync) {
  WalkLayout L{};
  const int64_t nseg = row_segments(rows, V);
  L.partial_off = 0;
  L.slots_off = align256(static_cast<size_t>(rows * nseg) * 8);
  L.arrive_off = L.slots_off + align256(G > 1 ? static_cast<size_t>(B * max_sync * 2 * G) * 8 : 0);
  L.end = L.arrive_off + align256(G > 1 ? static_cast<size_t>(B * G) * 8 : 0);
  return L;
}

// Lazy chain statistics: the segments of one row fit the deciding block's LDS.
constexpr int kMaxChainSegs = static_cast<int>(kMaxSampleVocab / kSegElems);

struct ChainStatsArgs {
  const void* tgt;
  const void* dq;
  int64_t V;
  float c;
  int32_t B, k_max, t_rows, q_rows;
  const int32_t* t_rs;
  const int32_t* q_rs;
  const int32_t* ids;
  const int32_t* dlen;
  const float* u;        // [B, k_max + 1], or null: Philox stream (seed, offset)
  uint64_t seed, offset;
  int32_t nseg;
  int32_t row_hi;        // k_chain_stats: rows 0 .. row_hi - 1
  int32_t row_lo;        // k_chain_stats_tail: rows row_lo .. k_b
  uint32_t* stop;        // [B] kMaxChainRows - (first row that stops the round); 0: none
  uint32_t* count;       // [B, R] finished segments
  uint64_t* row_words;   // [B, R] row pairs
  uint64_t* seg_words;   // [B, R, nseg] segment pairs
  int32_t* status;
  int32_t spin_limit;
};

hipError_t launch_chain_stats(int t_dtype, int q_dtype, const ChainStatsArgs& a, hipStream_t stream);
// The rows from row_lo on of the requests still running, `blocks` blocks
// taking the items (kTailSegs segments of a row each) in turn (B <=
// kMaxTailRequests).
constexpr int kMaxTailRequests = 1024;
// Rows decided one by one (row-major blocks) before the rest of a lazy round
// go at once.
constexpr int kLazyRows = 2;
constexpr int kTailSegs = 4;  // segments per item of the rows after them
hipError_t launch_chain_stats_tail(int t_dtype, int q_dtype, const ChainStatsArgs& a, int64_t blocks,
                                   hipStream_t stream);

// ---- the draw of a sampled chain round (k_chain_draw) ----
// After the statistics kernel: the break row, the residual pass over it and
// the inverse-CDF draw.  Grid B x nblk blocks; block r of a request sums the
// kDrawTiles x tpw tiles from kDrawTiles tpw r on of the break row, wave w
// taking every kDrawTiles-th of them.
constexpr int kDrawTiles = 4;                  // waves per block
constexpr int kMaxDrawTpw = 64;                // tiles per wave at most
inline int32_t draw_blocks(int64_t V, int64_t tpw) {
  const int64_t per = static_cast<int64_t>(kDrawTiles) * tpw;
  return static_cast<int32_t>((sample_tiles(V) + per - 1) / per);
}

struct ChainDrawArgs {
  const void* tgt;
  const void* dq;
  int64_t V;
  float c;                   // log2(e) / T
  int32_t B, k_max, t_rows, q_rows;
  const int32_t* t_rs;
  const int32_t* q_rs;
  const int32_t* ids;
  const int32_t* dlen;
  const float* u;            // [B, k_max + 1], or null: Philox stream (seed, offset)
  uint64_t seed, offset;
  const int32_t* max_new;
  int32_t eos;
  int32_t nseg;              // statistics segments per row
  int32_t ntiles;            // 2048-element tiles per row
  int32_t nblk;              // draw blocks per request
  int32_t tpw;               // tiles per wave of a draw block
  int32_t spin_limit;
  // the break row: decided here from the partials of every row (partial
  // non-null), or by the lazy statistics (stop words and row pairs)
  const float2* partial;     // [t_rows, nseg]
  const uint32_t* stop;      // [B]
  const uint64_t* row_words; // [B, k_max + 1]
  // words zeroed by the statistics kernel (or a fill kernel) before the draw
  uint32_t* rcnt;            // [B] finished draw blocks
  uint64_t* tile_w;          // [B, ntiles] tile sums of the draw weights
  uint64_t* tile_p;          // [B, ntiles] tile sums of p (zero-mass fallback)
  uint64_t* blk_q;           // [B, nblk] class of the draft row's sum over each block's tiles
  // outputs
  int32_t* out_tok;
  int32_t* out_cnt;
  int32_t* out_acc;
  float* resid;
  int32_t* status;
};

hipError_t launch_chain_draw(int t_dtype, int q_dtype, const ChainDrawArgs& a, hipStream_t stream);
// Resident draw blocks per CU (occupancy query, cached per dtype pair and LDS size).
int draw_occupancy(int t_dtype, int q_dtype, size_t lds);

// Workspace of the sampled chain verify, carved per call (every part 256-byte
// aligned): softmax partials of every row [t_rows, nseg] float2; then the
// words zeroed before each call's draw: draw counts [B], tile sums [B, ntiles]
// twice and block classes [B, nblk]; then, for the lazy statistics (R =
// k_max + 1 rows per request, 0 otherwise): stop words [B], finished-segment
// counts [B, R], row pairs [B, R] and segment pairs [B, R, nseg].
struct ChainLayout {
  size_t partial_off, rcnt_off, tw_off, tp_off, bq_off, stop_off, count_off, rows_off, segs_off, end;
};

inline ChainLayout chain_layout(int64_t B, int64_t t_rows, int64_t V, int64_t lazy_R) {
  ChainLayout L{};
  // (the draw's block classes are sized for one tile per wave, the most blocks)
  const int64_t nseg = row_segments(t_rows, V), nt = sample_tiles(V), nblk = draw_blocks(V, 1);
  L.partial_off = 0;
  L.rcnt_off = align256(static_cast<size_t>(t_rows * nseg) * 8);
  L.tw_off = L.rcnt_off + align256(static_cast<size_t>(B) * 4);
  L.tp_off = L.tw_off + align256(static_cast<size_t>(B * nt) * 8);
  L.bq_off = L.tp_off + align256(static_cast<size_t>(B * nt) * 8);
  L.stop_off = L.bq_off + align256(static_cast<size_t>(B * nblk) * 8);
  L.count_off = L.stop_off + align256(static_cast<size_t>(lazy_R > 0 ? B : 0) * 4);
  L.rows_off = L.count_off + align256(static_cast<size_t>(B * lazy_R) * 4);
  L.segs_off = L.rows_off + align256(static_cast<size_t>(B * lazy_R) * 8);
  L.end = L.segs_off + align256(static_cast<size_t>(B * lazy_R * nseg) * 8);
  return L;
}
hipError_t launch_clear(void* p, size_t bytes, hipStream_t stream);

// Walk variants over a draft tree: speculative sampling, every candidate
// tested as a point mass on its own token, and the greedy (T = 0) tree.
enum WalkMode : int { kWalkTree = 1, kWalkPoint = 2, kWalkGreedy = 3 };

struct WalkArgs {
  const void* tgt;
  const void* dq;
  int64_t V;
  float c;                  // log2(e) / T
  int32_t B;
  const float* u;           // [B, slots], or null: Philox stream (seed, offset)
  uint64_t seed, offset;
  // chain: request b has k_b = dlen[b] drafts, rows t_rs[b] + i and q_rs[b] + i
  int32_t t_rows, q_rows;
  const int32_t* t_rs;
  const int32_t* q_rs;
  const int32_t* ids;
  const int32_t* dlen;
  int32_t k_max;
  const int32_t* max_new;
  int32_t eos;
  float* resid;
  // tree: N nodes per request, rows b * N + c
  const int32_t* parent;
  const int32_t* token;
  int32_t N;
  int32_t* out_path;
  // outputs
  int32_t* out_tok;
  int32_t* out_cnt;
  int32_t* out_acc;
  int32_t* status;
  float* diag;
  const float2* partial;    // softmax partials of every row (diagnostics only)
  int32_t nseg;
  // the split
  int32_t ntiles;
  int32_t G;
  uint64_t* slots;          // [B, max_sync, 2 G] exchange words (G > 1)
  // tree walks: each workgroup zeroes its own exchange words, then stores
  // `ticket` (unique to the call) into arrive[b, g]; the first exchange of a
  // request waits for all G tickets.  Null: the words were zeroed before.
  uint64_t* arrive;
  uint64_t ticket;
  int32_t max_sync;
  int32_t spin_limit;
  int32_t node_cap;         // LDS capacity in nodes (>= nodes of any request)
  int32_t tile_cap;         // LDS capacity in tiles (>= tiles of any slice)
  int32_t cache;            // sampled tree walk: nonzero when LDS holds a copy of the slice's draw inputs
};

// Dynamic LDS of a walk workgroup; with_cache adds the sampled tree walk's
// copy of its slice's p and q (16 KB per tile).
size_t walk_lds_bytes(int node_cap, int tile_cap, bool with_cache = false);
// Resident walk workgroups per CU at this much dynamic LDS (0: none fits).
int walk_occupancy(int mode, int t_dtype, int q_dtype, size_t lds);
// Launches a tree walk (and the diagnostics, when asked for).  clear_slots:
// zero the exchange words first (not needed when the statistics kernel or the
// walk itself does it).  The point-mass and greedy walks read no draft rows
// (q_dtype is ignored).
hipError_t launch_walk(int mode, int t_dtype, int q_dtype, const WalkArgs& a, size_t lds,
                       bool clear_slots, hipStream_t stream);
// A sampled chain round with a one-tile vocabulary (V <= 2048): one wave per
// request from the partials of every row (k_walk_small), and the diagnostics
// when asked for.
hipError_t launch_walk_small(int t_dtype, int q_dtype, const WalkArgs& a, hipStream_t stream);
// Diagnostics of a sampled chain (M, S, p(x), q(x) per row) from a.partial.
hipError_t launch_chain_diag(int t_dtype, int q_dtype, const WalkArgs& a, hipStream_t stream);

struct GreedyArgs {
  const void* tgt;
  int64_t V;
  int32_t t_rows;
  const int32_t* t_rs;
  const int32_t* ids;
  const int32_t* dlen;
  int32_t B, k_max;
  const int32_t* max_new;
  int32_t eos;
  int32_t* out_tok;
  int32_t* out_cnt;
  int32_t* out_acc;
  int32_t* status;
  const uint64_t* keys;
  int32_t nseg;
};


// Softmax partials of every row; optionally zeroes clear_words 8-byte words
// at `clear` (16-byte aligned) on the side.
hipError_t launch_row_stats(int dtype, const void* rows, int64_t n_rows, int64_t V, int32_t nseg,
                            float c, float2* partial, hipStream_t stream, uint64_t* clear = nullptr,
                            int64_t clear_words = 0);
// A pure streaming read of `bytes` (a multiple of 16) at buf, one 32-bit fold
// per block into out: the HBM read ceiling (measurement tool).
inline int64_t read_blocks(int64_t bytes) { return (bytes / 16 + 4 * kSegElems / 8 - 1) / (4 * kSegElems / 8); }
hipError_t launch_read_ceiling(const void* buf, int64_t bytes, uint32_t* out, hipStream_t stream);
hipError_t launch_row_argmax(int dtype, const void* rows, int64_t n_rows, int64_t V, int32_t nseg,
                             uint64_t* keys, hipStream_t stream);
hipError_t launch_greedy_resolve(const GreedyArgs& a, hipStream_t stream);
// ---- EAGLE-2 draft tree on the device ----
constexpr int kMaxTreeCand = 1024;   // candidates per request (one finalize thread each)
constexpr int kMaxTreeExpand = 64;   // expanded nodes per request and round
constexpr int kMaxTreeTop = 16;      // children per expanded node

// Segments per row of the top-k pass: about 16 Ki elements per block, and at
// least ~1024 blocks in total when rows are few (never below 2 Ki elements).
inline int32_t tree_topk_segments(int64_t rows, int64_t V) {
  int64_t nseg = (V + 16383) / 16384;
  if (rows > 0 && rows * nseg < 1024) {
    const int64_t want = (1024 + rows - 1) / rows;
    const int64_t cap = (V + 2047) / 2048;
    nseg = std::max<int64_t>(nseg, std::min(want, cap));
  }
  if (nseg < 1) nseg = 1;
  if (nseg > 64) nseg = 64;
  return static_cast<int32_t>(nseg);
}

struct TreeRoundArgs {
  int32_t B, n_exp, top, expand_next, max_cand, nseg;
  bool first;             // the roots' round: node 0 is created here and expanded
  const int32_t* exp;     // [B, n_exp] candidates whose rows are given (-1: none)
  uint64_t* keys;         // [B * n_exp, nseg, top] segment keys (workspace)
  int32_t* token;         // candidates [B, max_cand] ...
  int32_t* parent;
  int32_t* depth;
  float* conf;
  double* value;
  int32_t* count;         // [B]
  int32_t* next;          // [B, expand_next]
  int32_t* status;
};

struct TreeFinalArgs {
  int32_t B, max_cand, n_nodes;
  const int32_t* token;
  const int32_t* parent;
  const int32_t* depth;
  const float* conf;
  const double* value;
  const int32_t* count;
  int32_t* out_parent;    // [B, n_nodes] flat arrays
  int32_t* out_token;
  int32_t* out_depth;
  int32_t* out_cand;
  uint8_t* out_mask;      // [B, n_nodes, n_nodes] or null
  int32_t* status;
};

hipError_t launch_tree_expand(int dtype, const void* rows, int64_t n_rows, int64_t V, const TreeRoundArgs& a,
                              hipStream_t stream);
hipError_t launch_tree_finalize(const TreeFinalArgs& a, hipStream_t stream);

// ---- vocabulary shards ----
constexpr int kMaxShards = 64;

struct ShardBounds {
  int32_t G;                      // shards
  int64_t b[kMaxShards + 1];      // shard g holds columns [b[g], b[g+1])
};

struct ShardArgs {
  const void* tgt;                // this shard's columns of the target rows [t_rows, width]
  const void* dq;                 // ... and of the draft rows [q_rows, width]
  int64_t V;                      // the whole vocabulary
  float c;                        // log2(e) / T
  int32_t B, k_max, t_rows, q_rows;
  const int32_t* t_rs;
  const int32_t* q_rs;
  const int32_t* ids;
  const int32_t* dlen;
  const float* u;                 // [B, k_max + 1], or null: Philox stream (seed, offset)
  uint64_t seed, offset;
  const int32_t* max_new;
  int32_t eos;
  int32_t shard;
  ShardBounds sb;
  const float* pairs;             // [G, t_rows, 2] every shard's pairs
  const float* at;                // [G, B, k_max, 2] every shard's gathered (logit, q)
  int64_t* state;                 // [B, 2] this shard's decision (m or -1, status bits)
  double* mass;                   // [G, B, 3] every shard's (residual, p, q) sums
  double* tiles;                  // [B, tile_cap, 2] this shard's tile sums
  int32_t tile_cap;
  int32_t* out_tok;
  int32_t* out_cnt;
  int32_t* out_acc;
  float* resid;
  int32_t* status;
};

hipError_t launch_shard_fold(const float2* partial, int64_t rows, int32_t nseg, float* pairs, hipStream_t stream);
// step 1: gather the drafted tokens' values (at); step 2: decisions and this
// shard's weight sums; step 3: the draw and the outputs.
hipError_t launch_shard_step(int step, int t_dtype, int q_dtype, const ShardArgs& a, float* at, hipStream_t stream);

// Fill u [B, slots] with the Philox stream (seed, offset).
hipError_t launch_philox_fill(uint64_t seed, uint64_t offset, int32_t B, int32_t slots, float* u,
                              hipStream_t stream);
hipError_t launch_ngram(const int32_t* ctx, const int32_t* ctx_len, int32_t B, int32_t stride,
                        int32_t window, int32_t k, int32_t* ids, int32_t* lens, int32_t* status,
                        hipStream_t stream);

}  // namespace sv
