// Host-side launchers of the verify kernels and the workspace layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

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

// The sampled verify's inverse-CDF unit: one wave sums one tile.
constexpr int kSampleTile = 2048;
inline int64_t sample_tiles(int64_t V) { return (V + kSampleTile - 1) / kSampleTile; }
constexpr int kMaxTreeTiles = 512;     // tree vocab <= 512 * 2048

// Tree walk: workgroups per request (G) and the exchange words between them.
constexpr int kMaxTreeGroups = 32;
constexpr int kCoopBlocks = 256;       // B * G never exceeds this (nor the device's CU count)
constexpr int kSpinLimit = 1 << 20;    // polls of one exchange before giving up

inline int32_t tree_groups(int64_t B, int64_t V, int cu_count) {
  const int64_t cap = cu_count < kCoopBlocks ? cu_count : kCoopBlocks;
  int64_t g = B > 0 ? cap / B : 1;
  const int64_t nt = sample_tiles(V);
  if (g > kMaxTreeGroups) g = kMaxTreeGroups;
  if (g > nt) g = nt;
  return static_cast<int32_t>(g < 1 ? 1 : g);
}

// Upper bound of G over devices (the workspace query knows no device).
inline int64_t tree_groups_bound(int64_t B) {
  int64_t g = B > 0 ? kCoopBlocks / B : 1;
  if (g > kMaxTreeGroups) g = kMaxTreeGroups;
  return g < 1 ? 1 : g;
}

// At most one exchange per visited node and one per weight pass: 2 N.
inline int64_t tree_max_sync(int64_t N) { return 2 * N; }

struct TreeLayout {
  size_t partial_off, slots_off, bytes;
};

inline TreeLayout tree_layout(int64_t B, int64_t rows, int64_t V) {
  TreeLayout L{};
  const int64_t N = B > 0 ? rows / B : 0;
  const int64_t G = tree_groups_bound(B);
  L.partial_off = 0;
  L.slots_off = align256(static_cast<size_t>(rows * row_segments(rows, V)) * 8);
  const size_t slots = G > 1 ? static_cast<size_t>(B * tree_max_sync(N) * 2 * G) * 8 : 0;
  L.bytes = L.slots_off + align256(slots);
  return L;
}

struct SampleLayout {
  size_t partial_off, tiles_off, records_off, bytes;
};

inline SampleLayout sample_layout(int64_t B, int64_t t_rows, int64_t V) {
  SampleLayout L{};
  const int64_t nseg = row_segments(t_rows, V);
  L.partial_off = 0;
  L.tiles_off = align256(static_cast<size_t>(t_rows * nseg) * 8);
  L.records_off = L.tiles_off + align256(static_cast<size_t>(B * sample_tiles(V)) * 3 * 8);
  L.bytes = L.records_off + align256(static_cast<size_t>(B) * 16);
  return L;
}

struct SampleArgs {
  const void* tgt;
  const void* dq;
  int64_t V;
  int32_t t_rows, q_rows;
  const int32_t* t_rs;
  const int32_t* q_rs;
  const int32_t* ids;
  const int32_t* dlen;
  int32_t B, k_max;
  float c;      // log2(e) / T
  const float* u;
  const int32_t* max_new;
  int32_t eos;
  int32_t* out_tok;
  int32_t* out_cnt;
  int32_t* out_acc;
  float* diag;
  float* resid;
  int32_t* status;
  const float2* partial;
  int32_t nseg;
  double* tiles;     // [B, ntiles, 3] sums of (draw weights, p, q) per tile
  int4* records;     // [B] (status bits, m, scaled max, 1/normaliser) of the draw row
  int32_t ntiles;
};

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

struct TreeArgs {
  const void* tgt;
  const void* dq;
  int64_t V;
  const int32_t* parent;
  const int32_t* token;
  int32_t B, N;
  float c;      // log2(e) / T
  const float* u;
  int32_t* out_tok;
  int32_t* out_cnt;
  int32_t* out_acc;
  int32_t* out_path;
  float* diag;
  int32_t* status;
  const float2* partial;   // softmax partials of every row (diagnostics only)
  int32_t nseg;
  int32_t ntiles;
  uint64_t* slots;         // [B, max_sync, 2 G] exchange words (G > 1)
  int32_t G;               // workgroups per request
  int32_t max_sync;
  int32_t spin_limit;
};

hipError_t launch_row_stats(int dtype, const void* rows, int64_t n_rows, int64_t V, int32_t nseg,
                            float c, float2* partial, hipStream_t stream);
hipError_t launch_sample_resolve(int t_dtype, int q_dtype, const SampleArgs& a,
                                 hipStream_t stream);
hipError_t launch_row_argmax(int dtype, const void* rows, int64_t n_rows, int64_t V, int32_t nseg,
                             uint64_t* keys, hipStream_t stream);
hipError_t launch_greedy_resolve(const GreedyArgs& a, hipStream_t stream);
hipError_t launch_ngram(const int32_t* ctx, const int32_t* ctx_len, int32_t B, int32_t stride,
                        int32_t window, int32_t k, int32_t* ids, int32_t* lens, int32_t* status,
                        hipStream_t stream);
hipError_t launch_tree_walk(int t_dtype, int q_dtype, const TreeArgs& a, hipStream_t stream);

}  // namespace sv
