// libspecverify C ABI: argument checks, workspace layout, kernel launches.
// The operations and their contracts are documented in include/specverify.h.
#include "specverify.h"
#include "specverify_debug.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "api_internal.hpp"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

// Measurement hook (sv_debug_time_kernel_once): the events that take the
// start and end times of the streaming kernel of this thread's next verify
// call.
thread_local hipEvent_t g_stat_ev[2] = {nullptr, nullptr};

// Hands the armed hook's events to this thread's next timed kernel launch
// (the call's streaming kernel launches next).
void time_next_kernel() {
  if (g_stat_ev[0] != nullptr) sv::g_timed = sv::TimedEvents{g_stat_ev[0], g_stat_ev[1]};
}

sv_status fail(sv_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

sv_status device_fail(hipError_t e, const char* what) {
  return fail(SV_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool dtype_ok(int32_t d) { return d == SV_F32 || d == SV_BF16; }

// Disarms the measurement hook when a verify call returns (it serves that
// call at most).
struct HookDone {
  ~HookDone() {
    g_stat_ev[0] = g_stat_ev[1] = nullptr;
    sv::g_timed = sv::TimedEvents{};
  }
};

sv_status check_workspace(const void* ws, size_t have, size_t need) {
  if (need == 0) return SV_OK;
  if (ws == nullptr) return fail(SV_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(SV_E_WORKSPACE, "workspace is not 256-byte aligned");
  if (have < need) return fail(SV_E_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return SV_OK;
}

constexpr int64_t kMaxGrid = 0x7fffffff;

// A 64-bit value that no earlier call of this process has used, never 0: the
// tree walks' per-call ticket.  The start is mixed from the clock and an
// address (SplitMix64 finaliser), so another process's leftovers in a reused
// allocation match a ticket only by a 2^-64 chance.
uint64_t next_ticket() {
  static std::atomic<uint64_t> next{[] {
    uint64_t z = static_cast<uint64_t>(std::chrono::steady_clock::now().time_since_epoch().count()) ^
                 reinterpret_cast<uintptr_t>(&g_err);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
  }()};
  uint64_t t;
  do {
    t = next.fetch_add(1, std::memory_order_relaxed);
  } while (t == 0);
  return t;
}

// A device attribute of the current device, cached per device (0 on error).
int device_attr(hipDeviceAttribute_t attr, std::atomic<int>* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) {
    if (const int n = cache[dev].load(std::memory_order_relaxed)) return n;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, attr, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Compute units of the current device (0 if unknown).
int cu_count() {
  static std::atomic<int> cache[64];
  return device_attr(hipDeviceAttributeMultiprocessorCount, cache);
}

// LDS bytes one workgroup may allocate.
int max_lds_per_block() {
  static std::atomic<int> cache[64];
  return device_attr(hipDeviceAttributeMaxSharedMemoryPerBlock, cache);
}


// Whether a sampled chain call takes the lazy statistics (k_chain_stats):
// requests own their rows (enough rows for every request's own), and a row
// has at least two waves of statistics blocks (8 resident blocks per CU), so
// a row's decision is known before the next row's blocks start; with fewer,
// streaming every row is faster.  Diagnostics need every row's statistics.
bool chain_lazy(int64_t B, int64_t t_rows, int64_t V, int64_t k_max, bool diag) {
  const int64_t nseg = sv::row_segments(t_rows, V);
  return !diag && sv::sample_tiles(V) > 1 && t_rows >= k_max + 1 && 2 * t_rows >= B * (k_max + 1) &&
         B * nseg >= 2 * 8 * static_cast<int64_t>(std::max(cu_count(), 1)) && (k_max + 1) * B * nseg <= kMaxGrid;
}

// Workspace of a sampled chain call with these sizes (either statistics path).
size_t chain_need(int64_t B, int64_t t_rows, int64_t V, int64_t k_max) {
  if (B == 0) return 0;
  const int64_t R = std::max<int64_t>(1, std::min<int64_t>(t_rows, k_max + 1));
  return sv::chain_layout(B, t_rows, V, R).end;
}

// The sampled chain verify: the statistics kernel (the partials of every
// row, which zeroes the draw's words on the side, or a fill kernel and the
// lazy statistics), then the draw (k_chain_draw); a one-tile vocabulary is one
// wave's work per request (k_walk_small).
sv_status launch_chain_call(int32_t t_dtype, int32_t q_dtype, sv::WalkArgs& a, void* workspace, hipStream_t st,
                            const char* what) {
  const int64_t ntiles = sv::sample_tiles(a.V);
  const bool lazy = chain_lazy(a.B, a.t_rows, a.V, a.k_max, a.diag != nullptr);
  const sv::ChainLayout L = sv::chain_layout(a.B, a.t_rows, a.V, lazy ? a.k_max + 1 : 0);
  char* ws = static_cast<char*>(workspace);
  float2* partial = reinterpret_cast<float2*>(ws + L.partial_off);
  // tiles per wave of the draw: the fewest that keep every draw block resident
  // at once (each block pays its prologue's load rounds once)
  const size_t draw_lds = static_cast<size_t>(ntiles) * sizeof(double);
  const int64_t resident =
      static_cast<int64_t>(sv::draw_occupancy(t_dtype, q_dtype, draw_lds)) * std::max(cu_count(), 1);
  const int64_t quads = (ntiles + sv::kDrawTiles - 1) / sv::kDrawTiles;
  const int64_t tpw = std::min<int64_t>(sv::kMaxDrawTpw, std::max<int64_t>(1, (a.B * quads + resident - 1) / resident));
  const int64_t nblk = sv::draw_blocks(a.V, tpw);
  if (static_cast<int64_t>(a.B) * nblk > kMaxGrid) return fail(SV_E_ARG, "too many requests");
  (void)hipGetLastError();
  hipError_t e = hipSuccess;
  if (lazy) {
    e = sv::launch_clear(ws + L.rcnt_off, L.end - L.rcnt_off, st);
    if (e != hipSuccess) return device_fail(e, what);
    sv::ChainStatsArgs c{};
    c.tgt = a.tgt;
    c.dq = a.dq;
    c.V = a.V;
    c.c = a.c;
    c.B = a.B;
    c.k_max = a.k_max;
    c.t_rows = a.t_rows;
    c.q_rows = a.q_rows;
    c.t_rs = a.t_rs;
    c.q_rs = a.q_rs;
    c.ids = a.ids;
    c.dlen = a.dlen;
    c.u = a.u;
    c.seed = a.seed;
    c.offset = a.offset;
    c.nseg = a.nseg;
    c.stop = reinterpret_cast<uint32_t*>(ws + L.stop_off);
    c.count = reinterpret_cast<uint32_t*>(ws + L.count_off);
    c.row_words = reinterpret_cast<uint64_t*>(ws + L.rows_off);
    c.seg_words = reinterpret_cast<uint64_t*>(ws + L.segs_off);
    c.status = a.status;
    c.spin_limit = sv::kSpinLimit;
    // rows 0 .. kLazyRows - 1 one by one, then the rest of every round still
    // running at once (a fixed grid of blocks taking their segments in turn)
    const int R = a.k_max + 1;
    const bool tail = R > sv::kLazyRows && a.B <= sv::kMaxTailRequests;
    c.row_hi = tail ? sv::kLazyRows : R;
    c.row_lo = sv::kLazyRows;
    time_next_kernel();
    e = sv::launch_chain_stats(t_dtype, q_dtype, c, st);
    if (e != hipSuccess) return device_fail(e, what);
    if (tail) {
      const int64_t items = static_cast<int64_t>(a.B) * (R - sv::kLazyRows) * ((a.nseg + sv::kTailSegs - 1) / sv::kTailSegs);
      e = sv::launch_chain_stats_tail(t_dtype, q_dtype, c,
                                      std::min<int64_t>(items, 8 * static_cast<int64_t>(std::max(cu_count(), 1))), st);
      if (e != hipSuccess) return device_fail(e, what);
    }
  } else {
    const bool small = ntiles == 1;  // k_walk_small reads only the partials
    if (!small) time_next_kernel();
    e = sv::launch_row_stats(t_dtype, a.tgt, a.t_rows, a.V, a.nseg, a.c, partial, st,
                             small ? nullptr : reinterpret_cast<uint64_t*>(ws + L.rcnt_off),
                             small ? 0 : static_cast<int64_t>(L.stop_off - L.rcnt_off) / 8);
    if (e != hipSuccess) return device_fail(e, what);
    if (small) {  // one tile: one wave per request does the whole round
      a.partial = partial;
      a.ntiles = 1;
      time_next_kernel();
      e = sv::launch_walk_small(t_dtype, q_dtype, a, st);
      return e == hipSuccess ? SV_OK : device_fail(e, what);
    }
    if (a.diag != nullptr) {
      a.partial = partial;
      e = sv::launch_chain_diag(t_dtype, q_dtype, a, st);
      if (e != hipSuccess) return device_fail(e, what);
    }
  }
  sv::ChainDrawArgs d{};
  d.tgt = a.tgt;
  d.dq = a.dq;
  d.V = a.V;
  d.c = a.c;
  d.B = a.B;
  d.k_max = a.k_max;
  d.t_rows = a.t_rows;
  d.q_rows = a.q_rows;
  d.t_rs = a.t_rs;
  d.q_rs = a.q_rs;
  d.ids = a.ids;
  d.dlen = a.dlen;
  d.u = a.u;
  d.seed = a.seed;
  d.offset = a.offset;
  d.max_new = a.max_new;
  d.eos = a.eos;
  d.nseg = a.nseg;
  d.ntiles = static_cast<int32_t>(ntiles);
  d.nblk = static_cast<int32_t>(nblk);
  d.tpw = static_cast<int32_t>(tpw);
  d.spin_limit = sv::kSpinLimit;
  d.partial = lazy ? nullptr : partial;
  d.stop = lazy ? reinterpret_cast<const uint32_t*>(ws + L.stop_off) : nullptr;
  d.row_words = lazy ? reinterpret_cast<const uint64_t*>(ws + L.rows_off) : nullptr;
  d.rcnt = reinterpret_cast<uint32_t*>(ws + L.rcnt_off);
  d.tile_w = reinterpret_cast<uint64_t*>(ws + L.tw_off);
  d.tile_p = reinterpret_cast<uint64_t*>(ws + L.tp_off);
  d.blk_q = reinterpret_cast<uint64_t*>(ws + L.bq_off);
  d.out_tok = a.out_tok;
  d.out_cnt = a.out_cnt;
  d.out_acc = a.out_acc;
  d.resid = a.resid;
  d.status = a.status;
  e = sv::launch_chain_draw(t_dtype, q_dtype, d, st);
  return e == hipSuccess ? SV_OK : device_fail(e, what);
}

// Shared tail of the three tree verifies: the split into G workgroups per
// request, the workspace carve-up and the launches.  The walk computes a
// node's statistics when it gets there; only diagnostics need the partials
// of every row.
sv_status launch_walk_call(int mode, int32_t t_dtype, int32_t q_dtype, sv::WalkArgs& a, int64_t rows,
                           int64_t nodes, int64_t node_cap, void* workspace, hipStream_t st,
                           const char* what) {
  const int64_t ntiles = sv::sample_tiles(a.V);
  const int64_t max_sync = sv::walk_max_sync(nodes);
  char* ws = static_cast<char*>(workspace);
  // G from the occupancy at the largest slice this kernel may get
  const size_t lds_max = sv::walk_lds_bytes(static_cast<int>(node_cap), static_cast<int>(ntiles));
  const int occ = sv::walk_occupancy(mode, t_dtype, q_dtype, lds_max);
  const int64_t resident = static_cast<int64_t>(occ) * std::max(cu_count(), 1);
  a.G = std::min<int32_t>(sv::walk_groups(a.B, a.V, resident),
                          static_cast<int32_t>(sv::walk_groups_bound(a.B)));
  // The point-mass walk makes one pass per visited node and then only
  // exchanges per rejected candidate: the fewest workgroups that still give
  // every wave at most one tile per pass (measured 7% faster on the 60-node
  // trees at V = 128,256 than one workgroup per CU).
  if (mode == sv::kWalkPoint) {
    constexpr int kWaves = sv::kWalkBlock / 64;
    a.G = std::min<int32_t>(a.G, static_cast<int32_t>(std::max<int64_t>(1, (ntiles + kWaves - 1) / kWaves)));
  }
  const sv::WalkLayout L = sv::walk_layout(a.B, rows, a.V, a.G, max_sync);
  a.ntiles = static_cast<int32_t>(ntiles);
  a.tile_cap = static_cast<int32_t>((ntiles + a.G - 1) / a.G);
  a.node_cap = static_cast<int32_t>(node_cap);
  a.max_sync = static_cast<int32_t>(max_sync);
  a.spin_limit = sv::kSpinLimit;
  a.slots = reinterpret_cast<uint64_t*>(ws + L.slots_off);
  a.partial = reinterpret_cast<const float2*>(ws + L.partial_off);
  if (static_cast<int64_t>(a.B) * a.G > kMaxGrid) return fail(SV_E_ARG, "too many requests");
  (void)hipGetLastError();
  bool clear_slots = true;
  if (a.diag != nullptr) {  // the diagnostics read every row's partials
    const int64_t slot_words = static_cast<int64_t>(L.end - L.slots_off) / 8;
    const hipError_t e = sv::launch_row_stats(t_dtype, a.tgt, rows, a.V, a.nseg, a.c,
                                              reinterpret_cast<float2*>(ws + L.partial_off), st,
                                              a.slots, slot_words);
    if (e != hipSuccess) return device_fail(e, what);
    clear_slots = false;  // the statistics kernel zeroed the exchange words
  }
  // The walks zero their own exchange words, certified by a ticket unique to
  // the call.  A captured call would replay one ticket, so under stream
  // capture the words are zeroed by a kernel before the walk instead.
  a.arrive = nullptr;
  a.ticket = 0;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusActive;
  if (a.G > 1 && hipStreamIsCapturing(st, &cap) == hipSuccess && cap == hipStreamCaptureStatusNone) {
    a.arrive = reinterpret_cast<uint64_t*>(ws + L.arrive_off);
    a.ticket = next_ticket();
    clear_slots = false;
  }
  // The sampled tree walk keeps its slice's p and q in LDS for a node's later
  // residual passes when that fits and leaves the grid resident.
  size_t lds = sv::walk_lds_bytes(a.node_cap, a.tile_cap);
  a.cache = 0;
  if (mode == sv::kWalkTree) {
    const size_t with = sv::walk_lds_bytes(a.node_cap, a.tile_cap, true);
    if (with <= static_cast<size_t>(max_lds_per_block()) &&
        static_cast<int64_t>(a.B) * a.G <=
            static_cast<int64_t>(sv::walk_occupancy(mode, t_dtype, q_dtype, with)) * std::max(cu_count(), 1)) {
      a.cache = 1;
      lds = with;
    }
  }
  time_next_kernel();
  const hipError_t e = sv::launch_walk(mode, t_dtype, q_dtype, a, lds, clear_slots, st);
  return e == hipSuccess ? SV_OK : device_fail(e, what);
}
}  // namespace

namespace sv {

thread_local TimedEvents g_timed;

sv_status set_error(sv_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

size_t sample_need(int64_t B, int64_t t_rows, int64_t V, int64_t k_max) { return chain_need(B, t_rows, V, k_max); }

}  // namespace sv

extern "C" {

int sv_abi_version(void) { return SV_ABI_VERSION; }

const char* sv_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_E_ARG: return "invalid argument";
    case SV_E_DTYPE: return "unsupported dtype";
    case SV_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case SV_E_DEVICE: return "HIP device error";
    default: return "unknown status";
  }
}

const char* sv_last_error(void) { return g_err; }

size_t sv_workspace_bytes(int op, int64_t batch, int64_t total_rows, int64_t vocab) {
  if (batch < 0 || total_rows < 0 || vocab <= 0) return 0;
  switch (op) {
    case SV_OP_GREEDY:
      return sv::align256(static_cast<size_t>(total_rows * sv::argmax_segments(total_rows, vocab)) * 8);
    case SV_OP_TREE:
      if (batch == 0) return 0;
      return sv::walk_layout(batch, total_rows, vocab, sv::walk_groups_bound(batch),
                             sv::walk_max_sync(total_rows / batch)).end;
    case SV_OP_TREE_EXPAND:  // total_rows = batch * expanded nodes per request
      return sv::align256(static_cast<size_t>(total_rows * sv::tree_topk_segments(total_rows, vocab)) *
                          sv::kMaxTreeTop * 8);
    case SV_OP_SHARD: {  // total_rows = t_rows, vocab = the shard's column count
      const size_t partials = static_cast<size_t>(total_rows * sv::row_segments(total_rows, vocab)) * 8;
      const size_t state = sv::align256(static_cast<size_t>(batch) * 16);
      const size_t tiles = static_cast<size_t>(batch * sv::sample_tiles(vocab)) * 16;
      return sv::align256(std::max(partials, state + tiles));
    }
    case SV_OP_SAMPLE:  // any k_max the rows allow (a request has at most min(t_rows, 256) rows)
      return chain_need(batch, total_rows, vocab, std::min<int64_t>(total_rows, sv::kMaxChainRows) - 1);
    default:
      return 0;
  }
}

size_t sv_sample_workspace_bytes(int64_t batch, int64_t t_rows, int64_t vocab, int32_t k_max) {
  if (batch < 0 || t_rows < 0 || vocab <= 0 || k_max < 0 || k_max >= sv::kMaxChainRows) return 0;
  return chain_need(batch, t_rows, vocab, k_max);
}

sv_status sv_debug_time_kernel_once(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr)) return fail(SV_E_ARG, "give both events or neither");
  g_stat_ev[0] = static_cast<hipEvent_t>(before);
  g_stat_ev[1] = static_cast<hipEvent_t>(after);
  return SV_OK;
}

int64_t sv_debug_read_blocks(int64_t bytes) { return bytes <= 0 ? 0 : sv::read_blocks(bytes); }

sv_status sv_debug_read_ceiling(const void* buf, int64_t bytes, uint32_t* out, void* stream) {
  HookDone hook_done;
  if (bytes < 0 || (bytes & 15) != 0) return fail(SV_E_ARG, "bytes must be a non-negative multiple of 16");
  if (bytes == 0) return SV_OK;
  if (buf == nullptr || out == nullptr || (reinterpret_cast<uintptr_t>(buf) & 15u) != 0)
    return fail(SV_E_ARG, "buf (16-byte aligned) and out are needed");
  (void)hipGetLastError();
  time_next_kernel();
  const hipError_t e = sv::launch_read_ceiling(buf, bytes, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : device_fail(e, "sv_debug_read_ceiling");
}

int32_t sv_softmax_segments(int64_t n_rows, int64_t vocab) {
  if (n_rows < 0 || vocab < 1) return 0;
  return sv::row_segments(n_rows, vocab);
}

sv_status sv_softmax_partials(const void* rows, int32_t dtype, int64_t n_rows, int64_t vocab,
                              float temperature, float* out_partials, void* stream) {
  if (!dtype_ok(dtype)) return fail(SV_E_DTYPE, "dtype must be SV_F32 or SV_BF16");
  if (n_rows < 0 || vocab < 1) return fail(SV_E_ARG, "n_rows must be >= 0 and vocab >= 1");
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(SV_E_ARG, "temperature must be finite and > 0");
  if (n_rows == 0) return SV_OK;
  if (rows == nullptr || out_partials == nullptr) return fail(SV_E_ARG, "null pointer argument");
  const int32_t nseg = sv::row_segments(n_rows, vocab);
  if (n_rows * nseg > kMaxGrid) return fail(SV_E_ARG, "too many rows");
  (void)hipGetLastError();
  const hipError_t e = sv::launch_row_stats(dtype, rows, n_rows, vocab, nseg, sv::kLog2e / temperature,
                                            reinterpret_cast<float2*>(out_partials),
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : device_fail(e, "sv_softmax_partials launch");
}

sv_status sv_ngram_draft(const int32_t* ctx, const int32_t* ctx_len, int32_t batch,
                         int32_t ctx_stride, int32_t window, int32_t k, int32_t* draft_ids,
                         int32_t* draft_len, int32_t* dev_status, void* stream) {
  HookDone hook_done;
  if (batch < 0) return fail(SV_E_ARG, "batch < 0");
  if (ctx_stride < 1) return fail(SV_E_ARG, "ctx_stride < 1");
  if (window < 1 || window > sv::kMaxWindow) return fail(SV_E_ARG, "window must be in [1, 64]");
  if (k < 0 || k > 1024) return fail(SV_E_ARG, "k must be in [0, 1024]");
  if (batch == 0) return SV_OK;
  if (ctx == nullptr || ctx_len == nullptr || draft_len == nullptr || (k > 0 && draft_ids == nullptr))
    return fail(SV_E_ARG, "null pointer argument");
  (void)hipGetLastError();
  time_next_kernel();
  const hipError_t e = sv::launch_ngram(ctx, ctx_len, batch, ctx_stride, window, k, draft_ids, draft_len,
                                        dev_status, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : device_fail(e, "sv_ngram_draft launch");
}

sv_status sv_verify_greedy(const void* target_logits, int32_t t_dtype, int32_t t_rows, int64_t vocab,
                           const int32_t* t_row_start, const int32_t* draft_ids,
                           const int32_t* draft_len, int32_t batch, int32_t k_max,
                           const int32_t* max_new, int32_t eos_id, int32_t* out_tokens,
                           int32_t* out_count, int32_t* out_accepted, int32_t* dev_status,
                           void* workspace, size_t workspace_bytes, void* stream) {
  HookDone hook_done;
  if (!dtype_ok(t_dtype)) return fail(SV_E_DTYPE, "t_dtype must be SV_F32 or SV_BF16");
  if (batch < 0) return fail(SV_E_ARG, "batch < 0");
  if (vocab < 1 || vocab > INT32_MAX) return fail(SV_E_ARG, "vocab must be in [1, 2^31)");
  if (k_max < 0 || k_max >= sv::kMaxChainRows) return fail(SV_E_ARG, "k_max must be in [0, 255]");
  if (t_rows < 0) return fail(SV_E_ARG, "t_rows < 0");
  if (batch == 0) return SV_OK;
  if (t_rows < 1) return fail(SV_E_ARG, "t_rows < 1");
  if (target_logits == nullptr || t_row_start == nullptr || draft_len == nullptr ||
      out_tokens == nullptr || out_count == nullptr || out_accepted == nullptr ||
      (k_max > 0 && draft_ids == nullptr))
    return fail(SV_E_ARG, "null pointer argument");
  const int32_t nseg = sv::argmax_segments(t_rows, vocab);
  if (static_cast<int64_t>(t_rows) * nseg > kMaxGrid) return fail(SV_E_ARG, "too many rows");
  const size_t need = sv_workspace_bytes(SV_OP_GREEDY, batch, t_rows, vocab);
  if (sv_status s = check_workspace(workspace, workspace_bytes, need)) return s;

  const hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  uint64_t* keys = static_cast<uint64_t*>(workspace);
  time_next_kernel();
  hipError_t e = sv::launch_row_argmax(t_dtype, target_logits, t_rows, vocab, nseg, keys, st);
  if (e != hipSuccess) return device_fail(e, "sv_verify_greedy argmax launch");
  sv::GreedyArgs a{};
  a.tgt = target_logits;
  a.V = vocab;
  a.t_rows = t_rows;
  a.t_rs = t_row_start;
  a.ids = draft_ids;
  a.dlen = draft_len;
  a.B = batch;
  a.k_max = k_max;
  a.max_new = max_new;
  a.eos = eos_id;
  a.out_tok = out_tokens;
  a.out_cnt = out_count;
  a.out_acc = out_accepted;
  a.status = dev_status;
  a.keys = keys;
  a.nseg = nseg;
  e = sv::launch_greedy_resolve(a, st);
  return e == hipSuccess ? SV_OK : device_fail(e, "sv_verify_greedy resolve launch");
}

// Sampled chain verify, with the uniforms from the caller (uniforms != null)
// or from the Philox stream (seed, offset).
static sv_status sample_impl(const void* target_logits, int32_t t_dtype, int32_t t_rows,
                             const void* draft_probs, int32_t q_dtype, int32_t q_rows, int64_t vocab,
                             const int32_t* t_row_start, const int32_t* q_row_start,
                             const int32_t* draft_ids, const int32_t* draft_len, int32_t batch,
                             int32_t k_max, float temperature, const float* uniforms, bool philox,
                             uint64_t seed, uint64_t offset, const int32_t* max_new, int32_t eos_id,
                             int32_t* out_tokens, int32_t* out_count, int32_t* out_accepted,
                             float* out_diag, float* out_resid, int32_t* dev_status, void* workspace,
                             size_t workspace_bytes, void* stream, const char* what) {
  HookDone hook_done;
  if (!dtype_ok(t_dtype) || !dtype_ok(q_dtype))
    return fail(SV_E_DTYPE, "t_dtype and q_dtype must be SV_F32 or SV_BF16");
  if (batch < 0) return fail(SV_E_ARG, "batch < 0");
  if (vocab < 1 || vocab > sv::kMaxSampleVocab) return fail(SV_E_ARG, "vocab must be in [1, 4194304]");
  if (k_max < 0 || k_max >= sv::kMaxChainRows) return fail(SV_E_ARG, "k_max must be in [0, 255]");
  if (t_rows < 0 || q_rows < 0) return fail(SV_E_ARG, "t_rows and q_rows must be >= 0");
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(SV_E_ARG, "temperature must be finite and > 0 (T = 0 is sv_verify_greedy)");
  if (batch == 0) return SV_OK;
  if (t_rows < 1) return fail(SV_E_ARG, "t_rows < 1");
  if (target_logits == nullptr || t_row_start == nullptr || q_row_start == nullptr ||
      draft_len == nullptr || (!philox && uniforms == nullptr) || out_tokens == nullptr || out_count == nullptr ||
      out_accepted == nullptr || (k_max > 0 && draft_ids == nullptr) ||
      (q_rows > 0 && draft_probs == nullptr))
    return fail(SV_E_ARG, "null pointer argument");
  const int32_t nseg = sv::row_segments(t_rows, vocab);
  if (static_cast<int64_t>(t_rows) * nseg > kMaxGrid) return fail(SV_E_ARG, "too many rows");
  const size_t need = chain_need(batch, t_rows, vocab, k_max);
  if (sv_status s = check_workspace(workspace, workspace_bytes, need)) return s;

  sv::WalkArgs a{};
  a.tgt = target_logits;
  a.dq = draft_probs;
  a.V = vocab;
  a.c = sv::kLog2e / temperature;
  a.B = batch;
  a.u = philox ? nullptr : uniforms;
  a.seed = seed;
  a.offset = offset;
  a.t_rows = t_rows;
  a.q_rows = q_rows;
  a.t_rs = t_row_start;
  a.q_rs = q_row_start;
  a.ids = draft_ids;
  a.dlen = draft_len;
  a.k_max = k_max;
  a.max_new = max_new;
  a.eos = eos_id;
  a.resid = out_resid;
  a.out_tok = out_tokens;
  a.out_cnt = out_count;
  a.out_acc = out_accepted;
  a.status = dev_status;
  a.diag = out_diag;
  a.nseg = nseg;
  return launch_chain_call(t_dtype, q_dtype, a, workspace, static_cast<hipStream_t>(stream), what);
}

}  // extern "C"

sv_status sv::verify_sample_on(const void* target_logits, int32_t t_dtype, int32_t t_rows, const void* draft_probs,
                               int32_t q_dtype, int32_t q_rows, int64_t vocab, const int32_t* t_row_start,
                               const int32_t* q_row_start, const int32_t* draft_ids, const int32_t* draft_len,
                               int32_t batch, int32_t k_max, float temperature, const float* uniforms,
                               const int32_t* max_new, int32_t eos_id, int32_t* out_tokens, int32_t* out_count,
                               int32_t* out_accepted, float* out_diag, float* out_resid, int32_t* dev_status,
                               void* workspace, size_t workspace_bytes, void* stream, const char* what) {
  return sample_impl(target_logits, t_dtype, t_rows, draft_probs, q_dtype, q_rows, vocab, t_row_start, q_row_start,
                     draft_ids, draft_len, batch, k_max, temperature, uniforms, false, 0, 0, max_new, eos_id,
                     out_tokens, out_count, out_accepted, out_diag, out_resid, dev_status, workspace,
                     workspace_bytes, stream, what);
}

extern "C" {

sv_status sv_verify_sample(const void* target_logits, int32_t t_dtype, int32_t t_rows,
                           const void* draft_probs, int32_t q_dtype, int32_t q_rows, int64_t vocab,
                           const int32_t* t_row_start, const int32_t* q_row_start,
                           const int32_t* draft_ids, const int32_t* draft_len, int32_t batch,
                           int32_t k_max, float temperature, const float* uniforms,
                           const int32_t* max_new, int32_t eos_id, int32_t* out_tokens,
                           int32_t* out_count, int32_t* out_accepted, float* out_diag,
                           float* out_resid, int32_t* dev_status, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return sample_impl(target_logits, t_dtype, t_rows, draft_probs, q_dtype, q_rows, vocab, t_row_start,
                     q_row_start, draft_ids, draft_len, batch, k_max, temperature, uniforms, false, 0, 0,
                     max_new, eos_id, out_tokens, out_count, out_accepted, out_diag, out_resid, dev_status,
                     workspace, workspace_bytes, stream, "sv_verify_sample");
}

sv_status sv_verify_sample_philox(const void* target_logits, int32_t t_dtype, int32_t t_rows,
                                  const void* draft_probs, int32_t q_dtype, int32_t q_rows, int64_t vocab,
                                  const int32_t* t_row_start, const int32_t* q_row_start,
                                  const int32_t* draft_ids, const int32_t* draft_len, int32_t batch,
                                  int32_t k_max, float temperature, uint64_t seed, uint64_t offset,
                                  const int32_t* max_new, int32_t eos_id, int32_t* out_tokens,
                                  int32_t* out_count, int32_t* out_accepted, float* out_diag,
                                  float* out_resid, int32_t* dev_status, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return sample_impl(target_logits, t_dtype, t_rows, draft_probs, q_dtype, q_rows, vocab, t_row_start,
                     q_row_start, draft_ids, draft_len, batch, k_max, temperature, nullptr, true, seed,
                     offset, max_new, eos_id, out_tokens, out_count, out_accepted, out_diag, out_resid,
                     dev_status, workspace, workspace_bytes, stream, "sv_verify_sample_philox");
}

sv_status sv_philox_uniforms(uint64_t seed, uint64_t offset, int32_t batch, int32_t slots, float* out,
                             void* stream) {
  if (batch < 0 || slots < 0) return fail(SV_E_ARG, "batch and slots must be >= 0");
  if (static_cast<int64_t>(batch) * slots == 0) return SV_OK;
  if (out == nullptr) return fail(SV_E_ARG, "null pointer argument");
  if (static_cast<int64_t>(batch) * slots > kMaxGrid * 256) return fail(SV_E_ARG, "too many slots");
  (void)hipGetLastError();
  const hipError_t e = sv::launch_philox_fill(seed, offset, batch, slots, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : device_fail(e, "sv_philox_uniforms");
}

sv_status sv_verify_tree(const void* target_logits, int32_t t_dtype, const void* draft_probs,
                         int32_t q_dtype, int64_t vocab, const int32_t* parent,
                         const int32_t* node_token, int32_t batch, int32_t n_nodes,
                         float temperature, const float* uniforms, int32_t* out_tokens,
                         int32_t* out_count, int32_t* out_accepted, int32_t* out_path,
                         float* out_diag, int32_t* dev_status, void* workspace,
                         size_t workspace_bytes, void* stream) {
  HookDone hook_done;
  if (!dtype_ok(t_dtype) || !dtype_ok(q_dtype))
    return fail(SV_E_DTYPE, "t_dtype and q_dtype must be SV_F32 or SV_BF16");
  if (batch < 0) return fail(SV_E_ARG, "batch < 0");
  if (n_nodes < 1 || n_nodes > sv::kMaxTreeNodes) return fail(SV_E_ARG, "n_nodes must be in [1, 1024]");
  if (vocab < 1 || vocab > sv::kMaxSampleVocab) return fail(SV_E_ARG, "tree vocab must be in [1, 4194304]");
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(SV_E_ARG, "temperature must be finite and > 0");
  if (batch == 0) return SV_OK;
  if (target_logits == nullptr || draft_probs == nullptr || parent == nullptr ||
      node_token == nullptr || uniforms == nullptr || out_tokens == nullptr ||
      out_count == nullptr || out_accepted == nullptr || out_path == nullptr)
    return fail(SV_E_ARG, "null pointer argument");
  const int64_t rows = static_cast<int64_t>(batch) * n_nodes;
  if (rows > INT32_MAX) return fail(SV_E_ARG, "too many rows");
  const int32_t nseg = sv::row_segments(rows, vocab);
  if (rows * nseg > kMaxGrid) return fail(SV_E_ARG, "too many rows");
  const size_t need = sv_workspace_bytes(SV_OP_TREE, batch, rows, vocab);
  if (sv_status s = check_workspace(workspace, workspace_bytes, need)) return s;

  sv::WalkArgs a{};
  a.tgt = target_logits;
  a.dq = draft_probs;
  a.V = vocab;
  a.c = sv::kLog2e / temperature;
  a.B = batch;
  a.u = uniforms;
  a.parent = parent;
  a.token = node_token;
  a.N = n_nodes;
  a.out_path = out_path;
  a.out_tok = out_tokens;
  a.out_cnt = out_count;
  a.out_acc = out_accepted;
  a.status = dev_status;
  a.diag = out_diag;
  a.nseg = nseg;
  return launch_walk_call(sv::kWalkTree, t_dtype, q_dtype, a, rows, n_nodes, n_nodes, workspace,
                          static_cast<hipStream_t>(stream), "sv_verify_tree");
}

// Greedy and point-mass tree verify: the same walk without draft rows.
static sv_status tree_variant(int mode, const void* target_logits, int32_t t_dtype, int64_t vocab,
                              const int32_t* parent, const int32_t* node_token, int32_t batch,
                              int32_t n_nodes, float temperature, const float* uniforms,
                              int32_t* out_tokens, int32_t* out_count, int32_t* out_accepted,
                              int32_t* out_path, int32_t* dev_status, void* workspace,
                              size_t workspace_bytes, void* stream, const char* what) {
  HookDone hook_done;
  if (!dtype_ok(t_dtype)) return fail(SV_E_DTYPE, "t_dtype must be SV_F32 or SV_BF16");
  if (batch < 0) return fail(SV_E_ARG, "batch < 0");
  if (n_nodes < 1 || n_nodes > sv::kMaxTreeNodes) return fail(SV_E_ARG, "n_nodes must be in [1, 1024]");
  if (vocab < 1 || vocab > sv::kMaxSampleVocab) return fail(SV_E_ARG, "tree vocab must be in [1, 4194304]");
  const bool greedy = mode == sv::kWalkGreedy;
  if (!greedy && (!(temperature > 0.f) || !std::isfinite(temperature)))
    return fail(SV_E_ARG, "temperature must be finite and > 0");
  if (batch == 0) return SV_OK;
  if (target_logits == nullptr || parent == nullptr || node_token == nullptr ||
      (!greedy && uniforms == nullptr) || out_tokens == nullptr || out_count == nullptr ||
      out_accepted == nullptr || out_path == nullptr)
    return fail(SV_E_ARG, "null pointer argument");
  const int64_t rows = static_cast<int64_t>(batch) * n_nodes;
  if (rows > INT32_MAX) return fail(SV_E_ARG, "too many rows");
  const int32_t nseg = sv::row_segments(rows, vocab);
  if (rows * nseg > kMaxGrid) return fail(SV_E_ARG, "too many rows");
  const size_t need = sv_workspace_bytes(SV_OP_TREE, batch, rows, vocab);
  if (sv_status s = check_workspace(workspace, workspace_bytes, need)) return s;

  sv::WalkArgs a{};
  a.tgt = target_logits;
  a.V = vocab;
  a.c = greedy ? 1.f : sv::kLog2e / temperature;
  a.B = batch;
  a.u = uniforms;
  a.parent = parent;
  a.token = node_token;
  a.N = n_nodes;
  a.out_path = out_path;
  a.out_tok = out_tokens;
  a.out_cnt = out_count;
  a.out_acc = out_accepted;
  a.status = dev_status;
  a.nseg = nseg;
  return launch_walk_call(mode, t_dtype, t_dtype, a, rows, n_nodes, n_nodes, workspace,
                          static_cast<hipStream_t>(stream), what);
}

sv_status sv_verify_tree_greedy(const void* target_logits, int32_t t_dtype, int64_t vocab,
                                const int32_t* parent, const int32_t* node_token, int32_t batch,
                                int32_t n_nodes, int32_t* out_tokens, int32_t* out_count,
                                int32_t* out_accepted, int32_t* out_path, int32_t* dev_status,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return tree_variant(sv::kWalkGreedy, target_logits, t_dtype, vocab, parent, node_token, batch, n_nodes,
                      0.f, nullptr, out_tokens, out_count, out_accepted, out_path, dev_status, workspace,
                      workspace_bytes, stream, "sv_verify_tree_greedy");
}

sv_status sv_verify_tree_pointmass(const void* target_logits, int32_t t_dtype, int64_t vocab,
                                   const int32_t* parent, const int32_t* node_token, int32_t batch,
                                   int32_t n_nodes, float temperature, const float* uniforms,
                                   int32_t* out_tokens, int32_t* out_count, int32_t* out_accepted,
                                   int32_t* out_path, int32_t* dev_status, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return tree_variant(sv::kWalkPoint, target_logits, t_dtype, vocab, parent, node_token, batch, n_nodes,
                      temperature, uniforms, out_tokens, out_count, out_accepted, out_path, dev_status,
                      workspace, workspace_bytes, stream, "sv_verify_tree_pointmass");
}

sv_status sv_tree_expand(const void* draft_rows, int32_t q_dtype, int64_t vocab, int32_t batch,
                         int32_t n_exp, const int32_t* exp_node, int32_t top_children,
                         int32_t expand_next, int32_t max_cand, int32_t* cand_token,
                         int32_t* cand_parent, int32_t* cand_depth, float* cand_conf,
                         double* cand_value, int32_t* cand_count, int32_t* next_exp,
                         int32_t* dev_status, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(q_dtype)) return fail(SV_E_DTYPE, "q_dtype must be SV_F32 or SV_BF16");
  if (batch < 0) return fail(SV_E_ARG, "batch < 0");
  if (n_exp < 1 || n_exp > sv::kMaxTreeExpand) return fail(SV_E_ARG, "n_exp must be in [1, 64]");
  if (exp_node == nullptr && n_exp != 1) return fail(SV_E_ARG, "the first round expands one root per request");
  if (top_children < 1 || top_children > sv::kMaxTreeTop) return fail(SV_E_ARG, "top_children must be in [1, 16]");
  if (vocab < top_children || vocab > INT32_MAX) return fail(SV_E_ARG, "vocab must be in [top_children, 2^31)");
  if (expand_next < 1 || expand_next > sv::kMaxTreeExpand) return fail(SV_E_ARG, "expand_next must be in [1, 64]");
  if (max_cand < 1 || max_cand > sv::kMaxTreeCand) return fail(SV_E_ARG, "max_cand must be in [1, 1024]");
  if (batch == 0) return SV_OK;
  if (draft_rows == nullptr || cand_token == nullptr || cand_parent == nullptr || cand_depth == nullptr ||
      cand_conf == nullptr || cand_value == nullptr || cand_count == nullptr || next_exp == nullptr)
    return fail(SV_E_ARG, "null pointer argument");
  const int64_t rows = static_cast<int64_t>(batch) * n_exp;
  const int32_t nseg = sv::tree_topk_segments(rows, vocab);
  if (rows * nseg > kMaxGrid) return fail(SV_E_ARG, "too many rows");
  const size_t need = sv_workspace_bytes(SV_OP_TREE_EXPAND, batch, rows, vocab);
  if (sv_status s = check_workspace(workspace, workspace_bytes, need)) return s;
  sv::TreeRoundArgs a{};
  a.B = batch;
  a.n_exp = n_exp;
  a.top = top_children;
  a.expand_next = expand_next;
  a.max_cand = max_cand;
  a.nseg = nseg;
  a.first = exp_node == nullptr;
  a.exp = exp_node;
  a.keys = static_cast<uint64_t*>(workspace);
  a.token = cand_token;
  a.parent = cand_parent;
  a.depth = cand_depth;
  a.conf = cand_conf;
  a.value = cand_value;
  a.count = cand_count;
  a.next = next_exp;
  a.status = dev_status;
  (void)hipGetLastError();
  const hipError_t e = sv::launch_tree_expand(q_dtype, draft_rows, rows, vocab, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : device_fail(e, "sv_tree_expand");
}

sv_status sv_tree_finalize(int32_t batch, int32_t max_cand, const int32_t* cand_token,
                           const int32_t* cand_parent, const int32_t* cand_depth, const float* cand_conf,
                           const double* cand_value, const int32_t* cand_count, int32_t n_nodes,
                           int32_t* out_parent, int32_t* out_token, int32_t* out_depth, int32_t* out_cand,
                           uint8_t* out_mask, int32_t* dev_status, void* stream) {
  if (batch < 0) return fail(SV_E_ARG, "batch < 0");
  if (max_cand < 1 || max_cand > sv::kMaxTreeCand) return fail(SV_E_ARG, "max_cand must be in [1, 1024]");
  if (n_nodes < 1 || n_nodes > sv::kMaxTreeNodes) return fail(SV_E_ARG, "n_nodes must be in [1, 1024]");
  if (batch == 0) return SV_OK;
  if (cand_token == nullptr || cand_parent == nullptr || cand_depth == nullptr || cand_conf == nullptr ||
      cand_value == nullptr || cand_count == nullptr || out_parent == nullptr || out_token == nullptr ||
      out_depth == nullptr || out_cand == nullptr)
    return fail(SV_E_ARG, "null pointer argument");
  sv::TreeFinalArgs a{};
  a.B = batch;
  a.max_cand = max_cand;
  a.n_nodes = n_nodes;
  a.token = cand_token;
  a.parent = cand_parent;
  a.depth = cand_depth;
  a.conf = cand_conf;
  a.value = cand_value;
  a.count = cand_count;
  a.out_parent = out_parent;
  a.out_token = out_token;
  a.out_depth = out_depth;
  a.out_cand = out_cand;
  a.out_mask = out_mask;
  a.status = dev_status;
  (void)hipGetLastError();
  const hipError_t e = sv::launch_tree_finalize(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : device_fail(e, "sv_tree_finalize");
}

// ---- vocabulary shards ----

// Checks shared by the three shard steps; fills the common fields of a.
static sv_status shard_setup(const void* target_cols, int32_t t_dtype, int32_t t_rows, const void* draft_cols,
                             int32_t q_dtype, int32_t q_rows, int64_t vocab, const int64_t* bounds,
                             int32_t n_shards, int32_t shard, const int32_t* t_row_start,
                             const int32_t* q_row_start, const int32_t* draft_ids, const int32_t* draft_len,
                             int32_t batch, int32_t k_max, float temperature, void* workspace,
                             size_t workspace_bytes, sv::ShardArgs& a) {
  if (!dtype_ok(t_dtype) || !dtype_ok(q_dtype))
    return fail(SV_E_DTYPE, "t_dtype and q_dtype must be SV_F32 or SV_BF16");
  if (batch < 0) return fail(SV_E_ARG, "batch < 0");
  if (k_max < 0 || k_max >= sv::kMaxChainRows) return fail(SV_E_ARG, "k_max must be in [0, 255]");
  if (t_rows < 1 || q_rows < 0) return fail(SV_E_ARG, "t_rows must be >= 1 and q_rows >= 0");
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(SV_E_ARG, "temperature must be finite and > 0");
  if (bounds == nullptr || n_shards < 1 || n_shards > sv::kMaxShards)
    return fail(SV_E_ARG, "bounds (host) with 1 <= n_shards <= 64 are needed");
  if (shard < 0 || shard >= n_shards) return fail(SV_E_ARG, "shard must be in [0, n_shards)");
  if (bounds[0] != 0 || bounds[n_shards] != vocab) return fail(SV_E_ARG, "bounds must run from 0 to vocab");
  for (int g = 0; g < n_shards; ++g)
    if (bounds[g + 1] <= bounds[g]) return fail(SV_E_ARG, "bounds must increase");
  const int64_t width = bounds[shard + 1] - bounds[shard];
  if (vocab > INT32_MAX || width > sv::kMaxSampleVocab)
    return fail(SV_E_ARG, "a shard holds at most 4194304 columns");
  if (batch > 0 && (target_cols == nullptr || t_row_start == nullptr || q_row_start == nullptr ||
                    draft_len == nullptr || (k_max > 0 && draft_ids == nullptr) ||
                    (q_rows > 0 && draft_cols == nullptr)))
    return fail(SV_E_ARG, "null pointer argument");
  if (static_cast<int64_t>(t_rows) * sv::row_segments(t_rows, width) > kMaxGrid)
    return fail(SV_E_ARG, "too many rows");
  const size_t need = sv_workspace_bytes(SV_OP_SHARD, batch, t_rows, width);
  if (batch > 0)
    if (sv_status st = check_workspace(workspace, workspace_bytes, need)) return st;
  a.tgt = target_cols;
  a.dq = draft_cols;
  a.V = vocab;
  a.c = sv::kLog2e / temperature;
  a.B = batch;
  a.k_max = k_max;
  a.t_rows = t_rows;
  a.q_rows = q_rows;
  a.t_rs = t_row_start;
  a.q_rs = q_row_start;
  a.ids = draft_ids;
  a.dlen = draft_len;
  a.shard = shard;
  a.sb.G = n_shards;
  for (int g = 0; g <= n_shards; ++g) a.sb.b[g] = bounds[g];
  a.tile_cap = static_cast<int32_t>(sv::sample_tiles(width));
  char* ws = static_cast<char*>(workspace);
  a.state = reinterpret_cast<int64_t*>(ws);
  a.tiles = reinterpret_cast<double*>(ws + sv::align256(static_cast<size_t>(batch) * 16));
  return SV_OK;
}

sv_status sv_shard_stats(const void* target_cols, int32_t t_dtype, int32_t t_rows, const void* draft_cols,
                         int32_t q_dtype, int32_t q_rows, int64_t vocab, const int64_t* bounds,
                         int32_t n_shards, int32_t shard, const int32_t* t_row_start,
                         const int32_t* q_row_start, const int32_t* draft_ids, const int32_t* draft_len,
                         int32_t batch, int32_t k_max, float temperature, float* out_pairs, float* out_at,
                         void* workspace, size_t workspace_bytes, void* stream) {
  sv::ShardArgs a{};
  if (sv_status st = shard_setup(target_cols, t_dtype, t_rows, draft_cols, q_dtype, q_rows, vocab, bounds,
                                 n_shards, shard, t_row_start, q_row_start, draft_ids, draft_len, batch, k_max,
                                 temperature, workspace, workspace_bytes, a))
    return st;
  if (batch == 0) return SV_OK;
  if (out_pairs == nullptr || (k_max > 0 && out_at == nullptr)) return fail(SV_E_ARG, "null pointer argument");
  const int64_t width = bounds[shard + 1] - bounds[shard];
  const int32_t nseg = sv::row_segments(t_rows, width);
  float2* partial = static_cast<float2*>(workspace);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipError_t e = sv::launch_row_stats(t_dtype, target_cols, t_rows, width, nseg, a.c, partial, st);
  if (e == hipSuccess) e = sv::launch_shard_fold(partial, t_rows, nseg, out_pairs, st);
  if (e == hipSuccess) e = sv::launch_shard_step(1, t_dtype, q_dtype, a, out_at, st);
  return e == hipSuccess ? SV_OK : device_fail(e, "sv_shard_stats");
}

sv_status sv_shard_residual(const void* target_cols, int32_t t_dtype, int32_t t_rows, const void* draft_cols,
                            int32_t q_dtype, int32_t q_rows, int64_t vocab, const int64_t* bounds,
                            int32_t n_shards, int32_t shard, const int32_t* t_row_start,
                            const int32_t* q_row_start, const int32_t* draft_ids, const int32_t* draft_len,
                            int32_t batch, int32_t k_max, float temperature, const float* uniforms,
                            const float* all_pairs, const float* all_at, double* mass, void* workspace,
                            size_t workspace_bytes, void* stream) {
  sv::ShardArgs a{};
  if (sv_status st = shard_setup(target_cols, t_dtype, t_rows, draft_cols, q_dtype, q_rows, vocab, bounds,
                                 n_shards, shard, t_row_start, q_row_start, draft_ids, draft_len, batch, k_max,
                                 temperature, workspace, workspace_bytes, a))
    return st;
  if (batch == 0) return SV_OK;
  if (uniforms == nullptr || all_pairs == nullptr || (k_max > 0 && all_at == nullptr) || mass == nullptr)
    return fail(SV_E_ARG, "null pointer argument");
  a.u = uniforms;
  a.pairs = all_pairs;
  a.at = all_at;
  a.mass = mass;
  (void)hipGetLastError();
  const hipError_t e = sv::launch_shard_step(2, t_dtype, q_dtype, a, nullptr, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : device_fail(e, "sv_shard_residual");
}

sv_status sv_shard_draw(const void* target_cols, int32_t t_dtype, int32_t t_rows, const void* draft_cols,
                        int32_t q_dtype, int32_t q_rows, int64_t vocab, const int64_t* bounds, int32_t n_shards,
                        int32_t shard, const int32_t* t_row_start, const int32_t* q_row_start,
                        const int32_t* draft_ids, const int32_t* draft_len, int32_t batch, int32_t k_max,
                        float temperature, const float* uniforms, const float* all_pairs, const double* mass,
                        const int32_t* max_new, int32_t eos_id, int32_t* out_tokens, int32_t* out_count,
                        int32_t* out_accepted, float* out_resid, int32_t* dev_status, void* workspace,
                        size_t workspace_bytes, void* stream) {
  sv::ShardArgs a{};
  if (sv_status st = shard_setup(target_cols, t_dtype, t_rows, draft_cols, q_dtype, q_rows, vocab, bounds,
                                 n_shards, shard, t_row_start, q_row_start, draft_ids, draft_len, batch, k_max,
                                 temperature, workspace, workspace_bytes, a))
    return st;
  if (batch == 0) return SV_OK;
  if (uniforms == nullptr || all_pairs == nullptr || mass == nullptr || out_tokens == nullptr ||
      out_count == nullptr || out_accepted == nullptr)
    return fail(SV_E_ARG, "null pointer argument");
  a.u = uniforms;
  a.pairs = all_pairs;
  a.mass = const_cast<double*>(mass);
  a.max_new = max_new;
  a.eos = eos_id;
  a.out_tok = out_tokens;
  a.out_cnt = out_count;
  a.out_acc = out_accepted;
  a.resid = out_resid;
  a.status = dev_status;
  (void)hipGetLastError();
  const hipError_t e = sv::launch_shard_step(3, t_dtype, q_dtype, a, nullptr, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : device_fail(e, "sv_shard_draw");
}

}  // extern "C"
