/*
 * libspecverify -- the verify step of speculative decoding on AMD Instinct
 * MI355X (gfx950).
 *
 * The operations, each following the pages that define it:
 *
 *   sv_ngram_draft    history n-gram (prompt-lookup) drafter
 *                     ("第 13 篇：推理引擎一次猜几个字——草稿 + 验证", notes under
 *                     section ③: take the context's last tokens as a window,
 *                     find the same fragment earlier, propose what followed).
 *   sv_verify_greedy  greedy (T = 0) prefix verify
 *                     (same article, section ③ pseudocode; "Speculative
 *                     decoding explained", four-case table).
 *   sv_verify_sample  speculative sampling: keep draft x with probability
 *                     min(1, p(x)/q(x)), stop at the first rejection, draw the
 *                     replacement from norm(max(0, p - q)), or one extra token
 *                     from p when every draft is kept
 *                     ("投机解码:为什么一个字都不改", sections "改进" and
 *                     "一轮能出几个 token"; p = softmax(logits / T) per the
 *                     figure "一次目标前向验 k 个草稿 token").
 *   sv_verify_tree    recursive speculative sampling over a flattened draft
 *                     tree, siblings tried in order with the residual update
 *                     in between ("Speculative Decoding II", EAGLE section:
 *                     the SpecInfer-style tree verify; EAGLE-2 worked example
 *                     for the flattened layout).
 *   sv_verify_tree_greedy     the same tree at T = 0 (argmax picks).
 *   sv_verify_tree_pointmass  the same tree with each candidate tested as a
 *                     point mass on its own token (deterministic top-k
 *                     candidates).
 *   sv_philox_uniforms, sv_verify_sample_philox  the verify's uniforms from a
 *                     counter-based generator on the device.
 *   sv_tree_expand, sv_tree_finalize  the EAGLE-2 draft tree the tree verify
 *                     takes, built on the device ("Speculative Decoding II",
 *                     EAGLE-2 section).
 *   sv_shard_stats, sv_shard_residual, sv_shard_draw  the sampled chain verify
 *                     on one device's column shard of the vocabulary.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All array arguments are DEVICE pointers on the current HIP device, except
 *   where marked "host".  `stream` is a hipStream_t (NULL = the default
 *   stream).  Every call only enqueues work on `stream` and returns; outputs,
 *   `dev_status` and the workspace are valid after the caller synchronises
 *   that stream.
 * - The caller owns every buffer.  The library allocates nothing, keeps no
 *   pointer after returning, and holds no mutable state that affects results:
 *   only the thread-local text behind sv_last_error(), per-device caches of
 *   launch parameters (compute-unit counts, kernel occupancy), and a
 *   process-wide counter that gives each tree-walk call a unique 64-bit
 *   ticket (outputs do not depend on its value).  (Measurement hooks for
 *   timing a call's streaming kernel and the read ceiling are declared apart,
 *   in specverify_debug.h; they are not part of the verify operations.)
 * - Row data: `t_dtype` / `q_dtype` select SV_F32 (float) or SV_BF16 (bfloat16
 *   bit patterns).  A row is `vocab` consecutive elements; row r starts at
 *   element r * vocab.  Any alignment is accepted; 16-byte aligned rows take the
 *   fastest path.
 * - Host-side argument checks return an error code and launch nothing.  Data
 *   problems found on the device never trap: they OR an SV_FLAG_* bit into
 *   *dev_status (if not NULL; the caller clears it) and the affected request
 *   gets a defined output.  A request with SV_FLAG_BAD_REQUEST, BAD_TOKEN,
 *   NONFINITE or BAD_TREE is invalid: count 0, accepted 0, all tokens -1.
 * - Workspace (greedy, sample, tree): caller-owned device memory of at least
 *   sv_workspace_bytes(...) bytes (sampled chains: sv_sample_workspace_bytes,
 *   which also knows k_max), 256-byte aligned.  Its contents need not be
 *   initialised: each call writes everything it later reads, so one buffer
 *   can serve calls of any shape in turn on one stream.  Calls that
 *   may run concurrently (different streams) need separate workspaces.
 * - HIP graphs: no entry point allocates, synchronises or records a memset,
 *   so calls can be captured on a stream and replayed.  The tree walks
 *   certify the zeroing of their exchange words with a ticket unique to the
 *   call; a captured call would replay its ticket, so under capture they zero
 *   the words with a kernel before the walk instead (the library asks the
 *   stream whether it is capturing).
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_ABI_VERSION 1

typedef enum {
  SV_OK = 0,
  SV_E_ARG = 1,        /* bad argument (null pointer, size out of range, T <= 0, ...) */
  SV_E_DTYPE = 2,      /* unsupported dtype */
  SV_E_WORKSPACE = 3,  /* workspace missing, misaligned or too small */
  SV_E_DEVICE = 4      /* a HIP call failed; sv_last_error() has its text */
} sv_status;

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

typedef enum {
  SV_OP_GREEDY = 0,
  SV_OP_SAMPLE = 1,
  SV_OP_TREE = 2,
  SV_OP_TREE_EXPAND = 3,
  SV_OP_SHARD = 4
} sv_op;

/* dev_status bits */
#define SV_FLAG_BAD_REQUEST 1   /* draft count outside [0,k_max], row index out of range,
                                   context length outside [0,stride] */
#define SV_FLAG_BAD_TOKEN 2     /* a draft / node token outside [0,vocab) */
#define SV_FLAG_NONFINITE 4     /* sampled / tree: a target row the verify reads (chain:
                                   rows 0..m; tree: the visited nodes) whose normaliser
                                   sum exp(l/T - M) is not finite and positive; the draft
                                   row a residual is taken from sums to NaN; a non-finite
                                   residual mass.  greedy: a NaN in a target row */
#define SV_FLAG_OVER_BUDGET 8   /* more drafts than max_new[b] (output still produced,
                                   truncated to max_new[b]) */
#define SV_FLAG_FALLBACK 16     /* a residual max(0, p - q) had zero mass: the token was
                                   drawn from p (chain) / p was left unchanged (tree) */
#define SV_FLAG_BAD_TREE 32     /* parent[b,0] != -1, or parent[b,c] not in [0,c) */
#define SV_FLAG_SYNC_TIMEOUT 64 /* tree verifies: the workgroups sharing a request did not
                                   all report within the bounded wait (2^20 polls, about a
                                   second); that request's outputs are undefined.  The
                                   walk's grid is sized to be resident at once on an idle
                                   device; kernels of other streams that hold compute
                                   units delay the rest of the grid only until they end,
                                   so the bit needs a kernel that runs (or spins) for the
                                   whole wait beside the walk.  The chain verifies never
                                   wait for a workgroup to be scheduled and report this
                                   bit only if a word another workgroup stored never
                                   becomes visible */

int sv_abi_version(void);
const char* sv_status_string(int status);
/* Text of the last non-OK return on the calling thread ("" if none). */
const char* sv_last_error(void);

/* Workspace bytes for op (SV_OP_GREEDY / SV_OP_SAMPLE / SV_OP_TREE /
 * SV_OP_TREE_EXPAND / SV_OP_SHARD), for a call with `batch` requests,
 * `total_rows` rows (greedy/sample/shard: t_rows; tree: batch * n_nodes;
 * tree expand: batch * n_exp draft rows) and `vocab` columns (shard: the
 * shard's column count).  Host function.  0 on bad input. */
size_t sv_workspace_bytes(int op, int64_t batch, int64_t total_rows, int64_t vocab);

/* Workspace bytes of one sv_verify_sample / sv_verify_sample_philox call with
 * these sizes (batch requests, t_rows target rows, vocab columns, k_max drafts
 * per request at most): what the call itself checks for, never more than
 * sv_workspace_bytes(SV_OP_SAMPLE, batch, t_rows, vocab), which covers any
 * k_max.  Host function.  0 on bad input (k_max outside [0, 255]) or batch 0. */
size_t sv_sample_workspace_bytes(int64_t batch, int64_t t_rows, int64_t vocab, int32_t k_max);

/* Streaming first pass of sv_verify_sample and sv_verify_tree, exposed on its
 * own: the temperature softmax of every row needs max(l)/T and
 * sum exp(l/T - max) over the whole vocabulary
 * ("投机解码:为什么一个字都不改", figure "一次目标前向验 k 个草稿 token").
 * Each of n_rows rows is split into sv_softmax_segments(n_rows, vocab) segments;
 * out_partials [n_rows, nseg, 2] float receives, per segment, the pair
 * (m = max over the segment of l * log2(e)/T, s = sum 2^(l * log2(e)/T - m)).
 * A row's pairs combine as m = max_j m_j, s = sum_j s_j * 2^(m_j - m); then
 * max(l)/T = m * ln 2 and sum exp(l/T - max(l)/T) = s.  temperature finite > 0. */
int32_t sv_softmax_segments(int64_t n_rows, int64_t vocab);
sv_status sv_softmax_partials(const void* rows, int32_t dtype, int64_t n_rows, int64_t vocab,
                              float temperature, float* out_partials, void* stream);

/* History n-gram drafter.
 * ctx [batch, ctx_stride] int32 tokens; ctx_len [batch]: tokens of request b are
 * ctx[b, 0..ctx_len[b]).  Key = the last `window` tokens.  The most recent
 * earlier occurrence of the key that is followed by at least one token (start j
 * <= n - window - 1) wins; the draft is the up-to-k tokens after it (it stops at
 * the context end).  No occurrence, or n < window + 1: draft_len = 0.
 * Outputs: draft_ids [batch, k] int32 (-1 padded), draft_len [batch].
 * Limits: 1 <= window <= 64, 0 <= k <= 1024, batch >= 0 (0: nothing launched),
 * ctx_stride >= 1.  A ctx_len outside [0, ctx_stride] gives draft_len 0 and
 * SV_FLAG_BAD_REQUEST. */
sv_status sv_ngram_draft(const int32_t* ctx, const int32_t* ctx_len, int32_t batch,
                         int32_t ctx_stride, int32_t window, int32_t k,
                         int32_t* draft_ids, int32_t* draft_len,
                         int32_t* dev_status, void* stream);

/* Greedy (T = 0) verify.
 * target_logits: t_rows rows of `vocab` scores.  Request b (draft count
 * k_b = draft_len[b], drafts draft_ids[b, 0..k_b), row stride k_max) uses rows
 * t_row_start[b] .. t_row_start[b] + k_b.  a_i = argmax of row i (lowest id
 * among equal maxima; +0 and -0 are equal).  m = first i < k_b with
 * draft_ids[b,i] != a_i, else k_b.  Emitted: draft_ids[b,0..m) then a_m,
 * cut after the first eos_id (if eos_id >= 0) and at max_new[b] tokens (if
 * max_new is not NULL).
 * Outputs: out_tokens [batch, k_max+1] int32 (-1 padded), out_count [batch],
 * out_accepted [batch] (= m).  draft_ids may be NULL when k_max == 0. */
sv_status sv_verify_greedy(const void* target_logits, int32_t t_dtype, int32_t t_rows,
                           int64_t vocab, const int32_t* t_row_start,
                           const int32_t* draft_ids, const int32_t* draft_len,
                           int32_t batch, int32_t k_max, const int32_t* max_new,
                           int32_t eos_id, int32_t* out_tokens, int32_t* out_count,
                           int32_t* out_accepted, int32_t* dev_status,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Speculative-sampling chain verify.
 * target_logits [t_rows, vocab]; draft_probs [q_rows, vocab] holds the draft's
 * probabilities (used as given, not renormalised).  Request b uses target rows
 * t_row_start[b] + i (i = 0..k_b) and draft rows q_row_start[b] + i (i < k_b);
 * requests may share rows.  p_i = softmax(target row i / temperature).
 * uniforms [batch, k_max+1] float in [0,1): u[b,i] (i < k_b) tests draft i,
 * which is kept iff u * q_i(x_i) < p_i(x_i); m = first draft not kept (else k_b).
 * u[b,k_b] draws the last token: from max(0, p_m - q_m) if m < k_b (from p_m,
 * with SV_FLAG_FALLBACK, if that has zero mass), else from p_{k_b}: the
 * smallest id whose running mass exceeds u times the total.  Emission,
 * eos_id, max_new and outputs as for sv_verify_greedy.
 * Optional outputs (NULL to skip): out_diag [batch, k_max+1, 4] float =
 * (M_i = max(l/T), S_i = sum exp(l/T - M_i), p_i(x_i), q_i(x_i)) for i <= k_b
 * (p, q = 0 at i = k_b; rows beyond k_b untouched); out_resid [batch] = total
 * mass of the weights the last token was drawn from.
 * The round reads target rows 0..k_b (0..m when the lazy statistics apply:
 * requests own their rows, many statistics blocks per row, no out_diag), draft
 * row m and the entries at the drafted tokens.  No workgroup of the call waits
 * for another to be scheduled, so the call needs the device to itself in no
 * way: it gives the same outputs beside any other work.  temperature must be
 * finite and > 0; 1 <= vocab <= 4194304. */
sv_status sv_verify_sample(const void* target_logits, int32_t t_dtype, int32_t t_rows,
                           const void* draft_probs, int32_t q_dtype, int32_t q_rows,
                           int64_t vocab, const int32_t* t_row_start,
                           const int32_t* q_row_start, const int32_t* draft_ids,
                           const int32_t* draft_len, int32_t batch, int32_t k_max,
                           float temperature, const float* uniforms,
                           const int32_t* max_new, int32_t eos_id,
                           int32_t* out_tokens, int32_t* out_count, int32_t* out_accepted,
                           float* out_diag, float* out_resid, int32_t* dev_status,
                           void* workspace, size_t workspace_bytes, void* stream);

/* sv_verify_sample for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops that must not call hipMalloc, and
 * harnesses that forbid it.  Arguments, outputs and results as for
 * sv_verify_sample, without the workspace: the call uses a static device
 * array of 8 MiB that each GPU the library runs on holds until the process
 * ends (its address is looked up on the first call on each device).  It
 * calls no allocating routine.  A call whose workspace need
 * (sv_sample_workspace_bytes) exceeds 8 MiB returns SV_E_WORKSPACE and
 * launches nothing.  Every call on one device shares that device's array:
 * calls that may overlap on one device (other streams, other threads) race,
 * and the caller must serialise them; what an earlier call left in the array
 * never affects a later one. */
sv_status sv_verify_sample_noalloc(const void* target_logits, int32_t t_dtype, int32_t t_rows,
                                   const void* draft_probs, int32_t q_dtype, int32_t q_rows,
                                   int64_t vocab, const int32_t* t_row_start,
                                   const int32_t* q_row_start, const int32_t* draft_ids,
                                   const int32_t* draft_len, int32_t batch, int32_t k_max,
                                   float temperature, const float* uniforms,
                                   const int32_t* max_new, int32_t eos_id, int32_t* out_tokens,
                                   int32_t* out_count, int32_t* out_accepted, float* out_diag,
                                   float* out_resid, int32_t* dev_status, void* stream);

/* Counter-based uniforms (Philox4x64-10; Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3", SC 2011), so that a serving
 * loop need not generate and upload the verify's uniforms.  Slot i of request
 * b is word i mod 4 of the Philox block at counter (i div 4, b, offset, 0)
 * under key (seed, 0), its top 24 bits times 2^-24: a value on the 2^-24 grid
 * in [0, 1), exact in float.  Use a new offset (or seed) for every round.
 * sv_philox_uniforms writes out [batch, slots] float (batch, slots >= 0). */
sv_status sv_philox_uniforms(uint64_t seed, uint64_t offset, int32_t batch, int32_t slots,
                             float* out, void* stream);

/* sv_verify_sample with its uniforms drawn on the device: u[b, i] is slot i
 * of request b of the Philox stream (seed, offset) above, with
 * slots = k_max + 1 (the same values sv_philox_uniforms writes); everything
 * else as for sv_verify_sample. */
sv_status sv_verify_sample_philox(const void* target_logits, int32_t t_dtype, int32_t t_rows,
                                  const void* draft_probs, int32_t q_dtype, int32_t q_rows,
                                  int64_t vocab, const int32_t* t_row_start,
                                  const int32_t* q_row_start, const int32_t* draft_ids,
                                  const int32_t* draft_len, int32_t batch, int32_t k_max,
                                  float temperature, uint64_t seed, uint64_t offset,
                                  const int32_t* max_new, int32_t eos_id,
                                  int32_t* out_tokens, int32_t* out_count,
                                  int32_t* out_accepted, float* out_diag, float* out_resid,
                                  int32_t* dev_status, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Tree verify.
 * Node c of request b (flattened order, node 0 = root) owns target row
 * b*n_nodes + c and draft row b*n_nodes + c; the draft row of a node is the q
 * its children were proposed from.  parent [batch, n_nodes] int32 (root -1,
 * else an earlier node); node_token [batch, n_nodes] (root entry ignored).
 * uniforms [batch, n_nodes]: u[b,c-1] tests node c, u[b,n_nodes-1] draws the
 * last token.  Walk: cur = root, p = softmax(target row of cur / T),
 * q = draft row of cur; children of cur in index order: keep c iff
 * u * q(x_c) < p(x_c); kept -> emit x_c, descend, reload p and q; not kept ->
 * p <- norm(max(0, p - q)) before the next sibling.  When no child is kept the
 * last token is drawn from the current p.
 * Outputs: out_tokens [batch, n_nodes] (-1 padded), out_count, out_accepted
 * (kept nodes), out_path [batch, n_nodes] (kept node ids, -1 padded).
 * Optional out_diag [batch, n_nodes, 4] = (M_c, S_c, p_parent(x_c),
 * q_parent(x_c)) with the parent's softmax before any residual update
 * (p, q = 0 at the root).  1 <= n_nodes <= 1024, 1 <= vocab <= 4194304.
 * Only the rows the walk reads are touched: the target rows of the visited
 * nodes and the draft rows of nodes whose children were rejected (out_diag,
 * when asked for, reads every row). */
sv_status sv_verify_tree(const void* target_logits, int32_t t_dtype,
                         const void* draft_probs, int32_t q_dtype, int64_t vocab,
                         const int32_t* parent, const int32_t* node_token,
                         int32_t batch, int32_t n_nodes, float temperature,
                         const float* uniforms, int32_t* out_tokens, int32_t* out_count,
                         int32_t* out_accepted, int32_t* out_path, float* out_diag,
                         int32_t* dev_status, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Greedy (T = 0) tree verify.
 * "Speculative Decoding II", EAGLE section: the flattened tree is verified in
 * one target forward and the kept path is the one the target itself would
 * produce; at T = 0 the target's pick at a node is the argmax of the node's
 * row ("第 13 篇：推理引擎一次猜几个字——草稿 + 验证", section ③).
 * Walk: cur = root; a = argmax of cur's target row (lowest id among equal
 * maxima, +0 and -0 equal); the first child of cur (index order) whose token
 * is a is kept (emit a, descend); when none is, emit a and stop (at a leaf:
 * the extra token from the leaf's row).  Layout, parent / node_token checks,
 * outputs and workspace (SV_OP_TREE) as for sv_verify_tree; no draft rows,
 * no temperature, no uniforms.  Only the target rows of visited nodes are
 * read; a NaN in one of them makes the request invalid (SV_FLAG_NONFINITE).
 * 1 <= n_nodes <= 1024, 1 <= vocab <= 4194304. */
sv_status sv_verify_tree_greedy(const void* target_logits, int32_t t_dtype, int64_t vocab,
                                const int32_t* parent, const int32_t* node_token,
                                int32_t batch, int32_t n_nodes, int32_t* out_tokens,
                                int32_t* out_count, int32_t* out_accepted, int32_t* out_path,
                                int32_t* dev_status, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Tree verify with every candidate taken as a point mass on its own token.
 * The recursive speculative sampling of "Speculative Decoding II" (EAGLE
 * section, as in SpecInfer) applied with q = delta_x for each candidate x, as
 * suits candidates chosen deterministically (EAGLE-2's top-k tree): keep x
 * with probability p(x); after a rejection p <- norm(max(0, p - delta_x)), x's
 * mass removed and the rest renormalised ("投机解码:为什么一个字都不改",
 * section "改进", with q = delta_x).  Every step is then that section's
 * identity, so the emitted tokens follow the target for any candidate set.
 * Walk: cur = root, p = softmax(target row of cur / T); children of cur in
 * index order, u = uniforms[b, c-1]: keep c iff u < p(x_c) (p the current,
 * renormalised distribution; a candidate already removed at this node has
 * p = 0); kept -> emit x_c, descend, reload p; not kept -> remove x_c (if the
 * rest has no mass, p is left as it was and SV_FLAG_FALLBACK is set).  When no
 * child is kept the last token is drawn from the current p with
 * uniforms[b, n_nodes-1] (smallest id whose running mass exceeds u times the
 * total).  Layout, checks, outputs and workspace (SV_OP_TREE) as for
 * sv_verify_tree; no draft rows.  Reads the target rows of the visited
 * nodes only; a visited row whose normaliser is not finite and positive makes
 * the request invalid (SV_FLAG_NONFINITE).  temperature finite and > 0;
 * 1 <= n_nodes <= 1024, 1 <= vocab <= 4194304. */
sv_status sv_verify_tree_pointmass(const void* target_logits, int32_t t_dtype, int64_t vocab,
                                   const int32_t* parent, const int32_t* node_token,
                                   int32_t batch, int32_t n_nodes, float temperature,
                                   const float* uniforms, int32_t* out_tokens,
                                   int32_t* out_count, int32_t* out_accepted, int32_t* out_path,
                                   int32_t* dev_status, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* EAGLE-2 dynamic draft tree, built on the device ("Speculative Decoding II",
 * EAGLE-2 section "Context-Aware Dynamic Draft Tree" and its worked example).
 * A request's candidates live in caller-owned arrays [batch, max_cand]
 * (index = creation order; 0 = the root): cand_token, cand_parent (candidate
 * index, -1 at the root), cand_depth (root 0), cand_conf (float: the draft's
 * probability of the token at its parent), cand_value (double: the product
 * of the confidences on the path, 1 at the root); cand_count [batch].
 *
 * sv_tree_expand: one round.  draft_rows [batch * n_exp, vocab] (q_dtype):
 * row b * n_exp + e is the draft's distribution at candidate
 * exp_node[b, e] (-1: none, that row is ignored).  exp_node == NULL is the
 * first round: n_exp must be 1, the root of each request is created (count
 * 1) and expanded with its row.  Each expanded node gets top_children
 * children: the ids of its row with the largest probabilities (lower id
 * first among equals; a value is clamped into [0, 1], NaN counts as 0),
 * appended in the order given, best first, with value = parent value x
 * confidence (fp64).  next_exp [batch, expand_next] receives the best
 * candidates appended in this round by (-value, depth, creation order),
 * best first, -1 padded: the nodes whose rows the next round expands.  A
 * round that would exceed max_cand, or names a candidate that does not
 * exist, appends nothing and sets SV_FLAG_BAD_REQUEST.
 * Limits: 1 <= n_exp, expand_next <= 64; 1 <= top_children <= min(16, vocab);
 * 1 <= max_cand <= 1024.  Workspace: SV_OP_TREE_EXPAND with
 * total_rows = batch * n_exp.
 *
 * sv_tree_finalize: keep the root and the best n_nodes - 1 candidates by
 * (-value, depth, creation order) (a value never exceeds its parent's and
 * ties go to the shallower node, so the kept set is connected) and flatten
 * them breadth-first, each depth ordered by (parent's flat index,
 * -confidence, token, creation order).  Outputs [batch, n_nodes]: out_parent
 * (flat index, -1 at the root), out_token (-1 at the root), out_depth (the
 * position offset), out_cand (candidate index); with fewer candidates than
 * n_nodes the tail is -1.  out_mask [batch, n_nodes, n_nodes] uint8 (NULL to
 * skip): row i has 1 at i and at each ancestor of i, else 0.  The flat
 * arrays feed sv_verify_tree (parent, token).  1 <= n_nodes <= 1024. */
sv_status sv_tree_expand(const void* draft_rows, int32_t q_dtype, int64_t vocab, int32_t batch,
                         int32_t n_exp, const int32_t* exp_node, int32_t top_children,
                         int32_t expand_next, int32_t max_cand, int32_t* cand_token,
                         int32_t* cand_parent, int32_t* cand_depth, float* cand_conf,
                         double* cand_value, int32_t* cand_count, int32_t* next_exp,
                         int32_t* dev_status, void* workspace, size_t workspace_bytes,
                         void* stream);
sv_status sv_tree_finalize(int32_t batch, int32_t max_cand, const int32_t* cand_token,
                           const int32_t* cand_parent, const int32_t* cand_depth,
                           const float* cand_conf, const double* cand_value,
                           const int32_t* cand_count, int32_t n_nodes, int32_t* out_parent,
                           int32_t* out_token, int32_t* out_depth, int32_t* out_cand,
                           uint8_t* out_mask, int32_t* dev_status, void* stream);

/* Sampled chain verify over a vocabulary split into column shards, as a
 * vocabulary-parallel LM head leaves the logits: device g holds columns
 * [bounds[g], bounds[g+1]) of every target and draft row ("投机解码:为什么一个字
 * 都不改", sections "改进" and "一轮能出几个 token"; the softmax of the figure
 * "一次目标前向验 k 个草稿 token" spans the whole vocabulary, so its max and
 * normaliser are combined from the shards' pairs).  The result is the
 * sv_verify_sample round; only the data movement differs.
 *
 * Common arguments: target_cols [t_rows, width] and draft_cols [q_rows, width]
 * are this shard's columns (width = bounds[shard+1] - bounds[shard]); bounds
 * is a HOST array of n_shards + 1 column offsets, 0 = bounds[0] < ... <
 * bounds[n_shards] = vocab, 1 <= n_shards <= 64; row starts, drafts, batch,
 * k_max, temperature as for sv_verify_sample.  Workspace: SV_OP_SHARD with
 * total_rows = t_rows and vocab = width; the same workspace must serve one
 * shard's three steps of a round.
 *
 * Step 1, sv_shard_stats: out_pairs [t_rows, 2] float = the shard's
 * scaled-domain softmax pair of every target row (m = max over its columns
 * of l log2(e)/T, s = sum 2^(l log2(e)/T - m)); out_at [batch, k_max, 2] =
 * (target logit, draft probability) at each drafted token the shard holds
 * (other entries are not written).
 * Exchange: all_pairs [n_shards, t_rows, 2] and all_at [n_shards, batch,
 * k_max, 2] hold every shard's step-1 outputs (an all-gather).
 * Step 2, sv_shard_residual: every shard takes the same decisions (rows'
 * pairs combined in shard order, p(x_i) from the shard holding x_i, the
 * accept scan with uniforms [batch, k_max+1]) and writes its row of
 * mass [n_shards, batch, 3] = (sum of max(0, p_m - q_m) over its columns, or
 * of p_k after a full accept; sum of p; sum of q) in float64.
 * Exchange: every shard's row of mass (an all-gather).
 * Step 3, sv_shard_draw: the shard whose columns hold u[b, k_b] times the
 * total (shard order) draws the token and writes request b's outputs
 * (tokens [batch, k_max+1], count, accepted, optional resid, status bits);
 * shard 0 writes the outputs of invalid requests; other shards write nothing
 * for b.  Status bits and invalid requests as for sv_verify_sample. */
sv_status sv_shard_stats(const void* target_cols, int32_t t_dtype, int32_t t_rows,
                         const void* draft_cols, int32_t q_dtype, int32_t q_rows, int64_t vocab,
                         const int64_t* bounds, int32_t n_shards, int32_t shard,
                         const int32_t* t_row_start, const int32_t* q_row_start,
                         const int32_t* draft_ids, const int32_t* draft_len, int32_t batch,
                         int32_t k_max, float temperature, float* out_pairs, float* out_at,
                         void* workspace, size_t workspace_bytes, void* stream);
sv_status sv_shard_residual(const void* target_cols, int32_t t_dtype, int32_t t_rows,
                            const void* draft_cols, int32_t q_dtype, int32_t q_rows,
                            int64_t vocab, const int64_t* bounds, int32_t n_shards,
                            int32_t shard, const int32_t* t_row_start,
                            const int32_t* q_row_start, const int32_t* draft_ids,
                            const int32_t* draft_len, int32_t batch, int32_t k_max,
                            float temperature, const float* uniforms, const float* all_pairs,
                            const float* all_at, double* mass, void* workspace,
                            size_t workspace_bytes, void* stream);
sv_status sv_shard_draw(const void* target_cols, int32_t t_dtype, int32_t t_rows,
                        const void* draft_cols, int32_t q_dtype, int32_t q_rows, int64_t vocab,
                        const int64_t* bounds, int32_t n_shards, int32_t shard,
                        const int32_t* t_row_start, const int32_t* q_row_start,
                        const int32_t* draft_ids, const int32_t* draft_len, int32_t batch,
                        int32_t k_max, float temperature, const float* uniforms,
                        const float* all_pairs, const double* mass, const int32_t* max_new,
                        int32_t eos_id, int32_t* out_tokens, int32_t* out_count,
                        int32_t* out_accepted, float* out_resid, int32_t* dev_status,
                        void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
