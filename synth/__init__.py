"""Seeded synthetic inputs for the speculative-decoding verify step.

This module only *produces inputs*: target logit rows, draft probability rows
(the simulated draft model's output), draft tokens drawn from those rows,
uniform random numbers, token contexts for the prompt-lookup drafter, and draft
trees.  It contains no part of the verify method itself: no target-side
softmax, no acceptance test, no residual, no inverse-CDF resample of the target.
Both the HIP library and the CPU oracle consume exactly the arrays returned
here, so the two sides see identical bits.

Every generator is deterministic in its seed.  Seeds come from
``np.random.SeedSequence([2026, cfg])`` spawned into named children in the fixed
order ``STREAMS``; a generator asks for the stream by name.

Stored value formats
--------------------
* ``f32`` rows are ``np.float32`` arrays.
* ``bf16`` rows are ``np.uint16`` arrays holding bfloat16 bit patterns, obtained
  by rounding the float64 value to float32 (round-to-nearest-even) and then to
  bfloat16 (round-to-nearest-even on the upper 16 bits).
* Uniforms are float32 multiples of 2**-24 in [0, 1): exactly representable in
  float32 and in float64, so both sides compare the same number.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np

SEED_ROOT = 2026
STREAMS = ("target", "boost", "draft_noise", "draft_draw", "uniforms",
           "per_request", "contexts", "tree")


def streams(cfg: int, salt: int = 0) -> dict:
    """Named, independent generators for config ``cfg`` (``salt`` gives replicates)."""
    ss = np.random.SeedSequence([SEED_ROOT, cfg, salt])
    kids = ss.spawn(len(STREAMS))
    return {name: np.random.default_rng(k) for name, k in zip(STREAMS, kids)}


# ----------------------------------------------------------------------------
# value encodings
# ----------------------------------------------------------------------------
def to_bf16_bits(x) -> np.ndarray:
    """float64/float32 -> bfloat16 bit patterns (uint16), RNE via float32."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    b = f.view(np.uint32).astype(np.uint64)
    out = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = ((f.view(np.uint32)[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(h) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (used by the generator
    itself to read back what it stored, e.g. to draw tokens from stored rows)."""
    h = np.ascontiguousarray(np.asarray(h, dtype=np.uint16))
    return (h.astype(np.uint32) << 16).view(np.float32)


def encode(x, kind: str) -> np.ndarray:
    if kind == "f32":
        return np.asarray(x, dtype=np.float32)
    if kind == "bf16":
        return to_bf16_bits(x)
    raise ValueError(kind)


def decode(a, kind: str) -> np.ndarray:
    """Stored row -> float64 (exact for both formats)."""
    if kind == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    return bf16_bits_to_f32(a).astype(np.float64)


def uniform_grid(rng: np.random.Generator, shape) -> np.ndarray:
    """U[0,1) on the 2**-24 grid, as float32 (exact)."""
    return (rng.integers(0, 1 << 24, size=shape, dtype=np.int64)
            .astype(np.float64) / float(1 << 24)).astype(np.float32)


# ----------------------------------------------------------------------------
# simulated models
# ----------------------------------------------------------------------------
def target_logits(rng_t, rng_b, V: int, sd: float, n_boost: int = 0,
                  boost: float = 0.0) -> np.ndarray:
    """One target logit row (float64): N(0, sd^2) plus ``boost`` on ``n_boost``
    distinct random ids (the row's 'likely' tokens)."""
    l = rng_t.standard_normal(V) * sd
    if n_boost:
        ids = rng_b.choice(V, size=n_boost, replace=False)
        l[ids] += boost
    return l


def draft_distribution(logits: np.ndarray, T: float) -> np.ndarray:
    """The simulated draft model's output distribution for one position:
    softmax(draft_logits / T) in float64.  (This is the draft side's own
    sampling distribution q, an *input* to verification.)"""
    z = logits / T
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def draw_from_stored(rng: np.random.Generator, stored_row: np.ndarray, kind: str,
                     size=None):
    """Draw draft tokens from a stored draft row (renormalised in float64):
    this is what the draft model does when it proposes a token."""
    q = decode(stored_row, kind)
    q = np.where(q > 0, q, 0.0)
    return rng.choice(q.shape[0], size=size, p=q / q.sum())


# ----------------------------------------------------------------------------
# chain inputs
# ----------------------------------------------------------------------------
@dataclass
class ChainInputs:
    """Inputs of one chain verify call (greedy or sampled).

    target[t_rows, V] and draft[q_rows, V] are stored rows; request b's target
    rows are t_row_start[b] .. t_row_start[b]+draft_len[b] and its draft rows are
    q_row_start[b] .. q_row_start[b]+draft_len[b]-1.  draft_ids[b, i] (i <
    draft_len[b]) is the i-th drafted token, -1 beyond.  uniforms[b, i] for i <
    draft_len[b] drives the test of draft i; uniforms[b, draft_len[b]] drives the
    final draw.
    """
    name: str
    V: int
    t_kind: str
    target: np.ndarray
    q_kind: str
    draft: Optional[np.ndarray]
    t_row_start: np.ndarray
    q_row_start: np.ndarray
    draft_ids: np.ndarray
    draft_len: np.ndarray
    k_max: int
    T: float
    uniforms: np.ndarray
    max_new: Optional[np.ndarray] = None
    eos_id: int = -1
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.draft_len.shape[0])


def _row_starts(ks: np.ndarray):
    ks = np.asarray(ks, dtype=np.int64)
    t_rs = np.concatenate([[0], np.cumsum(ks + 1)[:-1]]).astype(np.int32)
    q_rs = np.concatenate([[0], np.cumsum(ks)[:-1]]).astype(np.int32)
    return t_rs, q_rs


def sampled_chain(cfg: int, B: int, ks, V: int, T: float, *, sd: float,
                  n_boost: int, boost: float, sigma, kind: str = "bf16",
                  salt: int = 0, name: str = "") -> ChainInputs:
    """Packed (possibly ragged) sampled-chain inputs.

    Request b has ks[b] drafts.  Its target rows are fresh N(0, sd^2) rows with
    a ``boost`` on ``n_boost`` ids; its draft row for position i is the draft
    model's distribution softmax((l_i + N(0, sigma_b^2)) / T), stored in
    ``kind``; draft token i is drawn from that stored row.
    """
    st = streams(cfg, salt)
    ks = np.asarray(ks, dtype=np.int64)
    sig = np.broadcast_to(np.asarray(sigma, dtype=np.float64), (B,))
    k_max = int(ks.max()) if B else 0
    t_rows, q_rows = int((ks + 1).sum()), int(ks.sum())
    store_dt = np.float32 if kind == "f32" else np.uint16
    target = np.empty((t_rows, V), dtype=store_dt)
    draft = np.empty((max(q_rows, 1), V), dtype=store_dt)
    t_rs, q_rs = _row_starts(ks)
    ids = np.full((B, max(k_max, 1)), -1, dtype=np.int32)
    for b in range(B):
        for i in range(int(ks[b]) + 1):
            l = target_logits(st["target"], st["boost"], V, sd, n_boost, boost)
            target[t_rs[b] + i] = encode(l, kind)
            if i < ks[b]:
                dl = l + st["draft_noise"].standard_normal(V) * sig[b]
                qrow = encode(draft_distribution(dl, T), kind)
                draft[q_rs[b] + i] = qrow
                ids[b, i] = draw_from_stored(st["draft_draw"], qrow, kind)
    u = uniform_grid(st["uniforms"], (B, k_max + 1))
    return ChainInputs(name or f"cfg{cfg}", V, kind, target, kind, draft,
                       t_rs, q_rs, ids, ks.astype(np.int32), k_max, T, u,
                       meta=dict(cfg=cfg, salt=salt, sd=sd, n_boost=n_boost,
                                 boost=boost))


def c1_chain(rounds: int = 200_000, V: int = 2048, k: int = 4, T: float = 1.0,
             salt: int = 0) -> ChainInputs:
    """Chain verify, one fixed prefix, fp32: 5 target rows l ~ N(0, 2^2) and 4
    draft rows softmax(l + N(0, 1)) shared by ``rounds`` independent rounds
    (every request's row starts are 0); each round draws its own draft tokens
    from the draft rows and its own uniforms."""
    st = streams(1, salt)
    target = np.empty((k + 1, V), dtype=np.float32)
    draft = np.empty((k, V), dtype=np.float32)
    ids = np.empty((rounds, k), dtype=np.int32)
    for i in range(k + 1):
        l = target_logits(st["target"], st["boost"], V, 2.0)
        target[i] = encode(l, "f32")
        if i < k:
            q = draft_distribution(l + st["draft_noise"].standard_normal(V), T)
            draft[i] = encode(q, "f32")
            ids[:, i] = draw_from_stored(st["draft_draw"], draft[i], "f32", size=rounds)
    u = uniform_grid(st["uniforms"], (rounds, k + 1))
    zeros = np.zeros(rounds, dtype=np.int32)
    return ChainInputs("c1_chain", V, "f32", target, "f32", draft, zeros, zeros.copy(),
                       ids, np.full(rounds, k, dtype=np.int32), k, T, u,
                       meta=dict(cfg=1, salt=salt))


def c3_sampled(B: int = 64, k: int = 4, V: int = 248_320, T: float = 0.7,
               salt: int = 0) -> ChainInputs:
    """Sampled chain: bf16 target N(0, 2.5^2) + 6 on 5 ids/row; draft noise
    N(0, 1.5^2); T = 0.7."""
    return sampled_chain(3, B, np.full(B, k), V, T, sd=2.5, n_boost=5, boost=6.0,
                         sigma=1.5, salt=salt, name="c3_sampled")


def c4_ragged(B: int = 256, V: int = 151_936, T: float = 1.0, k_hi: int = 8,
              salt: int = 0) -> ChainInputs:
    """Ragged sampled chain: k_b ~ U{1..k_hi}, draft noise sigma_b ~ U[0.5, 3]."""
    st = streams(4, salt)
    ks = st["per_request"].integers(1, k_hi + 1, size=B)
    sig = st["per_request"].uniform(0.5, 3.0, size=B)
    return sampled_chain(4, B, ks, V, T, sd=2.5, n_boost=5, boost=6.0, sigma=sig,
                         salt=salt, name="c4_ragged")


# ----------------------------------------------------------------------------
# greedy + prompt-lookup inputs
# ----------------------------------------------------------------------------
def zipf_probs(V: int, s: float) -> np.ndarray:
    r = np.arange(1, V + 1, dtype=np.float64)
    w = r ** (-s)
    return w / w.sum()


def token_stream(rng: np.random.Generator, length: int, pz: np.ndarray,
                 p_repeat: float = 0.3, span=(8, 32)) -> np.ndarray:
    """Zipf tokens emitted in spans of U{span} tokens; a span is, with
    probability p_repeat once enough history exists, a copy of an earlier window
    of the stream (a planted repeat)."""
    seq: list = []
    V = pz.shape[0]
    while len(seq) < length:
        L = int(rng.integers(span[0], span[1] + 1))
        if len(seq) >= L and rng.random() < p_repeat:
            s = int(rng.integers(0, len(seq) - L + 1))
            seq.extend(seq[s:s + L])
        else:
            seq.extend(rng.choice(V, size=L, p=pz).tolist())
    return np.asarray(seq[:length], dtype=np.int32)


@dataclass
class GreedyInputs:
    """Contexts for the prompt-lookup drafter plus the target rows for the greedy
    verify that follows it.  Request b owns target rows b*(k+1) .. b*(k+1)+k."""
    V: int
    ctx: np.ndarray          # int32 [B, ctx_stride]
    ctx_len: np.ndarray      # int32 [B]
    truth: np.ndarray        # int32 [B, k+1] the true continuation
    target: np.ndarray       # bf16 bits [B*(k+1), V]
    t_kind: str
    k: int
    window: int
    forced: np.ndarray       # bool [B, k+1]

    @property
    def B(self) -> int:
        return int(self.ctx_len.shape[0])


def c2_greedy(B: int = 64, n: int = 4096, V: int = 32_000, k: int = 4, window: int = 3,
              s: float = 1.1, p_force: float = 0.7, sd: float = 3.0, salt: int = 0,
              ctx_lens=None) -> GreedyInputs:
    st = streams(2, salt)
    pz = zipf_probs(V, s)
    lens = np.full(B, n, dtype=np.int32) if ctx_lens is None else np.asarray(ctx_lens, np.int32)
    stride = int(max(int(lens.max()), 1))
    ctx = np.zeros((B, stride), dtype=np.int32)
    truth = np.empty((B, k + 1), dtype=np.int32)
    for b in range(B):
        seq = token_stream(st["contexts"], int(lens[b]) + k + 1, pz)
        ctx[b, :lens[b]] = seq[:lens[b]]
        truth[b] = seq[lens[b]:lens[b] + k + 1]
    rows = np.empty((B * (k + 1), V), dtype=np.uint16)
    forced = st["per_request"].random((B, k + 1)) < p_force
    for b in range(B):
        for i in range(k + 1):
            l = st["target"].standard_normal(V) * sd
            if forced[b, i]:
                l[truth[b, i]] = l.max() + 1.0
            rows[b * (k + 1) + i] = to_bf16_bits(l)
    return GreedyInputs(V, ctx, lens, truth, rows, "bf16", k, window, forced)


# ----------------------------------------------------------------------------
# draft trees (EAGLE-2 style construction, used to *produce* tree inputs)
# ----------------------------------------------------------------------------
@dataclass
class TreeNode:
    cid: int            # creation order
    parent: int         # parent's creation id (-1 at the root)
    depth: int
    token: int
    c: float            # draft confidence of this token under the parent
    value: float        # product of confidences on the path from the root


def build_draft_tree(propose: Callable[[TreeNode], list], top_children: int,
                     expand_per_layer: int, max_depth: int, keep: int):
    """Dynamic draft tree: expansion of the best nodes of the newest layer by
    path value, then a global rerank keeping the best ``keep`` nodes (root
    included), then breadth-first flattening.

    ``propose(node)`` returns the node's candidate children as (token,
    confidence) pairs, best first.  Returns (flat nodes, parent index array in
    flat order, depth array).  Ordering rules: layer selection and the rerank
    sort by (-value, depth, creation id); flattening sorts by (depth, parent's
    flat index, -confidence, token, creation id).
    """
    root = TreeNode(0, -1, 0, -1, 1.0, 1.0)
    nodes = [root]
    layer = [root]
    for depth in range(1, max_depth + 1):
        frontier = layer if depth == 1 else sorted(
            layer, key=lambda n: (-n.value, n.depth, n.cid))[:expand_per_layer]
        new_layer = []
        for par in frontier:
            for tok, c in propose(par)[:top_children]:
                node = TreeNode(len(nodes), par.cid, depth, int(tok), float(c),
                                par.value * float(c))
                nodes.append(node)
                new_layer.append(node)
        if not new_layer:
            break
        layer = new_layer
    rest = sorted(nodes[1:], key=lambda n: (-n.value, n.depth, n.cid))[:keep - 1]
    kept = [root] + rest
    kept_ids = {n.cid for n in kept}
    flat_index = {0: 0}
    flat = [root]
    for depth in range(1, max_depth + 1):
        lvl = [n for n in kept if n.depth == depth]
        assert all(n.parent in kept_ids for n in lvl), "rerank broke connectivity"
        lvl.sort(key=lambda n: (flat_index[n.parent], -n.c, n.token, n.cid))
        for n in lvl:
            flat_index[n.cid] = len(flat)
            flat.append(n)
    parent = np.array([-1] + [flat_index[n.parent] for n in flat[1:]], dtype=np.int32)
    depth = np.array([n.depth for n in flat], dtype=np.int32)
    return flat, parent, depth


@dataclass
class TreeInputs:
    """Inputs of one tree verify call.  Node c of request b (flattened order,
    node 0 = root) owns target row b*N+c and draft row b*N+c; the draft row of a
    node is the draft distribution its children were proposed from.
    uniforms[b, c-1] drives the test of node c and uniforms[b, N-1] the final
    draw."""
    name: str
    V: int
    N: int
    t_kind: str
    target: np.ndarray
    q_kind: str
    draft: np.ndarray
    parent: np.ndarray   # int32 [B, N]
    token: np.ndarray    # int32 [B, N] (root entry unused, -1)
    depth: np.ndarray    # int32 [B, N]
    T: float
    uniforms: np.ndarray  # float32 [B, N]
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.parent.shape[0])


def c5_tree(B: int = 32, N: int = 60, V: int = 128_256, T: float = 1.0,
            top_children: int = 4, expand_per_layer: int = 4, max_depth: int = 6,
            sigma: float = 1.5, salt: int = 0, kind: str = "bf16") -> TreeInputs:
    """Tree inputs: every node's target row is a fresh N(0, 2.5^2) row with +6 on
    5 ids; its draft row is softmax((l + N(0, sigma^2)) / T) stored in ``kind``.
    Children are the top tokens of the node's stored draft row (confidence =
    stored probability, ties to the lower id).  Node rows are seeded by
    (request, creation id), so they do not depend on which nodes get kept."""
    store_dt = np.float32 if kind == "f32" else np.uint16
    target = np.empty((B * N, V), dtype=store_dt)
    draft = np.empty((B * N, V), dtype=store_dt)
    parent = np.empty((B, N), dtype=np.int32)
    token = np.empty((B, N), dtype=np.int32)
    depth = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        cache = {}

        def rows(cid, b=b, cache=cache):
            if cid not in cache:
                ss = np.random.SeedSequence([SEED_ROOT, 5, salt, b, cid])
                r_t, r_b, r_n = (np.random.default_rng(s) for s in ss.spawn(3))
                l = target_logits(r_t, r_b, V, 2.5, 5, 6.0)
                q = encode(draft_distribution(l + r_n.standard_normal(V) * sigma, T), kind)
                cache[cid] = (encode(l, kind), q)
            return cache[cid]

        def propose(node, rows=rows):
            q = decode(rows(node.cid)[1], kind)
            order = np.lexsort((np.arange(V), -q))[:top_children]
            return [(int(t), float(q[t])) for t in order]

        flat, par, dep = build_draft_tree(propose, top_children, expand_per_layer,
                                          max_depth, N)
        if len(flat) != N:
            raise ValueError(f"tree has {len(flat)} nodes, wanted {N}")
        for j, node in enumerate(flat):
            t_row, q_row = rows(node.cid)
            target[b * N + j] = t_row
            draft[b * N + j] = q_row
        parent[b] = par
        depth[b] = dep
        token[b] = [n.token for n in flat]
    u = uniform_grid(streams(5, salt)["uniforms"], (B, N))
    return TreeInputs("c5_tree", V, N, kind, target, kind, draft, parent, token, depth,
                      T, u, meta=dict(cfg=5, salt=salt))
