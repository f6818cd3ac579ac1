"""Tree verification (EAGLE / SpecInfer style) in float64.

TEST INFRASTRUCTURE (see the package docstring).
"""
from functools import lru_cache

import numpy as np

from .rows import (widen, FLAG_BAD_TOKEN, FLAG_NONFINITE, FLAG_FALLBACK,
                   FLAG_BAD_TREE)
from .chain import softmax_T, inverse_cdf


def verify_tree(target, t_kind, draft, q_kind, V, parent, token, T, uniforms,
                with_diag=True):
    """Verify a flattened draft tree per request.

    "Speculative Decoding II", EAGLE section: one target forward (with tree
    attention) gives the target distribution at every node, and speculative
    sampling is applied recursively at the tree's nodes, either keeping a
    candidate or adjusting the distribution, the same way SpecInfer does, so
    that the output follows the target model.  The EAGLE-2 worked example on
    the same page flattens the tree breadth-first; siblings are candidates for
    the same position.

    Steps, per request (node 0 is the root; node c's parent is parent[b, c] and
    its token token[b, c]; node c's target row gives p at c, its draft row gives
    the q its children were drawn from):

    1. cur = root, p = softmax(target row of cur / T), q = draft row of cur.
    2. For each child c of cur, in flattened order, with uniform u = u[b, c-1]:
       keep c iff u * q(x_c) < p(x_c) (the chain test of
       "投机解码:为什么一个字都不改", section "改进").  If kept: emit x_c, cur = c,
       reload p and q from c's rows, go to 2.  If not: p <- norm(max(0, p - q))
       and try the next sibling with the same q.  (If that residual has zero
       mass, p is left as it was and the fallback bit is set.)
    3. When no child is kept, or cur has no children, draw the last token from
       the current p with u[b, N-1].

    Returns tokens [B, N] (-1 padded), count [B], accepted [B] (nodes kept),
    path [B, N] (ids of kept nodes, -1 padded), flags [B], margins [B, N]
    (indexed like the uniforms) and, if ``with_diag``, diag [B, N, 4] =
    (M_c, S_c, p_parent(x_c), q_parent(x_c)) with the parent's original p, and
    zeros in the p, q slots at the root.
    """
    parent = np.asarray(parent)
    token = np.asarray(token)
    B, N = parent.shape
    tokens = np.full((B, N), -1, dtype=np.int64)
    count = np.zeros(B, dtype=np.int64)
    accepted = np.zeros(B, dtype=np.int64)
    path = np.full((B, N), -1, dtype=np.int64)
    flags = np.zeros(B, dtype=np.int64)
    margins = np.full((B, N), np.nan, dtype=np.float64)
    diag = np.zeros((B, N, 4), dtype=np.float64) if with_diag else None

    @lru_cache(maxsize=8)
    def dist(row):
        return softmax_T(widen(target[row], t_kind), T)

    @lru_cache(maxsize=8)
    def qrow(row):
        return widen(draft[row], q_kind)

    for b in range(B):
        par = [int(v) for v in parent[b]]
        tok = [int(v) for v in token[b]]
        if par[0] != -1 or any(not (0 <= par[c] < c) for c in range(1, N)):
            flags[b] |= FLAG_BAD_TREE
            continue
        if any(not (0 <= tok[c] < V) for c in range(1, N)):
            flags[b] |= FLAG_BAD_TOKEN
            continue
        if with_diag:
            for c in range(N):
                _, M, S = dist(b * N + c)
                diag[b, c, 0], diag[b, c, 1] = M, S
                if c > 0:
                    pp = dist(b * N + par[c])[0]
                    diag[b, c, 2] = pp[tok[c]]
                    diag[b, c, 3] = qrow(b * N + par[c])[tok[c]]
        children = [[] for _ in range(N)]
        for c in range(1, N):
            children[par[c]].append(c)
        u = np.asarray(uniforms[b], dtype=np.float64)

        cur = 0
        p, _, S = dist(b * N + cur)
        ok = np.isfinite(S) and S > 0
        emitted, kept = [], []
        while ok:
            q = qrow(b * N + cur) if children[cur] else None
            nxt = None
            for c in children[cur]:
                x = tok[c]
                keep = u[c - 1] * q[x] < p[x]
                margins[b, c - 1] = abs(u[c - 1] - p[x] / q[x]) if q[x] > 0 else np.inf
                if keep:
                    nxt = c
                    break
                if np.isnan(np.sum(q)):
                    ok = False
                    break
                r = np.maximum(p - q, 0.0)
                R = np.sum(r)
                if not np.isfinite(R):
                    ok = False
                    break
                if R > 0.0:
                    p = r / R
                else:
                    flags[b] |= FLAG_FALLBACK
            if not ok or nxt is None:
                break
            emitted.append(tok[nxt])
            kept.append(nxt)
            cur = nxt
            p, _, S = dist(b * N + cur)
            ok = np.isfinite(S) and S > 0
        if not ok:
            flags[b] |= FLAG_NONFINITE
            continue
        y, _, marg = inverse_cdf(p, u[N - 1])
        margins[b, N - 1] = marg
        emitted.append(y)
        tokens[b, :len(emitted)] = emitted
        count[b] = len(emitted)
        accepted[b] = len(kept)
        path[b, :len(kept)] = kept
    out = dict(tokens=tokens, count=count, accepted=accepted, path=path,
               flags=flags, margins=margins)
    if with_diag:
        out["diag"] = diag
    return out


def _tree_shape_flags(par, tok, V, N):
    """FLAG_BAD_TREE / FLAG_BAD_TOKEN of one request's tree, else 0."""
    if par[0] != -1 or any(not (0 <= par[c] < c) for c in range(1, N)):
        return FLAG_BAD_TREE
    if any(not (0 <= tok[c] < V) for c in range(1, N)):
        return FLAG_BAD_TOKEN
    return 0


def verify_tree_greedy(target, t_kind, V, parent, token):
    """Greedy (T = 0) tree verify.

    "Speculative Decoding II", EAGLE section: the flattened tree is verified in
    one target forward and the kept path is the one the target model itself
    would have produced; at T = 0 the target's pick at a node is the argmax of
    that node's row ("第 13 篇：推理引擎一次猜几个字——草稿 + 验证", section ③:
    the model's own next token at each drafted position), so verification
    follows the target's picks down the tree.

    Steps, per request (node 0 is the root):

    1. cur = root; a = argmax of cur's target row (the lowest id among equal
       maxima; a row holding a NaN makes the request invalid).
    2. The first child c of cur, in flattened order, whose token is a is kept:
       emit a, cur = c, go to 1.  If no child carries a, emit a and stop (at a
       leaf this is the extra token from the leaf's own row).

    Only the rows of the visited nodes are read.  Returns tokens [B, N] (-1
    padded), count [B], accepted [B], path [B, N] (kept node ids, -1 padded),
    flags [B].
    """
    parent = np.asarray(parent)
    token = np.asarray(token)
    B, N = parent.shape
    tokens = np.full((B, N), -1, dtype=np.int64)
    count = np.zeros(B, dtype=np.int64)
    accepted = np.zeros(B, dtype=np.int64)
    path = np.full((B, N), -1, dtype=np.int64)
    flags = np.zeros(B, dtype=np.int64)
    for b in range(B):
        par = [int(v) for v in parent[b]]
        tok = [int(v) for v in token[b]]
        bad = _tree_shape_flags(par, tok, V, N)
        if bad:
            flags[b] |= bad
            continue
        children = [[] for _ in range(N)]
        for c in range(1, N):
            children[par[c]].append(c)
        cur, emitted, kept = 0, [], []
        while True:
            row = widen(target[b * N + cur], t_kind)
            if np.isnan(row).any():
                flags[b] |= FLAG_NONFINITE
                break
            a = int(np.argmax(row))
            emitted.append(a)
            nxt = next((c for c in children[cur] if tok[c] == a), None)
            if nxt is None:
                break
            kept.append(nxt)
            cur = nxt
        if flags[b] & FLAG_NONFINITE:
            continue
        tokens[b, :len(emitted)] = emitted
        count[b] = len(emitted)
        accepted[b] = len(kept)
        path[b, :len(kept)] = kept
    return dict(tokens=tokens, count=count, accepted=accepted, path=path, flags=flags)


def verify_tree_pointmass(target, t_kind, V, parent, token, T, uniforms):
    """Tree verify with every sibling taken as a point mass.

    The recursive speculative sampling of "Speculative Decoding II" (EAGLE
    section, verification as in SpecInfer) keeps the target's law when each
    candidate is a draw from the q it is tested against.  EAGLE-2's dynamic
    tree (same page, worked example) picks its candidates deterministically
    (top-k by confidence), so each one is tested here as a draw from the point
    mass q = delta_x on its own token: keep x with probability
    min(1, p(x)/1) = p(x); after a rejection p <- norm(max(0, p - delta_x)),
    i.e. x's mass is removed and the rest renormalised (the residual step of
    "投机解码:为什么一个字都不改", section "改进", with q = delta_x).  Each
    step is then the identity min(p, q) + (1 - alpha) norm(max(0, p - q)) = p
    of that section, so the output follows p for any candidate set.

    Steps, per request:

    1. cur = root, p = softmax(target row of cur / T).
    2. For each child c of cur in flattened order, u = u[b, c-1]: keep c iff
       u < p(x_c).  Kept: emit x_c, cur = c, reload p, go to 2.  Not kept:
       r = p with x_c's entry set to 0; if sum r > 0, p <- r / sum r, else p
       is left as it was and the fallback bit is set.
    3. When no child is kept, or cur is a leaf, draw the last token from the
       current p with u[b, N-1] (inverse CDF).

    Returns tokens, count, accepted, path, flags and margins [B, N] (distance
    of each used uniform to its decision edge) like ``verify_tree``.
    """
    parent = np.asarray(parent)
    token = np.asarray(token)
    B, N = parent.shape
    tokens = np.full((B, N), -1, dtype=np.int64)
    count = np.zeros(B, dtype=np.int64)
    accepted = np.zeros(B, dtype=np.int64)
    path = np.full((B, N), -1, dtype=np.int64)
    flags = np.zeros(B, dtype=np.int64)
    margins = np.full((B, N), np.nan, dtype=np.float64)
    for b in range(B):
        par = [int(v) for v in parent[b]]
        tok = [int(v) for v in token[b]]
        bad = _tree_shape_flags(par, tok, V, N)
        if bad:
            flags[b] |= bad
            continue
        children = [[] for _ in range(N)]
        for c in range(1, N):
            children[par[c]].append(c)
        u = np.asarray(uniforms[b], dtype=np.float64)
        cur = 0
        p, _, S = softmax_T(widen(target[b * N + cur], t_kind), T)
        ok = np.isfinite(S) and S > 0
        emitted, kept = [], []
        while ok:
            nxt = None
            for c in children[cur]:
                x = tok[c]
                margins[b, c - 1] = abs(u[c - 1] - p[x])
                if u[c - 1] < p[x]:
                    nxt = c
                    break
                r = p.copy()
                r[x] = 0.0
                R = np.sum(r)
                if R > 0.0:
                    p = r / R
                else:
                    flags[b] |= FLAG_FALLBACK
            if nxt is None:
                break
            emitted.append(tok[nxt])
            kept.append(nxt)
            cur = nxt
            p, _, S = softmax_T(widen(target[b * N + cur], t_kind), T)
            ok = np.isfinite(S) and S > 0
        if not ok:
            flags[b] |= FLAG_NONFINITE
            continue
        y, _, marg = inverse_cdf(p, u[N - 1])
        margins[b, N - 1] = marg
        emitted.append(y)
        tokens[b, :len(emitted)] = emitted
        count[b] = len(emitted)
        accepted[b] = len(kept)
        path[b, :len(kept)] = kept
    return dict(tokens=tokens, count=count, accepted=accepted, path=path,
                flags=flags, margins=margins)
