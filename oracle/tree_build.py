"""EAGLE-2 dynamic draft tree: expansion, rerank, flattening, ancestor mask.

TEST INFRASTRUCTURE (see the package docstring).

"Speculative Decoding II", EAGLE-2 section ("Context-Aware Dynamic Draft
Tree") and its worked example: a node's value is the product of the draft's
confidences along its path from the root (the root's value is 1); each round
the best nodes of the newest layer (by value) are expanded, each proposing its
top-k tokens under the draft's distribution at that node; after the last round
the whole tree is reranked by value and the best nodes are kept (a node's
value never exceeds its parent's, and ties go to the shallower node, so the
kept set stays connected); the kept tree is flattened breadth-first for the
target's one forward, each node attending to itself and its ancestors, at
position = depth.

Readings where the page is silent (used identically by the kernels):
* a node's children are the top-k ids of its draft row by stored probability,
  lower id first among equals; a stored value is clamped into [0, 1] and a
  NaN counts as 0, so a value never exceeds its parent's and the kept set
  is connected for any input;
* values are float64 products, parent value times the child's confidence;
* layer selection and the rerank order candidates by (-value, depth,
  creation order); creation order = the order candidates are appended
  (expanded nodes in the order given, each one's children best first);
* flattening orders each depth by (parent's flat index, -confidence, token,
  creation order);
* the ancestor mask row of node i has ones at i and at every ancestor of i.
"""
import numpy as np

from .rows import widen


def topk_children(row, kind, k):
    """The k ids of a stored draft row with the largest probabilities (lower id
    first among equals; values clamped into [0, 1], NaN counts as 0), with
    their confidences (float64)."""
    p = widen(row, kind)
    p = np.clip(np.where(np.isnan(p), 0.0, p), 0.0, 1.0)
    order = np.lexsort((np.arange(p.shape[0]), -p))[:k]
    return [(int(i), float(p[i])) for i in order]


class DraftTree:
    """Candidates of one request: token, parent (candidate index, -1 at the
    root), depth, confidence, value; index = creation order."""

    def __init__(self):
        self.token, self.parent, self.depth = [-1], [-1], [0]
        self.conf, self.value = [1.0], [1.0]

    def __len__(self):
        return len(self.token)

    def expand(self, nodes, rows, kind, top_children, expand_next):
        """Append the top_children children of each candidate in ``nodes`` (whose
        draft rows are ``rows``, in the same order) and return the indices of
        the expand_next best candidates appended now (the next round's
        frontier), best first."""
        first = len(self)
        for n, row in zip(nodes, rows):
            for tok, c in topk_children(row, kind, top_children):
                self.token.append(tok)
                self.parent.append(n)
                self.depth.append(self.depth[n] + 1)
                self.conf.append(c)
                self.value.append(self.value[n] * c)
        new = list(range(first, len(self)))
        new.sort(key=lambda i: (-self.value[i], self.depth[i], i))
        return new[:expand_next]

    def finalize(self, n_nodes):
        """Keep the root and the best n_nodes - 1 candidates, flatten them
        breadth-first.  Returns (parent [n], token [n], depth [n], candidate
        id [n], ancestor mask [n, n] uint8); with fewer candidates than
        n_nodes the tail of each array is -1 / 0."""
        rest = sorted(range(1, len(self)), key=lambda i: (-self.value[i], self.depth[i], i))
        kept = [0] + rest[:n_nodes - 1]
        kset = set(kept)
        flat_of = {0: 0}
        flat = [0]
        for d in range(1, max(self.depth[i] for i in kept) + 1):
            lvl = [i for i in kept if self.depth[i] == d]
            assert all(self.parent[i] in kset for i in lvl), "rerank broke connectivity"
            lvl.sort(key=lambda i: (flat_of[self.parent[i]], -self.conf[i], self.token[i], i))
            for i in lvl:
                flat_of[i] = len(flat)
                flat.append(i)
        n = len(flat)
        parent = np.full(n_nodes, -1, dtype=np.int64)
        token = np.full(n_nodes, -1, dtype=np.int64)
        depth = np.full(n_nodes, -1, dtype=np.int64)
        cand = np.full(n_nodes, -1, dtype=np.int64)
        mask = np.zeros((n_nodes, n_nodes), dtype=np.uint8)
        for f, i in enumerate(flat):
            parent[f] = flat_of[self.parent[i]] if i else -1
            token[f] = self.token[i]
            depth[f] = self.depth[i]
            cand[f] = i
        for f in range(n):
            j = f
            while j >= 0:
                mask[f, j] = 1
                j = parent[j]
        return parent, token, depth, cand, mask


def build_tree(row_of, kind, top_children, expand_per_layer, max_depth, n_nodes):
    """A whole EAGLE-2 round for one request: ``row_of(candidate index)``
    returns the draft row at that candidate; rounds expand the root, then the
    best expand_per_layer candidates of the newest layer, up to max_depth
    layers; then finalize."""
    t = DraftTree()
    frontier = [0]
    for _ in range(max_depth):
        if not frontier:
            break
        frontier = t.expand(frontier, [row_of(i) for i in frontier], kind, top_children,
                            expand_per_layer)
    return t, t.finalize(n_nodes)
