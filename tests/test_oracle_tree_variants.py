"""Pins of the oracle's greedy and point-mass tree verifies (CPU only).

Each is checked against something other than itself: the exact output law
the pages state (recursive speculative sampling keeps the target's
distribution, "Speculative Decoding II", EAGLE section; the acceptance/residual
identity of "投机解码:为什么一个字都不改", section "改进"), special cases that
reduce to the already pinned chain and tree verifies, and brute force.
"""
import itertools

import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

import oracle
from tests.exact_law import tree_round_law


def _logits(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, dtype=np.float64))


def _random_parents(rng, N):
    return np.array([-1] + [int(rng.integers(0, c)) for c in range(1, N)], dtype=np.int32)


# ---------------------------------------------------------------------------
# point-mass tree: exact law
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("tokens", [(-1, 2, 2, 5, 6), (-1, 5, 2, 5, 2), (-1, 3, 3, 3, 3)])
def test_pointmass_tree_keeps_the_target_law(tokens):
    """Node 1 has child 4; nodes 2 and 3 are leaves under the root.  Whatever
    the (fixed, possibly repeated) candidate tokens, the first emitted token
    follows the root's row and every later token follows the row of the node
    it is drawn at: P(t1, t2, ...) = P0(t1) P_{n1}(t2) ... along the kept path."""
    rng = np.random.default_rng(7)
    V = 8
    P = rng.dirichlet(np.ones(V) * 0.8, size=5)
    parent = np.array([-1, 0, 0, 0, 1])
    law = tree_round_law(_logits(P), "f64", None, None, V, 1.0, parent, np.array([tokens]),
                         np.array([1.0]), pointmass=True)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    children = {0: [1, 2, 3], 1: [4], 2: [], 3: [], 4: []}

    def expected(seq):
        # walk the kept path the sequence implies: after node n, the token t is
        # a kept child of n iff some child of n carries t (the first such child
        # is the one kept, a later duplicate never is), else the round ends
        pr, n = 1.0, 0
        for i, t in enumerate(seq):
            pr *= P[n][t]
            kid = next((c for c in children[n] if tokens[c] == t), None)
            if kid is None:
                return pr if i == len(seq) - 1 else 0.0
            n = kid
        return 0.0   # a sequence must end with a drawn token

    for seq, pr in law.items():
        assert abs(pr - expected(seq)) < 1e-12, (seq, pr, expected(seq))
    # and every sequence of positive expected probability is present
    total = sum(expected(s) for s in law)
    assert abs(total - 1.0) < 1e-12


def test_pointmass_tree_first_token_law_many_siblings():
    """Root with five fixed candidates (two repeated) and nothing below: the
    emitted token follows the root's row exactly."""
    rng = np.random.default_rng(8)
    V = 8
    P = rng.dirichlet(np.ones(V), size=6)
    parent = np.array([-1, 0, 0, 0, 0, 0])
    law = tree_round_law(_logits(P), "f64", None, None, V, 0.7, parent,
                         np.array([[-1, 4, 1, 4, 7, 1]]), np.array([1.0]), pointmass=True)
    Pt = scipy_softmax(_logits(P[0]) / 0.7)
    first = np.zeros(V)
    for seq, pr in law.items():
        first[seq[0]] += pr
    np.testing.assert_allclose(first, Pt, rtol=0, atol=1e-12)


def test_pointmass_equals_sampled_tree_with_one_hot_draft_rows():
    """A chain-shaped tree whose draft row at every node is one-hot at its one
    child's token is the same round for both verifies (q = delta_x)."""
    rng = np.random.default_rng(9)
    B, N, V, T = 40, 6, 300, 0.9
    tgt = rng.standard_normal((B * N, V)) * 2.0
    parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    tok = np.full((B, N), -1, dtype=np.int32)
    dft = np.zeros((B * N, V))
    for b in range(B):
        for c in range(1, N):
            row = tgt[b * N + c - 1]
            tok[b, c] = int(np.argmax(row)) if rng.random() < 0.5 else int(rng.integers(0, V))
            dft[b * N + c - 1, tok[b, c]] = 1.0
        dft[b * N + N - 1, 0] = 1.0
    u = rng.random((B, N))
    a = oracle.verify_tree(tgt, "f64", dft, "f64", V, parent, tok, T, u, with_diag=False)
    p = oracle.verify_tree_pointmass(tgt, "f64", V, parent, tok, T, u)
    for key in ("tokens", "count", "accepted", "path", "flags"):
        assert np.array_equal(a[key], p[key]), key
    assert 0 < a["accepted"].mean() < N - 1


def test_pointmass_never_emits_zero_mass_or_rejected_tokens():
    """u = 0 keeps any candidate with p > 0; a candidate with p = 0, or one
    already rejected at the same node, is never kept; the last draw never
    returns an id with p = 0 or one rejected at its node."""
    V = 6
    p = np.array([0.0, 0.5, 0.0, 0.3, 0.2, 0.0])
    parent = np.array([-1, 0, 0, 0])
    cases, uu = [], []
    for toks in itertools.product(range(V), repeat=3):
        for us in ((0.0, 0.0, 0.0), (0.9, 0.9, 0.0), (0.6, 0.99, 0.999), (0.95, 0.95, 0.5)):
            cases.append((-1,) + toks)
            uu.append(us + (0.999,))
    B = len(cases)
    tok = np.array(cases, dtype=np.int32)
    out = oracle.verify_tree_pointmass(np.tile(_logits(p), (B * 4, 1)), "f64", V,
                                       np.tile(parent, (B, 1)), tok, 1.0, np.array(uu))
    for b in range(B):
        n = int(out["count"][b])
        assert n >= 1
        first = int(out["tokens"][b, 0])
        assert p[first] > 0
        if out["accepted"][b] == 0:  # drawn: not one of the rejected candidates
            assert first not in set(tok[b, 1:])


# ---------------------------------------------------------------------------
# greedy tree
# ---------------------------------------------------------------------------
def test_greedy_chain_as_tree_equals_greedy_chain():
    rng = np.random.default_rng(10)
    B, k, V = 30, 4, 1000
    N = k + 1
    tgt = rng.standard_normal((B * N, V)).astype(np.float32)
    ids = np.zeros((B, k), dtype=np.int32)
    for b in range(B):
        for i in range(k):
            row = tgt[b * N + i]
            ids[b, i] = int(np.argmax(row)) if rng.random() < 0.7 else int(rng.integers(0, V))
    trs = (np.arange(B) * N).astype(np.int32)
    ch = oracle.verify_greedy(tgt, "f32", V, trs, ids, np.full(B, k, np.int32), k)
    parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    tok = np.concatenate([np.full((B, 1), -1, np.int32), ids], axis=1)
    tr = oracle.verify_tree_greedy(tgt, "f32", V, parent, tok)
    assert np.array_equal(ch["tokens"], tr["tokens"])
    assert np.array_equal(ch["count"], tr["count"])
    assert np.array_equal(ch["accepted"], tr["accepted"])
    for b in range(B):
        m = int(tr["accepted"][b])
        assert list(tr["path"][b, :m]) == list(range(1, m + 1))
    assert len(set(ch["accepted"])) > 2


def test_greedy_tree_equals_sampled_tree_on_one_hot_targets():
    """With every target row one-hot at a_c, the sampled tree keeps the first
    child carrying a_c (u q(a) < 1 = p(a)), rejects the others (p(x) = 0, and
    the residual is one-hot at a_c again), and draws a_c when none carries it:
    the greedy tree's walk."""
    rng = np.random.default_rng(11)
    B, N, V = 60, 14, 40
    parent = np.stack([_random_parents(rng, N) for _ in range(B)])
    tok = rng.integers(0, V, size=(B, N)).astype(np.int32)
    tok[:, 0] = -1
    tgt = np.full((B * N, V), -np.inf)
    for b in range(B):
        for c in range(N):
            kids = [d for d in range(1, N) if parent[b, d] == c]
            a = int(tok[b, kids[int(rng.integers(0, len(kids)))]]) if kids and rng.random() < 0.7 \
                else int(rng.integers(0, V))
            tgt[b * N + c, a] = 0.0
    q = rng.dirichlet(np.ones(V), size=B * N)
    u = rng.random((B, N))
    s = oracle.verify_tree(tgt, "f64", q, "f64", V, parent, tok, 1.0, u, with_diag=False)
    g = oracle.verify_tree_greedy(tgt, "f64", V, parent, tok)
    for key in ("tokens", "count", "accepted", "path", "flags"):
        assert np.array_equal(s[key], g[key]), key
    assert g["accepted"].max() >= 3


def _greedy_brute(rows, parent, tok):
    """Every node's root path; keep the valid ones (each node's token is the
    argmax of its parent's row); among the valid paths that no valid child
    extends, the lexicographically smallest index sequence; emitted = its
    tokens + the argmax of its last node's row."""
    N = len(parent)
    amax = [int(np.argmax(r)) for r in rows]
    paths = []
    for c in range(N):
        p, n = [], c
        while n > 0:
            p.append(n)
            n = parent[n]
        paths.append(tuple(reversed(p)))
    valid = [p for p in paths if all(tok[n] == amax[parent[n]] for n in p)]
    vset = set(valid)
    maximal = [p for p in valid
               if not any(parent[d] == (p[-1] if p else 0) and p + (d,) in vset for d in range(1, N))]
    best = min(maximal)
    last = best[-1] if best else 0
    return [tok[n] for n in best] + [amax[last]], list(best)


def test_greedy_tree_brute_force():
    rng = np.random.default_rng(12)
    V = 4
    for trial in range(300):
        N = int(rng.integers(1, 13))
        parent = _random_parents(rng, N)
        tok = rng.integers(0, V, size=N).astype(np.int32)
        tok[0] = -1
        rows = rng.standard_normal((N, V))
        rows[rng.random((N, V)) < 0.2] = 0.5   # ties
        out = oracle.verify_tree_greedy(rows, "f64", V, parent[None, :], tok[None, :])
        want, path = _greedy_brute(rows, parent, tok)
        n = int(out["count"][0])
        assert list(out["tokens"][0, :n]) == want, trial
        assert list(out["path"][0, :n - 1]) == path, trial
        assert int(out["accepted"][0]) == len(path)


def test_greedy_tree_nan_counts_only_in_visited_rows():
    V = 5
    parent = np.array([[-1, 0, 0, 1]], dtype=np.int32)
    tok = np.array([[-1, 2, 3, 4]], dtype=np.int32)
    rows = np.zeros((4, V))
    rows[0, 3] = 1.0         # root picks 3 -> node 2 (a leaf)
    rows[1, :] = np.nan      # node 1 is never visited
    rows[3, :] = np.nan
    rows[2, 1] = 2.0         # node 2 picks 1
    out = oracle.verify_tree_greedy(rows, "f64", V, parent, tok)
    assert int(out["flags"][0]) == 0
    assert list(out["tokens"][0, :2]) == [3, 1] and int(out["count"][0]) == 2
    rows[2, 0] = np.nan      # now a visited row holds a NaN
    out = oracle.verify_tree_greedy(rows, "f64", V, parent, tok)
    assert int(out["flags"][0]) == oracle.FLAG_NONFINITE and int(out["count"][0]) == 0
