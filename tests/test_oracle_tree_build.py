"""Pins of the oracle's EAGLE-2 tree builder (CPU only): the worked example the
page prints, brute force, an independent implementation, and invariants."""
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _example():
    children, kept, flat, pos = {}, None, None, None
    with open(os.path.join(GOLD, "p4_eagle2_example.txt"), encoding="utf-8") as f:
        for ln in f:
            w = ln.split()
            if not w or w[0].startswith("#"):
                continue
            if w[0] == "child":
                children.setdefault(w[1], []).append((w[2], float(w[3]), float(w[4])))
            elif w[0] == "kept":
                kept = w[1:]
            elif w[0] == "flat":
                flat = w[1:]
            elif w[0] == "positions":
                pos = [int(x) for x in w[1:]]
    return children, kept, flat, pos


def test_eagle2_worked_example():
    """Top-2 children per expanded node, the best 2 of the newest layer expanded,
    3 rounds, 8 nodes kept (root included): the page's values, kept set,
    flattened order and positions."""
    children, kept_want, flat_want, pos_want = _example()
    names = ["I"] + sorted({c for kids in children.values() for c, _, _ in kids})
    ids = {n: i for i, n in enumerate(names)}
    V = 16
    rows = {}
    for par, kids in children.items():
        r = np.zeros(V)
        for c, conf, _ in kids:
            r[ids[c]] = conf
        rest = [i for i in range(V) if r[i] == 0.0]
        r[rest] = (1.0 - r.sum()) / len(rest)      # below every listed child
        assert r[rest].max() < min(conf for _, conf, _ in kids)
        rows[par] = r
    flat_row = lambda name: rows.get(name, np.full(V, 1.0 / V))

    t = oracle.DraftTree()
    frontier = [0]
    for _ in range(3):
        frontier = t.expand(frontier, [flat_row(names[t.token[i]] if i else "I") for i in frontier], "f64",
                            2, 2)
    # every child the page lists, with its confidence and value
    got = {(names[t.token[t.parent[i]]] if t.parent[i] else "I", names[t.token[i]]): (t.conf[i], t.value[i])
           for i in range(1, len(t))}
    want = {(p, c): (conf, v) for p, kids in children.items() for c, conf, v in kids}
    assert set(got) == set(want)
    for key, (conf, v) in want.items():
        assert got[key][0] == pytest.approx(conf, abs=1e-12)
        assert got[key][1] == pytest.approx(v, abs=1e-12)
    parent, token, depth, cand, mask = t.finalize(8)
    flat_names = ["I" if tok < 0 else names[tok] for tok in token]
    assert flat_names == flat_want
    assert sorted(flat_names) == sorted(kept_want)
    assert list(depth) == pos_want
    # ancestor mask: "now" (flat 6) sees I, do, it and itself
    assert [flat_names[j] for j in np.nonzero(mask[6])[0]] == ["I", "do", "it", "now"]


def test_topk_brute_force():
    rng = np.random.default_rng(4)
    for trial in range(200):
        V = int(rng.integers(1, 12))
        p = rng.choice([0.0, 0.1, 0.25, 0.5, np.nan, -0.3, 1.0, 1.7], size=V) if trial % 2 else rng.random(V)
        k = int(rng.integers(1, V + 1))
        got = oracle.topk_children(p, "f64", k)
        q = np.array([0.0 if v != v else min(max(v, 0.0), 1.0) for v in p])
        # id i is chosen iff fewer than k ids beat it (larger, or equal with a lower id)
        beaten = [sum(1 for j in range(V) if q[j] > q[i] or (q[j] == q[i] and j < i)) for i in range(V)]
        want = sorted((i for i in range(V) if beaten[i] < k), key=lambda i: beaten[i])
        assert [i for i, _ in got] == want
        assert all(c == q[i] for i, c in got)


@pytest.mark.parametrize("top,exp,depth,keep", [(4, 4, 6, 60), (2, 2, 3, 8), (3, 1, 5, 12), (5, 3, 4, 30)])
def test_builder_matches_the_input_generators_builder(top, exp, depth, keep):
    """The workload generator has its own EAGLE-2 builder (written separately,
    used to produce the tree inputs); on the same draft rows both give the
    same flattened tree."""
    rng = np.random.default_rng(top * 100 + exp * 10 + depth)
    V = 50
    for b in range(6):
        cache = {}

        def row(cid, b=b):
            if cid not in cache:
                r = rng.dirichlet(np.ones(V) * 0.3)
                if b % 2:  # ties (not at the top, where they would hide the order by value)
                    srt = np.sort(r)
                    r[rng.integers(0, V, size=3)] = srt[-5]
                cache[cid] = synth.encode(r, "bf16")
            return cache[cid]

        def propose(node):
            q = synth.decode(row(node.cid), "bf16")
            order = np.lexsort((np.arange(V), -q))[:top]
            return [(int(i), float(q[i])) for i in order]

        flat, par, dep = synth.build_draft_tree(propose, top, exp, depth, keep)
        t, (parent, token, d, cand, mask) = oracle.build_tree(row, "bf16", top, exp, depth, keep)
        n = len(flat)
        assert list(parent[:n]) == list(par)
        assert list(d[:n]) == list(dep)
        assert list(token[1:n]) == [node.token for node in flat[1:]]
        assert list(cand[:n]) == [node.cid for node in flat]


def test_builder_invariants():
    rng = np.random.default_rng(5)
    for trial in range(40):
        V = int(rng.integers(3, 30))
        top, exp, depth = int(rng.integers(1, 5)), int(rng.integers(1, 5)), int(rng.integers(1, 7))
        rows = {}

        def row(cid):
            if cid not in rows:
                rows[cid] = rng.dirichlet(np.ones(V))
            return rows[cid]

        t, _ = oracle.build_tree(row, "f64", top, exp, depth, 1)
        n_nodes = int(rng.integers(1, len(t) + 3))
        parent, token, d, cand, mask = t.finalize(n_nodes)
        n = int((cand >= 0).sum())
        assert n == min(n_nodes, len(t))
        for f in range(1, n):
            assert 0 <= parent[f] < f
            assert d[f] == d[parent[f]] + 1
            assert d[f] >= d[f - 1]
            assert t.value[cand[f]] <= t.value[cand[parent[f]]]
        assert np.array_equal(mask[:n, :n].sum(axis=1), d[:n] + 1)
        assert not mask[n:].any() and not mask[:, n:].any()
        # the kept candidates are the best by (-value, depth, creation order)
        order = sorted(range(1, len(t)), key=lambda i: (-t.value[i], t.depth[i], i))
        assert set(cand[1:n]) == set(order[:n - 1])


def test_rerank_ties_go_to_the_shallower_node():
    """A child whose confidence is 1 has its parent's value; the rerank keeps
    the parent first (the page: ties to the shallower node keep the kept set
    connected), and the frontier choice among equal values follows creation
    order."""
    V = 10
    rows = {
        0: np.array([0.0, 0.5, 0.3, 0.2, 0, 0, 0, 0, 0, 0]),   # root: ids 1, 2, 3
        1: np.eye(V)[7],                                      # under id 1: id 7 with c = 1
        2: np.eye(V)[8],                                      # under id 2: id 8 with c = 1
        3: np.eye(V)[9],
    }
    t = oracle.DraftTree()
    frontier = t.expand([0], [rows[0]], "f64", 3, 2)
    assert frontier == [1, 2]
    assert [t.token[i] for i in frontier] == [1, 2]
    frontier = t.expand(frontier, [rows[t.token[i]] for i in frontier], "f64", 1, 2)
    assert [t.value[i] for i in frontier] == [0.5, 0.3]
    for keep, want in ((2, [-1, 1]), (3, [-1, 1, 7]), (4, [-1, 1, 2, 7]), (5, [-1, 1, 2, 7, 8])):
        parent, token, depth, cand, mask = t.finalize(keep)
        assert list(token[:keep]) == want, keep
