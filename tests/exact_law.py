"""Exact output laws of the oracle, by integration over its uniforms.

The oracle is used as a black box: every decision it takes is monotone in its
own uniform (a draft is kept for u below a threshold; the drawn token is a
non-decreasing step function of the final uniform), so the measure of each
outcome is found by bisecting on the uniform with the oracle in the loop, all
cases of one step in a single batched call.  No formula of the method is used
here; the tests compare the resulting laws with what the pages state.
"""
from collections import defaultdict

import numpy as np

import oracle

ONE_MINUS = 1.0 - 2.0 ** -53
ITERS = 54


def thresholds(f, n, iters=ITERS):
    """For n monotone predicates (True below a threshold, False at and above it),
    find the n thresholds in [0, 1]; ``f(u)`` evaluates all n at once."""
    at0 = np.asarray(f(np.zeros(n)), dtype=bool)
    at1 = np.asarray(f(np.full(n, ONE_MINUS)), dtype=bool)
    lo, hi = np.zeros(n), np.ones(n)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        r = np.asarray(f(mid), dtype=bool)
        lo = np.where(r, mid, lo)
        hi = np.where(r, hi, mid)
    th = hi.copy()
    th[~at0] = 0.0
    th[at1] = 1.0
    return th


def chain_round_law(target, t_kind, draft, q_kind, V, k, T, seqs, weights):
    """Law of the emitted token sequence of one chain round whose k drafts are
    ``seqs[s]`` with probability ``weights[s]`` (rows: target 0..k, draft 0..k-1,
    shared by every case).  Returns {tuple(tokens): probability}."""
    seqs = np.asarray(seqs, dtype=np.int32).reshape(-1, k)
    S = seqs.shape[0]

    def run(ids, u):
        n = ids.shape[0]
        z = np.zeros(n, dtype=np.int32)
        return oracle.verify_sample(target, t_kind, draft, q_kind, V, z, z, ids,
                                    np.full(n, k, dtype=np.int32), k, T, u)

    theta = np.ones((S, k))
    for i in range(k):
        def f(uu, i=i):
            u = np.zeros((S, k + 1))
            u[:, i] = uu
            u[:, k] = 0.5
            return run(seqs, u)["accepted"] > i
        theta[:, i] = thresholds(f, S)

    law = defaultdict(float)
    for m in range(k + 1):
        pm = np.asarray(weights, dtype=np.float64) * np.prod(theta[:, :m], axis=1)
        if m < k:
            pm = pm * (1.0 - theta[:, m])
        live = np.nonzero(pm > 0)[0]
        if live.size == 0:
            continue
        idx = np.repeat(live, V - 1)
        ys = np.tile(np.arange(1, V), live.size)

        def g(uu, idx=idx, ys=ys, m=m):
            u = np.zeros((idx.size, k + 1))
            if m < k:
                u[:, m] = ONE_MINUS
            u[:, k] = uu
            out = run(seqs[idx], u)
            assert np.all(out["accepted"] == m)
            return out["tokens"][np.arange(idx.size), m] < ys

        bounds = thresholds(g, idx.size).reshape(live.size, V - 1)
        cells = np.diff(np.concatenate([np.zeros((live.size, 1)), bounds,
                                        np.ones((live.size, 1))], axis=1), axis=1)
        for j, s in enumerate(live):
            for y in range(V):
                if cells[j, y] > 0:
                    law[tuple(int(t) for t in seqs[s, :m]) + (y,)] += pm[s] * cells[j, y]
    return dict(law)


def tree_round_law(target, t_kind, draft, q_kind, V, T, parent, tokens_list, weights,
                   pointmass=False):
    """Law of the emitted tokens of one tree round.  All cases share the tree
    shape ``parent`` (N nodes) and rows (node c uses target/draft row c); case s
    has node tokens ``tokens_list[s]`` with probability ``weights[s]``.
    ``pointmass``: the round is ``oracle.verify_tree_pointmass`` (no draft
    rows) instead of ``oracle.verify_tree``.

    Decisions are integrated in the walk's order: the node-c test uses
    u[c-1]; the final draw uses u[N-1]."""
    parent = np.asarray(parent, dtype=np.int32)
    N = parent.shape[0]
    toks = np.asarray(tokens_list, dtype=np.int32).reshape(-1, N)
    S = toks.shape[0]

    def run(tok_rows, u):
        n = tok_rows.shape[0]
        # every case reads the same rows: rows are indexed b*N + c, so give
        # each case a copy of the shared rows
        tgt = np.tile(target, (n, 1))
        if pointmass:
            return oracle.verify_tree_pointmass(tgt, t_kind, V, np.tile(parent, (n, 1)), tok_rows, T, u)
        dft = np.tile(draft, (n, 1))
        return oracle.verify_tree(tgt, t_kind, dft, q_kind, V,
                                  np.tile(parent, (n, 1)), tok_rows, T, u,
                                  with_diag=False)

    # enumerate decision outcomes as partial assignments of the node uniforms:
    # each state is (case index, dict slot->value, probability).  A slot gets
    # 0.0 (keep: inside [0, theta)) or ONE_MINUS (reject) after its threshold
    # is measured.
    states = [(s, {}, float(weights[s])) for s in range(S) if weights[s] > 0]
    finals = []
    while states:
        # find, for each state, the next undecided test the walk reaches
        probe = np.full((len(states), N), 0.5)
        for j, (s, fixed, _) in enumerate(states):
            for slot, val in fixed.items():
                probe[j, slot] = val
            probe[j, N - 1] = 0.0
        # the walk's next test is the first node whose slot is not fixed and
        # that the walk reaches; find it by running with unfixed slots at 0.5
        # and recording which unfixed node tests were taken
        nxt = []
        for j, (s, fixed, _) in enumerate(states):
            walk = _reached_tests(parent, fixed)
            nxt.append(walk)
        new_states = []
        pend = [(j, c) for j, c in enumerate(nxt) if c is not None]
        done = [j for j, c in enumerate(nxt) if c is None]
        for j in done:
            finals.append(states[j])
        if pend:
            jj = np.array([j for j, _ in pend])
            cc = np.array([c for _, c in pend])

            def f(uu, jj=jj, cc=cc):
                u = probe[jj].copy()
                u[np.arange(jj.size), cc - 1] = uu
                out = run(toks[[states[j][0] for j in jj]], u)
                # kept iff the node appears on the kept path
                return np.array([cc[t] in out["path"][t] for t in range(jj.size)])

            th = thresholds(f, jj.size)
            for t, (j, c) in enumerate(pend):
                s, fixed, pr = states[j]
                if th[t] > 0:
                    new_states.append((s, {**fixed, c - 1: 0.0}, pr * th[t]))
                if th[t] < 1:
                    new_states.append((s, {**fixed, c - 1: ONE_MINUS}, pr * (1 - th[t])))
        states = new_states

    law = defaultdict(float)
    if not finals:
        return {}
    idx = np.repeat(np.arange(len(finals)), V - 1)
    ys = np.tile(np.arange(1, V), len(finals))
    base = np.full((len(finals), N), 0.5)
    for j, (s, fixed, _) in enumerate(finals):
        for slot, val in fixed.items():
            base[j, slot] = val
    case = np.array([finals[j][0] for j in range(len(finals))])
    ref = run(toks[case], np.concatenate([base[:, :N - 1], np.zeros((len(finals), 1))], axis=1))

    def g(uu):
        u = base[idx].copy()
        u[:, N - 1] = uu
        out = run(toks[case[idx]], u)
        last = ref["count"][idx] - 1
        return out["tokens"][np.arange(idx.size), last] < ys

    bounds = thresholds(g, idx.size).reshape(len(finals), V - 1)
    cells = np.diff(np.concatenate([np.zeros((len(finals), 1)), bounds,
                                    np.ones((len(finals), 1))], axis=1), axis=1)
    for j, (s, fixed, pr) in enumerate(finals):
        head = tuple(int(t) for t in ref["tokens"][j, :ref["count"][j] - 1])
        for y in range(V):
            if cells[j, y] > 0:
                law[head + (y,)] += pr * cells[j, y]
    return dict(law)


def _reached_tests(parent, fixed):
    """The next node test a tree walk reaches, given decided slots (slot c-1 ->
    0.0 kept / ONE_MINUS rejected); None when the walk ends.  Walks the shape
    only: children in index order, a kept child is descended into."""
    N = parent.shape[0]
    children = [[] for _ in range(N)]
    for c in range(1, N):
        children[parent[c]].append(c)
    cur = 0
    while True:
        moved = False
        for c in children[cur]:
            v = fixed.get(c - 1)
            if v is None:
                return c
            if v == 0.0:
                cur = c
                moved = True
                break
        if not moved:
            return None
