"""Pins of the oracle's edge readings (CPU only): the end-token cut, the
budget cut, the zero-residual fallback and the outputs of invalid requests.

Each case is small enough to work out by hand from the pages' rules, so the
expected tokens, counts and status bits below are written out literally (they
do not come from the oracle).  Target rows are given as float64 logits; a
one-hot distribution is a row of -inf with one 0, so every accept decision and
every draw in these cases is forced whatever the uniform.

Readings pinned here:
* emission stops after the first end token, which is emitted ("第 13 篇：推理
  引擎一次猜几个字——草稿 + 验证", section ③: the loop runs while no end token
  has been met), and at the request's remaining budget ("Speculative decoding
  explained", four-case table: a finished path adds nothing);
* a residual max(0, p - q) with no mass (possible when the stored draft row
  sums to more than 1) draws the chain's token from p_m and sets the fallback
  bit; a tree leaves p as it was, sets the bit and tests the next sibling
  against it ("投机解码:为什么一个字都不改", section "改进": the draw comes
  from the target's side);
* an invalid request (a token outside [0, V), a draft count outside
  [0, k_max], a row range outside the buffers, a tree whose parents do not
  precede their children) gets count 0, accepted 0, every token -1 and its
  status bit, and nothing else is computed for it.
"""
import numpy as np
import pytest

import oracle

NEG = -np.inf
V = 8


def one_hot_logits(tok, V=V):
    row = np.full(V, NEG)
    row[tok] = 0.0
    return row


def chain_case(drafts, picks, k_max=None, q_rows=None):
    """One request: target rows 0..k one-hot at picks[i] (picks has k + 1
    entries), draft rows uniform over the vocabulary (every drafted token has
    q = 1/V > 0)."""
    k = len(drafts)
    k_max = k if k_max is None else k_max
    target = np.stack([one_hot_logits(t) for t in picks])
    draft = np.full((max(k, 1), V), 1.0 / V) if q_rows is None else q_rows
    ids = np.full((1, max(k_max, 1)), -1, dtype=np.int64)
    ids[0, :k] = drafts
    return target, draft, ids, np.array([k]), k_max


def run_sample(target, draft, ids, dlen, k_max, u=None, max_new=None, eos=-1, ts=0, qs=0, T=1.0):
    u = np.full((1, k_max + 1), 0.5) if u is None else np.asarray(u, dtype=np.float64).reshape(1, -1)
    mn = None if max_new is None else np.array([max_new])
    return oracle.verify_sample(target, "f64", draft, "f64", target.shape[1], np.array([ts]), np.array([qs]),
                                ids[:, :k_max] if k_max else ids[:, :0], dlen, k_max, T, u, max_new=mn,
                                eos_id=eos)


def run_greedy(target, ids, dlen, k_max, max_new=None, eos=-1, ts=0):
    mn = None if max_new is None else np.array([max_new])
    return oracle.verify_greedy(target, "f64", target.shape[1], np.array([ts]),
                                ids[:, :k_max] if k_max else ids[:, :0], dlen, k_max, max_new=mn, eos_id=eos)


def emitted(out):
    c = int(out["count"][0])
    toks = [int(t) for t in out["tokens"][0]]
    assert all(t == -1 for t in toks[c:]), "slots after the count are -1"
    return toks[:c]


# drafts 5, 3, 6 all kept (each row is one-hot at its draft), bonus 2 from row 3
FULL = dict(drafts=[5, 3, 6], picks=[5, 3, 6, 2])
# EOS cut: (eos id, emitted tokens).  The end token itself is emitted; only
# the first occurrence counts; an end token that never appears changes nothing.
EOS_CASES = [(-1, [5, 3, 6, 2]), (7, [5, 3, 6, 2]), (5, [5]), (3, [5, 3]), (6, [5, 3, 6]), (2, [5, 3, 6, 2])]


@pytest.mark.parametrize("eos,want", EOS_CASES)
@pytest.mark.parametrize("kind", ["sample", "greedy"])
def test_eos_cut_is_inclusive_and_first_only(kind, eos, want):
    t, d, ids, dl, km = chain_case(**FULL)
    out = run_sample(t, d, ids, dl, km, eos=eos) if kind == "sample" else run_greedy(t, ids, dl, km, eos=eos)
    assert emitted(out) == want
    assert int(out["accepted"][0]) == 3          # accepted counts the kept drafts, cut or not
    assert int(out["flags"][0]) == 0


@pytest.mark.parametrize("kind", ["sample", "greedy"])
def test_eos_first_occurrence_among_repeats(kind):
    t, d, ids, dl, km = chain_case(drafts=[3, 3, 6], picks=[3, 3, 6, 2])
    out = run_sample(t, d, ids, dl, km, eos=3) if kind == "sample" else run_greedy(t, ids, dl, km, eos=3)
    assert emitted(out) == [3]


@pytest.mark.parametrize("kind", ["sample", "greedy"])
def test_eos_after_a_rejection(kind):
    """Draft 4 at position 1 has p = 0 under a row one-hot at 3: rejected, and
    the residual max(0, p - q) keeps only token 3, so the round emits 5, 3."""
    t, d, ids, dl, km = chain_case(drafts=[5, 4, 6], picks=[5, 3, 6, 2])
    run = (lambda **kw: run_sample(t, d, ids, dl, km, **kw)) if kind == "sample" else \
        (lambda **kw: run_greedy(t, ids, dl, km, **kw))
    assert emitted(run()) == [5, 3]
    assert emitted(run(eos=5)) == [5]
    assert emitted(run(eos=3)) == [5, 3]
    assert emitted(run(eos=6)) == [5, 3]          # a rejected draft is never emitted
    assert int(run(eos=5)["accepted"][0]) == 1


# Budget cut: (max_new, eos, emitted, flags).  More drafts than the budget is
# flagged (over budget, 8) but still verified; a budget equal to k leaves no
# room for the bonus (the four-case table's finished path); the budget and the
# end token cut independently, whichever comes first.
BUDGET_CASES = [(4, -1, [5, 3, 6, 2], 0), (9, -1, [5, 3, 6, 2], 0), (3, -1, [5, 3, 6], 0),
                (2, -1, [5, 3], 8), (1, -1, [5], 8), (0, -1, [], 8), (-4, -1, [], 8),
                (2, 6, [5, 3], 8), (3, 3, [5, 3], 0), (4, 6, [5, 3, 6], 0)]


@pytest.mark.parametrize("max_new,eos,want,flags", BUDGET_CASES)
@pytest.mark.parametrize("kind", ["sample", "greedy"])
def test_budget_cut(kind, max_new, eos, want, flags):
    t, d, ids, dl, km = chain_case(**FULL)
    out = run_sample(t, d, ids, dl, km, max_new=max_new, eos=eos) if kind == "sample" else \
        run_greedy(t, ids, dl, km, max_new=max_new, eos=eos)
    assert emitted(out) == want
    assert int(out["flags"][0]) == flags


# ---------------------------------------------------------------------------
# zero residual mass
# ---------------------------------------------------------------------------
P = np.array([0.3, 0.7])
Q = np.array([0.5, 0.9])      # stored draft row summing to 1.4: p <= q everywhere


def test_chain_zero_residual_draws_from_p_and_flags():
    """k = 1, draft 0: u q(0) = 0.9 * 0.5 = 0.45 >= p(0) = 0.3, so the draft is
    rejected; max(0, p - q) = 0 everywhere, so the token is drawn from p_0 with
    u_1 = 0.35: cumulative p = 0.3, 1.0 -> token 1.  Drawing from q instead
    (cumulative 0.5, 1.4 against 0.35 * 1.4 = 0.49) would give 0, and drawing
    from the bonus row (one-hot at 0) would give 0 too."""
    target = np.stack([np.log(P), one_hot_logits(0, 2)])
    out = oracle.verify_sample(target, "f64", Q[None, :], "f64", 2, np.array([0]), np.array([0]),
                               np.array([[0]]), np.array([1]), 1, 1.0, np.array([[0.9, 0.35]]))
    assert emitted(out) == [1]
    assert int(out["accepted"][0]) == 0
    assert int(out["flags"][0]) == oracle.FLAG_FALLBACK
    assert abs(out["resid"][0] - 1.0) < 1e-12      # the mass drawn from is p's


def test_chain_positive_residual_sets_no_fallback():
    """The same rejection against a draft row that sums to 1 (q = 0.5, 0.5):
    the residual is (0, 0.2), token 1, mass 0.2, no flag."""
    target = np.stack([np.log(P), one_hot_logits(0, 2)])
    out = oracle.verify_sample(target, "f64", np.array([[0.5, 0.5]]), "f64", 2, np.array([0]), np.array([0]),
                               np.array([[0]]), np.array([1]), 1, 1.0, np.array([[0.9, 0.35]]))
    assert emitted(out) == [1]
    assert int(out["flags"][0]) == 0
    assert abs(out["resid"][0] - 0.2) < 1e-12


def test_tree_zero_residual_keeps_p_for_the_next_sibling():
    """Root with children node 1 (token 0) and node 2 (token 1); root p = (0.3,
    0.7), root q = (0.5, 0.9).  Node 1: 0.9 * 0.5 >= 0.3, rejected; the residual
    has no mass, so p stays (0.3, 0.7) and the fallback bit is set.  Node 2:
    0.7 * 0.9 = 0.63 < 0.7, kept.  Node 2 is a leaf: the last token comes from
    its own row (one-hot at 0).  Renormalising the empty residual (0/0) would
    make node 2's test fail; dropping to the zero vector would too."""
    target = np.stack([np.log(P), one_hot_logits(1, 2), one_hot_logits(0, 2)])
    draft = np.stack([Q, np.array([0.5, 0.5]), np.array([0.5, 0.5])])
    out = oracle.verify_tree(target, "f64", draft, "f64", 2, np.array([[-1, 0, 0]]), np.array([[-1, 0, 1]]),
                             1.0, np.array([[0.9, 0.7, 0.5]]), with_diag=False)
    assert emitted(out) == [1, 0]
    assert [int(v) for v in out["path"][0]] == [2, -1, -1]
    assert int(out["accepted"][0]) == 1
    assert int(out["flags"][0]) == oracle.FLAG_FALLBACK


def test_tree_zero_residual_then_draw_from_unchanged_p():
    """Both children rejected: node 1 as above; node 2 (token 1) with u = 0.8:
    0.8 * 0.9 = 0.72 >= 0.7, rejected, again no residual mass.  The last token
    is drawn from the unchanged root p with u = 0.2: cumulative 0.3 > 0.2 ->
    token 0."""
    target = np.stack([np.log(P), one_hot_logits(1, 2), one_hot_logits(1, 2)])
    draft = np.stack([Q, np.array([0.5, 0.5]), np.array([0.5, 0.5])])
    out = oracle.verify_tree(target, "f64", draft, "f64", 2, np.array([[-1, 0, 0]]), np.array([[-1, 0, 1]]),
                             1.0, np.array([[0.9, 0.8, 0.2]]), with_diag=False)
    assert emitted(out) == [0]
    assert int(out["accepted"][0]) == 0
    assert int(out["flags"][0]) == oracle.FLAG_FALLBACK


# ---------------------------------------------------------------------------
# invalid requests
# ---------------------------------------------------------------------------
def assert_invalid(out, bits, width):
    assert int(out["count"][0]) == 0
    assert int(out["accepted"][0]) == 0
    assert [int(t) for t in out["tokens"][0]] == [-1] * width
    assert int(out["flags"][0]) == bits


@pytest.mark.parametrize("kind", ["sample", "greedy"])
@pytest.mark.parametrize("bad", [8, 99, -1])
def test_bad_token_invalidates_the_request(kind, bad):
    """A drafted id outside [0, V) anywhere in the draft, also after a draft
    that would be rejected (row 0 is one-hot at 2, draft 0 is 5)."""
    t, d, ids, dl, km = chain_case(drafts=[5, bad], picks=[2, 3, 4])
    out = run_sample(t, d, ids, dl, km) if kind == "sample" else run_greedy(t, ids, dl, km)
    assert_invalid(out, oracle.FLAG_BAD_TOKEN, km + 1)


@pytest.mark.parametrize("kind", ["sample", "greedy"])
def test_draft_count_outside_k_max(kind):
    t, d, ids, _, _ = chain_case(drafts=[5, 3], picks=[5, 3, 2], k_max=2)
    for k in (3, -1):
        dl = np.array([k])
        out = run_sample(t, d, ids, dl, 2) if kind == "sample" else run_greedy(t, ids, dl, 2)
        assert_invalid(out, oracle.FLAG_BAD_REQUEST, 3)


@pytest.mark.parametrize("kind", ["sample", "greedy"])
def test_row_range_outside_the_buffers(kind):
    """k = 2 needs target rows ts..ts+2 (3 rows exist) and draft rows qs..qs+1
    (2 rows exist)."""
    t, d, ids, dl, km = chain_case(drafts=[5, 3], picks=[5, 3, 2])
    for ts, qs in ((1, 0), (-1, 0), (0, 1), (0, -1)):
        if kind == "greedy" and ts == 0:
            continue      # the greedy verify reads no draft rows
        out = run_sample(t, d, ids, dl, km, ts=ts, qs=qs) if kind == "sample" else \
            run_greedy(t, ids, dl, km, ts=ts)
        assert_invalid(out, oracle.FLAG_BAD_REQUEST, km + 1)
    # the same request at its proper rows is valid
    out = run_sample(t, d, ids, dl, km)
    assert emitted(out) == [5, 3, 2]


TREE_T = np.stack([one_hot_logits(1), one_hot_logits(2), one_hot_logits(3), one_hot_logits(4)])
TREE_Q = np.full((4, V), 1.0 / V)


@pytest.mark.parametrize("parent,token,bits", [
    ([0, 0, 1, 2], [-1, 1, 2, 3], oracle.FLAG_BAD_TREE),     # root's parent is not -1
    ([-1, 0, 2, 1], [-1, 1, 2, 3], oracle.FLAG_BAD_TREE),    # node 2's parent is itself
    ([-1, 0, 3, 1], [-1, 1, 2, 3], oracle.FLAG_BAD_TREE),    # node 2's parent comes later
    ([-1, -1, 1, 2], [-1, 1, 2, 3], oracle.FLAG_BAD_TREE),   # a second root
    ([-1, 0, 1, 2], [-1, 1, 8, 3], oracle.FLAG_BAD_TOKEN),   # token outside [0, V)
    ([-1, 0, 1, 5], [-1, 9, 2, 3], oracle.FLAG_BAD_TREE),    # both: the tree bit alone
])
@pytest.mark.parametrize("kind", ["tree", "greedy", "pointmass"])
def test_tree_invalid_outputs(kind, parent, token, bits):
    par, tok = np.array([parent]), np.array([token])
    u = np.full((1, 4), 0.5)
    if kind == "tree":
        out = oracle.verify_tree(TREE_T, "f64", TREE_Q, "f64", V, par, tok, 1.0, u, with_diag=False)
    elif kind == "greedy":
        out = oracle.verify_tree_greedy(TREE_T, "f64", V, par, tok)
    else:
        out = oracle.verify_tree_pointmass(TREE_T, "f64", V, par, tok, 1.0, u)
    assert_invalid(out, bits, 4)
    assert [int(v) for v in out["path"][0]] == [-1] * 4


@pytest.mark.parametrize("kind", ["tree", "greedy", "pointmass"])
def test_tree_valid_chain_reference(kind):
    """The same rows as a valid chain tree 0 -> 1 -> 2 -> 3 with tokens 1, 2, 3:
    every node is kept (each row is one-hot at its child's token) and the leaf
    adds its own pick 4."""
    par, tok = np.array([[-1, 0, 1, 2]]), np.array([[-1, 1, 2, 3]])
    u = np.full((1, 4), 0.5)
    if kind == "tree":
        out = oracle.verify_tree(TREE_T, "f64", TREE_Q, "f64", V, par, tok, 1.0, u, with_diag=False)
    elif kind == "greedy":
        out = oracle.verify_tree_greedy(TREE_T, "f64", V, par, tok)
    else:
        out = oracle.verify_tree_pointmass(TREE_T, "f64", V, par, tok, 1.0, u)
    assert emitted(out) == [1, 2, 3, 4]
    assert [int(v) for v in out["path"][0]] == [1, 2, 3, -1]
    assert int(out["flags"][0]) == 0
