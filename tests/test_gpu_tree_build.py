"""The EAGLE-2 draft tree built on the device (sv_tree_expand /
sv_tree_finalize) against the oracle's builder, on an MI355X, through the C
ABI: candidates, values, frontiers, the flattened tree and the ancestor mask
bit for bit."""
import numpy as np
import pytest
import torch

import draft_verify_sampling_amd as sv
import oracle
import synth
from tests.gpu_util import say, rows_to_dev, i32, f32, compare_tokens, DEV

pytestmark = pytest.mark.gpu


def _draft_rows(rng, n, V, kind, sharp=2.0, special=False):
    l = rng.standard_normal((n, V)) * sharp
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    if special:  # ties, NaN, values outside [0, 1]
        for r in range(n):
            idx = rng.choice(V, size=6, replace=False)
            p[r, idx[:3]] = p[r].max()
            p[r, idx[3]] = np.nan
            p[r, idx[4]] = 1.5
            p[r, idx[5]] = -0.5
    return synth.encode(p, kind)


def _build(rng, B, V, kind, top, exp, depth, N, max_cand, special=False):
    """Both builders on the same rows; returns (gpu outputs, oracle trees, rounds' rows)."""
    state = sv.DraftTreeState(B, max_cand)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    trees = [oracle.DraftTree() for _ in range(B)]
    fronts = [[0] for _ in range(B)]
    nxt = None
    for r in range(depth):
        n_exp = 1 if r == 0 else exp
        rows = _draft_rows(rng, B * n_exp, V, kind, special=special)
        nxt = sv.sv_tree_expand(rows_to_dev(rows, kind), nxt, top, exp, state, dev_status=st)
        for b in range(B):
            fr = fronts[b]
            if fr:
                fronts[b] = trees[b].expand(fr, [rows[b * n_exp + e] for e in range(len(fr))], kind, top, exp)
        got_next = nxt.cpu().numpy()
        for b in range(B):
            want = fronts[b] + [-1] * (exp - len(fronts[b]))
            assert list(got_next[b]) == want, (r, b)
    torch.cuda.synchronize()
    parent, token, dep, cand, mask = sv.sv_tree_finalize(state, N, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return state, (parent, token, dep, cand, mask), trees


def _compare(state, outs, trees, N):
    cnt = state.count.cpu().numpy()
    tok, par, dep = state.token.cpu().numpy(), state.parent.cpu().numpy(), state.depth.cpu().numpy()
    conf, val = state.conf.cpu().numpy(), state.value.cpu().numpy()
    parent, token, depth, cand, mask = (t.cpu().numpy() for t in outs)
    for b, t in enumerate(trees):
        n = len(t)
        assert cnt[b] == n
        assert list(tok[b, :n]) == t.token and list(par[b, :n]) == t.parent and list(dep[b, :n]) == t.depth
        assert np.array_equal(conf[b, :n].astype(np.float64), np.array(t.conf))
        assert np.array_equal(val[b, :n], np.array(t.value))          # fp64 products, bit for bit
        wp, wt, wd, wc, wm = t.finalize(N)
        assert np.array_equal(parent[b], wp) and np.array_equal(token[b], wt)
        assert np.array_equal(depth[b], wd) and np.array_equal(cand[b], wc)
        assert np.array_equal(mask[b], wm)


def test_gpu_tree_build_eagle2_shape():
    say("device tree builder: 32 requests, V=128256 bf16, top 4, expand 4, 6 rounds, keep 60")
    rng = np.random.default_rng(1)
    state, outs, trees = _build(rng, 32, 128_256, "bf16", 4, 4, 6, 60, 85)
    _compare(state, outs, trees, 60)


@pytest.mark.parametrize("B,V,kind,top,exp,depth,N,max_cand", [
    (50, 37, "f32", 3, 2, 5, 20, 64), (7, 5001, "bf16", 16, 3, 4, 100, 200),
    (3, 70_001, "f32", 2, 8, 3, 10, 64), (300, 300, "bf16", 1, 1, 8, 9, 9)])
def test_gpu_tree_build_shapes(B, V, kind, top, exp, depth, N, max_cand):
    say(f"device tree builder B={B} V={V} {kind} top={top} expand={exp} rounds={depth} N={N}")
    rng = np.random.default_rng(V + B)
    state, outs, trees = _build(rng, B, V, kind, top, exp, depth, N, max_cand, special=True)
    _compare(state, outs, trees, N)


def test_gpu_tree_build_overflow_and_bad_nodes():
    say("device tree builder: candidate overflow and bad node ids")
    rng = np.random.default_rng(3)
    B, V = 4, 1000
    state = sv.DraftTreeState(B, 9)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    nxt = sv.sv_tree_expand(rows_to_dev(_draft_rows(rng, B, V, "f32"), "f32"), None, 4, 2, state, dev_status=st)
    assert state.count.cpu().tolist() == [5] * B and int(st.item()) == 0
    nxt[1, 0] = 17                       # no such candidate
    nxt2 = sv.sv_tree_expand(rows_to_dev(_draft_rows(rng, 2 * B, V, "f32"), "f32"), nxt, 4, 2, state,
                             dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == sv.FLAG_BAD_REQUEST
    # 5 + 2 * 4 = 13 > 9: nothing appended anywhere; request 1 named a missing node
    assert state.count.cpu().tolist() == [5] * B
    assert (nxt2.cpu().numpy() == -1).all()
    parent, token, depth, cand, mask = sv.sv_tree_finalize(state, 8)
    c = cand.cpu().numpy()
    assert (c[:, :5] >= 0).all() and (c[:, 5:] == -1).all()
    assert (mask.cpu().numpy()[:, 5:, :] == 0).all()


def test_gpu_tree_build_then_verify():
    """The built tree feeds the tree verify: the flat parent / token arrays and
    the rows of the kept nodes (draft rows = the rows each node was expanded
    with) give the oracle's verify result on the oracle-built tree."""
    say("device tree builder feeding the tree verify")
    rng = np.random.default_rng(4)
    B, V, top, exp, depth, N, kind = 16, 4096, 3, 3, 4, 24, "bf16"
    state = sv.DraftTreeState(B, 64)
    trees = [oracle.DraftTree() for _ in range(B)]
    fronts = [[0] for _ in range(B)]
    rows_of = [dict() for _ in range(B)]
    nxt = None
    for r in range(depth):
        n_exp = 1 if r == 0 else exp
        rows = _draft_rows(rng, B * n_exp, V, kind)
        nxt = sv.sv_tree_expand(rows_to_dev(rows, kind), nxt, top, exp, state)
        for b in range(B):
            for e, node in enumerate(fronts[b]):
                rows_of[b][node] = rows[b * n_exp + e]
            if fronts[b]:
                fronts[b] = trees[b].expand(fronts[b], [rows_of[b][n] for n in fronts[b]], kind, top, exp)
    parent, token, dep, cand, mask = sv.sv_tree_finalize(state, N)
    torch.cuda.synchronize()
    cand_np = cand.cpu().numpy()
    # rows per flat node: target = fresh logits, draft = the node's expansion row
    # (a node never expanded gets a uniform draft row; it has no children)
    tgt = synth.encode(rng.standard_normal((B * N, V)) * 2.0, kind)
    dft = np.zeros((B * N, V), dtype=np.uint16)
    uni = synth.encode(np.full(V, 1.0 / V), kind)
    for b in range(B):
        for f in range(N):
            dft[b * N + f] = rows_of[b].get(int(cand_np[b, f]), uni)
    u = synth.uniform_grid(rng, (B, N))
    tok_t, cnt_t, acc_t, pth_t, _ = sv.sv_verify_tree(rows_to_dev(tgt, kind), rows_to_dev(dft, kind), parent,
                                                      token, 1.0, f32(u))
    torch.cuda.synchronize()
    wp = np.stack([t.finalize(N)[0] for t in trees])
    wt = np.stack([t.finalize(N)[1] for t in trees])
    want = oracle.verify_tree(tgt, kind, dft, kind, V, wp, wt, 1.0, u, with_diag=False)
    got = dict(tokens=tok_t.cpu().numpy(), count=cnt_t.cpu().numpy(), accepted=acc_t.cpu().numpy(),
               path=pth_t.cpu().numpy())
    nb, bad = compare_tokens(got, want, keys=("tokens", "count", "accepted", "path"))
    assert bad.size == 0 and nb <= 2
