"""The tree walks' exchange words, on an MI355X, through the C ABI.

A tree walk's workgroups zero their own exchange words at the start of a
call and certify that with a ticket unique to the call; the first exchange
reads no word before every ticket of the request is there.  These tests give
the walks workspaces whose every byte is 0xFF (every exchange word looks
written, every ticket is wrong) and require the outputs of a fresh workspace
and of the float64 oracle; they replay a captured tree walk (under capture
the words are zeroed by a kernel instead) with eager tree walks on the same
workspace in between; and they run the walks on one workspace with the shape
changing from call to call."""
import numpy as np
import pytest
import torch

import draft_verify_sampling_amd as sv
import oracle
import synth
from tests.gpu_util import say, compare_tokens, rows_to_dev, i32, f32, DEV

pytestmark = pytest.mark.gpu

KIND = "bf16"
T = 0.9


def _inputs(seed, B=8, N=24, V=20_000):
    """Trees whose children carry, with probability 0.6, their parent row's
    argmax (often kept), else a random id; a draft close to the target."""
    rng = np.random.default_rng(seed)
    l = rng.standard_normal((B * N, V)) * 2.5
    for r in range(B * N):
        l[r, rng.choice(V, size=3, replace=False)] += 5.0
    q = np.exp((l + rng.standard_normal(l.shape)) / T)
    q /= q.sum(axis=1, keepdims=True)
    target, draft = synth.encode(l, KIND), synth.encode(q, KIND)
    parent = np.zeros((B, N), dtype=np.int32)
    token = np.full((B, N), -1, dtype=np.int32)
    for b in range(B):
        parent[b, 0] = -1
        for c in range(1, N):
            p = int(rng.integers(max(0, c - 6), c))
            parent[b, c] = p
            row = synth.decode(target[b * N + p], KIND)
            token[b, c] = int(np.argmax(row)) if rng.random() < 0.6 else int(rng.integers(0, V))
    u = rng.random((B, N)).astype(np.float32)
    return target, draft, parent, token, u


def _np(ts):
    return [t.cpu().numpy() for t in ts]


def _poisoned(B, N, V):
    ws = sv.Workspace()
    n = sv.workspace_bytes(sv.SV_OP_TREE, B, B * N, V)
    ws.buf = torch.full((max(n, 256),), 255, dtype=torch.uint8, device=DEV)
    return ws


def _flags(want):
    out = 0
    for f in np.asarray(want["flags"]).ravel():
        out |= int(f)
    return out


def test_gpu_tree_walks_ignore_words_left_in_the_workspace():
    say("tree walks on workspaces filled with 0xFF")
    target, draft, parent, token, u = _inputs(91)
    B, N = parent.shape
    V = target.shape[1]
    tgt, dft = rows_to_dev(target, KIND), rows_to_dev(draft, KIND)
    par, tok = i32(parent), i32(token)

    fresh = _np(sv.sv_verify_tree(tgt, dft, par, tok, T, f32(u))[:4])
    want = oracle.verify_tree(target, KIND, draft, KIND, V, parent, token, T, u, with_diag=False)
    nb, bad = compare_tokens(dict(tokens=fresh[0], count=fresh[1], accepted=fresh[2], path=fresh[3]), want)
    assert bad.size == 0 and nb <= 1
    for rep in range(3):
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        got = _np(sv.sv_verify_tree(tgt, dft, par, tok, T, f32(u), dev_status=st, workspace=_poisoned(B, N, V))[:4])
        torch.cuda.synchronize()
        for g, f in zip(got, fresh):
            assert np.array_equal(g, f), rep
        assert int(st.item()) == _flags(want)

    g_fresh = _np(sv.sv_verify_tree_greedy(tgt, par, tok))
    g_want = oracle.verify_tree_greedy(target, KIND, V, parent, token)
    assert np.array_equal(g_fresh[0], g_want["tokens"]) and np.array_equal(g_fresh[3], g_want["path"])
    p_fresh = _np(sv.sv_verify_tree_pointmass(tgt, par, tok, T, f32(u)))
    for rep in range(2):
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        got = _np(sv.sv_verify_tree_greedy(tgt, par, tok, dev_status=st, workspace=_poisoned(B, N, V)))
        for g, f in zip(got, g_fresh):
            assert np.array_equal(g, f), rep
        got = _np(sv.sv_verify_tree_pointmass(tgt, par, tok, T, f32(u), dev_status=st, workspace=_poisoned(B, N, V)))
        for g, f in zip(got, p_fresh):
            assert np.array_equal(g, f), rep
        torch.cuda.synchronize()
        assert int(st.item()) & 64 == 0  # no sync timeout


def test_gpu_tree_walk_graph_replay():
    """A captured sv_verify_tree replayed four times, with eager tree walks of
    another tree on the same workspace between the replays, and the workspace
    refilled with 0xFF before some of them; every replay equals the eager
    result."""
    say("graph capture and replay of sv_verify_tree")
    a = _inputs(92)
    b = _inputs(93)
    B, N = a[2].shape
    V = a[0].shape[1]
    args = [rows_to_dev(a[0], KIND), rows_to_dev(a[1], KIND), i32(a[2]), i32(a[3])]
    ua = f32(a[4])
    want = [t.clone() for t in sv.sv_verify_tree(*args, T, ua)[:4]]
    torch.cuda.synchronize()
    oargs = [rows_to_dev(b[0], KIND), rows_to_dev(b[1], KIND), i32(b[2]), i32(b[3])]
    ub = f32(b[4])
    ws = _poisoned(B, N, V)
    out = tuple(torch.empty_like(t) for t in want) + (None,)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sv.sv_verify_tree(*args, T, ua, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sv.sv_verify_tree(*args, T, ua, workspace=ws, out=out)
    for rep in range(4):
        for t in out[:4]:
            t.fill_(-7)
        if rep % 2 == 1:
            ws.buf.fill_(255)
        g.replay()
        torch.cuda.synchronize()
        for got, w in zip(out[:4], want):
            assert torch.equal(got, w), rep
        sv.sv_verify_tree(*oargs, T, ub, workspace=ws)   # eager work on the same words in between
        torch.cuda.synchronize()


def test_gpu_tree_walks_changing_shapes_one_workspace():
    """36 calls of the three tree walks on one workspace, each with another
    shape (B, N, V, dtypes, T), so the split into workgroups, the number of
    exchanges and the workspace layout change from call to call and every
    call finds the previous call's words and tickets at other places."""
    say("tree walks with changing shapes on one workspace")
    rng = np.random.default_rng(94)
    ws = sv.Workspace()
    for case in range(36):
        B = int(rng.choice([1, 3, 8, 17]))
        N = int(rng.choice([2, 5, 24, 60]))
        V = int(rng.choice([2049, 5000, 20000, 70000]))
        tk, qk = str(rng.choice(["bf16", "f32"])), str(rng.choice(["bf16", "f32"]))
        T = float(rng.choice([0.5, 1.0, 1.7]))
        N = min(N, max(2, 12_000_000 // (B * V)))
        l = rng.standard_normal((B * N, V)) * 2.5
        for r in range(B * N):
            l[r, rng.choice(V, size=3, replace=False)] += 5.0
        q = np.exp((l + rng.standard_normal(l.shape)) / T)
        q /= q.sum(axis=1, keepdims=True)
        target, draft = synth.encode(l, tk), synth.encode(q, qk)
        parent = np.zeros((B, N), dtype=np.int32)
        token = np.full((B, N), -1, dtype=np.int32)
        for b in range(B):
            parent[b, 0] = -1
            for c in range(1, N):
                p = int(rng.integers(max(0, c - 6), c))
                parent[b, c] = p
                row = synth.decode(target[b * N + p], tk)
                token[b, c] = int(np.argmax(row)) if rng.random() < 0.5 else int(rng.integers(0, V))
        u = rng.random((B, N)).astype(np.float32)
        tgt, dft, par, tok = rows_to_dev(target, tk), rows_to_dev(draft, qk), i32(parent), i32(token)
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        mode = case % 3
        if mode == 0:
            o = _np(sv.sv_verify_tree(tgt, dft, par, tok, T, f32(u), dev_status=st, workspace=ws)[:4])
            want = oracle.verify_tree(target, tk, draft, qk, V, parent, token, T, u, with_diag=False)
            nb, bad = compare_tokens(dict(tokens=o[0], count=o[1], accepted=o[2], path=o[3]), want)
            assert bad.size == 0 and nb <= 1, (case, B, N, V, tk, qk, T)
        elif mode == 1:
            o = _np(sv.sv_verify_tree_greedy(tgt, par, tok, dev_status=st, workspace=ws))
            want = oracle.verify_tree_greedy(target, tk, V, parent, token)
            assert np.array_equal(o[0], want["tokens"]) and np.array_equal(o[3], want["path"]), case
        else:
            o = _np(sv.sv_verify_tree_pointmass(tgt, par, tok, T, f32(u), dev_status=st, workspace=ws))
            want = oracle.verify_tree_pointmass(target, tk, V, parent, token, T, u)
            nb, bad = compare_tokens(dict(tokens=o[0], count=o[1], accepted=o[2]), want)
            assert bad.size == 0 and nb <= 1, (case, B, N, V, tk, qk, T)
        torch.cuda.synchronize()
        assert int(st.item()) & 64 == 0, case  # no exchange timed out
