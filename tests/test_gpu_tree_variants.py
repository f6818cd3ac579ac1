"""Parity of the greedy and point-mass tree verifies with the float64 oracle,
on an MI355X, through the C ABI.

Greedy: bit-exact (tokens, counts, paths, status bits).  Point mass: token
ids, counts and paths equal except in requests where a uniform lies within
1e-6 of its decision edge (counted, and required to be rare).
"""
import numpy as np
import pytest
import torch

import draft_verify_sampling_amd as sv
import oracle
import synth
from tests.gpu_util import say, compare_tokens, rows_to_dev, i32, f32, DEV

pytestmark = pytest.mark.gpu


def _status():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def _or(flags):
    out = 0
    for f in np.asarray(flags).ravel():
        out |= int(f)
    return out


def _np(t):
    return t.cpu().numpy()


def run_greedy_tree(target, kind, parent, token, status=None):
    tok, cnt, acc, pth = sv.sv_verify_tree_greedy(rows_to_dev(target, kind), i32(parent), i32(token),
                                                  dev_status=status)
    torch.cuda.synchronize()
    return dict(tokens=_np(tok), count=_np(cnt), accepted=_np(acc), path=_np(pth))


def run_point_tree(target, kind, parent, token, T, u, status=None):
    tok, cnt, acc, pth = sv.sv_verify_tree_pointmass(rows_to_dev(target, kind), i32(parent), i32(token), T,
                                                     f32(u), dev_status=status)
    torch.cuda.synchronize()
    return dict(tokens=_np(tok), count=_np(cnt), accepted=_np(acc), path=_np(pth))


def _random_trees(rng, B, N, V, target, kind, dup=0.25, hit=0.5):
    """Random shapes; a child's token is, with probability `hit`, one of the
    three largest entries of its parent's target row (often kept), else a
    random id; with probability `dup` it repeats an earlier sibling's token."""
    parent = np.zeros((B, N), dtype=np.int32)
    token = np.full((B, N), -1, dtype=np.int32)
    for b in range(B):
        parent[b, 0] = -1
        for c in range(1, N):
            parent[b, c] = int(rng.integers(0, c))
            p = int(parent[b, c])
            sib = [int(token[b, d]) for d in range(1, c) if parent[b, d] == p]
            if sib and rng.random() < dup:
                token[b, c] = sib[int(rng.integers(0, len(sib)))]
            elif rng.random() < hit:
                row = synth.decode(target[b * N + p], kind)
                top = np.argsort(-row, kind="stable")[:3]
                token[b, c] = int(top[int(rng.integers(0, 3))])
            else:
                token[b, c] = int(rng.integers(0, V))
    return parent, token


def _rows(rng, n, V, kind, sd=2.5):
    l = rng.standard_normal((n, V)) * sd
    for r in range(n):
        l[r, rng.choice(V, size=3, replace=False)] += 5.0
    return synth.encode(l, kind)


# ---------------------------------------------------------------------------
# greedy tree
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def c5():
    return synth.c5_tree()


def test_gpu_tree_greedy_c5(c5):
    say("greedy tree B=32 N=60 V=128256 bf16")
    st = _status()
    got = run_greedy_tree(c5.target, c5.t_kind, c5.parent, c5.token, status=st)
    want = oracle.verify_tree_greedy(c5.target, c5.t_kind, c5.V, c5.parent, c5.token)
    say(f"greedy c5: mean kept {want['accepted'].mean():.2f}")
    for key in ("tokens", "count", "accepted", "path"):
        assert np.array_equal(got[key], want[key]), key
    assert int(st.item()) == _or(want["flags"])


@pytest.mark.parametrize("kind,V,N,B", [("bf16", 5000, 24, 30), ("f32", 70_001, 12, 3), ("bf16", 7, 9, 40),
                                        ("bf16", 70_000, 16, 1), ("f32", 2049, 30, 300)])
def test_gpu_tree_greedy_random(kind, V, N, B):
    say(f"greedy tree random kind={kind} V={V} N={N} B={B}")
    rng = np.random.default_rng(V + N + B)
    target = _rows(rng, B * N, V, kind)
    if V > 100:  # exact ties between the largest values, lowest id must win
        for r in range(0, B * N, 3):
            row = synth.decode(target[r], kind)
            m = int(np.argmax(row))
            target[r, (m + 7) % V] = target[r, m]
    parent, token = _random_trees(rng, B, N, V, target, kind, hit=0.7)
    st = _status()
    got = run_greedy_tree(target, kind, parent, token, status=st)
    want = oracle.verify_tree_greedy(target, kind, V, parent, token)
    for key in ("tokens", "count", "accepted", "path"):
        assert np.array_equal(got[key], want[key]), key
    assert int(st.item()) == _or(want["flags"])
    assert want["accepted"].max() >= 1


def test_gpu_tree_greedy_edge_cases():
    say("greedy tree: NaN in visited / unvisited rows, signed zeros, -inf rows, bad trees")
    V, N, B = 3000, 6, 8
    kind = "f32"
    target = np.zeros((B * N, V), dtype=np.float32)
    parent = np.tile(np.array([-1, 0, 0, 1, 1, 2], dtype=np.int32), (B, 1))
    token = np.tile(np.array([-1, 10, 20, 30, 40, 50], dtype=np.int32), (B, 1))
    for b in range(B):
        target[b * N + 0, 20] = 1.0                 # root picks 20 -> node 2
        target[b * N + 2, 50] = 1.0                 # node 2 picks 50 -> node 5 (a leaf)
        target[b * N + 5, 2999] = 3.0               # leaf row: extra token 2999
    target[0 * N + 1, :] = np.nan                   # unvisited row: no effect
    target[1 * N + 2, 5] = np.nan                   # visited row: invalid
    target[2 * N + 5, :] = -np.inf                  # all -inf: argmax 0
    target[3 * N + 5, :] = -0.0                     # all equal (signed zeros): id 0
    target[3 * N + 5, 100] = 0.0
    parent[4, 3] = 3                                # bad tree (parent not earlier)
    token[5, 4] = V                                 # bad token
    target[6 * N + 0, :] = np.float32(-1.0)         # root ties everywhere: id 0, no child
    st = _status()
    got = run_greedy_tree(target, kind, parent, token, status=st)
    want = oracle.verify_tree_greedy(target, kind, V, parent, token)
    for key in ("tokens", "count", "accepted", "path"):
        assert np.array_equal(got[key], want[key]), key
    assert list(want["count"]) == [3, 0, 3, 3, 0, 0, 1, 3]
    assert int(st.item()) == _or(want["flags"])


# ---------------------------------------------------------------------------
# point-mass tree
# ---------------------------------------------------------------------------
def _check_point(name, got, want, B, frac=1e-3):
    nb, bad = compare_tokens(got, want, keys=("tokens", "count", "accepted", "path"))
    say(f"{name}: {B} requests, {nb} boundary cases, mean kept {want['accepted'].mean():.2f}")
    assert bad.size == 0, f"{name}: mismatching requests {bad[:10]}"
    assert nb <= max(2, frac * B)


def test_gpu_tree_pointmass_c5(c5):
    say("point-mass tree B=32 N=60 V=128256 bf16 T=1")
    st = _status()
    got = run_point_tree(c5.target, c5.t_kind, c5.parent, c5.token, c5.T, c5.uniforms, status=st)
    want = oracle.verify_tree_pointmass(c5.target, c5.t_kind, c5.V, c5.parent, c5.token, c5.T, c5.uniforms)
    _check_point("pointmass c5", got, want, c5.B)
    assert int(st.item()) == _or(want["flags"])
    again = run_point_tree(c5.target, c5.t_kind, c5.parent, c5.token, c5.T, c5.uniforms)
    for key in ("tokens", "count", "accepted", "path"):
        assert np.array_equal(got[key], again[key]), key


@pytest.mark.parametrize("kind,V,N,B,T", [("bf16", 5000, 24, 40, 1.0), ("f32", 70_001, 12, 3, 0.8),
                                          ("bf16", 9, 9, 60, 1.3), ("bf16", 70_000, 16, 1, 0.7),
                                          ("f32", 2049, 30, 300, 1.0)])
def test_gpu_tree_pointmass_random(kind, V, N, B, T):
    say(f"point-mass tree random kind={kind} V={V} N={N} B={B} T={T}")
    rng = np.random.default_rng(10 * V + N + B)
    target = _rows(rng, B * N, V, kind, sd=1.0 if V < 100 else 2.5)
    parent, token = _random_trees(rng, B, N, V, target, kind)
    u = synth.uniform_grid(rng, (B, N))
    st = _status()
    got = run_point_tree(target, kind, parent, token, T, u, status=st)
    want = oracle.verify_tree_pointmass(target, kind, V, parent, token, T, u)
    _check_point(f"pointmass {kind}/{V}/{N}/{B}", got, want, B, frac=0.02)
    assert int(st.item()) == _or(want["flags"])


def test_gpu_tree_pointmass_many_rejections_one_node():
    """A root with 40 candidates (repeats included) that are mostly rejected:
    the distribution loses one id after another; the last draw must skip all
    of them."""
    say("point-mass tree: 40 siblings under the root")
    rng = np.random.default_rng(5)
    V, N, B, kind = 20_000, 41, 16, "bf16"
    target = _rows(rng, B * N, V, kind, sd=1.0)
    for b in range(B):  # mass concentrated on a few ids the candidates cover
        row = synth.decode(target[b * N], kind)
        hot = rng.choice(V, size=12, replace=False)
        row[hot] += 9.0
        target[b * N] = synth.encode(row, kind)
    parent = np.zeros((B, N), dtype=np.int32)
    parent[:, 0] = -1
    token = np.full((B, N), -1, dtype=np.int32)
    for b in range(B):
        row = synth.decode(target[b * N], kind)
        top = np.argsort(-row, kind="stable")[:30]
        token[b, 1:] = rng.choice(top, size=N - 1)
    u = synth.uniform_grid(rng, (B, N))
    u[:, :N - 1] = np.maximum(u[:, :N - 1], 0.97)  # reject nearly everything
    st = _status()
    got = run_point_tree(target, kind, parent, token, 1.0, u, status=st)
    want = oracle.verify_tree_pointmass(target, kind, V, parent, token, 1.0, u)
    _check_point("pointmass 40 siblings", got, want, B, frac=0.1)
    assert int(st.item()) == _or(want["flags"])
    drawn = want["accepted"] == 0
    assert drawn.sum() >= 4
    for b in np.nonzero(drawn)[0]:
        assert want["tokens"][b, 0] not in set(token[b, 1:])


def test_gpu_tree_pointmass_nonfinite_rows():
    say("point-mass tree: non-finite rows visited / not visited")
    rng = np.random.default_rng(6)
    V, N, B, kind = 4099, 7, 12, "f32"
    target = _rows(rng, B * N, V, kind)
    parent, token = _random_trees(rng, B, N, V, target, kind, dup=0.0, hit=0.0)
    u = synth.uniform_grid(rng, (B, N))
    u[:, :N - 1] = 0.999                     # nothing kept: only the root row is read
    target[0 * N + 0, 11] = np.nan           # root row (read)
    target[1 * N + 3, :] = np.nan            # never read
    target[2 * N + 0, 7] = np.inf            # root row: S = inf
    st = _status()
    got = run_point_tree(target, kind, parent, token, 1.0, u, status=st)
    with np.errstate(invalid="ignore", over="ignore"):
        want = oracle.verify_tree_pointmass(target, kind, V, parent, token, 1.0, u)
    _check_point("pointmass nonfinite", got, want, B)
    assert list(want["count"][:3]) == [0, 1, 0]
    assert int(st.item()) == _or(want["flags"])
