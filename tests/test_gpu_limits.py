"""The library at its documented limits and on empty batches, on an MI355X,
through the C ABI, against the float64 oracle: the largest vocabulary
(4,194,304 ids), the deepest chain (k_max = 255, sampled and greedy), the
largest tree (1024 nodes, all three walk variants), the most vocabulary
shards (64), the tree builder's largest candidate set and frontier (1024
candidates, 64 expanded nodes), the prompt-lookup drafter's largest draft
(k = 1024) over long unaligned contexts, and batches of zero requests."""
import numpy as np
import pytest
import torch

import draft_verify_sampling_amd as sv
import oracle
import synth
from tests.gpu_util import say, compare_tokens, close, rows_to_dev, i32, f32, DEV, run_sample, run_greedy

pytestmark = pytest.mark.gpu

MAX_V = 4_194_304


def _status():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def _or(flags):
    out = 0
    for f in np.asarray(flags).ravel():
        out |= int(f)
    return out


def _oracle_sample(ci, **kw):
    return oracle.verify_sample(ci.target, ci.t_kind, ci.draft, ci.q_kind, ci.V, ci.t_row_start,
                                ci.q_row_start, ci.draft_ids[:, :ci.k_max], ci.draft_len, ci.k_max,
                                ci.T, ci.uniforms, **kw)


def _check_sample(ci, got, want, status):
    nb, bad = compare_tokens(got, want)
    assert bad.size == 0, bad[:10]
    assert nb <= 1
    assert status == _or(want["flags"])
    same = (got["count"] == want["count"]) & (got["accepted"] == want["accepted"]) & (want["count"] > 0)
    assert close(got["resid"][same], want["resid"][same], rtol=1e-5, atol=1e-12).all()


def test_gpu_sample_largest_vocabulary():
    """V = 4,194,304 (2048 tiles, 512 statistics segments per row), bf16."""
    say("sampled chain at V = 4,194,304 bf16")
    ci = synth.sampled_chain(71, 3, np.array([2, 0, 1]), MAX_V, 0.9, sd=2.0, n_boost=3, boost=5.0, sigma=1.0,
                             kind="bf16")
    want = _oracle_sample(ci)
    for diag in (True, False):
        st = _status()
        got = run_sample(ci, status=st, diag=diag)
        _check_sample(ci, got, want, int(st.item()))
    say(f"  accepted {want['accepted'].tolist()}")


def test_gpu_greedy_largest_vocabulary():
    say("greedy chain at V = 4,194,304 f32")
    rng = np.random.default_rng(72)
    B, k = 2, 2
    rows = rng.standard_normal((B * (k + 1), MAX_V)).astype(np.float32)
    rows[1, 17] = rows[1].max()  # a tie for the argmax: the lower id wins
    am = np.argmax(rows, axis=1)
    ids = np.array([[am[0], am[1]], [am[3], (am[4] + 1) % MAX_V]], dtype=np.int32)
    ts = np.array([0, k + 1], dtype=np.int32)
    lens = np.array([k, k], dtype=np.int32)
    st = _status()
    got = run_greedy(rows, "f32", ts, ids, lens, status=st)
    want = oracle.verify_greedy(rows, "f32", MAX_V, ts, ids, lens, k)
    for key in ("tokens", "count", "accepted"):
        assert np.array_equal(got[key], want[key]), key
    assert int(st.item()) == _or(want["flags"])


def test_gpu_sample_deepest_chain():
    """k_max = 255: request 0 keeps every draft (u = 0) and draws the bonus
    token from row 255; request 1 stops early; request 2 has no drafts."""
    say("sampled chain with k_max = 255")
    V = 3000
    ci = synth.sampled_chain(73, 3, np.array([255, 255, 0]), V, 1.0, sd=2.0, n_boost=3, boost=4.0, sigma=1.0,
                             kind="f32")
    ci.uniforms[0, :255] = 0.0
    want = _oracle_sample(ci)
    assert want["accepted"][0] == 255 and want["count"][0] == 256
    for diag in (True, False):
        st = _status()
        got = run_sample(ci, status=st, diag=diag)
        _check_sample(ci, got, want, int(st.item()))


def _tree_inputs(rng, B, N, V, kind):
    target = rng.standard_normal((B * N, V)) * 2.0
    for r in range(B * N):
        target[r, rng.choice(V, size=3, replace=False)] += 5.0
    target = synth.encode(target, kind)
    l = rng.standard_normal((B * N, V)) * 2.0
    q = np.exp(l - l.max(axis=1, keepdims=True))
    q /= q.sum(axis=1, keepdims=True)
    draft = synth.encode(q, kind)
    parent = np.zeros((B, N), dtype=np.int32)
    token = np.full((B, N), -1, dtype=np.int32)
    for b in range(B):
        parent[b, 0] = -1
        for c in range(1, N):
            # deep, bushy trees: most nodes hang under one of the last few
            p = int(rng.integers(max(0, c - 8), c))
            parent[b, c] = p
            row = synth.decode(target[b * N + p], kind)
            token[b, c] = int(np.argmax(row)) if rng.random() < 0.6 else int(rng.integers(0, V))
    return target, draft, parent, token


def test_gpu_tree_largest():
    """1024 nodes per request: the sampled tree walk, the greedy tree and the
    point-mass tree."""
    say("tree verify with 1024 nodes")
    rng = np.random.default_rng(74)
    B, N, V, kind, T = 2, 1024, 2500, "bf16", 1.0
    target, draft, parent, token = _tree_inputs(rng, B, N, V, kind)
    u = rng.random((B, N)).astype(np.float32)
    u[0, :N - 1] *= 0.05  # request 0 keeps most candidates it tries
    tgt, dft = rows_to_dev(target, kind), rows_to_dev(draft, kind)

    st = _status()
    tok, cnt, acc, pth, _ = sv.sv_verify_tree(tgt, dft, i32(parent), i32(token), T, f32(u), dev_status=st)
    torch.cuda.synchronize()
    got = dict(tokens=tok.cpu().numpy(), count=cnt.cpu().numpy(), accepted=acc.cpu().numpy(), path=pth.cpu().numpy())
    want = oracle.verify_tree(target, kind, draft, kind, V, parent, token, T, u, with_diag=False)
    nb, bad = compare_tokens(got, want)
    assert bad.size == 0 and nb <= 1
    if nb == 0:
        assert np.array_equal(got["path"], want["path"])
    assert int(st.item()) == _or(want["flags"])
    say(f"  sampled: accepted {want['accepted'].tolist()}")

    st = _status()
    tok, cnt, acc, pth = sv.sv_verify_tree_greedy(tgt, i32(parent), i32(token), dev_status=st)
    torch.cuda.synchronize()
    want = oracle.verify_tree_greedy(target, kind, V, parent, token)
    assert np.array_equal(tok.cpu().numpy(), want["tokens"]) and np.array_equal(pth.cpu().numpy(), want["path"])
    assert np.array_equal(cnt.cpu().numpy(), want["count"]) and np.array_equal(acc.cpu().numpy(), want["accepted"])
    assert int(st.item()) == _or(want["flags"])
    say(f"  greedy: accepted {want['accepted'].tolist()}")

    st = _status()
    tok, cnt, acc, pth = sv.sv_verify_tree_pointmass(tgt, i32(parent), i32(token), T, f32(u), dev_status=st)
    torch.cuda.synchronize()
    got = dict(tokens=tok.cpu().numpy(), count=cnt.cpu().numpy(), accepted=acc.cpu().numpy(), path=pth.cpu().numpy())
    want = oracle.verify_tree_pointmass(target, kind, V, parent, token, T, u)
    nb, bad = compare_tokens(got, want)
    assert bad.size == 0 and nb <= 1
    assert int(st.item()) == _or(want["flags"])
    say(f"  point mass: accepted {want['accepted'].tolist()}")


def test_gpu_shards_most():
    """64 shards of uneven widths (the most the shard descriptor holds)."""
    from tests.test_gpu_shards import run_sharded, _check
    say("vocabulary-sharded verify over 64 shards")
    V = 64 * 97 + 13
    rng = np.random.default_rng(75)
    cuts = np.sort(rng.choice(np.arange(1, V), size=63, replace=False))
    bounds = [0] + [int(c) for c in cuts] + [V]
    ci = synth.sampled_chain(76, 9, rng.integers(0, 5, size=9), V, 0.8, sd=2.0, n_boost=3, boost=4.0,
                             sigma=1.0, kind="bf16")
    got, status = run_sharded(ci, bounds)
    _check("64 shards", ci, got, status)


def test_gpu_tree_build_largest():
    """1024 candidates per request, 64 nodes expanded in a round, and the
    finalize at 1024 nodes."""
    from tests.test_gpu_tree_build import _build, _compare
    say("device tree builder: 1024 candidates, frontier of 64, 1024 flat nodes")
    rng = np.random.default_rng(77)
    # 1 + 11 + 11 * 11 + 64 * 11 = 837 candidates after three rounds
    state, outs, trees = _build(rng, 2, 3000, "bf16", 11, 64, 3, 1024, 1024)
    _compare(state, outs, trees, 1024)
    assert int(state.count.cpu().numpy()[0]) == 837


def test_gpu_empty_batches():
    """Zero requests: every entry point returns without launching anything."""
    say("empty batches")
    z2 = lambda *s: torch.zeros(s, dtype=torch.int32, device=DEV)
    rows = torch.zeros((0, 100), dtype=torch.float32, device=DEV)
    st = _status()
    tok, cnt, acc, _, _ = sv.sv_verify_sample(rows, rows, z2(0), z2(0), z2(0, 3), z2(0), 1.0,
                                              torch.zeros((0, 4), dtype=torch.float32, device=DEV),
                                              diag=False, dev_status=st)
    assert tok.shape == (0, 4) and cnt.shape == (0,) and acc.shape == (0,)
    tok, cnt, acc, _, _ = sv.sv_verify_sample_philox(rows, rows, z2(0), z2(0), z2(0, 3), z2(0), 1.0, 5, 0,
                                                     diag=False, dev_status=st)
    assert tok.shape == (0, 4)
    tok, cnt, acc = sv.sv_verify_greedy(rows, z2(0), z2(0, 3), z2(0), dev_status=st)
    assert tok.shape == (0, 4)
    tok, cnt, acc, pth, _ = sv.sv_verify_tree(rows, rows, z2(0, 5), z2(0, 5), 1.0,
                                              torch.zeros((0, 5), dtype=torch.float32, device=DEV),
                                              diag=False, dev_status=st)
    assert tok.shape == (0, 5) and pth.shape == (0, 5)
    ids, lens = sv.sv_ngram_draft(z2(0, 8), z2(0), 2, 3, dev_status=st)
    assert ids.shape == (0, 3) and lens.shape == (0,)
    u = sv.sv_philox_uniforms(1, 2, 0, 5)
    assert u.shape == (0, 5)
    torch.cuda.synchronize()
    assert int(st.item()) == 0


def test_gpu_greedy_deepest_chain():
    """k_max = 255 in the greedy verify (one block per request, thread i
    holding row i): a full match, a mismatch at draft 200, an EOS kept at
    draft 100 (the round ends after it) and a budget cut, over rows of small
    integers (ties for the maximum are common; the lowest id wins)."""
    say("greedy chain with k_max = 255")
    rng = np.random.default_rng(78)
    B, k, V = 4, 255, 1000
    eos = V - 1
    rows = rng.integers(-40, 40, size=(B * (k + 1), V)).astype(np.float32)
    rows[:, eos] = -1000.0                    # no row picks the EOS id ...
    rows[2 * (k + 1) + 100, eos] = 1000.0     # ... except request 2's row 100
    am = np.argmax(rows, axis=1).reshape(B, k + 1)
    ids = am[:, :k].astype(np.int32).copy()
    ids[1, 200] = (ids[1, 200] + 1) % (V - 1)
    ts = np.arange(B, dtype=np.int32) * (k + 1)
    lens = np.full(B, k, dtype=np.int32)
    max_new = np.array([300, 300, 300, 57], dtype=np.int32)
    st = _status()
    got = run_greedy(rows, "f32", ts, ids, lens, max_new=max_new, eos_id=eos, status=st)
    want = oracle.verify_greedy(rows, "f32", V, ts, ids, lens, k, max_new=max_new, eos_id=eos)
    for key in ("tokens", "count", "accepted"):
        assert np.array_equal(got[key], want[key]), key
    assert int(st.item()) == _or(want["flags"])
    assert list(want["accepted"]) == [255, 200, 255, 255]
    assert list(want["count"]) == [256, 201, 101, 57]


def test_gpu_ngram_long_unaligned_contexts():
    """Contexts of up to 10,003 tokens in rows of an odd stride (no row is
    16-byte aligned), so the newest-first search crosses several 4,096-start
    chunks; repeats planted at distances from 10 to 9,000 tokens and contexts
    without any repeat; k up to 1,024 (the proposal may run to the context's
    end)."""
    say("prompt lookup over 10,003-token unaligned contexts")
    rng = np.random.default_rng(79)
    B, stride = 24, 10_003
    ctx = rng.integers(0, 1 << 30, size=(B, stride)).astype(np.int32)  # (almost) no chance repeats
    lens = rng.integers(stride - 50, stride + 1, size=B).astype(np.int32)
    lens[0] = 3
    lens[1] = 4100
    for b in range(2, B):
        n = int(lens[b])
        if b % 6 == 5:
            continue  # no repeat: every chunk is searched
        dist = [10, 900, 4100, 6000, 9000][b % 5] + int(rng.integers(0, 7))
        w = 8
        src = n - w
        dst = max(0, src - dist)
        ctx[b, dst:dst + w] = ctx[b, src:src + w]
    st = _status()
    for w, k in ((1, 1), (3, 7), (8, 1024), (64, 300)):
        got_ids, got_lens = sv.sv_ngram_draft(i32(ctx), i32(lens), w, k, dev_status=st)
        torch.cuda.synchronize()
        wi, wl, wf = oracle.ngram_draft(ctx, lens, w, k)
        assert np.array_equal(got_lens.cpu().numpy(), wl), (w, k)
        assert np.array_equal(got_ids.cpu().numpy(), wi), (w, k)
    assert int(st.item()) == 0
