"""A seeded random sweep of the verify entry points against the float64 oracle,
on an MI355X, through the C ABI: vocabulary sizes around the tile and segment
edges, both dtypes and their mixes, temperatures, ragged draft counts, row
starts in any order with gaps and rows shared between requests, EOS and
budgets, host or device uniforms, with and without diagnostics; greedy chains
with ties; trees of random shape in all three walk variants.  Token ids must
equal the oracle's except in requests where a uniform lies within 1e-6 of its
decision edge, which must be rare."""
import numpy as np
import pytest
import torch

import draft_verify_sampling_amd as sv
import oracle
import synth
from tests.gpu_util import say, compare_tokens, close, rows_to_dev, i32, f32, DEV, run_sample, run_greedy

pytestmark = pytest.mark.gpu

VOCABS = [1, 5, 63, 2047, 2048, 2049, 3001, 8191, 8192, 8193, 16385, 40000, 70001]


def _status():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def _or(flags):
    out = 0
    for f in np.asarray(flags).ravel():
        out |= int(f)
    return out


def _relayout(ci, rng, gaps, share):
    """Row blocks of the requests in a random order with random filler rows
    between them; with `share`, some requests reuse an earlier request's
    rows, drafts and draft count."""
    B, V = ci.B, ci.V
    if gaps:
        _gaps(ci, rng)
    if share:
        for b in range(1, B):
            if rng.random() < 0.2:
                a = int(rng.integers(0, b))
                ci.t_row_start[b], ci.q_row_start[b] = ci.t_row_start[a], ci.q_row_start[a]
                ci.draft_len[b] = ci.draft_len[a]
                ci.draft_ids[b] = ci.draft_ids[a]
    return ci


def _gaps(ci, rng):
    B, V = ci.B, ci.V
    filler = lambda n, kind: synth.encode(rng.standard_normal((n, V)) * 2.0, kind)
    t_blocks, q_blocks = [], []
    t_new, q_new = np.zeros(B, np.int32), np.zeros(B, np.int32)
    t_at = q_at = 0
    for b in rng.permutation(B):
        k = int(ci.draft_len[b])
        g = int(rng.integers(0, 3))
        if g:
            t_blocks.append(filler(g, ci.t_kind))
            q_blocks.append(filler(g, ci.q_kind))
            t_at += g
            q_at += g
        t_blocks.append(ci.target[ci.t_row_start[b]:ci.t_row_start[b] + k + 1])
        q_blocks.append(ci.draft[ci.q_row_start[b]:ci.q_row_start[b] + max(k, 0)])
        t_new[b], q_new[b] = t_at, q_at
        t_at += k + 1
        q_at += k
    ci.target = np.ascontiguousarray(np.concatenate(t_blocks))
    ci.draft = np.ascontiguousarray(np.concatenate(q_blocks)) if q_at else ci.draft[:1]
    ci.t_row_start, ci.q_row_start = t_new, q_new


@pytest.mark.parametrize("seed", range(36))
def test_gpu_random_sampled_chain(seed):
    rng = np.random.default_rng(5000 + seed)
    V = int(rng.choice(VOCABS))
    B = int(rng.integers(1, 90))
    k_max = int(rng.integers(0, 9))
    ks = rng.integers(0, k_max + 1, size=B)
    ks[int(rng.integers(0, B))] = k_max
    tk, qk = (str(x) for x in rng.choice(["f32", "bf16"], size=2))
    T = float(rng.uniform(0.3, 2.0))
    ci = synth.sampled_chain(6000 + seed, B, ks, V, T, sd=float(rng.uniform(0.5, 4.0)), n_boost=min(3, V),
                             boost=float(rng.uniform(0.0, 6.0)), sigma=float(rng.uniform(0.05, 2.0)), kind=tk)
    if qk != tk:  # (a batch without drafts has one unused, unset draft row)
        with np.errstate(invalid="ignore"):
            ci.draft = synth.encode(synth.decode(ci.draft, tk), qk)
        ci.q_kind = qk
    gaps, share = rng.random() < 0.4, rng.random() < 0.25
    ci = _relayout(ci, rng, gaps, share)
    if rng.random() < 0.3:  # uniforms at the ends of the grid
        mask = rng.random(ci.uniforms.shape) < 0.2
        ci.uniforms[mask] = rng.choice([0.0, 1.0 - 2.0 ** -24], size=int(mask.sum())).astype(np.float32)
    kw = {}
    if rng.random() < 0.4:
        kw["max_new"] = rng.integers(0, k_max + 3, size=B).astype(np.int32)
    if rng.random() < 0.4 and B > 0 and k_max > 0:
        kw["eos_id"] = int(ci.draft_ids[int(rng.integers(0, B)), 0])
    philox = rng.random() < 0.3
    diag = bool(rng.random() < 0.5)
    say(f"seed {seed}: B={B} k_max={k_max} V={V} {tk}/{qk} T={T:.2f} gaps={gaps} share={share} "
        f"philox={philox} diag={diag} {sorted(kw)}")
    st = _status()
    if philox:
        seed_, off = int(rng.integers(0, 2 ** 62)), int(rng.integers(0, 2 ** 40))
        ci.uniforms = oracle.philox_uniforms(seed_, off, B, k_max + 1)
        mn = i32(kw["max_new"]) if "max_new" in kw else None
        tok, cnt, acc, dg, rs = sv.sv_verify_sample_philox(
            rows_to_dev(ci.target, ci.t_kind), rows_to_dev(ci.draft, ci.q_kind), i32(ci.t_row_start),
            i32(ci.q_row_start), i32(ci.draft_ids[:, :k_max]), i32(ci.draft_len), T, seed_, off, max_new=mn,
            eos_id=kw.get("eos_id", -1), diag=diag, resid=True, dev_status=st)
        torch.cuda.synchronize()
        got = dict(tokens=tok.cpu().numpy(), count=cnt.cpu().numpy(), accepted=acc.cpu().numpy(),
                   resid=rs.cpu().numpy())
    else:
        got = run_sample(ci, status=st, diag=diag, **kw)
    with np.errstate(invalid="ignore", over="ignore"):
        want = oracle.verify_sample(ci.target, ci.t_kind, ci.draft, ci.q_kind, V, ci.t_row_start,
                                    ci.q_row_start, ci.draft_ids[:, :k_max], ci.draft_len, k_max, T,
                                    ci.uniforms, **kw)
    nb, bad = compare_tokens(got, want)
    assert bad.size == 0, (seed, bad[:10])
    assert nb <= max(2, 0.02 * B)
    assert int(st.item()) == _or(want["flags"])
    same = (got["count"] == want["count"]) & (got["accepted"] == want["accepted"]) & (want["count"] > 0)
    assert close(got["resid"][same], want["resid"][same], rtol=1e-5, atol=1e-12).all()


@pytest.mark.parametrize("seed", range(12))
def test_gpu_random_greedy_chain(seed):
    rng = np.random.default_rng(7000 + seed)
    V = int(rng.choice(VOCABS))
    B = int(rng.integers(1, 120))
    k_max = int(rng.integers(0, 9))
    ks = rng.integers(0, k_max + 1, size=B).astype(np.int32)
    kind = str(rng.choice(["f32", "bf16"]))
    rows = synth.encode(rng.standard_normal((int((ks + 1).sum()), V)) * 2.0, kind)
    dec = synth.decode(rows, kind)
    n_tie = min(V, 3)
    for r in range(rows.shape[0]):  # ties for the maximum in some rows
        if rng.random() < 0.3 and V > 1:
            idx = rng.choice(V, size=n_tie, replace=False)
            dec[r, idx] = dec[r].max()
    rows = synth.encode(dec, kind)
    am = np.argmax(synth.decode(rows, kind), axis=1)
    ts = np.concatenate([[0], np.cumsum(ks + 1)[:-1]]).astype(np.int32)
    ids = np.full((B, max(k_max, 1)), 0, dtype=np.int32)
    for b in range(B):
        for i in range(int(ks[b])):
            ids[b, i] = am[ts[b] + i] if rng.random() < 0.75 else int(rng.integers(0, V))
    kw = {}
    if rng.random() < 0.4:
        kw["max_new"] = rng.integers(0, k_max + 3, size=B).astype(np.int32)
    if rng.random() < 0.4:
        kw["eos_id"] = int(rng.integers(0, V))
    say(f"greedy seed {seed}: B={B} k_max={k_max} V={V} {kind} {sorted(kw)}")
    st = _status()
    got = run_greedy(rows, kind, ts, ids[:, :k_max], ks, status=st, **kw)
    want = oracle.verify_greedy(rows, kind, V, ts, ids[:, :k_max], ks, k_max, **kw)
    for key in ("tokens", "count", "accepted"):
        assert np.array_equal(got[key], want[key]), (seed, key)
    assert int(st.item()) == _or(want["flags"])


def _random_tree(rng, B, N, V, kind):
    target = synth.encode(rng.standard_normal((B * N, V)) * float(rng.uniform(0.5, 3.0)), kind)
    l = rng.standard_normal((B * N, V)) * 2.0
    q = np.exp(l - l.max(axis=1, keepdims=True))
    q /= q.sum(axis=1, keepdims=True)
    draft = synth.encode(q, kind)
    parent = np.zeros((B, N), dtype=np.int32)
    token = np.full((B, N), -1, dtype=np.int32)
    for b in range(B):
        parent[b, 0] = -1
        for c in range(1, N):
            p = int(rng.integers(max(0, c - int(rng.integers(1, 12))), c))
            parent[b, c] = p
            row = synth.decode(target[b * N + p], kind)
            sib = [int(token[b, d]) for d in range(1, c) if parent[b, d] == p]
            r = rng.random()
            if sib and r < 0.15:
                token[b, c] = sib[int(rng.integers(0, len(sib)))]
            elif r < 0.6:
                token[b, c] = int(np.argsort(-row, kind="stable")[int(rng.integers(0, min(3, V)))])
            else:
                token[b, c] = int(rng.integers(0, V))
    return target, draft, parent, token


@pytest.mark.parametrize("seed", range(12))
def test_gpu_random_trees(seed):
    rng = np.random.default_rng(8000 + seed)
    V = int(rng.choice([5, 2047, 2049, 8193, 40000]))
    B = int(rng.integers(1, 9))
    N = int(rng.integers(1, 160))
    kind = str(rng.choice(["f32", "bf16"]))
    T = float(rng.uniform(0.4, 1.8))
    target, draft, parent, token = _random_tree(rng, B, N, V, kind)
    u = rng.random((B, N)).astype(np.float32)
    u[:, :max(N - 1, 0)] *= float(rng.choice([1.0, 0.2, 0.02]))
    say(f"tree seed {seed}: B={B} N={N} V={V} {kind} T={T:.2f}")
    tgt, dft = rows_to_dev(target, kind), rows_to_dev(draft, kind)
    for variant in ("sampled", "greedy", "point"):
        st = _status()
        if variant == "sampled":
            tok, cnt, acc, pth, _ = sv.sv_verify_tree(tgt, dft, i32(parent), i32(token), T, f32(u), dev_status=st)
            want = oracle.verify_tree(target, kind, draft, kind, V, parent, token, T, u, with_diag=False)
        elif variant == "greedy":
            tok, cnt, acc, pth = sv.sv_verify_tree_greedy(tgt, i32(parent), i32(token), dev_status=st)
            want = oracle.verify_tree_greedy(target, kind, V, parent, token)
        else:
            tok, cnt, acc, pth = sv.sv_verify_tree_pointmass(tgt, i32(parent), i32(token), T, f32(u), dev_status=st)
            want = oracle.verify_tree_pointmass(target, kind, V, parent, token, T, u)
        torch.cuda.synchronize()
        got = dict(tokens=tok.cpu().numpy(), count=cnt.cpu().numpy(), accepted=acc.cpu().numpy(),
                   path=pth.cpu().numpy())
        if variant == "greedy":
            for key in ("tokens", "count", "accepted", "path"):
                assert np.array_equal(got[key], want[key]), (seed, variant, key)
        else:
            nb, bad = compare_tokens(got, want)
            assert bad.size == 0, (seed, variant, bad[:10])
            assert nb <= max(1, 0.1 * B)
        assert int(st.item()) == _or(want["flags"]), (seed, variant)
