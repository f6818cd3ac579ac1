"""Parity of the HIP verify path with the float64 oracle, on an MI355X.

Greedy and prompt-lookup results must be bit-exact.  Sampled results: the
normalisers, probabilities at the drafted tokens and the residual mass within
1e-5 relative; token ids equal except in requests where some uniform lies within
1e-6 of its decision edge (counted, and required to be rare).
"""
import os

import numpy as np
import pytest
import torch
from scipy.special import softmax as scipy_softmax

import oracle
import synth
from tests.gpu_util import (say, run_sample, run_greedy, run_tree, close, compare_tokens, same_round,
                            rows_to_dev, i32, f32, DEV, tv_at_noise_level)

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _status():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def _or(flags):
    out = 0
    for f in np.asarray(flags).ravel():
        out |= int(f)
    return out


def _check_chain(ci, got, want, name, max_boundary_frac=1e-3):
    nb, bad = compare_tokens(got, want)
    say(f"{name}: {ci.B} requests, {nb} boundary cases")
    assert bad.size == 0, f"{name}: mismatching requests {bad[:10]}"
    assert nb <= max(2, max_boundary_frac * ci.B)
    valid = want["count"] > 0
    for b in np.nonzero(valid)[0][:4096] if got["diag"] is not None else []:
        k = int(ci.draft_len[b])
        d, e = got["diag"][b, :k + 1], want["diag"][b, :k + 1]
        assert close(d[:, 0], e[:, 0], atol=1e-6).all(), (name, b, "M")
        assert close(d[:, 1], e[:, 1]).all(), (name, b, "S")
        assert close(d[:k, 2], e[:k, 2]).all(), (name, b, "p(x)")
        assert close(d[:k, 3], e[:k, 3]).all(), (name, b, "q(x)")
    same = (got["count"] == want["count"]) & (got["accepted"] == want["accepted"]) & valid
    assert close(got["resid"][same], want["resid"][same], rtol=1e-5, atol=1e-12).all(), name


def _oracle_sample(ci, **kw):
    return oracle.verify_sample(ci.target, ci.t_kind, ci.draft, ci.q_kind, ci.V, ci.t_row_start,
                                ci.q_row_start, ci.draft_ids[:, :ci.k_max], ci.draft_len, ci.k_max,
                                ci.T, ci.uniforms, **kw)


# ---------------------------------------------------------------------------
# greedy + prompt lookup
# ---------------------------------------------------------------------------
def test_gpu_greedy_four_case_table():
    say("greedy four-case table")
    rows = [ln.split() for ln in open(os.path.join(GOLD, "p3_four_cases.txt"), encoding="utf-8")
            if ln.strip() and not ln.startswith("#")]
    path = rows[0][1]
    sym = {s: i for i, s in enumerate("ABCDEFGX")}
    for r in rows[1:]:
        prefix, guess, kept, added, new = (("" if v == "-" else v) for v in r[1:])
        k = len(guess)
        tgt = np.zeros((k + 1, 8), dtype=np.float32)
        for i in range(k + 1):
            pos = len(prefix) + i
            tgt[i, sym[path[pos] if pos < len(path) else "A"]] = 1.0
        ids = np.array([[sym[s] for s in guess]], dtype=np.int32)
        out = run_greedy(tgt, "f32", [0], ids, [k], max_new=[len(path) - len(prefix)])
        got = "".join("ABCDEFGX"[t] for t in out["tokens"][0, :out["count"][0]])
        assert got == kept + added and prefix + got == new
        assert out["accepted"][0] == len(kept)


@pytest.fixture(scope="module")
def c2():
    return synth.c2_greedy()


def test_gpu_ngram_then_greedy_c2(c2):
    say("prompt lookup + greedy, B=64 ctx=4096 V=32000")
    import draft_verify_sampling_amd as sv
    st = _status()
    ids, lens = sv.sv_ngram_draft(i32(c2.ctx), i32(c2.ctx_len), c2.window, c2.k, dev_status=st)
    torch.cuda.synchronize()
    w_ids, w_lens, w_flags = oracle.ngram_draft(c2.ctx, c2.ctx_len, c2.window, c2.k)
    assert np.array_equal(lens.cpu().numpy(), w_lens)
    assert np.array_equal(ids.cpu().numpy(), w_ids)
    assert int(st.item()) == 0
    assert (w_lens > 0).sum() >= 8, "the planted repeats should give drafts"
    t_rs = np.arange(c2.B, dtype=np.int32) * (c2.k + 1)
    got = run_greedy(c2.target, "bf16", t_rs, w_ids, w_lens, status=st)
    want = oracle.verify_greedy(c2.target, "bf16", c2.V, t_rs, w_ids, w_lens, c2.k)
    for key in ("tokens", "count", "accepted"):
        assert np.array_equal(got[key], want[key]), key
    assert int(st.item()) == 0
    say(f"  mean accepted {want['accepted'].mean():.2f}, mean tokens {want['count'].mean():.2f}")


@pytest.mark.parametrize("kind,V", [("bf16", 4999), ("bf16", 8), ("f32", 3001), ("f32", 1)])
def test_gpu_greedy_ties_ragged_unaligned(kind, V):
    say(f"greedy ties/ragged kind={kind} V={V}")
    rng = np.random.default_rng(V)
    B, k_max = 97, 6
    ks = rng.integers(0, k_max + 1, size=B).astype(np.int32)
    t_rs = np.concatenate([[0], np.cumsum(ks + 1)[:-1]]).astype(np.int32)
    rows = int((ks + 1).sum())
    vals = rng.integers(-3, 4, size=(rows, V)).astype(np.float32)   # many ties
    vals[vals == 0] = rng.choice([0.0, -0.0], size=int((vals == 0).sum()))
    tgt = synth.to_bf16_bits(vals) if kind == "bf16" else vals
    dec = oracle.widen(tgt, kind)
    ids = np.full((B, k_max), -1, dtype=np.int32)
    for b in range(B):
        for i in range(ks[b]):
            a = int(np.argmax(dec[t_rs[b] + i]))
            ids[b, i] = a if rng.random() < 0.8 else int(rng.integers(0, V))
    max_new = rng.integers(0, k_max + 3, size=B).astype(np.int32)
    eos = int(rng.integers(0, V))
    for mn, eo in ((None, -1), (max_new, eos)):
        st = _status()
        got = run_greedy(tgt, kind, t_rs, ids, ks, max_new=mn, eos_id=eo, status=st)
        want = oracle.verify_greedy(tgt, kind, V, t_rs, ids, ks, k_max, max_new=mn, eos_id=eo)
        for key in ("tokens", "count", "accepted"):
            assert np.array_equal(got[key], want[key]), key
        assert int(st.item()) == _or(want["flags"])


def test_gpu_greedy_invalid_inputs():
    say("greedy invalid inputs")
    V, k = 300, 3
    rng = np.random.default_rng(0)
    tgt = rng.standard_normal((12, V)).astype(np.float32)
    tgt[5, 17] = np.nan                   # request 1 uses rows 4..7
    ids = rng.integers(0, V, size=(4, k)).astype(np.int32)
    ids[2, 1] = V                         # bad token
    t_rs = np.array([0, 4, 8, 11], dtype=np.int32)   # request 3: rows 11..14 out of range
    ks = np.array([3, 3, 3, 3], dtype=np.int32)
    st = _status()
    got = run_greedy(tgt, "f32", t_rs, ids, ks, status=st)
    want = oracle.verify_greedy(tgt, "f32", V, t_rs, ids, ks, k)
    for key in ("tokens", "count", "accepted"):
        assert np.array_equal(got[key], want[key]), key
    assert list(want["count"]) == [int(want["count"][0]), 0, 0, 0]
    assert int(st.item()) == _or(want["flags"]) == (oracle.FLAG_NONFINITE | oracle.FLAG_BAD_TOKEN |
                                                    oracle.FLAG_BAD_REQUEST)


def test_gpu_ngram_small_contexts():
    say("prompt lookup, brute-force-sized contexts")
    import draft_verify_sampling_amd as sv
    rng = np.random.default_rng(2)
    B, stride = 300, 700
    ctx = rng.integers(0, 3, size=(B, stride)).astype(np.int32)
    lens = rng.integers(0, stride + 1, size=B).astype(np.int32)
    lens[:5] = [0, 1, 2, 3, 4]
    lens[5] = stride + 1                 # bad length
    for w in (1, 2, 3, 7):
        for k in (0, 1, 4, 9):
            st = _status()
            ids, dl = sv.sv_ngram_draft(i32(ctx), i32(lens), w, k, dev_status=st)
            torch.cuda.synchronize()
            wi, wl, wf = oracle.ngram_draft(ctx, lens, w, k)
            assert np.array_equal(dl.cpu().numpy(), wl), (w, k)
            assert np.array_equal(ids.cpu().numpy(), wi), (w, k)
            assert int(st.item()) == _or(wf)


# ---------------------------------------------------------------------------
# sampled chain
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def c1():
    return synth.c1_chain()


def test_gpu_sample_c1_parity_and_tv(c1):
    say("sampled chain, fixed prefix, V=2048 fp32, 200,000 rounds")
    st = _status()
    got = run_sample(c1, status=st)
    want = _oracle_sample(c1)
    _check_chain(c1, got, want, "c1")
    assert int(st.item()) == 0
    rows = [scipy_softmax(c1.target[i].astype(np.float64) / c1.T) for i in range(c1.k_max + 1)]
    tv_at_noise_level(got["tokens"], c1.k_max + 1, rows, got["count"], np.random.default_rng(99))


@pytest.fixture(scope="module")
def c3():
    return synth.c3_sampled()


def test_gpu_sample_c3_full(c3):
    say("sampled chain B=64 k=4 V=248320 bf16 T=0.7")
    st = _status()
    got = run_sample(c3, status=st)
    want = _oracle_sample(c3)
    _check_chain(c3, got, want, "c3")
    assert int(st.item()) == 0
    say(f"  mean accepted {want['accepted'].mean():.2f}")
    say("  the same without diagnostics (statistics only of the rows the rounds read)")
    st = _status()
    lazy = run_sample(c3, status=st, diag=False)
    same_round(lazy, got)
    assert int(st.item()) == 0


def test_gpu_sample_deterministic(c3):
    say("sampled chain run twice (lazy statistics)")
    a = run_sample(c3, diag=False)
    b = run_sample(c3, diag=False)
    for key in ("tokens", "count", "accepted", "resid"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("tk,qk,V", [("bf16", "bf16", 4999), ("f32", "bf16", 12289),
                                     ("f32", "f32", 777), ("bf16", "f32", 4096), ("bf16", "bf16", 1)])
def test_gpu_sample_small_ragged(tk, qk, V):
    say(f"sampled ragged tk={tk} qk={qk} V={V}")
    ci = synth.sampled_chain(40 + V % 7, 41, np.random.default_rng(V).integers(0, 9, size=41), V,
                             0.9, sd=2.0, n_boost=min(3, V), boost=4.0, sigma=1.0, kind=tk)
    if qk != tk:
        dec = synth.decode(ci.draft, tk)
        ci.draft = synth.encode(dec, qk)
        ci.q_kind = qk
    st = _status()
    got = run_sample(ci, status=st)
    want = _oracle_sample(ci)
    _check_chain(ci, got, want, f"ragged {tk}/{qk}/{V}", max_boundary_frac=0.05)
    assert int(st.item()) == _or(want["flags"])
    st = _status()
    same_round(run_sample(ci, status=st, diag=False), got)
    assert int(st.item()) == _or(want["flags"])


@pytest.fixture(scope="module")
def c4():
    return synth.c4_ragged()


def test_gpu_sample_c4_full(c4):
    say("ragged sampled chain B=256 k in 1..8 V=151936 bf16 T=1")
    st = _status()
    got = run_sample(c4, status=st)
    want = _oracle_sample(c4)
    _check_chain(c4, got, want, "c4")
    assert int(st.item()) == 0
    say("  the same with lazy statistics")
    st = _status()
    same_round(run_sample(c4, status=st, diag=False), got)
    assert int(st.item()) == 0


def _edge_batch(B, V=5000):
    """Requests 0..12 are the edge cases below; the rest are ordinary rounds."""
    k = 3
    ks = np.full(B, 3, dtype=np.int32)
    ks[[0, 10]] = [0, 2]
    ci = synth.sampled_chain(90, B, ks, V, 1.0, sd=2.0, n_boost=3, boost=5.0, sigma=1.0, kind="f32")
    t = ci.target
    q = ci.draft
    # request 2: residual with zero mass -> fallback to p (draft row of position 0 all ones)
    q[ci.q_row_start[2]] = 1.0
    ci.uniforms[2, 0] = 0.99
    # request 3: NaN in a target row the round reads (u = 0 keeps draft 0)
    t[ci.t_row_start[3] + 1, 10] = np.nan
    ci.uniforms[3, 0] = 0.0
    # request 4: +inf in a target row the round reads (drafts 0 and 1 kept)
    t[ci.t_row_start[4] + 2, 11] = np.inf
    ci.uniforms[4, :2] = 0.0
    # request 12: NaN in a row after a forced break at 0: never read, valid
    ci.draft_ids[12, 0] = 13
    q[ci.q_row_start[12], 13] = 1.0
    ci.uniforms[12, 0] = 0.999
    t[ci.t_row_start[12] + 2, 10] = np.nan
    # request 5: NaN in the draft row at the break (force a rejection at 0)
    q[ci.q_row_start[5], 12] = np.nan
    ci.draft_ids[5, 0] = 13
    q[ci.q_row_start[5], 13] = 1.0
    ci.uniforms[5, 0] = 0.999
    # request 6: bad token
    ci.draft_ids[6, 1] = V + 3
    # request 7: row start out of range
    ci.t_row_start[7] = t.shape[0] - 2
    # request 8: -inf logits are allowed (zero probability)
    t[ci.t_row_start[8]:ci.t_row_start[8] + 4, :100] = -np.inf
    # request 9: u = 0 everywhere
    ci.uniforms[9] = 0.0
    ci.uniforms[11] = 0.0                # keep every draft with p > 0
    max_new = np.full(B, 5, dtype=np.int32)
    max_new[[10, 11]] = [1, 2]           # over budget
    eos = int(ci.draft_ids[1, 1])
    return ci, max_new, eos


@pytest.mark.parametrize("B,V", [(13, 5000), (4200, 5000), (900, 40_000), (1024, 40_000), (1025, 40_000)])
def test_gpu_sample_edge_cases(B, V):
    # B = 4200 (one segment a row) and B = 900 or more (five) have enough
    # statistics blocks per row for the lazy statistics; with B = 900 and
    # 1024 (the most requests its LDS layout holds) rows 2 and 3 go to the
    # kernel that reads every remaining row of the running rounds at once,
    # with B = 1025 every row is decided row-major
    say(f"sampled chain edge cases, B={B}, V={V}")
    ci, max_new, eos = _edge_batch(B, V)
    seen = {}
    for mn, eo, dg in ((None, -1, True), (max_new, eos, True), (None, -1, False), (max_new, eos, False)):
        st = _status()
        got = run_sample(ci, status=st, max_new=mn, eos_id=eo, diag=dg)
        # statistics of every row (diagnostics) and the lazy statistics (B =
        # 4200): the same pairs and weights, bit for bit
        if (mn is None) in seen:
            same_round(seen[mn is None], got)
        seen[mn is None] = got
        with np.errstate(invalid="ignore", over="ignore"):
            want = _oracle_sample(ci, max_new=mn, eos_id=eo)
        nb, bad = compare_tokens(got, want)
        assert bad.size == 0, (dg, bad[:10])
        assert nb <= max(2, 1e-3 * B)
        assert int(st.item()) == _or(want["flags"]), dg
    fl = want["flags"]
    assert fl[2] & oracle.FLAG_FALLBACK and fl[3] & oracle.FLAG_NONFINITE
    assert fl[4] & oracle.FLAG_NONFINITE and fl[5] & oracle.FLAG_NONFINITE
    assert fl[6] & oracle.FLAG_BAD_TOKEN and fl[7] & oracle.FLAG_BAD_REQUEST
    assert fl[11] & oracle.FLAG_OVER_BUDGET and got["count"][11] == 2
    assert fl[12] == 0 and want["accepted"][12] == 0 and got["count"][12] == 1


@pytest.mark.parametrize("V", [151_936, 248_320])
def test_gpu_sample_zero_mass_fallback_bf16(V):
    """bf16 rows at the large vocabularies: a draft row of all ones (q >= p
    everywhere) leaves the residual without mass, so the last token is drawn
    from p of the break row (the request's last draw block sums p over every
    tile of that row: 75 or 122 tiles)."""
    say(f"zero-mass residual fallback, bf16, V={V}")
    B = 24
    ci = synth.sampled_chain(93, B, np.full(B, 2, dtype=np.int32), V, 1.0, sd=2.0, n_boost=3, boost=5.0,
                             sigma=1.0, kind="bf16")
    one = 0x3F80                                      # 1.0 in bfloat16
    for b in range(8):                                # break at row 0
        ci.draft[ci.q_row_start[b]] = one
        ci.uniforms[b, 0] = 0.99
    for b in range(8, 12):                            # draft 0 kept, break at row 1
        ci.uniforms[b, 0] = 0.0
        ci.draft[ci.q_row_start[b] + 1] = one
        ci.uniforms[b, 1] = 0.99
    want = _oracle_sample(ci)
    assert all(f & oracle.FLAG_FALLBACK for f in want["flags"][:12])
    for dg in (True, False):
        st = _status()
        got = run_sample(ci, status=st, diag=dg)
        _check_chain(ci, got, want, f"fallback V={V}")
        assert int(st.item()) == _or(want["flags"])


def test_gpu_greedy_equals_sampling_on_one_hot():
    say("one-hot targets: sampled == greedy")
    rng = np.random.default_rng(31)
    V, k, B = 1000, 4, 64
    a = rng.integers(0, V, size=B * (k + 1))
    tgt = np.zeros((B * (k + 1), V), dtype=np.float32)
    tgt[np.arange(B * (k + 1)), a] = 800.0
    q = rng.dirichlet(np.ones(V), size=B * k).astype(np.float32) + 1e-6
    ids = np.where(rng.random((B, k)) < 0.6, a.reshape(B, k + 1)[:, :k],
                   rng.integers(0, V, size=(B, k))).astype(np.int32)
    ks = rng.integers(0, k + 1, size=B).astype(np.int32)
    t_rs = (np.arange(B) * (k + 1)).astype(np.int32)
    q_rs = (np.arange(B) * k).astype(np.int32)
    ci = synth.ChainInputs("onehot", V, "f32", tgt, "f32", q, t_rs, q_rs, ids, ks, k, 1.0,
                           rng.random((B, k + 1)).astype(np.float32))
    s = run_sample(ci)
    g = run_greedy(tgt, "f32", t_rs, ids, ks)
    for key in ("tokens", "count", "accepted"):
        assert np.array_equal(s[key], g[key]), key


# ---------------------------------------------------------------------------
# tree
# ---------------------------------------------------------------------------
def _check_tree(ti, got, want, name, max_boundary_frac=1e-3):
    nb, bad = compare_tokens(got, want, keys=("tokens", "count", "accepted", "path"))
    say(f"{name}: {ti.B} requests, {nb} boundary cases, mean kept {want['accepted'].mean():.2f}")
    assert bad.size == 0, f"{name}: mismatching requests {bad[:10]}"
    assert nb <= max(2, max_boundary_frac * ti.B)
    for b in np.nonzero(want["count"] > 0)[0]:
        d, e = got["diag"][b], want["diag"][b]
        assert close(d[:, 0], e[:, 0], atol=1e-6).all(), (name, b, "M")
        assert close(d[:, 1], e[:, 1]).all(), (name, b, "S")
        assert close(d[1:, 2], e[1:, 2]).all(), (name, b, "p(x)")
        assert close(d[1:, 3], e[1:, 3]).all(), (name, b, "q(x)")


def _oracle_tree(ti):
    return oracle.verify_tree(ti.target, ti.t_kind, ti.draft, ti.q_kind, ti.V, ti.parent, ti.token,
                              ti.T, ti.uniforms)


@pytest.fixture(scope="module")
def c5():
    return synth.c5_tree()


def _same_walk(a, b):
    for key in ("tokens", "count", "accepted", "path"):
        assert np.array_equal(a[key], b[key]), key


def test_gpu_tree_c5_full(c5):
    say("tree B=32 N=60 V=128256 bf16 T=1")
    st = _status()
    got = run_tree(c5, status=st)
    want = _oracle_tree(c5)
    _check_tree(c5, got, want, "c5")
    assert int(st.item()) == _or(want["flags"])
    # the walk reads only visited rows and never the diagnostics' statistics:
    # the same tokens with and without diagnostics, and on a repeat
    say("tree c5 without diagnostics, twice")
    _same_walk(run_tree(c5, diag=False), got)
    _same_walk(run_tree(c5, diag=False), got)


def test_gpu_tree_beside_another_stream(c5):
    """The walk's workgroups of one request wait for each other.  Copies
    queued on another stream just before the walk hold compute units while
    it starts; they never wait for the walk, so they only delay the rest of
    its grid: the outputs are the oracle's and no wait runs out (no sync
    timeout bit)."""
    say("tree c5 beside another stream's copies")
    want = _oracle_tree(c5)
    src = torch.empty(1 << 28, dtype=torch.uint8, device=DEV)
    dst = torch.empty_like(src)
    side = torch.cuda.Stream()
    for rep in range(3):
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(4):
                dst.copy_(src)
        st = _status()
        got = run_tree(c5, status=st, diag=False)
        nb, bad = compare_tokens(got, want, keys=("tokens", "count", "accepted", "path"))
        assert bad.size == 0 and nb <= 2, (rep, bad[:10])
        assert int(st.item()) == _or(want["flags"]), rep
    torch.cuda.synchronize()


@pytest.mark.parametrize("B", [1, 3, 300])
def test_gpu_tree_group_counts(B):
    # the library splits a request over G = min(32, 256 // B, tiles) workgroups:
    # B=1 -> 32, B=3 -> 32 (V=70000 has 35 tiles), B=300 -> 1
    say(f"tree B={B} N=9 V=70000 (workgroups per request vary with B)")
    ti = synth.c5_tree(B=B, N=9, V=70_000, top_children=2, expand_per_layer=2, max_depth=4,
                       sigma=0.8, salt=B)
    st = _status()
    got = run_tree(ti, status=st, diag=False)
    want = _oracle_tree(ti)
    nb, bad = compare_tokens(got, want, keys=("tokens", "count", "accepted", "path"))
    say(f"B={B}: {nb} boundary cases, mean kept {want['accepted'].mean():.2f}")
    assert bad.size == 0, bad[:10]
    assert nb <= max(2, 0.01 * B)
    assert int(st.item()) == _or(want["flags"])


def test_gpu_tree_nonfinite_rows():
    say("tree non-finite rows: visited ones invalidate, unvisited ones do not")
    ti = synth.c5_tree(B=40, N=10, V=4999, top_children=3, expand_per_layer=3, max_depth=3,
                       sigma=1.5, salt=77)
    base = _oracle_tree(ti)
    N, V = ti.N, ti.V
    rej = [b for b in range(ti.B) if base["accepted"][b] == 0 and base["count"][b] == 1]
    assert len(rej) >= 5, rej          # requests whose root rejects every child
    enc = lambda x, kind: synth.encode(np.array([x]), kind)[0]
    tgt, dft = ti.target.copy(), ti.draft.copy()
    r_t, r_unv, r_qnan, r_mix, r_pinf = rej[:5]
    tgt[r_t * N, 17] = enc(np.nan, ti.t_kind)            # visited target row (root)
    tgt[r_unv * N + N - 1, :] = enc(np.nan, ti.t_kind)   # a node the walk never reaches
    dft[r_qnan * N, 4000] = enc(np.nan, ti.q_kind)       # root draft row, used by a residual
    dft[r_mix * N, 5] = enc(np.inf, ti.q_kind)           # +inf and -inf in far apart slices
    dft[r_mix * N, V - 3] = enc(-np.inf, ti.q_kind)
    dft[r_pinf * N, 5] = enc(np.inf, ti.q_kind)          # +inf alone: zero residual weight there
    bad_ti = synth.TreeInputs(ti.name, V, N, ti.t_kind, tgt, ti.q_kind, dft, ti.parent, ti.token,
                              ti.depth, ti.T, ti.uniforms)
    st = _status()
    got = run_tree(bad_ti, status=st, diag=False)
    with np.errstate(invalid="ignore", over="ignore"):
        want = _oracle_tree(bad_ti)
    nb, bad = compare_tokens(got, want, keys=("tokens", "count", "accepted", "path"))
    assert bad.size == 0, bad
    assert [int(want["count"][r]) for r in (r_t, r_qnan, r_mix)] == [0, 0, 0]
    assert want["count"][r_unv] == 1 and want["count"][r_pinf] == 1
    assert int(st.item()) == _or(want["flags"])


@pytest.mark.parametrize("kind,V,N", [("bf16", 4999, 12), ("f32", 3000, 20), ("bf16", 9, 7)])
def test_gpu_tree_small(kind, V, N):
    say(f"tree small kind={kind} V={V} N={N}")
    ti = synth.c5_tree(B=24, N=N, V=V, top_children=3 if V > 9 else 2, expand_per_layer=3,
                       max_depth=4, sigma=0.7, salt=V, kind=kind)
    st = _status()
    got = run_tree(ti, status=st)
    want = _oracle_tree(ti)
    _check_tree(ti, got, want, f"tree {kind}/{V}/{N}", max_boundary_frac=0.05)
    assert int(st.item()) == _or(want["flags"])


def test_gpu_tree_invalid_and_chain_equivalence():
    say("tree invalid inputs; chain-as-tree equals chain")
    ch = synth.c3_sampled(B=20, k=4, V=6000, T=0.8, salt=4)
    B, k, V = ch.B, ch.k_max, ch.V
    N = k + 1
    tgt = np.zeros((B * N, V), dtype=np.uint16)
    dft = np.zeros((B * N, V), dtype=np.uint16)
    parent = np.tile(np.arange(-1, N - 1), (B, 1)).astype(np.int32)
    tok = np.full((B, N), -1, dtype=np.int32)
    for b in range(B):
        tgt[b * N:(b + 1) * N] = ch.target[ch.t_row_start[b]:ch.t_row_start[b] + N]
        dft[b * N:b * N + k] = ch.draft[ch.q_row_start[b]:ch.q_row_start[b] + k]
        tok[b, 1:] = ch.draft_ids[b, :k]
    ti = synth.TreeInputs("chain", V, N, "bf16", tgt, "bf16", dft, parent, tok,
                          np.tile(np.arange(N), (B, 1)), ch.T, ch.uniforms.copy())
    g_tree = run_tree(ti)
    g_chain = run_sample(ch)
    assert np.array_equal(g_tree["tokens"][:, :N], g_chain["tokens"])
    for key in ("count", "accepted"):
        assert np.array_equal(g_tree[key], g_chain[key]), key
    ti.parent[3, 2] = 3          # parent not before child
    ti.parent[4, 0] = 0          # root with a parent
    ti.token[5, 3] = V           # bad token
    st = _status()
    got = run_tree(ti, status=st)
    want = _oracle_tree(ti)
    nb, bad = compare_tokens(got, want, keys=("tokens", "count", "accepted", "path"))
    assert bad.size == 0
    assert list(got["count"][3:6]) == [0, 0, 0]
    assert int(st.item()) == _or(want["flags"]) == oracle.FLAG_BAD_TREE | oracle.FLAG_BAD_TOKEN


@pytest.mark.parametrize("kind,V,T", [("bf16", 248_320, 0.7), ("f32", 4099, 1.3), ("bf16", 7, 1.0)])
def test_gpu_softmax_partials(kind, V, T):
    say(f"softmax partials kind={kind} V={V} T={T}")
    import draft_verify_sampling_amd as sv
    rng = np.random.default_rng(V)
    rows = rng.standard_normal((9, V)) * 2.5
    rows[3, :V // 2] = -np.inf
    stored = synth.encode(rows, kind)
    part = sv.sv_softmax_partials(rows_to_dev(stored, kind), T).cpu().numpy().astype(np.float64)
    for r in range(rows.shape[0]):
        m = part[r, :, 0].max()
        s = (part[r, :, 1] * np.exp2(part[r, :, 0] - m)).sum()
        _, M, S = oracle.softmax_T(oracle.widen(stored[r], kind), T)
        assert close(m * np.log(2.0), M, atol=1e-6), r
        assert close(s, S), r


def test_gpu_graph_replay_matches_eager():
    """The sampled verify allocates nothing, synchronises nothing and issues no
    memset, so it can be captured in a HIP graph; every replay (with eager work
    and synchronisations in between) must equal the eager result."""
    say("graph capture and replay of sv_verify_sample")
    import draft_verify_sampling_amd as sv
    ci = synth.c3_sampled(B=16, k=4, V=20_000, T=0.8, salt=9)
    other = synth.c3_sampled(B=16, k=4, V=20_000, T=0.8, salt=10)
    args = [rows_to_dev(ci.target, "bf16"), rows_to_dev(ci.draft, "bf16"), i32(ci.t_row_start),
            i32(ci.q_row_start), i32(ci.draft_ids), i32(ci.draft_len)]
    u = f32(ci.uniforms)
    eager = sv.sv_verify_sample(*args, ci.T, u)
    torch.cuda.synchronize()
    want = [t.clone() for t in eager[:3]]
    ws = sv.Workspace()
    out = (torch.empty_like(want[0]), torch.empty_like(want[1]), torch.empty_like(want[2]), None, None)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sv.sv_verify_sample(*args, ci.T, u, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sv.sv_verify_sample(*args, ci.T, u, workspace=ws, out=out)
    oargs = [rows_to_dev(other.target, "bf16"), rows_to_dev(other.draft, "bf16"),
             i32(other.t_row_start), i32(other.q_row_start), i32(other.draft_ids), i32(other.draft_len)]
    for rep in range(4):
        for t in out[:3]:
            t.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for got, w in zip(out[:3], want):
            assert torch.equal(got, w), rep
        sv.sv_verify_sample(*oargs, other.T, f32(other.uniforms))   # eager work in between
        torch.cuda.synchronize()


def test_gpu_prepared_calls_match_direct_calls():
    """The pre-marshalled launchers enqueue exactly the calls they were
    prepared from: same outputs as the direct calls, call after call."""
    say("prepared sv_verify_sample / sv_softmax_partials launchers")
    import draft_verify_sampling_amd as sv
    ci = synth.c3_sampled(B=12, k=3, V=30_001, T=0.9, salt=21)
    args = [rows_to_dev(ci.target, "bf16"), rows_to_dev(ci.draft, "bf16"), i32(ci.t_row_start),
            i32(ci.q_row_start), i32(ci.draft_ids), i32(ci.draft_len)]
    u = f32(ci.uniforms)
    want = [t.clone() for t in sv.sv_verify_sample(*args, ci.T, u)[:3]]
    launch, outs = sv.prepare_verify_sample(*args, ci.T, u, workspace=sv.Workspace())
    part_want = sv.sv_softmax_partials(args[0], ci.T)
    part = torch.full_like(part_want, -5.0)
    plaunch = sv.prepare_softmax_partials(args[0], ci.T, part)
    for rep in range(3):
        for t in outs[:3]:
            t.fill_(-7)
        launch()
        plaunch()
        torch.cuda.synchronize()
        for got, w in zip(outs[:3], want):
            assert torch.equal(got, w), rep
        assert torch.equal(part, part_want), rep
    # tree and greedy entry points through the generic prepare()
    ti = synth.c5_tree(B=6, N=9, V=5000, top_children=2, expand_per_layer=2, max_depth=4, salt=3)
    targs = (rows_to_dev(ti.target, "bf16"), rows_to_dev(ti.draft, "bf16"), i32(ti.parent), i32(ti.token))
    tu = f32(ti.uniforms)
    direct = [t.clone() for t in sv.sv_verify_tree(*targs, ti.T, tu)[:4]]
    tl, touts = sv.prepare(sv.sv_verify_tree, *targs, ti.T, tu)
    gd = [t.clone() for t in sv.sv_verify_tree_greedy(targs[0], targs[2], targs[3])]
    gl, gouts = sv.prepare(sv.sv_verify_tree_greedy, targs[0], targs[2], targs[3])
    for rep in range(2):
        for t in list(touts[:4]) + list(gouts):
            t.fill_(-7)
        tl()
        gl()
        torch.cuda.synchronize()
        for got, w in zip(touts[:4], direct):
            assert torch.equal(got, w), rep
        for got, w in zip(gouts, gd):
            assert torch.equal(got, w), rep


def test_gpu_calls_on_a_side_stream():
    """Calls given a stream that is not torch's current one: the binding makes
    and fills their outputs, diagnostics and a fresh workspace on that stream,
    so they equal the same calls on the current stream, bit for bit, while the
    current stream is kept busy with copies."""
    import draft_verify_sampling_amd as sv
    say("sample and tree calls with diagnostics on a side stream")
    rng = np.random.default_rng(21)
    ks = rng.integers(0, 7, size=16)
    ci = synth.sampled_chain(311, 16, ks, 30_011, 0.9, sd=2.0, n_boost=3, boost=4.0, sigma=1.0, kind="bf16")
    sargs = (rows_to_dev(ci.target, ci.t_kind), rows_to_dev(ci.draft, ci.q_kind), i32(ci.t_row_start),
             i32(ci.q_row_start), i32(ci.draft_ids[:, :ci.k_max]), i32(ci.draft_len), ci.T, f32(ci.uniforms))
    ti = synth.c5_tree(B=8, N=20, V=30_000, top_children=3, expand_per_layer=3, max_depth=4, salt=5)
    targs = (rows_to_dev(ti.target, ti.t_kind), rows_to_dev(ti.draft, ti.q_kind), i32(ti.parent),
             i32(ti.token), ti.T, f32(ti.uniforms))
    ref_s = [t.cpu().numpy() for t in sv.sv_verify_sample(*sargs, diag=True)]
    ref_t = [t.cpu().numpy() for t in sv.sv_verify_tree(*targs, diag=True)]
    torch.cuda.synchronize()
    busy = torch.empty(1 << 28, dtype=torch.uint8, device=DEV)
    busy2 = torch.empty_like(busy)
    side = torch.cuda.Stream()
    for rep in range(3):
        for _ in range(4):
            busy2.copy_(busy)
        got_s = sv.sv_verify_sample(*sargs, diag=True, stream=side, workspace=sv.Workspace(DEV))
        got_t = sv.sv_verify_tree(*targs, diag=True, stream=side, workspace=sv.Workspace(DEV))
        side.synchronize()
        for name, g, w in zip(("tokens", "count", "accepted", "diag", "resid"), got_s, ref_s):
            assert np.array_equal(g.cpu().numpy(), w), ("sample", name, rep)
        for name, g, w in zip(("tokens", "count", "accepted", "path", "diag"), got_t, ref_t):
            assert np.array_equal(g.cpu().numpy(), w), ("tree", name, rep)
    torch.cuda.synchronize()
