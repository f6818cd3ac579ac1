"""The sampled chain round against the float64 oracle (MI355X, through the C
ABI): long chains (k_max 30 and 31) whose drafts are mostly kept, rounds that
keep every draft, empty drafts, vocabularies of 2^19 and one past it (a last
tile of one element), end-token and budget cuts, and the round running beside
another stream's kernels.

Every case runs twice: without diagnostics (the softmax statistics of every
target row, then the draw kernel: the accept scan, the residual's tile sums
and the inverse-CDF pick) and with them (the same statistics, the
diagnostics kernel, then the draw); the two must give the same round."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import say, compare_tokens, close, run_sample, same_round, DEV

pytestmark = pytest.mark.gpu


def _status():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def _or(flags):
    out = 0
    for f in np.asarray(flags).ravel():
        out |= int(f)
    return out


def _oracle(ci, **kw):
    return oracle.verify_sample(ci.target, ci.t_kind, ci.draft, ci.q_kind, ci.V, ci.t_row_start,
                                ci.q_row_start, ci.draft_ids[:, :ci.k_max], ci.draft_len, ci.k_max, ci.T,
                                ci.uniforms, **kw)


def _check(ci, label, max_boundary=2, **kw):
    st = _status()
    got = run_sample(ci, status=st, diag=False, **kw)
    want = _oracle(ci, **kw)
    nb, bad = compare_tokens(got, want)
    say(f"  {label}: mean accepted {want['accepted'].mean():.2f}, max {want['accepted'].max()}, "
        f"boundary {nb}")
    assert bad.size == 0, (label, bad[:10])
    assert nb <= max_boundary
    ok = (want["flags"] & oracle.INVALID_FLAGS) == 0
    assert np.all(close(got["resid"][ok], want["resid"][ok])), label
    assert int(st.item()) == _or(want["flags"]), label
    # with diagnostics: the same round
    st2 = _status()
    full = run_sample(ci, status=st2, diag=True, **kw)
    same_round(got, full)
    assert int(st2.item()) == int(st.item())
    return got, want


def test_gpu_round_long_chains_k30():
    """k_max = 30 with a draft close to the target (sigma 0.15), so many
    requests keep long runs of drafts and the break row lies far down the
    chain."""
    say("round: k_max = 30, close draft, V = 20,011")
    rng = np.random.default_rng(7)
    ks = rng.integers(0, 31, size=24)
    ks[0] = 30
    ci = synth.sampled_chain(301, 24, ks, 20_011, 1.0, sd=1.0, n_boost=3, boost=3.0, sigma=0.15, kind="bf16")
    got, want = _check(ci, "k30")
    assert want["accepted"].max() >= 8


def test_gpu_round_k31():
    say("round: k_max = 31, V = 9,000")
    rng = np.random.default_rng(8)
    ks = rng.integers(0, 32, size=12)
    ks[0] = 31
    ci = synth.sampled_chain(302, 12, ks, 9_000, 1.0, sd=1.0, n_boost=3, boost=3.0, sigma=0.2, kind="bf16")
    _check(ci, "k31")


def test_gpu_round_every_draft_kept_and_empty_drafts():
    """u = 0 keeps every draft with p(x) > 0 (the extra token then comes from
    row k); requests with no draft draw from row 0."""
    say("round: all kept, empty drafts, V = 33,333 f32")
    ks = np.array([0, 3, 5, 0, 1, 5, 2, 4], dtype=np.int64)
    ci = synth.sampled_chain(303, 8, ks, 33_333, 0.8, sd=2.0, n_boost=4, boost=5.0, sigma=1.0, kind="f32")
    ci.uniforms[[1, 2, 5]] = 0.0
    got, want = _check(ci, "all kept")
    assert want["accepted"][1] == 3 and want["accepted"][5] == 5
    assert np.all(got["count"][[0, 3]] == 1)


@pytest.mark.parametrize("V", [524_288, 524_289])
def test_gpu_round_vocab_limit(V):
    say(f"round: vocabulary {V}")
    ci = synth.sampled_chain(304, 4, np.array([3, 0, 2, 3]), V, 0.7, sd=2.5, n_boost=5, boost=6.0, sigma=1.5,
                             kind="bf16")
    _check(ci, f"V={V}")


def test_gpu_round_edges_eos_budget():
    """End token and budget cuts (drafts drawn from q: the end token is the
    second draft of the request with the most drafts)."""
    say("round: end token and budgets")
    rng = np.random.default_rng(9)
    ks = rng.integers(0, 7, size=48)
    ci = synth.sampled_chain(305, 48, ks, 12_345, 1.0, sd=1.0, n_boost=3, boost=3.0, sigma=0.3, kind="bf16")
    mn = rng.integers(0, 8, size=48).astype(np.int32)
    eos = int(ci.draft_ids[int(np.argmax(ks)), 1])
    _check(ci, "eos+budget", max_new=mn, eos_id=eos)


def test_gpu_round_beside_another_stream():
    """The round's blocks wait only for blocks launched before them, so it
    needs no particular residency: run it while another stream keeps the
    device busy with large copies, and compare with the oracle."""
    say("round beside another stream's copies")
    ci = synth.c3_sampled(B=64, k=4, V=248_320, T=0.7, salt=4)
    want = _oracle(ci)
    src = torch.empty(1 << 28, dtype=torch.uint8, device=DEV)
    dst = torch.empty_like(src)
    side = torch.cuda.Stream()
    for rep in range(3):
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(4):
                dst.copy_(src)
        st = _status()
        got = run_sample(ci, status=st, diag=False)
        nb, bad = compare_tokens(got, want)
        assert bad.size == 0 and nb <= 2, (rep, bad[:10])
        assert int(st.item()) == _or(want["flags"])
    torch.cuda.synchronize()
