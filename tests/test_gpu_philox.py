"""The verify's uniforms drawn on the device (Philox4x64-10), on an MI355X,
through the C ABI: the generator bit for bit against the oracle's, and the
sampled chain verify that draws them in-kernel against the oracle fed the
oracle's uniforms."""
import numpy as np
import pytest
import torch
from scipy.special import softmax as scipy_softmax

import draft_verify_sampling_amd as sv
import oracle
import synth
from tests.gpu_util import say, compare_tokens, close, rows_to_dev, i32, f32, DEV, tv_at_noise_level

pytestmark = pytest.mark.gpu

M64 = 2 ** 64 - 1


@pytest.mark.parametrize("seed,offset,B,slots", [(0, 0, 3, 5), (0xDEADBEEF, 41, 257, 9),
                                                 (M64, M64, 64, 1), (12345, 2 ** 40 + 3, 2000, 17)])
def test_gpu_philox_uniforms_bit_exact(seed, offset, B, slots):
    say(f"philox uniforms seed={seed} offset={offset} B={B} slots={slots}")
    got = sv.sv_philox_uniforms(seed, offset, B, slots).cpu().numpy().astype(np.float64)
    want = oracle.philox_uniforms(seed, offset, B, slots)
    assert np.array_equal(got, want)


def _oracle_chain(ci, u):
    return oracle.verify_sample(ci.target, ci.t_kind, ci.draft, ci.q_kind, ci.V, ci.t_row_start,
                                ci.q_row_start, ci.draft_ids[:, :ci.k_max], ci.draft_len, ci.k_max, ci.T, u)


def _run_philox(ci, seed, offset, diag):
    tok, cnt, acc, dg, rs = sv.sv_verify_sample_philox(
        rows_to_dev(ci.target, ci.t_kind), rows_to_dev(ci.draft, ci.q_kind), i32(ci.t_row_start),
        i32(ci.q_row_start), i32(ci.draft_ids[:, :ci.k_max]), i32(ci.draft_len), ci.T, seed, offset,
        diag=diag, resid=True)
    torch.cuda.synchronize()
    return dict(tokens=tok.cpu().numpy(), count=cnt.cpu().numpy(), accepted=acc.cpu().numpy(),
                resid=rs.cpu().numpy())


@pytest.mark.parametrize("name", ["c3", "ragged", "small"])
def test_gpu_sample_philox_parity(name):
    """All three chain paths: statistics of every row then the walk (diag),
    lazy statistics (ragged, many requests), one wave per request (V <= 2048)."""
    if name == "c3":
        ci = synth.c3_sampled()
    elif name == "ragged":
        ci = synth.c4_ragged(B=256, V=40_000, salt=5)
    else:
        ci = synth.sampled_chain(9, 500, np.random.default_rng(3).integers(0, 6, size=500), 1500, 0.9,
                                 sd=2.0, n_boost=3, boost=4.0, sigma=1.0, kind="f32", name="small")
    seed, offset = 0x5EED0000 + len(name), 77
    say(f"sampled chain with device uniforms: {name} B={ci.B} V={ci.V}")
    u = oracle.philox_uniforms(seed, offset, ci.B, ci.k_max + 1)
    want = _oracle_chain(ci, u)
    for diag in (True, False):
        got = _run_philox(ci, seed, offset, diag)
        nb, bad = compare_tokens(got, want)
        say(f"  diag={diag}: {nb} boundary cases, mean tokens {want['count'].mean():.3f}")
        assert bad.size == 0, bad[:10]
        assert nb <= max(2, 1e-3 * ci.B)
        same = (got["count"] == want["count"]) & (want["count"] > 0)
        assert close(got["resid"][same], want["resid"][same], atol=1e-12).all()
    # the same round as passing those uniforms in
    tok, cnt, acc, _, _ = sv.sv_verify_sample(
        rows_to_dev(ci.target, ci.t_kind), rows_to_dev(ci.draft, ci.q_kind), i32(ci.t_row_start),
        i32(ci.q_row_start), i32(ci.draft_ids[:, :ci.k_max]), i32(ci.draft_len), ci.T,
        sv.sv_philox_uniforms(seed, offset, ci.B, ci.k_max + 1))
    assert np.array_equal(tok.cpu().numpy(), got["tokens"])
    assert np.array_equal(cnt.cpu().numpy(), got["count"])


def test_gpu_sample_philox_tv_200k():
    """Fixed prefix, 200,000 rounds, device uniforms: the emitted token at
    every position follows the target row (TV at sampling-noise level)."""
    say("device uniforms: 200,000 rounds, V=2048, TV per position")
    c1 = synth.c1_chain()
    got = _run_philox(c1, 2026, 1, diag=False)
    rows = [scipy_softmax(c1.target[i].astype(np.float64) / c1.T) for i in range(c1.k_max + 1)]
    res = tv_at_noise_level(got["tokens"], c1.k_max + 1, rows, got["count"], np.random.default_rng(98))
    assert len(res) >= 3
