"""sv_verify_sample_noalloc (the sampled chain verify on the library's static
device scratch, for callers that cannot allocate) against sv_verify_sample on a
caller workspace, through the C ABI on an MI355X: two calls in a row, the
second with a smaller input, each bit for bit equal to the workspace call on
the same inputs; a call too large for the scratch is refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

import draft_verify_sampling_amd as sv
import synth
from tests.gpu_util import DEV, rows_to_dev, i32, f32, say

pytestmark = pytest.mark.gpu


def _inputs(ci):
    return (rows_to_dev(ci.target, ci.t_kind), rows_to_dev(ci.draft, ci.q_kind), i32(ci.t_row_start),
            i32(ci.q_row_start), i32(ci.draft_ids[:, :ci.k_max]), i32(ci.draft_len), ci.T, f32(ci.uniforms))


def _outs(B, k_max):
    return (torch.full((B, k_max + 1), -7, dtype=torch.int32, device=DEV),
            torch.full((B,), -7, dtype=torch.int32, device=DEV),
            torch.full((B,), -7, dtype=torch.int32, device=DEV), None,
            torch.full((B,), -7.0, dtype=torch.float32, device=DEV))


def _both(ci, **kw):
    args = _inputs(ci)
    st_a = torch.zeros(1, dtype=torch.int32, device=DEV)
    st_b = torch.zeros(1, dtype=torch.int32, device=DEV)
    a = sv.sv_verify_sample(*args, dev_status=st_a, out=_outs(ci.B, ci.k_max), resid=True, **kw)
    b = sv.sv_verify_sample_noalloc(*args, dev_status=st_b, out=_outs(ci.B, ci.k_max), resid=True, **kw)
    torch.cuda.synchronize()
    for name, x, y in zip(("tokens", "count", "accepted", "resid"), (a[0], a[1], a[2], a[4]),
                          (b[0], b[1], b[2], b[4])):
        assert torch.equal(x, y), name
    assert int(st_a.item()) == int(st_b.item())
    return b


def test_gpu_noalloc_matches_workspace_call_twice():
    say("scratch call 1: ragged chain B=256, k in 1..8, V=151,936 (lazy statistics)")
    c4 = synth.c4_ragged()
    got = _both(c4)
    assert int(got[1].min().item()) >= 1
    say("scratch call 2: smaller, B=8, k=4, V=20,000, with end token and budgets")
    c3 = synth.c3_sampled(B=8, k=4, V=20_000, T=0.7, salt=3)
    mn = torch.from_numpy(np.array([5, 1, 3, 0, 2, 5, 4, 1], dtype=np.int32)).to(DEV)
    got = _both(c3, max_new=mn, eos_id=int(c3.draft_ids[0, 1]))
    assert int(got[1].max().item()) <= 5


def test_gpu_noalloc_refuses_calls_beyond_the_scratch():
    """B = 4096 requests with 9 rows each at V = 248,320 need more than 8 MiB of
    words (their rows' softmax partials alone are 9.1 MB): refused on the host
    with SV_E_WORKSPACE, nothing launched (the pointers are never read)."""
    lib = sv.load()
    dummy = ctypes.c_void_p(256)
    st = lib.sv_verify_sample_noalloc(dummy, sv.SV_BF16, 4096 * 9, dummy, sv.SV_BF16, 4096 * 8, 248_320, dummy,
                                      dummy, dummy, dummy, 4096, 8, 1.0, dummy, None, -1, dummy, dummy, dummy,
                                      None, None, None, None)
    assert st == 3
    assert b"scratch" in lib.sv_last_error()
    say("  refused: " + lib.sv_last_error().decode())
    # the scratch still serves a call that fits
    c3 = synth.c3_sampled(B=4, k=3, V=9_000, T=1.0, salt=5)
    _both(c3)
