"""The measurement hooks of include/specverify_debug.h on an MI355X, through
the C ABI: the streaming read folds every 32-bit word of each 64 KiB chunk with
xor (so none of its loads can be dropped), and the timing hook hands its events
to the streaming kernel of the next call only."""
import numpy as np
import pytest
import torch

import draft_verify_sampling_amd as sv
import synth
from tests.gpu_util import say, rows_to_dev, i32, f32, DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 65536, (1 << 20) + 48, 3 * 65536 - 16])
def test_gpu_read_ceiling_folds_every_word(nbytes):
    say(f"read ceiling over {nbytes} bytes")
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32).copy()).to(DEV)
    out = sv.sv_debug_read_ceiling(buf)
    torch.cuda.synchronize()
    chunk = 65536 // 4
    pad = (-host.size) % chunk
    want = np.bitwise_xor.reduce(np.concatenate([host, np.zeros(pad, np.uint32)]).reshape(-1, chunk), axis=1)
    got = out.cpu().numpy().view(np.uint32)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def test_gpu_timing_hook_times_one_call():
    """Armed, the next call's streaming kernel takes the events (a positive
    duration below the whole call's); the call after that leaves them as they
    were (the hook disarms)."""
    say("timing hook around the statistics of one sampled call")
    rng = np.random.default_rng(5)
    ks = rng.integers(0, 5, size=32)
    ci = synth.sampled_chain(401, 32, ks, 65_536, 0.8, sd=2.0, n_boost=3, boost=4.0, sigma=1.0, kind="bf16")
    args = (rows_to_dev(ci.target, ci.t_kind), rows_to_dev(ci.draft, ci.q_kind), i32(ci.t_row_start),
            i32(ci.q_row_start), i32(ci.draft_ids[:, :ci.k_max]), i32(ci.draft_len), ci.T, f32(ci.uniforms))
    sv.sv_verify_sample(*args)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sv.sv_debug_time_kernel_once(e0, e1)
    c0.record()
    sv.sv_verify_sample(*args)
    c1.record()
    torch.cuda.synchronize()
    k_ms, call_ms = e0.elapsed_time(e1), c0.elapsed_time(c1)
    say(f"  kernel {1e3 * k_ms:.1f} us, call {1e3 * call_ms:.1f} us")
    assert 0.0 < k_ms < call_ms
    sv.sv_verify_sample(*args)   # disarmed: the events keep their times
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) == k_ms
