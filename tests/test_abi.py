"""The C-ABI library loads and exports what include/specverify.h declares; host-side
argument checks return their documented codes without launching anything
(CPU only: no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import draft_verify_sampling_amd as sv

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = [os.path.join(INCLUDE, h) for h in ("specverify.h", "specverify_debug.h")]


def _declared():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        names |= set(re.findall(r"^\s*(?:sv_status|int|int32_t|int64_t|size_t|const char\*)\s+(sv_\w+)\s*\(",
                                text, flags=re.M))
    return names


@pytest.fixture(scope="module")
def lib():
    return sv.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert names == set(sv.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strings(lib):
    assert sv.abi_version() == 1
    assert lib.sv_status_string(0) == b"ok"
    assert b"argument" in lib.sv_status_string(1)
    assert lib.sv_status_string(99) == b"unknown status"


def test_workspace_sizes(lib):
    assert sv.workspace_bytes(sv.SV_OP_SAMPLE, 64, 320, 248_320) % 256 == 0
    # softmax partials of every row (31 segments of 8192 at V = 248,320), then
    # the exchange words between the workgroups that share a request
    assert sv.workspace_bytes(sv.SV_OP_SAMPLE, 64, 320, 248_320) >= 320 * 31 * 8 + 64 * 6 * 2 * 8
    assert sv.workspace_bytes(sv.SV_OP_TREE, 32, 1920, 128_256) >= 1920 * 16 * 8 + 32 * 61 * 2 * 8
    assert sv.workspace_bytes(sv.SV_OP_GREEDY, 64, 320, 32_000) >= 320 * 8
    assert sv.workspace_bytes(sv.SV_OP_TREE, 32, 1920, 128_256) >= 1920 * 8
    assert sv.workspace_bytes(sv.SV_OP_SAMPLE, -1, 1, 1) == 0
    assert sv.workspace_bytes(7, 1, 1, 1) == 0


def test_sample_workspace_sizes_know_k_max(lib):
    """The exact query of a sampled chain call: the segment pairs and the
    draw's tile sums at the headline shape (B = 64, k = 4, V = 248,320) come to well under the
    any-k_max bound, which must still cover it; the bound covers every
    k_max; bad sizes give 0."""
    exact = sv.sample_workspace_bytes(64, 320, 248_320, 4)
    bound = sv.workspace_bytes(sv.SV_OP_SAMPLE, 64, 320, 248_320)
    assert exact % 256 == 0 and 0 < exact <= bound
    # segment pairs [64, 5, 31] and tile sums [64, 122] x 2 at least
    assert exact >= 64 * 5 * 31 * 8 + 2 * 64 * 122 * 8
    assert exact < 1 << 20 and bound > 8 * exact
    for k in (0, 1, 7, 30, 31, 63, 255):
        rows = 64 * (k + 1)
        assert 0 < sv.sample_workspace_bytes(64, rows, 151_936, k) <= \
            sv.workspace_bytes(sv.SV_OP_SAMPLE, 64, rows, 151_936)
    assert sv.sample_workspace_bytes(64, 320, 248_320, -1) == 0
    assert sv.sample_workspace_bytes(64, 320, 248_320, 256) == 0
    assert sv.sample_workspace_bytes(0, 320, 248_320, 4) == 0
    assert sv.sample_workspace_bytes(64, 320, 0, 4) == 0


def test_kernel_timing_hook_arguments(lib):
    # host-only: both events or neither (nothing is recorded without a call)
    assert lib.sv_debug_time_kernel_once(None, None) == 0
    assert lib.sv_debug_time_kernel_once(ctypes.c_void_p(256), None) == 1
    assert "both events" in lib.sv_last_error().decode()
    assert lib.sv_debug_time_kernel_once(None, None) == 0


def _err(lib):
    return lib.sv_last_error().decode()


def test_host_checks_sample(lib):
    f = lib.sv_verify_sample
    dummy = ctypes.c_void_p(256)  # never dereferenced: every call below fails on the host
    base = dict(tgt=dummy, tdt=0, t_rows=5, dq=dummy, qdt=0, q_rows=4, V=100, trs=dummy, qrs=dummy,
                ids=dummy, dlen=dummy, B=1, k_max=4, T=1.0, u=dummy, max_new=None, eos=-1,
                out=dummy, cnt=dummy, acc=dummy, diag=None, resid=None, st=None, ws=None, wsb=0,
                stream=None)

    def call(**kw):
        a = {**base, **kw}
        return f(*a.values())

    assert call(T=0.0) == 1 and "temperature" in _err(lib)
    assert call(T=float("nan")) == 1
    assert call(T=-1.0) == 1
    assert call(tdt=5) == 2
    assert call(qdt=-1) == 2
    assert call(k_max=256) == 1
    assert call(V=0) == 1
    assert call(V=(1 << 22) + 1) == 1 and "vocab" in _err(lib)
    assert call(B=-1) == 1
    assert call(tgt=None) == 1 and "null" in _err(lib)
    assert call() == 3 and "workspace" in _err(lib)                     # workspace NULL
    assert call(ws=ctypes.c_void_p(4096 + 8), wsb=1 << 30) == 3          # misaligned
    assert call(ws=ctypes.c_void_p(4096), wsb=16) == 3                   # too small
    assert call(B=0) == 0                                                # nothing to do


def test_host_checks_greedy_tree_ngram(lib):
    d = ctypes.c_void_p(256)
    g = lib.sv_verify_greedy
    assert g(d, 3, 5, 100, d, d, d, 1, 4, None, -1, d, d, d, None, None, 0, None) == 2
    assert g(d, 1, 5, 100, d, d, d, 1, 300, None, -1, d, d, d, None, None, 0, None) == 1
    assert g(d, 1, 5, 100, d, d, d, 1, 4, None, -1, d, d, d, None, None, 0, None) == 3
    t = lib.sv_verify_tree
    assert t(d, 1, d, 1, 100, d, d, 1, 0, 1.0, d, d, d, d, d, None, None, None, 0, None) == 1
    assert t(d, 1, d, 1, 100, d, d, 1, 2000, 1.0, d, d, d, d, d, None, None, None, 0, None) == 1
    assert t(d, 1, d, 1, (1 << 22) + 1, d, d, 1, 60, 1.0, d, d, d, d, d, None, None, None, 0, None) == 1
    assert t(d, 1, d, 1, 100, d, d, 1, 60, 0.0, d, d, d, d, d, None, None, None, 0, None) == 1
    assert t(d, 1, d, 1, 100, d, d, 1, 60, 1.0, d, d, d, d, d, None, None, None, 0, None) == 3
    tg = lib.sv_verify_tree_greedy
    assert tg(d, 3, 100, d, d, 1, 60, d, d, d, d, None, None, 0, None) == 2
    assert tg(d, 1, 100, d, d, 1, 0, d, d, d, d, None, None, 0, None) == 1
    assert tg(d, 1, 0, d, d, 1, 60, d, d, d, d, None, None, 0, None) == 1
    assert tg(None, 1, 100, d, d, 1, 60, d, d, d, d, None, None, 0, None) == 1
    assert tg(d, 1, 100, d, d, 1, 60, d, d, d, d, None, None, 0, None) == 3   # no workspace
    assert tg(d, 1, 100, d, d, 0, 60, d, d, d, d, None, None, 0, None) == 0   # nothing to do
    tp = lib.sv_verify_tree_pointmass
    assert tp(d, 1, 100, d, d, 1, 60, 0.0, d, d, d, d, d, None, None, 0, None) == 1
    assert tp(d, 1, 100, d, d, 1, 60, 1.0, None, d, d, d, d, None, None, 0, None) == 1
    assert tp(d, 1, (1 << 22) + 1, d, d, 1, 60, 1.0, d, d, d, d, d, None, None, 0, None) == 1
    assert tp(d, 1, 100, d, d, 1, 1025, 1.0, d, d, d, d, d, None, None, 0, None) == 1
    assert tp(d, 1, 100, d, d, 1, 60, 1.0, d, d, d, d, d, None, None, 0, None) == 3
    te = lib.sv_tree_expand
    base = [d, 1, 100, 2, 4, d, 4, 4, 85, d, d, d, d, d, d, d, None, None, 0, None]

    def expand(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return te(*a)

    assert expand(a1=7) == 2                                  # dtype
    assert expand(a4=0) == 1 and expand(a4=65) == 1           # n_exp
    assert expand(a5=None) == 1                               # first round needs n_exp == 1
    assert expand(a6=0) == 1 and expand(a6=17) == 1           # top_children
    assert expand(a2=3) == 1                                  # vocab < top_children
    assert expand(a7=0) == 1                                  # expand_next
    assert expand(a8=1025) == 1                               # max_cand
    assert expand(a9=None) == 1                               # null candidate array
    assert expand() == 3                                      # no workspace
    assert expand(a3=0) == 0                                  # nothing to do
    tf = lib.sv_tree_finalize
    assert tf(2, 85, d, d, d, d, d, d, 0, d, d, d, d, None, None, None) == 1
    assert tf(2, 2000, d, d, d, d, d, d, 60, d, d, d, d, None, None, None) == 1
    assert tf(2, 85, d, d, d, d, d, d, 60, None, d, d, d, None, None, None) == 1
    assert tf(0, 85, d, d, d, d, d, d, 60, d, d, d, d, None, None, None) == 0
    ss = lib.sv_shard_stats
    hb = (ctypes.c_int64 * 3)(0, 40, 100)

    def stats(**kw):
        a = [d, 1, 5, d, 1, 4, 100, hb, 2, 0, d, d, d, d, 1, 4, 1.0, d, d, d, 1 << 20, None]
        for i, v in kw.items():
            a[int(i[1:])] = v
        return ss(*a)

    assert stats(a1=9) == 2
    assert stats(a8=0) == 1 and stats(a8=65) == 1           # shard count
    assert stats(a9=2) == 1 and stats(a9=-1) == 1            # shard index
    assert stats(a6=99) == 1                                 # bounds must end at vocab
    assert stats(a7=None) == 1                               # bounds are required
    bad = (ctypes.c_int64 * 3)(0, 100, 100)
    assert stats(a7=bad) == 1                                # bounds must increase
    assert stats(a16=0.0) == 1
    assert stats(a15=256) == 1
    assert stats(a18=None, a19=None, a20=0) == 3             # workspace
    assert stats(a14=0) == 0
    n = lib.sv_ngram_draft
    assert n(d, d, 1, 16, 0, 4, d, d, None, None) == 1
    assert n(d, d, 1, 16, 65, 4, d, d, None, None) == 1
    assert n(d, d, 1, 16, 3, -1, d, d, None, None) == 1
    assert n(d, d, 1, 0, 3, 4, d, d, None, None) == 1
    assert n(None, d, 1, 16, 3, 4, d, d, None, None) == 1
    assert n(d, d, 0, 16, 3, 4, d, d, None, None) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    import importlib
    monkeypatch.setenv("SPECVERIFY_LIB", str(tmp_path / "nope.so"))
    mod = importlib.reload(sv)
    try:
        with pytest.raises(mod.SpecVerifyError):
            mod.load()
    finally:
        monkeypatch.delenv("SPECVERIFY_LIB")
        importlib.reload(sv)


def test_binding_rejects_mismatched_buffers():
    """Caller-provided outputs and index arrays must match the call's sizes
    (the kernels index them by B, k_max, N): a mismatch raises before any
    launch.  CPU tensors suffice, the shape checks come first."""
    import torch
    B, k, V = 4, 3, 50
    tgt = torch.zeros((B * (k + 1), V))
    dft = torch.zeros((B * k, V))
    trs = torch.zeros(B, dtype=torch.int32)
    ids = torch.zeros((B, k), dtype=torch.int32)
    dl = torch.full((B,), k, dtype=torch.int32)
    u = torch.zeros((B, k + 1))
    bad_out = (torch.zeros((B, k), dtype=torch.int32), torch.zeros(B, dtype=torch.int32),
               torch.zeros(B, dtype=torch.int32), None, None)
    with pytest.raises(sv.SpecVerifyError, match="out tokens must have shape"):
        sv.sv_verify_sample(tgt, dft, trs, trs, ids, dl, 1.0, u, out=bad_out)
    with pytest.raises(sv.SpecVerifyError, match="t_row_start must have shape"):
        sv.sv_verify_sample(tgt, dft, trs[:2], trs, ids, dl, 1.0, u)
    with pytest.raises(sv.SpecVerifyError, match="out must be"):
        sv.sv_softmax_partials(tgt, 1.0, out=torch.zeros((B, 1, 2)))
    par = torch.zeros((B, 5), dtype=torch.int32)
    with pytest.raises(sv.SpecVerifyError, match="node_token must have shape"):
        sv.sv_verify_tree_greedy(torch.zeros((B * 5, V)), par, par[:, :4])
    with pytest.raises(sv.SpecVerifyError, match="out path must have shape"):
        sv.sv_verify_tree_pointmass(torch.zeros((B * 5, V)), par, par, 1.0, torch.zeros((B, 5)),
                                    out=(par, par[:, 0], par[:, 0], par[:, :3]))
