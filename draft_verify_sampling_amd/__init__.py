"""Python binding of libspecverify (the verify step of speculative decoding on
MI355X / gfx950).

Argument marshalling only: every step of the verify path runs in the HIP
kernels of ``libspecverify.so``; torch supplies device memory (tensors) and
the current stream.  The functions carry the names of the C entry points
declared in ``include/specverify.h`` and follow its contracts.

There is no fallback: if the shared library is missing or cannot be loaded,
every call raises ``SpecVerifyError``.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

__all__ = [
    "SpecVerifyError", "lib_path", "load", "abi_version", "workspace_bytes",
    "sv_ngram_draft", "sv_verify_greedy", "sv_verify_sample", "sv_verify_tree",
    "sv_softmax_partials", "sv_softmax_segments", "SV_F32", "SV_BF16", "SV_OP_GREEDY", "SV_OP_SAMPLE", "SV_OP_TREE",
    "FLAG_BAD_REQUEST", "FLAG_BAD_TOKEN", "FLAG_NONFINITE", "FLAG_OVER_BUDGET",
    "FLAG_FALLBACK", "FLAG_BAD_TREE", "FLAG_SYNC_TIMEOUT", "EXPORTS",
]

SV_F32, SV_BF16 = 0, 1
SV_OP_GREEDY, SV_OP_SAMPLE, SV_OP_TREE = 0, 1, 2
FLAG_BAD_REQUEST, FLAG_BAD_TOKEN, FLAG_NONFINITE = 1, 2, 4
FLAG_OVER_BUDGET, FLAG_FALLBACK, FLAG_BAD_TREE, FLAG_SYNC_TIMEOUT = 8, 16, 32, 64

EXPORTS = ("sv_abi_version", "sv_status_string", "sv_last_error", "sv_workspace_bytes",
           "sv_softmax_segments", "sv_softmax_partials",
           "sv_ngram_draft", "sv_verify_greedy", "sv_verify_sample", "sv_verify_tree")

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None
_LOCK = threading.Lock()

P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64
SZ = ctypes.c_size_t
F32 = ctypes.c_float

_SIGS = {
    "sv_abi_version": (ctypes.c_int, []),
    "sv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sv_last_error": (ctypes.c_char_p, []),
    "sv_workspace_bytes": (SZ, [ctypes.c_int, I64, I64, I64]),
    "sv_softmax_segments": (I32, [I64, I64]),
    "sv_softmax_partials": (ctypes.c_int, [P, I32, I64, I64, F32, P, P]),
    "sv_ngram_draft": (ctypes.c_int, [P, P, I32, I32, I32, I32, P, P, P, P]),
    "sv_verify_greedy": (ctypes.c_int, [P, I32, I32, I64, P, P, P, I32, I32, P, I32,
                                        P, P, P, P, P, SZ, P]),
    "sv_verify_sample": (ctypes.c_int, [P, I32, I32, P, I32, I32, I64, P, P, P, P, I32, I32,
                                        F32, P, P, I32, P, P, P, P, P, P, P, SZ, P]),
    "sv_verify_tree": (ctypes.c_int, [P, I32, P, I32, I64, P, P, I32, I32, F32, P, P, P,
                                      P, P, P, P, P, SZ, P]),
}


class SpecVerifyError(RuntimeError):
    """A libspecverify call failed, or the library is not available."""


def lib_path() -> str:
    return os.environ.get("SPECVERIFY_LIB", os.path.join(_HERE, "libspecverify.so"))


def load():
    """Load libspecverify.so (once) and declare its signatures."""
    global _LIB
    with _LOCK:
        if _LIB is None:
            path = lib_path()
            if not os.path.exists(path):
                raise SpecVerifyError(
                    f"{path} is not built; run `python -m draft_verify_sampling_amd.build`")
            try:
                lib = ctypes.CDLL(path)
            except OSError as e:
                raise SpecVerifyError(f"cannot load {path}: {e}") from e
            for name, (res, args) in _SIGS.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _LIB = lib
    return _LIB


def abi_version() -> int:
    return int(load().sv_abi_version())


def workspace_bytes(op: int, batch: int, total_rows: int, vocab: int) -> int:
    return int(load().sv_workspace_bytes(op, batch, total_rows, vocab))


def _check(status: int, what: str):
    if status != 0:
        lib = load()
        raise SpecVerifyError(f"{what}: {lib.sv_status_string(status).decode()} "
                              f"({lib.sv_last_error().decode()})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise SpecVerifyError(f"unsupported row dtype {t.dtype}")


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, device=None):
    """Device pointer of a contiguous tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise SpecVerifyError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise SpecVerifyError(f"{name} must be on the GPU")
    if device is not None and t.device != device:
        raise SpecVerifyError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise SpecVerifyError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise SpecVerifyError(f"{name} must be contiguous")
    return t.data_ptr() if t.numel() else None


def _stream(stream) -> Optional[int]:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream or None


class Workspace:
    """Caller-side workspace: a device buffer grown on demand and reused across
    calls on one stream (the library needs no particular initial contents)."""

    def __init__(self, device=None):
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        self.buf = None

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf


_DEFAULT_WS: dict = {}


def _workspace(ws: Optional[Workspace], device, stream, nbytes: int) -> torch.Tensor:
    if ws is None:
        key = (str(device), _stream(stream))
        ws = _DEFAULT_WS.setdefault(key, Workspace(device))
    return ws.get(nbytes)


def sv_softmax_segments(n_rows: int, vocab: int) -> int:
    return int(load().sv_softmax_segments(n_rows, vocab))


def sv_softmax_partials(rows: torch.Tensor, temperature: float, out: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """Per-segment softmax pairs of every row: returns float32 [n_rows, nseg, 2]
    (scaled-domain max, sum); see include/specverify.h."""
    lib = load()
    n_rows, V = rows.shape
    nseg = sv_softmax_segments(n_rows, V)
    if out is None:
        out = torch.empty((n_rows, nseg, 2), dtype=torch.float32, device=rows.device)
    _check(lib.sv_softmax_partials(_dev(rows, "rows"), _dtype_code(rows), n_rows, V,
                                   float(temperature), _dev(out, "out", torch.float32, rows.device),
                                   _stream(stream)), "sv_softmax_partials")
    return out


def prepare_softmax_partials(rows: torch.Tensor, temperature: float, out: torch.Tensor, stream=None):
    """sv_softmax_partials with its arguments marshalled once: returns a
    callable that enqueues the same launch again (for tight launch loops
    whose host cost must stay below the kernel's run time).  The callable
    holds the tensors it points into."""
    lib = load()
    n_rows, V = rows.shape
    nseg = sv_softmax_segments(n_rows, V)
    if out.shape != (n_rows, nseg, 2):
        raise SpecVerifyError(f"out must be [{n_rows}, {nseg}, 2]")
    args = (_dev(rows, "rows"), _dtype_code(rows), n_rows, V, float(temperature),
            _dev(out, "out", torch.float32, rows.device), _stream(stream))
    fn = lib.sv_softmax_partials
    keep = (rows, out)

    def launch():
        _ = keep
        status = fn(*args)
        if status != 0:
            _check(status, "sv_softmax_partials")

    return launch


def sv_ngram_draft(ctx: torch.Tensor, ctx_len: torch.Tensor, window: int, k: int,
                   dev_status: Optional[torch.Tensor] = None, stream=None):
    """Prompt-lookup drafts: returns (draft_ids int32 [B, k], draft_len int32 [B])."""
    lib = load()
    B, stride = ctx.shape
    ids = torch.empty((B, k), dtype=torch.int32, device=ctx.device)
    lens = torch.empty((B,), dtype=torch.int32, device=ctx.device)
    _check(lib.sv_ngram_draft(_dev(ctx, "ctx", torch.int32), _dev(ctx_len, "ctx_len", torch.int32),
                              B, stride, window, k, _dev(ids, "draft_ids"), _dev(lens, "draft_len"),
                              _dev(dev_status, "dev_status", torch.int32), _stream(stream)),
           "sv_ngram_draft")
    return ids, lens


def sv_verify_greedy(target: torch.Tensor, t_row_start: torch.Tensor, draft_ids: torch.Tensor,
                     draft_len: torch.Tensor, max_new: Optional[torch.Tensor] = None,
                     eos_id: int = -1, dev_status: Optional[torch.Tensor] = None,
                     workspace: Optional[Workspace] = None, stream=None):
    """Greedy verify; returns (tokens [B, k_max+1], count [B], accepted [B])."""
    lib = load()
    t_rows, V = target.shape
    B = draft_len.shape[0]
    k_max = draft_ids.shape[1] if draft_ids.dim() == 2 else 0
    dev = target.device
    tok = torch.empty((B, k_max + 1), dtype=torch.int32, device=dev)
    cnt = torch.empty((B,), dtype=torch.int32, device=dev)
    acc = torch.empty((B,), dtype=torch.int32, device=dev)
    nb = workspace_bytes(SV_OP_GREEDY, B, t_rows, V)
    ws = _workspace(workspace, dev, stream, nb)
    _check(lib.sv_verify_greedy(_dev(target, "target"), _dtype_code(target), t_rows, V,
                                _dev(t_row_start, "t_row_start", torch.int32, dev),
                                _dev(draft_ids, "draft_ids", torch.int32, dev),
                                _dev(draft_len, "draft_len", torch.int32, dev), B, k_max,
                                _dev(max_new, "max_new", torch.int32, dev), eos_id,
                                _dev(tok, "out"), _dev(cnt, "cnt"), _dev(acc, "acc"),
                                _dev(dev_status, "dev_status", torch.int32, dev),
                                ws.data_ptr(), ws.numel(), _stream(stream)),
           "sv_verify_greedy")
    return tok, cnt, acc


def _sample_args(target, draft, t_row_start, q_row_start, draft_ids, draft_len, temperature, uniforms,
                 max_new, eos_id, diag, dev_status, workspace, stream, out, resid):
    """Checked, marshalled argument list of sv_verify_sample and its outputs."""
    t_rows, V = target.shape
    q_rows = draft.shape[0]
    if draft.shape[1] != V:
        raise SpecVerifyError("target and draft rows differ in length")
    B = draft_len.shape[0]
    k_max = draft_ids.shape[1] if draft_ids.dim() == 2 else 0
    if uniforms.shape != (B, k_max + 1):
        raise SpecVerifyError(f"uniforms must be [B, k_max+1] = [{B}, {k_max + 1}]")
    dev = target.device
    if out is None:
        tok = torch.empty((B, k_max + 1), dtype=torch.int32, device=dev)
        cnt = torch.empty((B,), dtype=torch.int32, device=dev)
        acc = torch.empty((B,), dtype=torch.int32, device=dev)
        dg = torch.zeros((B, k_max + 1, 4), dtype=torch.float32, device=dev) if diag else None
        want_resid = diag if resid is None else resid
        rs = torch.zeros((B,), dtype=torch.float32, device=dev) if want_resid else None
    else:
        tok, cnt, acc, dg, rs = out
    nb = workspace_bytes(SV_OP_SAMPLE, B, t_rows, V)
    ws = _workspace(workspace, dev, stream, nb)
    args = (_dev(target, "target"), _dtype_code(target), t_rows,
            _dev(draft, "draft"), _dtype_code(draft), q_rows, V,
            _dev(t_row_start, "t_row_start", torch.int32, dev),
            _dev(q_row_start, "q_row_start", torch.int32, dev),
            _dev(draft_ids, "draft_ids", torch.int32, dev),
            _dev(draft_len, "draft_len", torch.int32, dev), B, k_max,
            float(temperature), _dev(uniforms, "uniforms", torch.float32, dev),
            _dev(max_new, "max_new", torch.int32, dev), eos_id,
            _dev(tok, "out"), _dev(cnt, "cnt"), _dev(acc, "acc"),
            _dev(dg, "diag", torch.float32, dev), _dev(rs, "resid", torch.float32, dev),
            _dev(dev_status, "dev_status", torch.int32, dev),
            ws.data_ptr(), ws.numel(), _stream(stream))
    return args, (tok, cnt, acc, dg, rs), ws


def sv_verify_sample(target: torch.Tensor, draft: torch.Tensor, t_row_start: torch.Tensor,
                     q_row_start: torch.Tensor, draft_ids: torch.Tensor, draft_len: torch.Tensor,
                     temperature: float, uniforms: torch.Tensor,
                     max_new: Optional[torch.Tensor] = None, eos_id: int = -1,
                     diag: bool = False, dev_status: Optional[torch.Tensor] = None,
                     workspace: Optional[Workspace] = None, stream=None, out=None,
                     resid: Optional[bool] = None):
    """Speculative-sampling verify.  Returns (tokens [B, k_max+1], count, accepted,
    diag [B, k_max+1, 4] or None, resid [B] or None).  ``out`` may pass a
    preallocated (tokens, count, accepted, diag, resid) tuple.  ``resid``
    (default: same as ``diag``) asks for the residual masses."""
    lib = load()
    args, outs, _ = _sample_args(target, draft, t_row_start, q_row_start, draft_ids, draft_len, temperature,
                                 uniforms, max_new, eos_id, diag, dev_status, workspace, stream, out, resid)
    _check(lib.sv_verify_sample(*args), "sv_verify_sample")
    return outs


def prepare_verify_sample(target: torch.Tensor, draft: torch.Tensor, t_row_start: torch.Tensor,
                          q_row_start: torch.Tensor, draft_ids: torch.Tensor, draft_len: torch.Tensor,
                          temperature: float, uniforms: torch.Tensor,
                          max_new: Optional[torch.Tensor] = None, eos_id: int = -1,
                          diag: bool = False, dev_status: Optional[torch.Tensor] = None,
                          workspace: Optional[Workspace] = None, stream=None, out=None,
                          resid: Optional[bool] = None):
    """sv_verify_sample with its arguments checked and marshalled once.  Returns
    (launch, outputs): launch() enqueues the same call again on the same
    buffers, for loops whose host cost must stay below the GPU's.  The
    callable holds every tensor it points into (the workspace buffer too), so
    none is freed while it lives."""
    lib = load()
    args, outs, ws = _sample_args(target, draft, t_row_start, q_row_start, draft_ids, draft_len, temperature,
                                  uniforms, max_new, eos_id, diag, dev_status, workspace, stream, out, resid)
    fn = lib.sv_verify_sample
    keep = (target, draft, t_row_start, q_row_start, draft_ids, draft_len, uniforms, max_new, dev_status,
            outs, ws)

    def launch():
        _ = keep
        status = fn(*args)
        if status != 0:
            _check(status, "sv_verify_sample")

    return launch, outs


def sv_verify_tree(target: torch.Tensor, draft: torch.Tensor, parent: torch.Tensor,
                   node_token: torch.Tensor, temperature: float, uniforms: torch.Tensor,
                   diag: bool = False, dev_status: Optional[torch.Tensor] = None,
                   workspace: Optional[Workspace] = None, stream=None, out=None):
    """Tree verify.  target/draft rows [B*N, V]; parent/node_token/uniforms [B, N].
    Returns (tokens [B, N], count, accepted, path [B, N], diag [B, N, 4] or None)."""
    lib = load()
    B, N = parent.shape
    rows, V = target.shape
    if rows != B * N or draft.shape != target.shape:
        raise SpecVerifyError("target/draft must be [B*N, V]")
    dev = target.device
    if out is None:
        tok = torch.empty((B, N), dtype=torch.int32, device=dev)
        cnt = torch.empty((B,), dtype=torch.int32, device=dev)
        acc = torch.empty((B,), dtype=torch.int32, device=dev)
        pth = torch.empty((B, N), dtype=torch.int32, device=dev)
        dg = torch.zeros((B, N, 4), dtype=torch.float32, device=dev) if diag else None
    else:
        tok, cnt, acc, pth, dg = out
    nb = workspace_bytes(SV_OP_TREE, B, B * N, V)
    ws = _workspace(workspace, dev, stream, nb)
    _check(lib.sv_verify_tree(_dev(target, "target"), _dtype_code(target), _dev(draft, "draft"),
                              _dtype_code(draft), V, _dev(parent, "parent", torch.int32, dev),
                              _dev(node_token, "node_token", torch.int32, dev), B, N,
                              float(temperature), _dev(uniforms, "uniforms", torch.float32, dev),
                              _dev(tok, "out"), _dev(cnt, "cnt"), _dev(acc, "acc"), _dev(pth, "path"),
                              _dev(dg, "diag", torch.float32, dev),
                              _dev(dev_status, "dev_status", torch.int32, dev),
                              ws.data_ptr(), ws.numel(), _stream(stream)),
           "sv_verify_tree")
    return tok, cnt, acc, pth, dg
