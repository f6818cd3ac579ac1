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
import functools
import inspect
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
    "sv_verify_tree_greedy", "sv_verify_tree_pointmass", "prepare", "prepare_verify_sample",
    "sv_philox_uniforms", "sv_verify_sample_philox", "DraftTreeState", "sv_tree_expand",
    "sv_tree_finalize", "SV_OP_TREE_EXPAND", "SV_OP_SHARD", "sv_shard_stats", "sv_shard_residual",
    "sv_shard_draw",
    "prepare_softmax_partials", "sv_debug_time_kernel_once", "sv_debug_read_ceiling", "sample_workspace_bytes",
    "sv_verify_sample_noalloc",
]

SV_F32, SV_BF16 = 0, 1
SV_OP_GREEDY, SV_OP_SAMPLE, SV_OP_TREE, SV_OP_TREE_EXPAND, SV_OP_SHARD = 0, 1, 2, 3, 4
FLAG_BAD_REQUEST, FLAG_BAD_TOKEN, FLAG_NONFINITE = 1, 2, 4
FLAG_OVER_BUDGET, FLAG_FALLBACK, FLAG_BAD_TREE, FLAG_SYNC_TIMEOUT = 8, 16, 32, 64

EXPORTS = ("sv_abi_version", "sv_status_string", "sv_last_error", "sv_workspace_bytes",
           "sv_softmax_segments", "sv_softmax_partials",
           "sv_ngram_draft", "sv_verify_greedy", "sv_verify_sample", "sv_verify_tree",
           "sv_verify_tree_greedy", "sv_verify_tree_pointmass", "sv_philox_uniforms",
           "sv_verify_sample_philox", "sv_tree_expand", "sv_tree_finalize", "sv_shard_stats",
           "sv_shard_residual", "sv_shard_draw", "sv_sample_workspace_bytes", "sv_verify_sample_noalloc",
           "sv_debug_time_kernel_once", "sv_debug_read_blocks", "sv_debug_read_ceiling")

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None
_LOCK = threading.Lock()

P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64
SZ = ctypes.c_size_t
U64 = ctypes.c_uint64
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
    "sv_verify_tree_greedy": (ctypes.c_int, [P, I32, I64, P, P, I32, I32, P, P, P, P, P, P, SZ, P]),
    "sv_philox_uniforms": (ctypes.c_int, [U64, U64, I32, I32, P, P]),
    "sv_debug_time_kernel_once": (ctypes.c_int, [P, P]),
    "sv_debug_read_blocks": (I64, [I64]),
    "sv_debug_read_ceiling": (ctypes.c_int, [P, I64, P, P]),
    "sv_sample_workspace_bytes": (SZ, [I64, I64, I64, I32]),
    "sv_tree_expand": (ctypes.c_int, [P, I32, I64, I32, I32, P, I32, I32, I32, P, P, P, P, P, P, P, P,
                                      P, SZ, P]),
    "sv_tree_finalize": (ctypes.c_int, [I32, I32, P, P, P, P, P, P, I32, P, P, P, P, P, P, P]),
    "sv_shard_stats": (ctypes.c_int, [P, I32, I32, P, I32, I32, I64, P, I32, I32, P, P, P, P, I32, I32, F32,
                                      P, P, P, SZ, P]),
    "sv_shard_residual": (ctypes.c_int, [P, I32, I32, P, I32, I32, I64, P, I32, I32, P, P, P, P, I32, I32,
                                         F32, P, P, P, P, P, SZ, P]),
    "sv_shard_draw": (ctypes.c_int, [P, I32, I32, P, I32, I32, I64, P, I32, I32, P, P, P, P, I32, I32, F32,
                                     P, P, P, P, I32, P, P, P, P, P, P, SZ, P]),
    "sv_verify_sample_noalloc": (ctypes.c_int, [P, I32, I32, P, I32, I32, I64, P, P, P, P, I32, I32,
                                                F32, P, P, I32, P, P, P, P, P, P, P]),
    "sv_verify_sample_philox": (ctypes.c_int, [P, I32, I32, P, I32, I32, I64, P, P, P, P, I32, I32,
                                               F32, U64, U64, P, I32, P, P, P, P, P, P, P, SZ, P]),
    "sv_verify_tree_pointmass": (ctypes.c_int, [P, I32, I64, P, P, I32, I32, F32, P, P, P, P, P,
                                                P, P, SZ, P]),
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


def sample_workspace_bytes(batch: int, t_rows: int, vocab: int, k_max: int) -> int:
    """Workspace bytes one sampled chain call with these sizes checks for."""
    return int(load().sv_sample_workspace_bytes(batch, t_rows, vocab, k_max))


def sv_debug_time_kernel_once(before=None, after=None):
    """Arm the measurement hook (include/specverify_debug.h): the calling
    thread's next verify call hands torch.cuda.Event `before` / `after` to
    the launch of the kernel that streams its rows, so they take that
    kernel's own start and end (None, None disarms).  The events are created
    here if they are not yet."""
    if (before is None) != (after is None):
        raise SpecVerifyError("give both events or neither")
    ptrs = []
    for e in (before, after):
        if e is None:
            ptrs.append(None)
            continue
        if not e.cuda_event:  # torch creates its events on first use
            e.record()
        ptrs.append(ctypes.c_void_p(e.cuda_event))
    _check(load().sv_debug_time_kernel_once(*ptrs), "sv_debug_time_kernel_once")


def sv_debug_read_ceiling(buf: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """A pure streaming read of the bytes of `buf` (a measurement of the HBM
    read ceiling); returns the per-block fold values (uint32 as int32)."""
    nbytes = buf.numel() * buf.element_size()
    nb = int(load().sv_debug_read_blocks(nbytes))
    if out is None:
        out = torch.empty((max(nb, 1),), dtype=torch.int32, device=buf.device)
    args = (_dev(buf, "buf"), nbytes, _dev(out, "out"), _stream(stream))
    return _invoke("sv_debug_read_ceiling", args, (buf, out), out)


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


def _shape(t: Optional[torch.Tensor], name: str, shape, dtype=None):
    """A caller-provided tensor must have exactly the shape (and dtype) the
    call reads or writes: the kernels index it by the call's sizes."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise SpecVerifyError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise SpecVerifyError(f"{name} must be {dtype}, got {t.dtype}")


def _status_arg(t: Optional[torch.Tensor]):
    if t is not None and (t.numel() < 1 or t.dtype != torch.int32):
        raise SpecVerifyError("dev_status must be an int32 tensor with at least one element")


def _stream(stream) -> Optional[int]:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream or None


def _on_call_stream(fn):
    """Run a binding call with its `stream` argument as torch's current stream,
    so that every tensor the binding allocates or fills for the call (outputs,
    zeroed diagnostics, a grown workspace) is made on the stream the kernels
    run on: the fills are ordered before the kernels, and the caching
    allocator hands a freed buffer out again only after the work queued on
    that stream."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def call(*args, **kwargs):
        stream = sig.bind_partial(*args, **kwargs).arguments.get("stream")
        if stream is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(stream):
            return fn(*args, **kwargs)

    return call


class Workspace:
    """Caller-side workspace: a device buffer grown on demand and reused across
    calls on one stream (the library needs no particular initial contents)."""

    def __init__(self, device=None):
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        self.buf = None
        self.last_stream = None

    def get(self, nbytes: int) -> torch.Tensor:
        cur = torch.cuda.current_stream(self.device)
        if self.buf is None or self.buf.numel() < nbytes:
            if self.buf is not None:
                # the old buffer may still be in use by work queued on the
                # stream of its last call: free it only after that work
                self.buf.record_stream(self.last_stream)
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        self.last_stream = cur
        return self.buf


_DEFAULT_WS: dict = {}


def _workspace(ws: Optional[Workspace], device, stream, nbytes: int) -> torch.Tensor:
    if ws is None:
        key = (str(device), _stream(stream))
        ws = _DEFAULT_WS.setdefault(key, Workspace(device))
    return ws.get(nbytes)


# ---- calling the library -----------------------------------------------------
#
# Every entry point below checks its arguments, marshals them into one
# argument tuple and hands it to _invoke, which calls the C function -- or,
# inside prepare(), records the call so that it can be enqueued again later
# without the host work of checking and marshalling.

_CAPTURE = threading.local()


def _invoke(name: str, args: tuple, keep: tuple, result):
    rec = getattr(_CAPTURE, "calls", None)
    fn = getattr(load(), name)
    if rec is not None:
        rec.append((fn, args, keep, name))
    else:
        _check(fn(*args), name)
    return result


def prepare(fn, *args, **kwargs):
    """Check and marshal one call of a binding function (sv_verify_sample,
    sv_verify_tree, ...) without running it.  Returns (launch, result):
    launch() enqueues the identical call (same tensors, same stream, same
    workspace buffer) and result holds the output tensors it writes.  For
    loops whose host cost must stay below the GPU's run time.  The launcher
    holds every tensor it points into, so none is freed while it lives."""
    if getattr(_CAPTURE, "calls", None) is not None:
        raise SpecVerifyError("prepare() does not nest")
    _CAPTURE.calls = []
    try:
        result = fn(*args, **kwargs)
        calls = _CAPTURE.calls
    finally:
        _CAPTURE.calls = None

    def launch():
        for f, a, keep, name in calls:
            status = f(*a)
            if status != 0:
                _check(status, name)

    launch.held = [c[2] for c in calls]
    return launch, result


def sv_softmax_segments(n_rows: int, vocab: int) -> int:
    return int(load().sv_softmax_segments(n_rows, vocab))


@_on_call_stream
def sv_softmax_partials(rows: torch.Tensor, temperature: float, out: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """Per-segment softmax pairs of every row: returns float32 [n_rows, nseg, 2]
    (scaled-domain max, sum); see include/specverify.h."""
    n_rows, V = rows.shape
    nseg = sv_softmax_segments(n_rows, V)
    if out is None:
        out = torch.empty((n_rows, nseg, 2), dtype=torch.float32, device=rows.device)
    elif tuple(out.shape) != (n_rows, nseg, 2):
        raise SpecVerifyError(f"out must be [{n_rows}, {nseg}, 2], got {tuple(out.shape)}")
    args = (_dev(rows, "rows"), _dtype_code(rows), n_rows, V, float(temperature),
            _dev(out, "out", torch.float32, rows.device), _stream(stream))
    return _invoke("sv_softmax_partials", args, (rows, out), out)


def prepare_softmax_partials(rows: torch.Tensor, temperature: float, out: torch.Tensor, stream=None):
    """prepare(sv_softmax_partials, ...): the launcher alone."""
    return prepare(sv_softmax_partials, rows, temperature, out=out, stream=stream)[0]


@_on_call_stream
def sv_ngram_draft(ctx: torch.Tensor, ctx_len: torch.Tensor, window: int, k: int,
                   dev_status: Optional[torch.Tensor] = None, stream=None):
    """Prompt-lookup drafts: returns (draft_ids int32 [B, k], draft_len int32 [B])."""
    B, stride = ctx.shape
    _shape(ctx_len, "ctx_len", (B,))
    _status_arg(dev_status)
    ids = torch.empty((B, k), dtype=torch.int32, device=ctx.device)
    lens = torch.empty((B,), dtype=torch.int32, device=ctx.device)
    args = (_dev(ctx, "ctx", torch.int32), _dev(ctx_len, "ctx_len", torch.int32), B, stride, window, k,
            _dev(ids, "draft_ids"), _dev(lens, "draft_len"), _dev(dev_status, "dev_status", torch.int32),
            _stream(stream))
    return _invoke("sv_ngram_draft", args, (ctx, ctx_len, ids, lens, dev_status), (ids, lens))


@_on_call_stream
def sv_verify_greedy(target: torch.Tensor, t_row_start: torch.Tensor, draft_ids: torch.Tensor,
                     draft_len: torch.Tensor, max_new: Optional[torch.Tensor] = None,
                     eos_id: int = -1, dev_status: Optional[torch.Tensor] = None,
                     workspace: Optional[Workspace] = None, stream=None):
    """Greedy verify; returns (tokens [B, k_max+1], count [B], accepted [B])."""
    t_rows, V = target.shape
    B = draft_len.shape[0]
    k_max = draft_ids.shape[1] if draft_ids.dim() == 2 else 0
    _shape(t_row_start, "t_row_start", (B,))
    _shape(draft_ids, "draft_ids", (B, k_max))
    _shape(max_new, "max_new", (B,))
    _status_arg(dev_status)
    dev = target.device
    tok = torch.empty((B, k_max + 1), dtype=torch.int32, device=dev)
    cnt = torch.empty((B,), dtype=torch.int32, device=dev)
    acc = torch.empty((B,), dtype=torch.int32, device=dev)
    ws = _workspace(workspace, dev, stream, workspace_bytes(SV_OP_GREEDY, B, t_rows, V))
    args = (_dev(target, "target"), _dtype_code(target), t_rows, V,
            _dev(t_row_start, "t_row_start", torch.int32, dev),
            _dev(draft_ids, "draft_ids", torch.int32, dev),
            _dev(draft_len, "draft_len", torch.int32, dev), B, k_max,
            _dev(max_new, "max_new", torch.int32, dev), eos_id,
            _dev(tok, "out"), _dev(cnt, "cnt"), _dev(acc, "acc"),
            _dev(dev_status, "dev_status", torch.int32, dev),
            ws.data_ptr(), ws.numel(), _stream(stream))
    keep = (target, t_row_start, draft_ids, draft_len, max_new, dev_status, tok, cnt, acc, ws)
    return _invoke("sv_verify_greedy", args, keep, (tok, cnt, acc))


@_on_call_stream
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
    return _sample(target, draft, t_row_start, q_row_start, draft_ids, draft_len, temperature, uniforms,
                   None, max_new, eos_id, diag, dev_status, workspace, stream, out, resid)


@_on_call_stream
def sv_verify_sample_philox(target: torch.Tensor, draft: torch.Tensor, t_row_start: torch.Tensor,
                            q_row_start: torch.Tensor, draft_ids: torch.Tensor, draft_len: torch.Tensor,
                            temperature: float, seed: int, offset: int,
                            max_new: Optional[torch.Tensor] = None, eos_id: int = -1,
                            diag: bool = False, dev_status: Optional[torch.Tensor] = None,
                            workspace: Optional[Workspace] = None, stream=None, out=None,
                            resid: Optional[bool] = None):
    """sv_verify_sample with the uniforms of the Philox stream (seed, offset)
    drawn on the device (see sv_philox_uniforms)."""
    return _sample(target, draft, t_row_start, q_row_start, draft_ids, draft_len, temperature, None,
                   (int(seed), int(offset)), max_new, eos_id, diag, dev_status, workspace, stream, out, resid)


@_on_call_stream
def sv_philox_uniforms(seed: int, offset: int, batch: int, slots: int, out: Optional[torch.Tensor] = None,
                       device=None, stream=None) -> torch.Tensor:
    """The verify's uniforms u [batch, slots] of the Philox stream (seed, offset)."""
    if out is None:
        out = torch.empty((batch, slots), dtype=torch.float32,
                          device=device if device is not None else torch.device("cuda"))
    _shape(out, "out", (batch, slots), torch.float32)
    args = (int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 64 - 1), batch, slots,
            _dev(out, "out", torch.float32), _stream(stream))
    return _invoke("sv_philox_uniforms", args, (out,), out)


def _sample(target, draft, t_row_start, q_row_start, draft_ids, draft_len, temperature, uniforms, philox,
            max_new, eos_id, diag, dev_status, workspace, stream, out, resid, noalloc=False):
    t_rows, V = target.shape
    q_rows = draft.shape[0]
    if draft.shape[1] != V:
        raise SpecVerifyError("target and draft rows differ in length")
    B = draft_len.shape[0]
    k_max = draft_ids.shape[1] if draft_ids.dim() == 2 else 0
    if philox is None and uniforms.shape != (B, k_max + 1):
        raise SpecVerifyError(f"uniforms must be [B, k_max+1] = [{B}, {k_max + 1}]")
    _shape(t_row_start, "t_row_start", (B,))
    _shape(q_row_start, "q_row_start", (B,))
    _shape(max_new, "max_new", (B,))
    _status_arg(dev_status)
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
        _shape(tok, "out tokens", (B, k_max + 1), torch.int32)
        _shape(cnt, "out count", (B,), torch.int32)
        _shape(acc, "out accepted", (B,), torch.int32)
        _shape(dg, "out diag", (B, k_max + 1, 4), torch.float32)
        _shape(rs, "out resid", (B,), torch.float32)
    ws = None if noalloc else _workspace(workspace, dev, stream, sample_workspace_bytes(B, t_rows, V, k_max))
    head = (_dev(target, "target"), _dtype_code(target), t_rows,
            _dev(draft, "draft"), _dtype_code(draft), q_rows, V,
            _dev(t_row_start, "t_row_start", torch.int32, dev),
            _dev(q_row_start, "q_row_start", torch.int32, dev),
            _dev(draft_ids, "draft_ids", torch.int32, dev),
            _dev(draft_len, "draft_len", torch.int32, dev), B, k_max, float(temperature))
    if philox is None:
        rng = (_dev(uniforms, "uniforms", torch.float32, dev),)
    else:
        rng = (philox[0] & (2 ** 64 - 1), philox[1] & (2 ** 64 - 1))
    args = head + rng + (
            _dev(max_new, "max_new", torch.int32, dev), eos_id,
            _dev(tok, "out"), _dev(cnt, "cnt"), _dev(acc, "acc"),
            _dev(dg, "diag", torch.float32, dev), _dev(rs, "resid", torch.float32, dev),
            _dev(dev_status, "dev_status", torch.int32, dev)) + \
        (() if noalloc else (ws.data_ptr(), ws.numel())) + (_stream(stream),)
    keep = (target, draft, t_row_start, q_row_start, draft_ids, draft_len, uniforms, max_new, dev_status,
            tok, cnt, acc, dg, rs, ws)
    name = "sv_verify_sample_noalloc" if noalloc else (
        "sv_verify_sample" if philox is None else "sv_verify_sample_philox")
    return _invoke(name, args, keep, (tok, cnt, acc, dg, rs))


@_on_call_stream
def sv_verify_sample_noalloc(target: torch.Tensor, draft: torch.Tensor, t_row_start: torch.Tensor,
                             q_row_start: torch.Tensor, draft_ids: torch.Tensor, draft_len: torch.Tensor,
                             temperature: float, uniforms: torch.Tensor, max_new: Optional[torch.Tensor] = None,
                             eos_id: int = -1, diag: bool = False, dev_status: Optional[torch.Tensor] = None,
                             stream=None, out=None, resid: Optional[bool] = None):
    """sv_verify_sample on the library's static device scratch (no workspace;
    the C call allocates nothing).  Pass ``out`` to make the whole call free of
    allocations; the returned tuple is as for sv_verify_sample."""
    return _sample(target, draft, t_row_start, q_row_start, draft_ids, draft_len, temperature, uniforms, None,
                   max_new, eos_id, diag, dev_status, None, stream, out, resid, noalloc=True)


def prepare_verify_sample(*args, **kwargs):
    """prepare(sv_verify_sample, ...): (launch, outputs)."""
    return prepare(sv_verify_sample, *args, **kwargs)


@_on_call_stream
def sv_verify_tree(target: torch.Tensor, draft: torch.Tensor, parent: torch.Tensor,
                   node_token: torch.Tensor, temperature: float, uniforms: torch.Tensor,
                   diag: bool = False, dev_status: Optional[torch.Tensor] = None,
                   workspace: Optional[Workspace] = None, stream=None, out=None):
    """Tree verify.  target/draft rows [B*N, V]; parent/node_token/uniforms [B, N].
    Returns (tokens [B, N], count, accepted, path [B, N], diag [B, N, 4] or None)."""
    B, N = parent.shape
    rows, V = target.shape
    if rows != B * N or draft.shape != target.shape:
        raise SpecVerifyError("target/draft must be [B*N, V]")
    _shape(node_token, "node_token", (B, N))
    _shape(uniforms, "uniforms", (B, N))
    _status_arg(dev_status)
    dev = target.device
    if out is None:
        tok, cnt, acc, pth = _tree_outputs(B, N, dev, None)
        dg = torch.zeros((B, N, 4), dtype=torch.float32, device=dev) if diag else None
    else:
        tok, cnt, acc, pth, dg = out
        _tree_outputs(B, N, dev, (tok, cnt, acc, pth))
        _shape(dg, "out diag", (B, N, 4), torch.float32)
    ws = _workspace(workspace, dev, stream, workspace_bytes(SV_OP_TREE, B, B * N, V))
    args = (_dev(target, "target"), _dtype_code(target), _dev(draft, "draft"),
            _dtype_code(draft), V, _dev(parent, "parent", torch.int32, dev),
            _dev(node_token, "node_token", torch.int32, dev), B, N,
            float(temperature), _dev(uniforms, "uniforms", torch.float32, dev),
            _dev(tok, "out"), _dev(cnt, "cnt"), _dev(acc, "acc"), _dev(pth, "path"),
            _dev(dg, "diag", torch.float32, dev),
            _dev(dev_status, "dev_status", torch.int32, dev),
            ws.data_ptr(), ws.numel(), _stream(stream))
    keep = (target, draft, parent, node_token, uniforms, dev_status, tok, cnt, acc, pth, dg, ws)
    return _invoke("sv_verify_tree", args, keep, (tok, cnt, acc, pth, dg))


def _tree_outputs(B, N, dev, out):
    if out is not None:
        tok, cnt, acc, pth = out
        _shape(tok, "out tokens", (B, N), torch.int32)
        _shape(cnt, "out count", (B,), torch.int32)
        _shape(acc, "out accepted", (B,), torch.int32)
        _shape(pth, "out path", (B, N), torch.int32)
        return out
    return (torch.empty((B, N), dtype=torch.int32, device=dev), torch.empty((B,), dtype=torch.int32, device=dev),
            torch.empty((B,), dtype=torch.int32, device=dev), torch.empty((B, N), dtype=torch.int32, device=dev))


@_on_call_stream
def sv_verify_tree_greedy(target: torch.Tensor, parent: torch.Tensor, node_token: torch.Tensor,
                          dev_status: Optional[torch.Tensor] = None,
                          workspace: Optional[Workspace] = None, stream=None, out=None):
    """Greedy (T = 0) tree verify.  target rows [B*N, V]; parent/node_token [B, N].
    Returns (tokens [B, N], count, accepted, path [B, N])."""
    B, N = parent.shape
    rows, V = target.shape
    if rows != B * N:
        raise SpecVerifyError("target must be [B*N, V]")
    _shape(node_token, "node_token", (B, N))
    _status_arg(dev_status)
    dev = target.device
    tok, cnt, acc, pth = _tree_outputs(B, N, dev, out)
    ws = _workspace(workspace, dev, stream, workspace_bytes(SV_OP_TREE, B, B * N, V))
    args = (_dev(target, "target"), _dtype_code(target), V, _dev(parent, "parent", torch.int32, dev),
            _dev(node_token, "node_token", torch.int32, dev), B, N,
            _dev(tok, "out"), _dev(cnt, "cnt"), _dev(acc, "acc"), _dev(pth, "path"),
            _dev(dev_status, "dev_status", torch.int32, dev), ws.data_ptr(), ws.numel(), _stream(stream))
    keep = (target, parent, node_token, dev_status, tok, cnt, acc, pth, ws)
    return _invoke("sv_verify_tree_greedy", args, keep, (tok, cnt, acc, pth))


@_on_call_stream
def sv_verify_tree_pointmass(target: torch.Tensor, parent: torch.Tensor, node_token: torch.Tensor,
                             temperature: float, uniforms: torch.Tensor,
                             dev_status: Optional[torch.Tensor] = None,
                             workspace: Optional[Workspace] = None, stream=None, out=None):
    """Tree verify with every candidate tested as a point mass on its token.
    target rows [B*N, V]; parent/node_token/uniforms [B, N].  Returns (tokens
    [B, N], count, accepted, path [B, N])."""
    B, N = parent.shape
    rows, V = target.shape
    if rows != B * N:
        raise SpecVerifyError("target must be [B*N, V]")
    if uniforms.shape != (B, N):
        raise SpecVerifyError(f"uniforms must be [B, N] = [{B}, {N}]")
    _shape(node_token, "node_token", (B, N))
    _status_arg(dev_status)
    dev = target.device
    tok, cnt, acc, pth = _tree_outputs(B, N, dev, out)
    ws = _workspace(workspace, dev, stream, workspace_bytes(SV_OP_TREE, B, B * N, V))
    args = (_dev(target, "target"), _dtype_code(target), V, _dev(parent, "parent", torch.int32, dev),
            _dev(node_token, "node_token", torch.int32, dev), B, N,
            float(temperature), _dev(uniforms, "uniforms", torch.float32, dev),
            _dev(tok, "out"), _dev(cnt, "cnt"), _dev(acc, "acc"), _dev(pth, "path"),
            _dev(dev_status, "dev_status", torch.int32, dev), ws.data_ptr(), ws.numel(), _stream(stream))
    keep = (target, parent, node_token, uniforms, dev_status, tok, cnt, acc, pth, ws)
    return _invoke("sv_verify_tree_pointmass", args, keep, (tok, cnt, acc, pth))


class DraftTreeState:
    """Device candidates of a batch of EAGLE-2 draft trees (see sv_tree_expand):
    token, parent, depth [B, max_cand] int32, conf float32, value float64,
    count [B] int32."""

    def __init__(self, batch: int, max_cand: int, device=None):
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self.batch, self.max_cand = batch, max_cand
        self.token = torch.empty((batch, max_cand), dtype=torch.int32, device=dev)
        self.parent = torch.empty((batch, max_cand), dtype=torch.int32, device=dev)
        self.depth = torch.empty((batch, max_cand), dtype=torch.int32, device=dev)
        self.conf = torch.empty((batch, max_cand), dtype=torch.float32, device=dev)
        self.value = torch.empty((batch, max_cand), dtype=torch.float64, device=dev)
        self.count = torch.zeros((batch,), dtype=torch.int32, device=dev)


@_on_call_stream
def sv_tree_expand(draft_rows: torch.Tensor, exp_node: Optional[torch.Tensor], top_children: int,
                   expand_next: int, state: DraftTreeState, next_exp: Optional[torch.Tensor] = None,
                   dev_status: Optional[torch.Tensor] = None, workspace: Optional[Workspace] = None,
                   stream=None) -> torch.Tensor:
    """One EAGLE-2 round.  draft_rows [B * n_exp, V]: the draft's distribution at
    each node of exp_node [B, n_exp] (None: the first round, one root row per
    request).  Returns next_exp [B, expand_next]: the candidates to expand next."""
    B = state.batch
    rows, V = draft_rows.shape
    n_exp = 1 if exp_node is None else exp_node.shape[1]
    if rows != B * n_exp:
        raise SpecVerifyError(f"draft_rows must be [B * n_exp, V] = [{B * n_exp}, V]")
    _shape(exp_node, "exp_node", (B, n_exp))
    _status_arg(dev_status)
    dev = draft_rows.device
    if next_exp is None:
        next_exp = torch.empty((B, expand_next), dtype=torch.int32, device=dev)
    _shape(next_exp, "next_exp", (B, expand_next), torch.int32)
    ws = _workspace(workspace, dev, stream, workspace_bytes(SV_OP_TREE_EXPAND, B, rows, V))
    args = (_dev(draft_rows, "draft_rows"), _dtype_code(draft_rows), V, B, n_exp,
            _dev(exp_node, "exp_node", torch.int32, dev), top_children, expand_next, state.max_cand,
            _dev(state.token, "token"), _dev(state.parent, "parent"), _dev(state.depth, "depth"),
            _dev(state.conf, "conf"), _dev(state.value, "value"), _dev(state.count, "count"),
            _dev(next_exp, "next_exp"), _dev(dev_status, "dev_status", torch.int32, dev),
            ws.data_ptr(), ws.numel(), _stream(stream))
    keep = (draft_rows, exp_node, state, next_exp, dev_status, ws)
    return _invoke("sv_tree_expand", args, keep, next_exp)


@_on_call_stream
def sv_tree_finalize(state: DraftTreeState, n_nodes: int, mask: bool = True,
                     dev_status: Optional[torch.Tensor] = None, stream=None, out=None):
    """Rerank and flatten: returns (parent, token, depth, cand [B, n_nodes] int32,
    mask [B, n_nodes, n_nodes] uint8 or None)."""
    B = state.batch
    dev = state.token.device
    _status_arg(dev_status)
    if out is None:
        outs = [torch.empty((B, n_nodes), dtype=torch.int32, device=dev) for _ in range(4)]
        m = torch.empty((B, n_nodes, n_nodes), dtype=torch.uint8, device=dev) if mask else None
    else:
        *outs, m = out
        for t, nm in zip(outs, ("parent", "token", "depth", "cand")):
            _shape(t, f"out {nm}", (B, n_nodes), torch.int32)
        _shape(m, "out mask", (B, n_nodes, n_nodes), torch.uint8)
    args = (B, state.max_cand, _dev(state.token, "token"), _dev(state.parent, "parent"),
            _dev(state.depth, "depth"), _dev(state.conf, "conf"), _dev(state.value, "value"),
            _dev(state.count, "count"), n_nodes, *(_dev(t, "out") for t in outs), _dev(m, "mask"),
            _dev(dev_status, "dev_status", torch.int32, dev), _stream(stream))
    return _invoke("sv_tree_finalize", args, (state, outs, m, dev_status), (*outs, m))


def _shard_common(target_cols, draft_cols, bounds, shard, t_row_start, q_row_start, draft_ids, draft_len,
                  temperature):
    """Checked head of a shard step's argument list, the sizes, and the
    host bounds array (kept alive by the argument tuple)."""
    t_rows, width = target_cols.shape
    q_rows = draft_cols.shape[0]
    G = len(bounds) - 1
    if not 0 <= shard < G or bounds[shard + 1] - bounds[shard] != width or draft_cols.shape[1] != width:
        raise SpecVerifyError("target_cols / draft_cols must hold the shard's columns")
    B = draft_len.shape[0]
    k_max = draft_ids.shape[1] if draft_ids.dim() == 2 else 0
    _shape(t_row_start, "t_row_start", (B,))
    _shape(q_row_start, "q_row_start", (B,))
    _shape(draft_ids, "draft_ids", (B, k_max))
    dev = target_cols.device
    hb = (ctypes.c_int64 * (G + 1))(*[int(v) for v in bounds])
    head = (_dev(target_cols, "target_cols"), _dtype_code(target_cols), t_rows, _dev(draft_cols, "draft_cols"),
            _dtype_code(draft_cols), q_rows, int(bounds[-1]), hb, G, shard,
            _dev(t_row_start, "t_row_start", torch.int32, dev), _dev(q_row_start, "q_row_start", torch.int32, dev),
            _dev(draft_ids, "draft_ids", torch.int32, dev), _dev(draft_len, "draft_len", torch.int32, dev),
            B, k_max, float(temperature))
    return head, B, k_max, t_rows, width, G, dev


@_on_call_stream
def sv_shard_stats(target_cols, draft_cols, bounds, shard, t_row_start, q_row_start, draft_ids, draft_len,
                   temperature, out=None, workspace: Optional[Workspace] = None, stream=None):
    """Step 1 of the sharded verify: (pairs [t_rows, 2], at [B, k_max, 2]) of
    this shard (see include/specverify.h)."""
    head, B, k_max, t_rows, width, G, dev = _shard_common(target_cols, draft_cols, bounds, shard, t_row_start,
                                                          q_row_start, draft_ids, draft_len, temperature)
    if out is None:
        pairs = torch.empty((t_rows, 2), dtype=torch.float32, device=dev)
        at = torch.zeros((B, max(k_max, 1), 2), dtype=torch.float32, device=dev)
    else:
        pairs, at = out
        _shape(pairs, "pairs", (t_rows, 2), torch.float32)
        _shape(at, "at", (B, max(k_max, 1), 2), torch.float32)
    ws = _workspace(workspace, dev, stream, workspace_bytes(SV_OP_SHARD, B, t_rows, width))
    args = head + (_dev(pairs, "pairs"), _dev(at, "at"), ws.data_ptr(), ws.numel(), _stream(stream))
    return _invoke("sv_shard_stats", args, (target_cols, draft_cols, t_row_start, q_row_start, draft_ids,
                                            draft_len, pairs, at, ws), (pairs, at))


@_on_call_stream
def sv_shard_residual(target_cols, draft_cols, bounds, shard, t_row_start, q_row_start, draft_ids, draft_len,
                      temperature, uniforms, all_pairs, all_at, mass, workspace: Workspace, stream=None):
    """Step 2: writes this shard's row of mass [G, B, 3] (float64)."""
    head, B, k_max, t_rows, width, G, dev = _shard_common(target_cols, draft_cols, bounds, shard, t_row_start,
                                                          q_row_start, draft_ids, draft_len, temperature)
    _shape(uniforms, "uniforms", (B, k_max + 1), torch.float32)
    _shape(all_pairs, "all_pairs", (G, t_rows, 2), torch.float32)
    _shape(all_at, "all_at", (G, B, max(k_max, 1), 2), torch.float32)
    _shape(mass, "mass", (G, B, 3), torch.float64)
    ws = _workspace(workspace, dev, stream, workspace_bytes(SV_OP_SHARD, B, t_rows, width))
    args = head + (_dev(uniforms, "uniforms"), _dev(all_pairs, "all_pairs"), _dev(all_at, "all_at"),
                   _dev(mass, "mass"), ws.data_ptr(), ws.numel(), _stream(stream))
    return _invoke("sv_shard_residual", args, (target_cols, draft_cols, t_row_start, q_row_start, draft_ids,
                                               draft_len, uniforms, all_pairs, all_at, mass, ws), mass)


@_on_call_stream
def sv_shard_draw(target_cols, draft_cols, bounds, shard, t_row_start, q_row_start, draft_ids, draft_len,
                  temperature, uniforms, all_pairs, mass, out, max_new: Optional[torch.Tensor] = None,
                  eos_id: int = -1, dev_status: Optional[torch.Tensor] = None,
                  workspace: Optional[Workspace] = None, stream=None):
    """Step 3: the shard holding the draw writes request b's outputs into
    out = (tokens [B, k_max+1], count [B], accepted [B], resid [B] or None)."""
    head, B, k_max, t_rows, width, G, dev = _shard_common(target_cols, draft_cols, bounds, shard, t_row_start,
                                                          q_row_start, draft_ids, draft_len, temperature)
    tok, cnt, acc, rs = out
    _shape(tok, "out tokens", (B, k_max + 1), torch.int32)
    _shape(cnt, "out count", (B,), torch.int32)
    _shape(acc, "out accepted", (B,), torch.int32)
    _shape(rs, "out resid", (B,), torch.float32)
    _shape(max_new, "max_new", (B,))
    _status_arg(dev_status)
    _shape(uniforms, "uniforms", (B, k_max + 1), torch.float32)
    _shape(all_pairs, "all_pairs", (G, t_rows, 2), torch.float32)
    _shape(mass, "mass", (G, B, 3), torch.float64)
    ws = _workspace(workspace, dev, stream, workspace_bytes(SV_OP_SHARD, B, t_rows, width))
    args = head + (_dev(uniforms, "uniforms"), _dev(all_pairs, "all_pairs"), _dev(mass, "mass"),
                   _dev(max_new, "max_new", torch.int32, dev), eos_id, _dev(tok, "out"), _dev(cnt, "cnt"),
                   _dev(acc, "acc"), _dev(rs, "resid"), _dev(dev_status, "dev_status", torch.int32, dev),
                   ws.data_ptr(), ws.numel(), _stream(stream))
    return _invoke("sv_shard_draw", args, (target_cols, draft_cols, t_row_start, q_row_start, draft_ids,
                                           draft_len, uniforms, all_pairs, mass, out, max_new, dev_status, ws),
                   out)
