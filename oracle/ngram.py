"""History n-gram (prompt-lookup) drafter in plain Python.

TEST INFRASTRUCTURE (see the package docstring).
"""
import numpy as np

from .rows import FLAG_BAD_REQUEST


def ngram_draft(ctx, ctx_len, window, k):
    """Draft up to k tokens per request by looking the context's tail up in its
    own history.

    "第 13 篇：推理引擎一次猜几个字——草稿 + 验证", notes under section ③: the
    drafter needs no model; it takes the last few tokens of the context as a
    window, finds an identical fragment earlier in the history, and proposes
    the tokens that followed it.

    Readings where the page is silent: the window length is fixed (no shorter
    fallback); the most recent earlier occurrence wins; an occurrence must be
    followed by at least one token, so the tail never matches itself; the
    proposal stops at the end of the context and may be shorter than k; no
    occurrence (or a context shorter than window + 1) gives an empty draft.

    Returns (draft_ids int32 [B, k] padded with -1, draft_len int32 [B],
    flags [B]); a context length outside [0, stride] is a bad request.
    """
    ctx = np.asarray(ctx)
    B, stride = ctx.shape
    ids = np.full((B, k), -1, dtype=np.int32)
    lens = np.zeros(B, dtype=np.int32)
    flags = np.zeros(B, dtype=np.int64)
    for b in range(B):
        n = int(ctx_len[b])
        if n < 0 or n > stride:
            flags[b] |= FLAG_BAD_REQUEST
            continue
        if k <= 0 or n < window + 1:
            continue
        row = [int(t) for t in ctx[b, :n]]
        key = row[n - window:]
        for j in range(n - window - 1, -1, -1):      # most recent first
            if row[j:j + window] == key:
                cont = row[j + window:min(j + window + k, n)]
                ids[b, :len(cont)] = cont
                lens[b] = len(cont)
                break
    return ids, lens, flags
