"""Chain verification in float64: greedy (T = 0) and speculative sampling.

TEST INFRASTRUCTURE (see the package docstring).  Plain numpy, one request at
a time, in the order the pages give the steps.
"""
from functools import lru_cache

import numpy as np

from .rows import (widen, FLAG_BAD_REQUEST, FLAG_BAD_TOKEN, FLAG_NONFINITE,
                   FLAG_OVER_BUDGET, FLAG_FALLBACK)


def softmax_T(l: np.ndarray, T: float):
    """Target distribution of one position: p = softmax(l / T) over the whole
    vocabulary, with M = max(l / T) and S = sum exp(l / T - M).

    "投机解码:为什么一个字都不改", figure "一次目标前向验 k 个草稿 token": the
    target's k+1 rows are P = softmax(f_target([x1..xk]) / T); temperature
    divides the target scores before the softmax.
    """
    with np.errstate(invalid="ignore", over="ignore"):
        z = l / T
        M = np.max(z)
        e = np.exp(z - M)
        S = np.sum(e)
        p = e / S
    return p, M, S


def inverse_cdf(r: np.ndarray, u: float):
    """Draw from the (unnormalised, non-negative) weights ``r`` with the uniform
    ``u``: the smallest id x, ids ascending, whose running sum exceeds u times
    the total.  Returns (x, total, margin) where margin is the distance from u
    to the nearer edge of x's cell in the normalised CDF.

    The pages say only that the token is resampled from the distribution
    ("投机解码:为什么一个字都不改", section "改进"); ascending ids with a strict
    '>' is the plain inverse-CDF reading.
    """
    cdf = np.cumsum(r)
    total = cdf[-1]
    t = u * total
    x = int(np.searchsorted(cdf, t, side="right"))
    if x >= r.shape[0]:                       # rounding overshoot: last positive id
        x = int(np.nonzero(r > 0)[0][-1])
    hi = cdf[x] / total
    lo = cdf[x - 1] / total if x > 0 else 0.0
    return x, total, min(u - lo, hi - u)


def _emit(drafted, m, y, eos_id, budget):
    """Emitted tokens of one round: the m accepted drafts, then the target's own
    token at the break ("第 13 篇：推理引擎一次猜几个字——草稿 + 验证", section ③:
    append draft[0:m], then the model's true next token).  Cut after the first
    end token, and at the request's remaining budget ("Speculative decoding
    explained", four-case table: at the end of the path nothing is added)."""
    toks = [int(t) for t in drafted[:m]] + [int(y)]
    if eos_id >= 0 and eos_id in toks:
        toks = toks[:toks.index(eos_id) + 1]
    if budget is not None:
        toks = toks[:max(int(budget), 0)]
    return toks


def _check_request(b, k, k_max, ts, qs, t_rows, q_rows, need_q):
    if not (0 <= k <= k_max):
        return False
    if ts < 0 or ts + k >= t_rows:
        return False
    if need_q and k > 0 and (qs < 0 or qs + k > q_rows):
        return False
    return True


def verify_sample(target, t_kind, draft, q_kind, V, t_row_start, q_row_start,
                  draft_ids, draft_len, k_max, T, uniforms, max_new=None,
                  eos_id=-1, variant="residual"):
    """Speculative-sampling verify of a batch of chain drafts.

    For request b with k = draft_len[b] drafts x_0..x_{k-1}:

    1. p_i = softmax(target row i / T) for i = 0..k (k+1 rows from one target
       forward) -- "投机解码:为什么一个字都不改", figure "一次目标前向验 k 个草稿 token".
       The round reads rows 0..m (m below); a row it reads whose normaliser is
       not finite and positive makes the request invalid (FLAG_NONFINITE).
    2. Draft i is kept with probability min(1, p_i(x_i) / q_i(x_i)): with the
       uniform u_i, kept iff u_i * q_i(x_i) < p_i(x_i); stop at the first draft
       that is not kept (m = its index, else m = k) -- same page, section
       "改进:接受概率 min(1, p/q),拒绝时从残差重采".
    3. On a rejection the replacement is drawn from the residual
       norm(max(0, p_m - q_m)); if every draft was kept, one more token is
       drawn from p_k -- same page, sections "改进" and "一轮能出几个 token"
       (a full accept earns one extra token).  The draw uses u_k, k = draft_len.
    4. Emit x_0..x_{m-1} and the drawn token: m + 1 tokens, in [1, k + 1].

    ``variant="resample_from_p"`` is the wrong scheme the page warns about
    (section "常见误解": after a rejection, draw from p itself); it exists only as
    a negative control.

    Returns a dict of numpy arrays: tokens [B, k_max+1] (-1 padded), count [B],
    accepted [B] (= m), flags [B], diag [B, k_max+1, 4] = (M_i, S_i, p_i(x_i),
    q_i(x_i)) with zeros in the p, q slots at i = k, resid [B] (total mass of
    the distribution the last token was drawn from) and margins [B, k_max+1]
    (distance of each uniform to its decision boundary; NaN where unused).
    """
    B = int(np.asarray(draft_len).shape[0])
    t_rows = target.shape[0]
    q_rows = 0 if draft is None else draft.shape[0]
    tokens = np.full((B, k_max + 1), -1, dtype=np.int64)
    count = np.zeros(B, dtype=np.int64)
    accepted = np.zeros(B, dtype=np.int64)
    flags = np.zeros(B, dtype=np.int64)
    diag = np.zeros((B, k_max + 1, 4), dtype=np.float64)
    resid = np.zeros(B, dtype=np.float64)
    margins = np.full((B, k_max + 1), np.nan, dtype=np.float64)

    @lru_cache(maxsize=16)
    def target_dist(row):
        return softmax_T(widen(target[row], t_kind), T)

    @lru_cache(maxsize=16)
    def draw_weights(t_row, q_row):
        """Weights the final token is drawn from, and whether that needed the
        zero-mass fallback (or failed: None)."""
        p = target_dist(t_row)[0]
        if q_row < 0:
            return p, 0
        q = widen(draft[q_row], q_kind)
        if np.isnan(np.sum(q)):
            return None, FLAG_NONFINITE
        r = np.maximum(p - q, 0.0)
        R = np.sum(r)
        if not np.isfinite(R):
            return None, FLAG_NONFINITE
        if not R > 0.0:
            return p, FLAG_FALLBACK
        return r, 0

    for b in range(B):
        k = int(draft_len[b])
        ts, qs = int(t_row_start[b]), int(q_row_start[b])
        if not _check_request(b, k, k_max, ts, qs, t_rows, q_rows, True):
            flags[b] |= FLAG_BAD_REQUEST
            continue
        x = np.asarray(draft_ids[b, :k], dtype=np.int64)
        if np.any((x < 0) | (x >= V)):
            flags[b] |= FLAG_BAD_TOKEN
            continue
        budget = None if max_new is None else int(max_new[b])
        if budget is not None and k > budget:
            flags[b] |= FLAG_OVER_BUDGET
        stats = [target_dist(ts + i) for i in range(k + 1)]
        u = np.asarray(uniforms[b], dtype=np.float64)
        for i in range(k + 1):
            diag[b, i, 0], diag[b, i, 1] = stats[i][1], stats[i][2]
        for i in range(k):
            diag[b, i, 2] = stats[i][0][x[i]]
            diag[b, i, 3] = widen(draft[qs + i, x[i]:x[i] + 1], q_kind)[0]
        # position-by-position test, stopping at the first rejection; the
        # round reads target rows 0..m only, and a row it reads must have a
        # finite, positive normaliser (rows after the break play no part)
        m = k
        finite = True
        for i in range(k + 1):
            S = stats[i][2]
            if not (np.isfinite(S) and S > 0):
                finite = False
                break
            if i == k:
                break
            p_x, q_x = diag[b, i, 2], diag[b, i, 3]
            margins[b, i] = abs(u[i] - p_x / q_x) if q_x > 0 else np.inf
            if not u[i] * q_x < p_x:
                m = i
                break
        if not finite:
            flags[b] |= FLAG_NONFINITE
            margins[b] = np.nan
            continue
        if m < k:
            if variant == "resample_from_p":
                w, fl = stats[m][0], 0
            else:
                w, fl = draw_weights(ts + m, qs + m)
        else:
            w, fl = draw_weights(ts + k, -1)
        flags[b] |= fl
        if w is None:
            continue
        y, total, marg = inverse_cdf(w, u[k])
        margins[b, k] = marg
        resid[b] = total
        toks = _emit(x, m, y, eos_id, budget)
        tokens[b, :len(toks)] = toks
        count[b] = len(toks)
        accepted[b] = m
    return dict(tokens=tokens, count=count, accepted=accepted, flags=flags,
                diag=diag, resid=resid, margins=margins)


def verify_greedy(target, t_kind, V, t_row_start, draft_ids, draft_len, k_max,
                  max_new=None, eos_id=-1):
    """Greedy (T = 0) verify of a batch of chain drafts.

    "第 13 篇：推理引擎一次猜几个字——草稿 + 验证", section ③ and its notes: one
    target forward gives, at every drafted position, the token the model would
    pick; compare draft i with it left to right, stop at the first difference,
    keep the drafts before it and append the model's own token there.
    "Speculative decoding explained", four-case table: when all drafts match,
    the target's next token is appended too, unless the path has ended.

    The model's pick is the argmax of the row (the lowest id among equal
    maxima; a row holding a NaN makes the request invalid).  Returns tokens,
    count, accepted, flags and argmax [B, k_max+1] (-1 where unused).
    """
    B = int(np.asarray(draft_len).shape[0])
    t_rows = target.shape[0]
    tokens = np.full((B, k_max + 1), -1, dtype=np.int64)
    count = np.zeros(B, dtype=np.int64)
    accepted = np.zeros(B, dtype=np.int64)
    flags = np.zeros(B, dtype=np.int64)
    argmax = np.full((B, k_max + 1), -1, dtype=np.int64)
    for b in range(B):
        k = int(draft_len[b])
        ts = int(t_row_start[b])
        if not _check_request(b, k, k_max, ts, 0, t_rows, 0, False):
            flags[b] |= FLAG_BAD_REQUEST
            continue
        x = np.asarray(draft_ids[b, :k], dtype=np.int64)
        if np.any((x < 0) | (x >= V)):
            flags[b] |= FLAG_BAD_TOKEN
            continue
        budget = None if max_new is None else int(max_new[b])
        if budget is not None and k > budget:
            flags[b] |= FLAG_OVER_BUDGET
        rows = [widen(target[ts + i], t_kind) for i in range(k + 1)]
        if any(np.isnan(r).any() for r in rows):
            flags[b] |= FLAG_NONFINITE
            continue
        a = [int(np.argmax(r)) for r in rows]
        argmax[b, :k + 1] = a
        m = k
        for i in range(k):
            if x[i] != a[i]:
                m = i
                break
        toks = _emit(x, m, a[m], eos_id, budget)
        tokens[b, :len(toks)] = toks
        count[b] = len(toks)
        accepted[b] = m
    return dict(tokens=tokens, count=count, accepted=accepted, flags=flags,
                argmax=argmax)


def greedy_path_verify(path, prefix, guess):
    """The toy greedy verifier of "Speculative decoding explained" (section on
    the exercise contract and the four-case table): the target follows the
    fixed ``path``; compare the guess with the path from the left, keep it up to
    the first difference, add the path's symbol there and drop the rest; if the
    whole guess matches and the path continues, add the path's next symbol; at
    the end of the path add nothing.

    Per the page's function contract, an empty guess, a prefix that is not a
    prefix of the path or is the whole path, and a guess longer than the rest
    of the path are not allowed (ValueError).

    Returns (kept part of the guess, added symbol or None, new output).
    """
    path, prefix, guess = list(path), list(prefix), list(guess)
    if not guess:
        raise ValueError("empty guess")
    if prefix != path[:len(prefix)]:
        raise ValueError("prefix is not a prefix of the path")
    if len(prefix) == len(path):
        raise ValueError("path already finished")
    rest = path[len(prefix):]
    if len(guess) > len(rest):
        raise ValueError("guess longer than the remaining path")
    kept = []
    for g, t in zip(guess, rest):
        if g != t:
            return kept, t, prefix + kept + [t]
        kept.append(g)
    added = rest[len(guess)] if len(guess) < len(rest) else None
    return kept, added, prefix + kept + ([added] if added is not None else [])


def forward_accounting(accepts):
    """Target forwards and tokens gained over rounds with the given accepted
    counts: one target forward per round, m + 1 tokens per round
    ("第 13 篇：推理引擎一次猜几个字——草稿 + 验证", section ④ and its REPL
    version)."""
    accepts = [int(m) for m in accepts]
    return len(accepts), sum(m + 1 for m in accepts)


def naive_round(p, q, u_draft, u_target):
    """The naive sampled scheme ("投机解码:为什么一个字都不改", section
    "先自己设计:什么时候算「猜中」?"): the draft draws x from q, the target draws
    y from p, x is kept only if x == y; the emitted token is always y.  Returns
    (kept, emitted)."""
    x = inverse_cdf(np.asarray(q, dtype=np.float64), u_draft)[0]
    y = inverse_cdf(np.asarray(p, dtype=np.float64), u_target)[0]
    return x == y, y


def shard_pairs(l: np.ndarray, bounds, T: float):
    """Softmax pairs of column shards of one row of logits l: for each shard
    [bounds[g], bounds[g+1]), (m_g, s_g) = (max of l/T over the shard, sum
    exp(l/T - m_g) over it).  A vocabulary-parallel LM head leaves each device
    one shard; the full row's statistics follow from the pairs alone
    (combine_pairs)."""
    z = np.asarray(l, dtype=np.float64) / T
    out = []
    with np.errstate(invalid="ignore", over="ignore"):
        for g in range(len(bounds) - 1):
            seg = z[bounds[g]:bounds[g + 1]]
            m = np.max(seg) if seg.size else -np.inf
            s = np.sum(np.exp(seg - m)) if seg.size and np.isfinite(m) else 0.0
            out.append((m, s))
    return out


def combine_pairs(pairs):
    """(M, S) of the whole row from its shards' pairs: M = max m_g,
    S = sum s_g exp(m_g - M) (the softmax normaliser of the figure
    "一次目标前向验 k 个草稿 token", split over the vocabulary)."""
    ms = [m for m, _ in pairs]
    M = max(ms)
    with np.errstate(invalid="ignore", over="ignore"):
        S = sum(s * np.exp(m - M) for m, s in pairs if np.isfinite(m) or m == M)
    return M, S
