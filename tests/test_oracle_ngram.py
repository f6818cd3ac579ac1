"""Pins of the oracle's prompt-lookup drafter (CPU only): hand cases and brute
force over every window position on tiny contexts."""
import numpy as np
from numpy.lib.stride_tricks import sliding_window_view

import oracle


def _one(ctx, w, k, stride=None):
    stride = stride or max(len(ctx), 1)
    a = np.zeros((1, stride), dtype=np.int32)
    a[0, :len(ctx)] = ctx
    ids, lens, flags = oracle.ngram_draft(a, np.array([len(ctx)]), w, k)
    return list(ids[0, :lens[0]]), int(lens[0]), int(flags[0]), ids


def test_hand_cases():
    assert _one([1, 2, 3, 4, 5], 3, 4)[:2] == ([], 0)                 # no match
    assert _one([7, 7, 7, 7], 3, 4)[:2] == ([7], 1)                   # overlapping match
    assert _one([1, 2, 3, 9, 9, 1, 2, 3], 3, 4)[:2] == ([9, 9, 1, 2], 4)   # match at j = 0
    assert _one([1, 2, 3, 4, 1, 2, 3, 5, 1, 2, 3], 3, 4)[:2] == ([5, 1, 2, 3], 4)  # most recent
    assert _one([9, 5, 6, 7, 5, 6, 7], 3, 4)[:2] == ([5, 6, 7], 3)    # stops at the context end
    assert _one([1, 2, 3], 3, 4)[:2] == ([], 0)                       # shorter than window + 1
    assert _one([1, 2, 1, 2], 2, 0)[:2] == ([], 0)                    # k = 0
    assert _one([4, 4], 1, 3)[:2] == ([4], 1)
    _, _, _, ids = _one([1, 2, 3, 1, 2], 2, 5)
    assert list(ids[0]) == [3, 1, 2, -1, -1]                          # -1 padding


def test_bad_length_is_flagged():
    a = np.zeros((2, 4), dtype=np.int32)
    ids, lens, flags = oracle.ngram_draft(a, np.array([5, -1]), 2, 3)
    assert list(lens) == [0, 0]
    assert all(f & oracle.FLAG_BAD_REQUEST for f in flags)


def test_brute_force_small_contexts():
    rng = np.random.default_rng(1)
    B, stride = 400, 24
    ctx = rng.integers(0, 3, size=(B, stride)).astype(np.int32)
    lens = rng.integers(0, stride + 1, size=B)
    for w in (1, 2, 3):
        for k in (0, 1, 4, 6):
            ids, dl, flags = oracle.ngram_draft(ctx, lens, w, k)
            assert not flags.any()
            for b in range(B):
                n = int(lens[b])
                want = []
                if n >= w + 1 and k > 0:
                    win = sliding_window_view(ctx[b, :n - 1], w)      # windows ending before n-1
                    hits = np.nonzero((win == ctx[b, n - w:n]).all(axis=1))[0]
                    if hits.size:
                        j = int(hits.max())
                        want = list(ctx[b, j + w:min(j + w + k, n)])
                assert list(ids[b, :dl[b]]) == want
                assert np.all(ids[b, dl[b]:] == -1)
