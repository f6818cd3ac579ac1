"""Pins of the oracle's counter-based generator (CPU only).

numpy ships an implementation of the same published Philox4x64-10 function
(numpy.random.Philox) written independently of this repository: its raw
output stream for a key and a starting counter is the function applied to
counters start + 1, start + 2, ... (numpy advances the 256-bit counter before
each block).  The oracle must reproduce it bit for bit.
"""
import numpy as np
import pytest

import oracle

M64 = (1 << 64) - 1


def _np_blocks(key, counter, n):
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(counter, dtype=np.uint64))
    raw = [int(v) for v in bg.random_raw(4 * n)]
    return [tuple(raw[4 * i:4 * i + 4]) for i in range(n)]


def _plus(counter, k):
    v = sum(int(c) << (64 * i) for i, c in enumerate(counter)) + k
    v &= (1 << 256) - 1
    return tuple((v >> (64 * i)) & M64 for i in range(4))


@pytest.mark.parametrize("key", [(0, 0), (123, 456), (M64, M64), (0x0123456789ABCDEF, 7)])
@pytest.mark.parametrize("start", [(0, 0, 0, 0), (5, 9, 2, 1), (M64, 0, 0, 0), (M64, M64, M64, 3),
                                   (M64 - 1, 17, 0, M64)])
def test_philox_matches_numpy(key, start):
    blocks = _np_blocks(key, start, 3)
    for i, blk in enumerate(blocks):
        assert oracle.philox4x64_10(_plus(start, i + 1), key) == blk, (key, start, i)


def test_philox_uniform_mapping():
    seed, offset, B, slots = 0xDEADBEEF, 41, 5, 11
    u = oracle.philox_uniforms(seed, offset, B, slots)
    for b in range(B):
        for i in range(slots):
            words = oracle.philox4x64_10((i // 4, b, offset, 0), (seed, 0))
            assert u[b, i] == (words[i % 4] >> 40) / 2.0 ** 24
    g = oracle.philox_uniforms(7, 0, 200, 9)
    assert g.min() >= 0.0 and g.max() < 1.0
    assert np.all(g * 2 ** 24 == np.floor(g * 2 ** 24))          # on the 2^-24 grid
    assert np.all(g.astype(np.float32).astype(np.float64) == g)  # exact in float32
    # every request, slot and offset gets its own stream
    assert len({float(v) for v in g.ravel()}) > 0.99 * g.size
    assert not np.array_equal(oracle.philox_uniforms(7, 1, 200, 9), g)
    assert abs(g.mean() - 0.5) < 0.02
