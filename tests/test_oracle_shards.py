"""Pin of the oracle's shard statistics (CPU only): for any split of the
vocabulary into column shards, combining the shards' softmax pairs gives the
whole row's max and normaliser."""
import numpy as np

import oracle


def test_combined_shard_pairs_equal_the_full_row():
    rng = np.random.default_rng(8)
    for trial in range(200):
        V = int(rng.integers(1, 3000))
        l = rng.standard_normal(V) * rng.uniform(0.5, 6)
        if trial % 5 == 0:
            l[rng.random(V) < 0.5] = -np.inf
            l[int(rng.integers(0, V))] = 1.0
        T = float(rng.uniform(0.3, 2.0))
        G = int(rng.integers(1, min(V, 9) + 1))
        cuts = np.sort(rng.choice(np.arange(1, V), size=G - 1, replace=False)) if G > 1 else np.array([], int)
        bounds = [0, *cuts.tolist(), V]
        M, S = oracle.combine_pairs(oracle.shard_pairs(l, bounds, T))
        _, M0, S0 = oracle.softmax_T(l, T)
        assert M == M0
        assert abs(S - S0) <= 1e-12 * S0


def test_empty_and_all_masked_shards():
    l = np.array([-np.inf, -np.inf, 2.0, 1.0, -np.inf])
    M, S = oracle.combine_pairs(oracle.shard_pairs(l, [0, 2, 5], 1.0))
    assert M == 2.0 and abs(S - (1.0 + np.exp(-1.0))) < 1e-15
