"""Checks of the input generators (CPU only)."""
import os

import numpy as np
import torch

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_eagle2_worked_example_tree():
    """The tree construction reproduces the EAGLE-2 worked example of "Speculative
    Decoding II": values, kept set, flattened order and relative positions."""
    rows = [ln.split() for ln in open(os.path.join(GOLD, "p4_eagle2_example.txt"),
                                      encoding="utf-8")
            if ln.strip() and not ln.startswith("#")]
    kids = {}
    values = {}
    for r in rows:
        if r[0] == "child":
            kids.setdefault(r[1], []).append((r[2], float(r[3])))
            values[r[2]] = float(r[4])
    kept_want = [r for r in rows if r[0] == "kept"][0][1:]
    flat_want = [r for r in rows if r[0] == "flat"][0][1:]
    pos_want = [int(v) for v in [r for r in rows if r[0] == "positions"][0][1:]]
    vocab = sorted(values)

    def propose(node):
        name = "I" if node.cid == 0 else vocab[node.token]
        lst = sorted(kids.get(name, []), key=lambda t: -t[1])
        return [(vocab.index(nm), c) for nm, c in lst]

    flat, parent, depth = synth.build_draft_tree(propose, 2, 2, 3, 8)
    got = ["I"] + [vocab[n.token] for n in flat[1:]]
    assert got == flat_want
    assert list(depth) == pos_want
    assert sorted(got) == sorted(kept_want)
    for n in flat[1:]:
        assert abs(n.value - values[vocab[n.token]]) < 1e-12
    # parents: do, make under I; it, this under do; a under make; now under it; plan under a
    par_names = [None] + [got[parent[j]] for j in range(1, len(got))]
    assert par_names == [None, "I", "I", "do", "do", "make", "it", "a"]


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100_000) * 10,
                        1 + np.arange(16) * 2.0 ** -8,            # halfway cases
                        [0.0, -0.0, 1e-40, -1e-40, 3.4e38, np.inf, -np.inf]]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.to_bf16_bits(x), want)
    back = synth.bf16_bits_to_f32(want)
    assert np.array_equal(back, torch.from_numpy(want.view(np.int16)).view(torch.bfloat16)
                          .float().numpy())


def test_uniform_grid():
    u = synth.uniform_grid(np.random.default_rng(0), (1000, 7))
    assert u.dtype == np.float32
    assert np.all((u >= 0) & (u < 1))
    assert np.all(u.astype(np.float64) * 2 ** 24 == np.floor(u.astype(np.float64) * 2 ** 24))


def test_small_configs_shapes():
    c = synth.c3_sampled(B=3, k=4, V=1000)
    assert c.target.shape == (15, 1000) and c.draft.shape == (12, 1000)
    assert c.uniforms.shape == (3, 5)
    r = synth.c4_ragged(B=5, V=777)
    assert r.target.shape[0] == int((r.draft_len + 1).sum())
    assert np.all(r.t_row_start[1:] == np.cumsum(r.draft_len + 1)[:-1])
    t = synth.c5_tree(B=2, N=12, V=600, top_children=2, expand_per_layer=2, max_depth=4)
    assert t.target.shape == (24, 600)
    assert np.all(t.parent[:, 0] == -1)
    assert np.all(t.parent[:, 1:] < np.arange(1, 12))
    g = synth.c2_greedy(B=3, n=300, V=500)
    assert g.ctx.shape == (3, 300) and g.target.shape == (15, 500)
