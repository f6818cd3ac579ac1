"""The sampled chain verify over vocabulary shards (sv_shard_stats /
sv_shard_residual / sv_shard_draw), every shard run on one MI355X with the
exchanges as stacked arrays: the round must be the oracle's (token ids equal
except boundary cases, which must be rare) and the unsharded call's."""
import numpy as np
import pytest
import torch

import draft_verify_sampling_amd as sv
import oracle
import synth
from tests.gpu_util import say, compare_tokens, close, rows_to_dev, i32, f32, DEV

pytestmark = pytest.mark.gpu


def run_sharded(ci, bounds, max_new=None, eos_id=-1):
    G = len(bounds) - 1
    B, k = ci.B, ci.k_max
    trs, qrs = i32(ci.t_row_start), i32(ci.q_row_start)
    ids, dl = i32(ci.draft_ids[:, :k]), i32(ci.draft_len)
    u = f32(ci.uniforms)
    tcols = [rows_to_dev(np.ascontiguousarray(ci.target[:, bounds[g]:bounds[g + 1]]), ci.t_kind) for g in range(G)]
    qcols = [rows_to_dev(np.ascontiguousarray(ci.draft[:, bounds[g]:bounds[g + 1]]), ci.q_kind) for g in range(G)]
    wss = [sv.Workspace() for _ in range(G)]
    st1 = [sv.sv_shard_stats(tcols[g], qcols[g], bounds, g, trs, qrs, ids, dl, ci.T, workspace=wss[g])
           for g in range(G)]
    all_pairs = torch.stack([p for p, _ in st1])          # the all-gather of step 1
    all_at = torch.stack([a for _, a in st1])
    mass = torch.zeros((G, B, 3), dtype=torch.float64, device=DEV)
    for g in range(G):
        sv.sv_shard_residual(tcols[g], qcols[g], bounds, g, trs, qrs, ids, dl, ci.T, u, all_pairs, all_at, mass,
                             workspace=wss[g])
    out = (torch.full((B, k + 1), -9, dtype=torch.int32, device=DEV), torch.full((B,), -9, dtype=torch.int32, device=DEV),
           torch.full((B,), -9, dtype=torch.int32, device=DEV), torch.zeros((B,), dtype=torch.float32, device=DEV))
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    mn = i32(max_new) if max_new is not None else None
    for g in range(G):
        sv.sv_shard_draw(tcols[g], qcols[g], bounds, g, trs, qrs, ids, dl, ci.T, u, all_pairs, mass, out,
                         max_new=mn, eos_id=eos_id, dev_status=st, workspace=wss[g])
    torch.cuda.synchronize()
    return dict(tokens=out[0].cpu().numpy(), count=out[1].cpu().numpy(), accepted=out[2].cpu().numpy(),
                resid=out[3].cpu().numpy()), int(st.item())


def _oracle(ci, **kw):
    return oracle.verify_sample(ci.target, ci.t_kind, ci.draft, ci.q_kind, ci.V, ci.t_row_start, ci.q_row_start,
                                ci.draft_ids[:, :ci.k_max], ci.draft_len, ci.k_max, ci.T, ci.uniforms, **kw)


def _unsharded(ci, **kw):
    tok, cnt, acc, _, rs = sv.sv_verify_sample(rows_to_dev(ci.target, ci.t_kind), rows_to_dev(ci.draft, ci.q_kind),
                                               i32(ci.t_row_start), i32(ci.q_row_start),
                                               i32(ci.draft_ids[:, :ci.k_max]), i32(ci.draft_len), ci.T,
                                               f32(ci.uniforms), resid=True, **kw)
    torch.cuda.synchronize()
    return dict(tokens=tok.cpu().numpy(), count=cnt.cpu().numpy(), accepted=acc.cpu().numpy(), resid=rs.cpu().numpy())


def _check(name, ci, got, status, **kw):
    want = _oracle(ci, **kw)
    nb, bad = compare_tokens(got, want)
    say(f"{name}: {ci.B} requests, {nb} boundary cases, mean tokens {want['count'].mean():.3f}")
    assert bad.size == 0, bad[:10]
    assert nb <= max(2, 1e-3 * ci.B)
    flags = 0
    for f in want["flags"]:
        flags |= int(f)
    assert status == flags
    same = (got["count"] == want["count"]) & (want["count"] > 0)
    assert close(got["resid"][same], want["resid"][same], atol=1e-12).all()
    ref = _unsharded(ci, **{k: (i32(v) if k == "max_new" and v is not None else v) for k, v in kw.items()})
    for key in ("tokens", "count", "accepted"):
        assert np.array_equal(got[key][~np.isin(np.arange(ci.B), bad)], ref[key]), key


def test_gpu_shards_headline_eight_devices():
    ci = synth.c3_sampled()
    V = ci.V
    bounds = [V * g // 8 for g in range(9)]       # 31,040 columns each
    got, st = run_sharded(ci, bounds)
    _check("c3 over 8 shards", ci, got, st)


@pytest.mark.parametrize("G,V,kind", [(1, 5000, "bf16"), (3, 70_001, "f32"), (5, 2049, "bf16"), (8, 12_289, "f32")])
def test_gpu_shards_ragged_uneven(G, V, kind):
    rng = np.random.default_rng(G * 100 + V)
    B = 37
    ks = rng.integers(0, 7, size=B)
    ci = synth.sampled_chain(7, B, ks, V, 0.9, sd=2.5, n_boost=5, boost=6.0, sigma=rng.uniform(0.5, 3, size=B),
                             kind=kind, salt=G)
    cuts = np.sort(rng.choice(np.arange(1, V), size=G - 1, replace=False)).tolist() if G > 1 else []
    bounds = [0, *cuts, V]
    say(f"shards G={G} V={V} {kind}: widths {np.diff(bounds).tolist()}")
    got, st = run_sharded(ci, bounds)
    _check(f"ragged G={G}", ci, got, st)


def test_gpu_shards_edge_cases():
    """Bad tokens and rows, a NaN in a row that is read and in one that is
    not, budgets and EOS."""
    rng = np.random.default_rng(11)
    B, V = 24, 9000
    ks = rng.integers(0, 5, size=B)
    ci = synth.sampled_chain(8, B, ks, V, 1.0, sd=2.5, n_boost=5, boost=6.0, sigma=1.0, kind="f32", salt=3)
    ci.draft_ids[1, 0] = V + 5 if ks[1] > 0 else ci.draft_ids[1, 0]
    ci.target[ci.t_row_start[2], 17] = np.nan                    # row 0 of request 2: always read
    b_unread = int(np.argmax(ks >= 3))
    ci.uniforms[b_unread, 0] = 0.999999                           # rejects draft 0 (p < q likely)
    ci.target[ci.t_row_start[b_unread] + 2, :] = np.nan            # row 2: not read after a break at 0
    ci.draft_len[5] = 9                                           # more than k_max: bad request
    max_new = rng.integers(0, 6, size=B).astype(np.int32)
    eos = int(ci.draft_ids[7, 0]) if ks[7] > 0 else -1
    bounds = [0, 1000, 5000, 6001, V]
    with np.errstate(invalid="ignore", over="ignore"):
        got, st = run_sharded(ci, bounds, max_new=max_new, eos_id=eos)
        _check("edge cases", ci, got, st, max_new=max_new, eos_id=eos)
