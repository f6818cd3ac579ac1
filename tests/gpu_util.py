"""Helpers for the GPU tests: move generated inputs to the device, run the
library, compare with the oracle."""
import sys

import numpy as np
import torch

import draft_verify_sampling_amd as sv

DEV = "cuda"
BOUNDARY = 1e-6      # a uniform this close to a decision edge may flip it
RTOL = 1e-5          # probabilities, normalisers, ratios, residual mass


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def rows_to_dev(a, kind):
    if kind == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)
    bits = np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(bits).to(DEV).view(torch.bfloat16)


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def run_sample(ci, status=None, workspace=None, max_new=None, eos_id=-1, diag=True):
    """diag=True also asks for the per-row diagnostics, which makes the library
    compute every row's statistics; diag=False is the lazy path that skips the
    rows after the break (where rows are not shared between requests)."""
    tgt = rows_to_dev(ci.target, ci.t_kind)
    dft = rows_to_dev(ci.draft, ci.q_kind)
    mn = i32(max_new) if max_new is not None else None
    tok, cnt, acc, dg, rs = sv.sv_verify_sample(
        tgt, dft, i32(ci.t_row_start), i32(ci.q_row_start), i32(ci.draft_ids[:, :ci.k_max]),
        i32(ci.draft_len), ci.T, f32(ci.uniforms), max_new=mn, eos_id=eos_id, diag=diag,
        resid=True, dev_status=status, workspace=workspace)
    torch.cuda.synchronize()
    return dict(tokens=tok.cpu().numpy(), count=cnt.cpu().numpy(), accepted=acc.cpu().numpy(),
                diag=dg.cpu().numpy() if diag else None, resid=rs.cpu().numpy())


def same_round(a, b, keys=("tokens", "count", "accepted")):
    """The chain's statistics paths (the partials of every row, with or
    without the diagnostics kernel, or the lazy statistics of rows 0..m)
    combine the same segment pairs in the same order, and the draw kernel
    that follows each forms and totals the same tile sums, so tokens, counts
    and accepted counts are identical.  The residual mass is held to one unit
    in the last place of float32 (the bound a change of the totalling order
    would need)."""
    for k in keys:
        assert np.array_equal(a[k], b[k]), k
    ra, rb = np.asarray(a["resid"], dtype=np.float64), np.asarray(b["resid"], dtype=np.float64)
    assert np.all(np.abs(ra - rb) <= 2.0 ** -23 * np.abs(rb)), "resid"


def run_greedy(target, kind, t_row_start, draft_ids, draft_len, max_new=None, eos_id=-1,
               status=None):
    tok, cnt, acc = sv.sv_verify_greedy(rows_to_dev(target, kind), i32(t_row_start), i32(draft_ids),
                                        i32(draft_len), i32(max_new) if max_new is not None else None,
                                        eos_id, dev_status=status)
    torch.cuda.synchronize()
    return dict(tokens=tok.cpu().numpy(), count=cnt.cpu().numpy(), accepted=acc.cpu().numpy())


def run_tree(ti, status=None, diag=True):
    tok, cnt, acc, pth, dg = sv.sv_verify_tree(
        rows_to_dev(ti.target, ti.t_kind), rows_to_dev(ti.draft, ti.q_kind), i32(ti.parent),
        i32(ti.token), ti.T, f32(ti.uniforms), diag=diag, dev_status=status)
    torch.cuda.synchronize()
    return dict(tokens=tok.cpu().numpy(), count=cnt.cpu().numpy(), accepted=acc.cpu().numpy(),
                path=pth.cpu().numpy(), diag=dg.cpu().numpy() if diag else None)


def close(a, b, rtol=RTOL, atol=1e-30):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.abs(a - b) <= atol + rtol * np.abs(b)


def compare_tokens(got, want, keys=("tokens", "count", "accepted")):
    """Per request: equal, or a boundary case (some decision of the oracle lies
    within BOUNDARY of its edge), or a failure.  Returns (n_boundary, failures)."""
    B = want["count"].shape[0]
    same = np.ones(B, dtype=bool)
    for k in keys:
        g, w = got[k], want[k]
        same &= (g.reshape(B, -1) == w.reshape(B, -1)).all(axis=1)
    near = np.nanmin(np.where(np.isnan(want["margins"]), np.inf, want["margins"]), axis=1) < BOUNDARY
    bad = ~same & ~near
    return int((~same & near).sum()), np.nonzero(bad)[0]


def tv_at_noise_level(emitted, n_positions, p_rows, count, rng, family_alpha=0.01, reps=1000):
    """TV of the emitted token at each position (rounds that reach it) against
    the target row there, and the fraction of `reps` multinomial draws of the
    same size from that row whose TV is at least as large (a p-value).  The
    positions are tested together at family-wise level `family_alpha`
    (Bonferroni: each p-value must exceed family_alpha / positions tested).
    Returns [(position, n, tv, p-value)]; asserts the criterion."""
    res = []
    for i in range(n_positions):
        sel = count > i
        n = int(sel.sum())
        if n < 2000:
            continue
        p = p_rows[i]
        emp = np.bincount(emitted[sel, i], minlength=p.shape[0]) / n
        tv = 0.5 * np.abs(emp - p).sum()
        noise = np.array([0.5 * np.abs(rng.multinomial(n, p) / n - p).sum() for _ in range(reps)])
        res.append((i, n, float(tv), float((noise >= tv).mean())))
    for i, n, tv, pv in res:
        say(f"  position {i}: n={n} TV={tv:.4f} p-value {pv:.3f}")
    assert res, "no position reached often enough"
    assert min(pv for *_, pv in res) > family_alpha / len(res), res
    return res
