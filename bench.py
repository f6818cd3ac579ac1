"""Benchmark of the speculative-decoding verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]

A step is one sampled chain verify (sv_verify_sample: softmax statistics of
every target row, accept scan, residual and inverse-CDF draw) over one batch
of synthetic inputs already resident in HBM.  The default workload is the
sampled chain at B=64 requests, k=4 drafts, V=248,320, bf16 target logits and
bf16 draft probabilities, T=0.7; three input sets rotate so that no step finds
its rows in the 256 MB last-level cache.  Prints one JSON line.

Other workloads (``--workload c1|c2|c3p|c3s|c4|c5|c5g|c5p|tb``) print the same
kind of line for the other configurations (fixed-prefix chain, greedy + prompt
lookup, device uniforms, one vocabulary shard, ragged chain, sampled / greedy /
point-mass tree, EAGLE-2 tree build); their inputs also rotate over device
copies totalling more than twice that cache (the fixed-prefix chain, whose
rows are shared by all rounds by construction, excepted).
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified rounds/s + achieved HBM GB/s (% peak), B=64 k=4 V=248,320 bf16"
PEAK_HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "row_stats_c3_traffic.json")
# the sources the row-statistics kernel is compiled from (its counter summary
# holds while their hash is unchanged)
STATS_SRCS = [os.path.join(ROOT, "draft_verify_sampling_amd", "csrc", f)
              for f in ("k_stats.hip", "segment.hpp", "common.hpp", "words.hpp", "launch.hpp")]


def stats_source_hash():
    h = hashlib.sha1()
    for path in STATS_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _rows(a, kind, torch, dev):
    if kind == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(dev).view(
        torch.bfloat16)


def _i32(a, torch, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


# Input sets rotate so that a set is read again only after more than twice the
# 256 MB MALL of other sets has streamed through: n copies of `touched` bytes.
MALL_BYTES = 256 << 20


def rotation(touched):
    return max(2, -(-2 * MALL_BYTES // max(int(touched), 1)))


def chain_formula_bytes(ci):
    """Logit rows read once + draft rows + draft ids + uniforms."""
    st = 4 if ci.t_kind == "f32" else 2
    sq = 4 if ci.q_kind == "f32" else 2
    ks = ci.draft_len.astype(np.int64)
    return int(((ks + 1) * ci.V * st).sum() + (ks * ci.V * sq).sum() + 4 * ks.sum() + 4 * (ks + 1).sum())


def stats_traffic(step_kernel_src_hash):
    """HBM bytes per launch of the row-statistics kernel from the committed
    counter summary, or None if absent or taken on a different kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha1") != step_kernel_src_hash:
        return None
    return t.get("bytes_per_launch")


def timed(fn, steps, warmup, torch):
    """W untimed calls, then exactly K timed calls bracketed by synchronisations
    (host wall clock, and one HIP event pair on the current stream).  A second,
    untimed-for-the-result pass records an event pair around every call for the
    per-step distribution.  Returns (wall s, event ms over the K calls, per-call
    event ms list)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = e0.elapsed_time(e1)
    n = min(steps, 200)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        ev[i][0].record()
        fn(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return wall, total_ms, [a.elapsed_time(b) for a, b in ev]


def kernel_avg_us(launchers, steps, warmup, torch):
    """Average duration of one launch of a kernel, launched directly as the
    step launches it: `steps` back-to-back launches (rotating input sets, each
    a pre-marshalled call so that the host enqueues faster than the kernel
    runs and the queue never drains) between a pair of HIP events on the
    stream they run on."""
    n = len(launchers)
    for i in range(warmup):
        launchers[i % n]()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        launchers[i % n]()
    e1.record()
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / steps


def cpu_baseline_chain(ci, gpu_out, budget_s, philox=None):
    """The float64 oracle on the host on the same inputs: whole batches of this
    workload's requests, repeated until about budget_s seconds have passed.
    philox = (seed, offset): the GPU drew its uniforms on the device; the
    oracle draws the same ones with its own generator (outside the timing)."""
    import oracle
    u = ci.uniforms if philox is None else oracle.philox_uniforms(philox[0], philox[1], ci.B, ci.k_max + 1)
    reps, t0 = 0, time.perf_counter()
    want = None
    while True:
        want = oracle.verify_sample(ci.target, ci.t_kind, ci.draft, ci.q_kind, ci.V, ci.t_row_start,
                                    ci.q_row_start, ci.draft_ids[:, :ci.k_max], ci.draft_len,
                                    ci.k_max, ci.T, u)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    tok, cnt = gpu_out
    same = (cnt == want["count"]) & (tok == want["tokens"]).all(axis=1)
    near = np.nanmin(np.where(np.isnan(want["margins"]), np.inf, want["margins"]), axis=1) < 1e-6
    return dict(value=round(reps * ci.B / el, 3), unit="rounds/s", cores=1, kind="oracle",
                sample=f"{reps} x all {ci.B} requests of input set 0 ({el:.1f} s, numpy float64, "
                       f"one thread)"), dict(requests=int(ci.B), mismatched=int((~same & ~near).sum()),
                                             boundary=int((~same & near).sum()))


def summarize_counters(fetch_db, write_db, out_json):
    """Per-launch HBM traffic of the row-statistics kernel from two rocprofv3
    --pmc databases (FETCH_SIZE and WRITE_SIZE passes of
    `bench.py --calibrate-copy`), each counter scaled by what it reads for the
    run's 256 MiB device-to-device copies; writes a JSON summary."""
    import sqlite3

    def per_kernel(db, counter):
        cur = sqlite3.connect(db).cursor()
        rows = cur.execute("select kernel_name, value from counters_collection where counter_name = ?",
                           (counter,)).fetchall()
        out = {}
        for name, v in rows:
            out.setdefault(name, []).append(float(v))
        return out

    ref_kib = 256 * 1024
    res = {}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        k = per_kernel(db, counter)
        copies = [v for name, vals in k.items() if "copyBuffer" in name for v in vals]
        big = sorted(copies)[-8:]
        scale = (sum(big) / len(big)) / ref_kib
        stats = [vals for name, vals in k.items() if "k_row_stats" in name][0]
        res[counter] = dict(raw_kib_per_launch=sum(stats) / len(stats), copy_reading_kib=sum(big) / len(big),
                            copy_true_kib=ref_kib, scale=scale,
                            bytes_per_launch=sum(stats) / len(stats) / scale * 1024)
        res[counter + "_all_kernels_raw_kib"] = {n[:80]: sum(v) / len(v) for n, v in k.items()}
    res["kernel_source_sha1"] = stats_source_hash()
    res["bytes_per_launch"] = int(res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"])
    with open(out_json, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps({k: res[k] for k in ("bytes_per_launch", "kernel_source_sha1")}))


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        summarize_counters(sys.argv[2], sys.argv[3], sys.argv[4])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="c3", choices=["c1", "c2", "c3", "c3p", "c3s", "c4", "c5", "c5g", "c5p", "tb"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay one captured HIP graph per step instead of launching the step's "
                         "kernels directly (each replay adds a few microseconds on this stack)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run plain 256 MiB device-to-device copies (a counter calibration "
                         "reference for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import draft_verify_sampling_amd as sv
    import synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    sv.load()
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    src_hash = stats_source_hash()

    result = dict(metric=METRIC, n_gpus=1, steps=args.steps, warmup=args.warmup,
                  higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f32",
                  data="synthetic")
    W = args.workload
    philox = W == "c3p"  # the headline workload with its uniforms drawn on the device
    if philox:
        W = "c3"
    if W in ("c1", "c3", "c4"):
        log(f"generating {W} inputs")
        if W == "c3":
            sets = [synth.c3_sampled(salt=s) for s in (0, 1, 2)]
            cfg = dict(workload="sampled chain verify (speculative sampling): 64 requests, k=4 drafts, "
                                "V=248,320, bf16 target logits ~N(0,2.5^2)+6 on 5 ids, bf16 draft "
                                "probabilities, T=0.7" + (", uniforms drawn on the device (Philox4x64-10)"
                                                          if philox else ""),
                       batch=64, k=4, vocab=248_320, temperature=0.7, inputs="bf16", input_sets=3)
        elif W == "c4":
            sets = [synth.c4_ragged(salt=s) for s in (0, 1, 2)]
            cfg = dict(workload="ragged sampled chain verify: 256 requests, k in 1..8, V=151,936, bf16, "
                                "T=1", batch=256, vocab=151_936, temperature=1.0, inputs="bf16",
                       input_sets=3)
        else:
            sets = [synth.c1_chain()]
            cfg = dict(workload="fixed-prefix sampled chain: 200,000 rounds sharing 5 target and 4 draft "
                                "rows, k=4, V=2048, fp32, T=1", batch=200_000, k=4, vocab=2048,
                       temperature=1.0, inputs="f32", input_sets=1)
        ci0 = sets[0]
        dsets = []
        for ci in sets:
            dsets.append(dict(
                tgt=_rows(ci.target, ci.t_kind, torch, dev), dft=_rows(ci.draft, ci.q_kind, torch, dev),
                trs=_i32(ci.t_row_start, torch, dev), qrs=_i32(ci.q_row_start, torch, dev),
                ids=_i32(ci.draft_ids[:, :ci.k_max], torch, dev), dl=_i32(ci.draft_len, torch, dev),
                u=torch.from_numpy(ci.uniforms).to(dev)))
        B, k_max = ci0.B, ci0.k_max
        out = (torch.empty((B, k_max + 1), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev), None, None)
        ws = sv.Workspace(dev)

        # one pre-marshalled call per input set: the host enqueues a step in a
        # few microseconds, well below the step's GPU time
        if philox:
            calls = [sv.prepare(sv.sv_verify_sample_philox, d["tgt"], d["dft"], d["trs"], d["qrs"], d["ids"],
                                d["dl"], ci0.T, 2026, j, workspace=ws, out=out)[0] for j, d in enumerate(dsets)]
        else:
            calls = [sv.prepare_verify_sample(d["tgt"], d["dft"], d["trs"], d["qrs"], d["ids"], d["dl"], ci0.T,
                                              d["u"], workspace=ws, out=out)[0] for d in dsets]

        def eager(i):
            calls[i % len(calls)]()

        step = eager
        if args.graph:
            # one captured graph per input set: the step's kernels, replayed
            # without per-launch host work
            graphs = []
            side = torch.cuda.Stream()
            for j in range(len(dsets)):
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    eager(j)
                torch.cuda.current_stream().wait_stream(side)
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    eager(j)
                graphs.append(g)

            def step(i):
                graphs[i % len(graphs)].replay()

        log(f"timing {args.steps} steps")
        wall, tot_ms, ev_ms = timed(step, args.steps, args.warmup, torch)
        # one more call on set 0 for the parity sample and token counts
        step(0)
        torch.cuda.synchronize()
        tok0, cnt0 = out[0].cpu().numpy(), out[1].cpu().numpy()
        ms = 1e3 * wall / args.steps
        # the dominant kernel, the statistics of every target row: its duration
        # inside the steps, from HIP events the library records around it
        # (the measurement hook) over a pass of steps like the timed ones;
        # and, for reference, back-to-back stand-alone launches of it (the
        # input sets of a ragged workload differ in row count: one output
        # buffer per set, and the mean of their bytes per launch)
        esz = 4 if ci0.t_kind == "f32" else 2
        rows_bytes = int(round(np.mean([d["tgt"].shape[0] * ci0.V * esz for d in dsets])))
        in_step = None
        # (the ragged workload's steps take the lazy statistics, which read
        # rows 0..m only: there the all-rows kernel is timed stand-alone)
        if not args.graph and W in ("c1", "c3"):
            n = min(args.steps, 200)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            for e0, e1 in ev:
                e0.record()
                e1.record()
            torch.cuda.synchronize()
            for i in range(n):
                sv.sv_debug_time_kernel_once(*ev[i])
                step(i)
            torch.cuda.synchronize()
            in_step = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
        parts = [torch.empty((d["tgt"].shape[0], sv.sv_softmax_segments(d["tgt"].shape[0], ci0.V), 2),
                             dtype=torch.float32, device=dev) for d in dsets]
        stats = [sv.prepare_softmax_partials(d["tgt"], ci0.T, p) for d, p in zip(dsets, parts)]
        alone = kernel_avg_us(stats, args.steps, args.warmup, torch) * 1e-6
        st_avg = in_step if in_step is not None else alone
        achieved = rows_bytes / st_avg / 1e9
        fb = int(round(np.mean([chain_formula_bytes(ci) for ci in sets])))
        cfg["launch"] = "hip graph per step" if args.graph else "direct kernel launches per step"
        result.update(
            value=round(B / (ms * 1e-3), 1), unit="rounds/s", ms_per_step=round(ms, 5), config=cfg,
            tokens_per_s=round(float(cnt0.sum()) / (ms * 1e-3), 1),
            mean_tokens_per_round=round(float(cnt0.mean()), 4),
            event_ms_per_step=dict(timed_region=round(tot_ms / args.steps, 5),
                                   mean=round(float(np.mean(ev_ms)), 5),
                                   p10=round(float(np.percentile(ev_ms, 10)), 5),
                                   p50=round(float(np.percentile(ev_ms, 50)), 5),
                                   p90=round(float(np.percentile(ev_ms, 90)), 5)),
            formula_bytes_per_step=fb,
            formula_GBps=round(fb / (ms * 1e-3) / 1e9, 1),
            formula_frac_of_peak=round(fb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            roofline=dict(bound="hbm", kernel="k_row_stats (softmax statistics of every target row)",
                          achieved=round(achieved, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                          frac=round(achieved / PEAK_HBM_GBPS, 4),
                          traffic=stats_traffic(src_hash) if W == "c3" else None,
                          algorithmic_bytes_per_launch=rows_bytes,
                          avg_launch_us=round(st_avg * 1e6, 3),
                          timing="inside the steps (HIP events around the kernel)" if in_step is not None
                          else "back-to-back stand-alone launches",
                          stand_alone_avg_launch_us=round(alone * 1e6, 3)))
        if not args.no_cpu:
            log("timing the oracle on the host")
            cb, par = cpu_baseline_chain(ci0, (tok0, cnt0), args.cpu_seconds, (2026, 0) if philox else None)
            result["cpu_baseline"] = cb
            result["parity_sample"] = par
    elif W == "c5":
        log("generating c5 inputs")
        ti = synth.c5_tree()
        d = dict(tgt=_rows(ti.target, "bf16", torch, dev), dft=_rows(ti.draft, "bf16", torch, dev),
                 par=_i32(ti.parent, torch, dev), tok=_i32(ti.token, torch, dev),
                 u=torch.from_numpy(ti.uniforms).to(dev))
        ws = sv.Workspace(dev)
        B, N = ti.parent.shape
        out = (torch.empty((B, N), dtype=torch.int32, device=dev), torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev), torch.empty((B, N), dtype=torch.int32, device=dev),
               None)

        # a round reads the visited nodes' target rows and the rejected children's
        # draft rows (~15 MB): device copies of both row sets rotate
        nset = rotation(15 << 20)
        copies = [(d["tgt"], d["dft"])] + [(d["tgt"].clone(), d["dft"].clone()) for _ in range(nset - 1)]
        launches = [sv.prepare(sv.sv_verify_tree, t, q, d["par"], d["tok"], ti.T, d["u"], workspace=ws, out=out)[0]
                    for t, q in copies]

        def step(i):
            launches[i % nset]()

        wall, tot_ms, ev_ms = timed(step, args.steps, args.warmup, torch)
        ms = 1e3 * wall / args.steps
        acc = out[2].cpu().numpy()
        # rows the walk must read: the target row of every visited node (root and
        # kept path); draft rows are read only where a child was rejected
        visited_bytes = int((1 + acc).sum()) * ti.V * 2
        rows_bytes = B * N * ti.V * 2
        fb = 2 * rows_bytes + 2 * 4 * B * N
        result.update(value=round(B / (ms * 1e-3), 1), unit="rounds/s", ms_per_step=round(ms, 5),
                      config=dict(workload="tree verify: 32 requests, 60-node draft trees (depth <= 6, "
                                           "branching <= 4), V=128,256, bf16, T=1", batch=32, nodes=60,
                                  vocab=128_256, temperature=1.0, inputs="bf16", input_sets=nset),
                      tokens_per_s=round(float(out[1].sum().item()) / (ms * 1e-3), 1),
                      formula_bytes_per_step=fb, formula_GBps=round(fb / (ms * 1e-3) / 1e9, 1),
                      visited_target_row_bytes=visited_bytes,
                      event_ms_per_step=dict(timed_region=round(tot_ms / args.steps, 5),
                                             p50=round(float(np.percentile(ev_ms, 50)), 5)),
                      roofline=None)
    elif W in ("c5g", "c5p"):
        # the same trees, verified greedily (argmax picks) or with every
        # candidate tested as a point mass on its own token (no draft rows)
        log("generating c5 inputs")
        ti = synth.c5_tree()
        tgt = _rows(ti.target, "bf16", torch, dev)
        par, tok = _i32(ti.parent, torch, dev), _i32(ti.token, torch, dev)
        u = torch.from_numpy(ti.uniforms).to(dev)
        ws = sv.Workspace(dev)
        B, N = ti.parent.shape
        out = (torch.empty((B, N), dtype=torch.int32, device=dev), torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev), torch.empty((B, N), dtype=torch.int32, device=dev))
        # a round reads the visited nodes' target rows (~11 MB): device copies rotate
        nset = rotation(11 << 20)
        tgts = [tgt] + [tgt.clone() for _ in range(nset - 1)]
        if W == "c5g":
            launches = [sv.prepare(sv.sv_verify_tree_greedy, t, par, tok, workspace=ws, out=out)[0] for t in tgts]
            name = "greedy tree verify (argmax picks)"
        else:
            launches = [sv.prepare(sv.sv_verify_tree_pointmass, t, par, tok, ti.T, u, workspace=ws, out=out)[0]
                        for t in tgts]
            name = "point-mass tree verify (each candidate tested as a point mass)"

        def step(i):
            launches[i % nset]()

        wall, tot_ms, ev_ms = timed(step, args.steps, args.warmup, torch)
        ms = 1e3 * wall / args.steps
        acc = out[2].cpu().numpy()
        visited_bytes = int((1 + acc).sum()) * ti.V * 2
        result.update(value=round(B / (ms * 1e-3), 1), unit="rounds/s", ms_per_step=round(ms, 5),
                      config=dict(workload=f"{name}: 32 requests, 60-node draft trees (depth <= 6, "
                                           "branching <= 4), V=128,256, bf16 target rows, T=1", batch=32,
                                  nodes=60, vocab=128_256, temperature=1.0, inputs="bf16", input_sets=nset),
                      tokens_per_s=round(float(out[1].sum().item()) / (ms * 1e-3), 1),
                      mean_tokens_per_round=round(float(out[1].float().mean().item()), 4),
                      visited_target_row_bytes=visited_bytes,
                      visited_GBps=round(visited_bytes / (ms * 1e-3) / 1e9, 1),
                      event_ms_per_step=dict(timed_region=round(tot_ms / args.steps, 5),
                                             p50=round(float(np.percentile(ev_ms, 50)), 5)),
                      roofline=None)
    elif W == "c3s":
        # the headline round with the vocabulary split over 8 devices: one
        # device's share (31,040 columns of every row) through the three shard
        # steps; the exchanges between them (a few KB) are filled once
        log("generating c3 inputs for the sharded verify")
        ci = synth.c3_sampled()
        G, V, B, k = 8, ci.V, ci.B, ci.k_max
        bounds = [V * g // G for g in range(G + 1)]
        trs, qrs = _i32(ci.t_row_start, torch, dev), _i32(ci.q_row_start, torch, dev)
        ids, dl = _i32(ci.draft_ids[:, :k], torch, dev), _i32(ci.draft_len, torch, dev)
        u = torch.from_numpy(ci.uniforms).to(dev)
        cols = [(_rows(np.ascontiguousarray(ci.target[:, bounds[g]:bounds[g + 1]]), "bf16", torch, dev),
                 _rows(np.ascontiguousarray(ci.draft[:, bounds[g]:bounds[g + 1]]), "bf16", torch, dev))
                for g in range(G)]
        wss = [sv.Workspace(dev) for _ in range(G)]
        st1 = [sv.sv_shard_stats(cols[g][0], cols[g][1], bounds, g, trs, qrs, ids, dl, ci.T, workspace=wss[g])
               for g in range(G)]
        all_pairs = torch.stack([p for p, _ in st1])
        all_at = torch.stack([a for _, a in st1])
        mass = torch.zeros((G, B, 3), dtype=torch.float64, device=dev)
        for g in range(G):
            sv.sv_shard_residual(cols[g][0], cols[g][1], bounds, g, trs, qrs, ids, dl, ci.T, u, all_pairs, all_at,
                                 mass, workspace=wss[g])
        out = (torch.empty((B, k + 1), dtype=torch.int32, device=dev), torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev), None)
        for g in range(G):
            sv.sv_shard_draw(cols[g][0], cols[g][1], bounds, g, trs, qrs, ids, dl, ci.T, u, all_pairs, mass, out,
                             workspace=wss[g])
        # device copies of shard 0's columns rotate (40 MB a step)
        share = (bounds[1] - bounds[0]) * 2 * (ci.target.shape[0] + ci.draft.shape[0])
        nset = rotation(share)
        calls = []
        for j in range(nset):
            tg, qg = cols[0] if j == 0 else (cols[0][0].clone(), cols[0][1].clone())
            calls.append([sv.prepare(sv.sv_shard_stats, tg, qg, bounds, 0, trs, qrs, ids, dl, ci.T, out=st1[0],
                                     workspace=wss[0])[0],
                          sv.prepare(sv.sv_shard_residual, tg, qg, bounds, 0, trs, qrs, ids, dl, ci.T, u, all_pairs,
                                     all_at, mass, workspace=wss[0])[0],
                          sv.prepare(sv.sv_shard_draw, tg, qg, bounds, 0, trs, qrs, ids, dl, ci.T, u, all_pairs, mass,
                                     out, workspace=wss[0])[0]])

        def step(i):
            for c in calls[i % nset]:
                c()

        wall, tot_ms, ev_ms = timed(step, args.steps, args.warmup, torch)
        ms = 1e3 * wall / args.steps
        result.update(value=round(B / (ms * 1e-3), 1), unit="rounds/s", ms_per_step=round(ms, 5),
                      config=dict(workload="sampled chain verify on one of 8 vocabulary shards: 64 requests, k=4, "
                                           "31,040 of V=248,320 columns per device, bf16, T=0.7 (the three shard "
                                           "steps of one device; the all-gathers between them not included)",
                                  batch=B, k=k, vocab=V, shards=G, inputs="bf16", input_sets=nset),
                      shard_bytes=share,
                      event_ms_per_step=dict(timed_region=round(tot_ms / args.steps, 5),
                                             p50=round(float(np.percentile(ev_ms, 50)), 5)),
                      roofline=None)
    elif W == "tb":
        # the EAGLE-2 tree built on the device at the tree workload's shape:
        # 32 requests, top 4 children, the best 4 of each layer expanded, 6
        # rounds, 60 nodes kept; a step = the 6 rounds (each a top-k pass over
        # the expanded nodes' draft rows) and the finalize with the mask
        log("generating draft rows for the tree builder")
        B, V, top, exp, depth, N = 32, 128_256, 4, 4, 6, 60
        rng = np.random.default_rng(2026)
        rounds = []
        for r in range(depth):
            n = B * (1 if r == 0 else exp)
            l = rng.standard_normal((n, V)).astype(np.float32) * 1.5
            p = np.exp(l - l.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            rounds.append(_rows(synth.encode(p, "bf16"), "bf16", torch, dev))
        state = sv.DraftTreeState(B, 1 + top + (depth - 1) * exp * top, dev)
        ws = sv.Workspace(dev)
        nexts = [torch.empty((B, exp), dtype=torch.int32, device=dev) for _ in range(depth)]
        outs = ([torch.empty((B, N), dtype=torch.int32, device=dev) for _ in range(4)]
                + [torch.empty((B, N, N), dtype=torch.uint8, device=dev)])
        # device copies of the draft rows rotate (172 MB a build)
        row_bytes = sum(int(t.numel()) * 2 for t in rounds)
        nset = rotation(row_bytes)
        sets = [rounds] + [[t.clone() for t in rounds] for _ in range(nset - 1)]
        fin = sv.prepare(sv.sv_tree_finalize, state, N, out=outs)[0]
        calls = []
        for rs in sets:
            calls.append([sv.prepare(sv.sv_tree_expand, rs[r], None if r == 0 else nexts[r - 1], top, exp,
                                     state, next_exp=nexts[r], workspace=ws)[0] for r in range(depth)] + [fin])

        def step(i):
            for c in calls[i % nset]:
                c()

        wall, tot_ms, ev_ms = timed(step, args.steps, args.warmup, torch)
        ms = 1e3 * wall / args.steps
        result.update(value=round(B / (ms * 1e-3), 1), unit="trees/s", ms_per_step=round(ms, 5),
                      config=dict(workload="EAGLE-2 draft tree built on the device: 32 requests, V=128,256 bf16 "
                                           "draft rows, top 4 children, 4 nodes expanded per round, 6 rounds, "
                                           "60 nodes kept, ancestor mask", batch=B, vocab=V, top_children=top,
                                  expand_per_round=exp, rounds=depth, nodes=N, inputs="bf16", input_sets=nset),
                      draft_row_bytes_per_step=row_bytes,
                      row_GBps=round(row_bytes / (ms * 1e-3) / 1e9, 1),
                      event_ms_per_step=dict(timed_region=round(tot_ms / args.steps, 5),
                                             p50=round(float(np.percentile(ev_ms, 50)), 5)),
                      roofline=None)
    else:  # c2: prompt lookup + greedy verify
        log("generating c2 inputs")
        g = synth.c2_greedy()
        ctx = _i32(g.ctx, torch, dev)
        cl = _i32(g.ctx_len, torch, dev)
        tgt = _rows(g.target, "bf16", torch, dev)
        trs = _i32(np.arange(g.B) * (g.k + 1), torch, dev)
        ws = sv.Workspace(dev)

        # device copies of the contexts and target rows rotate (21.5 MB a step)
        nset = rotation(g.target.size * 2 + g.ctx.size * 4)
        pairs = []
        for j in range(nset):
            c_j, t_j = (ctx, tgt) if j == 0 else (ctx.clone(), tgt.clone())
            draft, (ids, lens) = sv.prepare(sv.sv_ngram_draft, c_j, cl, g.window, g.k)
            pairs.append((draft, sv.prepare(sv.sv_verify_greedy, t_j, trs, ids, lens, workspace=ws)[0]))

        def step(i):
            draft, verify = pairs[i % nset]
            draft()
            verify()

        wall, tot_ms, ev_ms = timed(step, args.steps, args.warmup, torch)
        ms = 1e3 * wall / args.steps
        fb = g.target.size * 2 + g.ctx.size * 4
        result.update(value=round(g.B / (ms * 1e-3), 1), unit="rounds/s", ms_per_step=round(ms, 5),
                      config=dict(workload="prompt-lookup draft + greedy verify: 64 requests, contexts of "
                                           "4,096 tokens, window 3, k=4, V=32,000, bf16", batch=64, k=4,
                                  vocab=32_000, inputs="bf16", input_sets=nset),
                      formula_bytes_per_step=fb, formula_GBps=round(fb / (ms * 1e-3) / 1e9, 1),
                      dtype="int32+f32", roofline=None)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
