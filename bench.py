"""Benchmark of the speculative-decoding verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]

A step is one pass of the verify path over one batch of synthetic input
already resident in HBM.  The default workload is the sampled chain verify
(sv_verify_sample: softmax statistics of the target rows, accept scan,
residual and inverse-CDF draw) at B=64 requests, k=4 drafts, V=248,320, bf16
target logits and bf16 draft probabilities, T=0.7; three input sets rotate so
that no step finds its rows in the 256 MB last-level cache.  Prints one JSON
line.

The other workloads print the same kind of line: c1 (fixed-prefix chain,
200,000 rounds, V=2048 f32, plus the latency of one B=1 call), c2 (prompt
lookup + greedy verify), c3p (the default workload with its uniforms drawn on
the device), c3s (one of 8 vocabulary shards of the default round), c4 (ragged
chain), c5 / c5g / c5p (sampled / greedy / point-mass tree verify), tb
(EAGLE-2 tree build) and ceiling (a pure streaming read: the practical HBM
read ceiling).  Their inputs rotate over device copies totalling more than
twice that cache (the fixed-prefix chain, whose rows every round shares by
construction, excepted).

Each line carries:
* value / unit: rounds (trees) per second, wall clock over the K timed steps,
  which are bracketed by synchronisations;
* roofline: the dominant kernel of the step, its algorithmic bytes per launch
  over its average duration inside the steps (HIP events that the library's
  measurement hook hands to that kernel's launch, on the step's stream, so
  they take the kernel's own start and end), against
  the 8 TB/s HBM peak; where no one kernel dominates (the shard steps, the
  tree build) the whole step; for the fixed-prefix chain, whose rows stay in
  cache, its fp32 work against the 157.3 TFLOP/s vector peak; `traffic` is
  the kernel's HBM bytes per launch from the committed rocprofv3 counter
  summary, when that summary was taken on the current kernel sources;
* cpu_baseline: the float64 oracle on the host on a bounded sample of the
  same requests, on one thread and over a pool of one process per available
  core (at most 16), with the CPU model.

Order of work: a settle phase of untimed steps (about a second, so the clocks
have ramped), the per-step event pass and the in-step kernel timing pass, then
the W warmup steps and the K timed steps.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified rounds/s + achieved HBM GB/s (% peak), B=64 k=4 V=248,320 bf16"
PEAK_HBM_GBPS = 8000.0
PEAK_FP32_TFLOPS = 157.3
MAX_POOL = 16  # the host cores one GPU's share of the machine has
TIMING = ("inside {n} steps like the timed ones: HIP events handed to the kernel's launch on the step's stream "
          "(the kernel's own start and end)")
CSRC = os.path.join(ROOT, "draft_verify_sampling_amd", "csrc")
# the source a kernel is compiled from: its counter summary holds while the
# code of that file and of the headers it includes (transitively) is unchanged
KERNEL_SRCS = {
    "k_row_stats": "k_stats.hip",
    "k_chain_stats": "k_stats.hip",
    "k_read_ceiling": "k_stats.hip",
    "k_row_argmax": "k_greedy.hip",
    "k_walk": "k_walk.hip",
}


def source_files(src):
    """`src` and the csrc headers it includes, transitively, in first-include
    order (each once)."""
    out, todo = [], [src]
    while todo:
        f = todo.pop(0)
        if f in out or not os.path.exists(os.path.join(CSRC, f)):
            continue
        out.append(f)
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            todo += re.findall(r'^\s*#include\s+"([^"]+)"', fh.read(), flags=re.M)
    return out


def _code_only(text):
    """C++ source without its comments and blank space (so a comment edit
    keeps a counter summary valid).  String literals in these sources hold no
    comment markers."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(kernel):
    """sha1 of the code (comments and blank space stripped) of the sources the
    kernel is compiled from."""
    h = hashlib.sha1()
    for f in source_files(KERNEL_SRCS[kernel]):
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def traffic_file(kernel, workload):
    return os.path.join(ROOT, "profiles", f"{kernel[2:]}_{workload}_traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _rows(a, kind, torch, dev):
    if kind == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(dev).view(torch.bfloat16)


def _i32(a, torch, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


# Input sets rotate so that a set is read again only after more than twice the
# 256 MB MALL of other sets has streamed through: n copies of `touched` bytes.
MALL_BYTES = 256 << 20


def rotation(touched):
    return max(2, -(-2 * MALL_BYTES // max(int(touched), 1)))


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------
def settle(step, seconds, torch):
    """Untimed steps for about `seconds` of wall clock (the device clocks ramp
    up under load); synchronises every 256 steps so the queue stays short."""
    t0, i = time.perf_counter(), 0
    while True:
        step(i)
        i += 1
        if i % 256 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                break
    torch.cuda.synchronize()
    return i


def event_pass(step, n, torch):
    """n steps, each between a pair of HIP events on the current stream: the
    per-step duration distribution (ms)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        ev[i][0].record()
        step(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def kernel_pass(step, n, sv, torch, arm_call):
    """n steps with the library's measurement hook armed right before the
    step's `arm_call`-th library call: the average duration (us) of the
    kernel that call streams its rows with (HIP events handed to its launch
    take its own start and end)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:  # the events exist before the hook records them
        a.record()
        b.record()
    torch.cuda.synchronize()
    for i in range(n):
        step(i, arm=(arm_call, lambda i=i: sv.sv_debug_time_kernel_once(*ev[i])))
    torch.cuda.synchronize()
    return 1e3 * float(np.mean([a.elapsed_time(b) for a, b in ev]))


def timed(step, steps, warmup, torch):
    """W untimed steps, then exactly K timed steps bracketed by
    synchronisations; returns the host wall clock (s) over the K steps.  No
    event is recorded inside the region (a pair cost ~13 us of wall clock per
    region here); the per-step event pass gives the device-side view."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None if absent or taken on different kernel sources."""
    try:
        with open(traffic_file(kernel, workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha1") != source_hash(kernel):
        return None
    return t.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# the float64 oracle on the host: one thread, and a pool of processes
# ---------------------------------------------------------------------------
def oracle_requests(kind, A, P, reqs):
    """The oracle on requests `reqs` of one input set (A: arrays, P: scalars),
    one request at a time; used alike by the one-thread run and the pool's
    workers.  Returns {request: (tokens, count)} for the chain kinds."""
    import oracle
    out = {}
    for b in reqs:
        b = int(b)
        if kind == "chain":
            r = oracle.verify_sample(A["target"], P["t_kind"], A["draft"], P["q_kind"], P["V"], A["t_rs"][b:b + 1],
                                     A["q_rs"][b:b + 1], A["ids"][b:b + 1], A["dlen"][b:b + 1], P["k_max"], P["T"],
                                     A["u"][b:b + 1])
            out[b] = (r["tokens"][0], int(r["count"][0]), float(np.nanmin(np.append(r["margins"][0], np.inf))))
        elif kind in ("tree", "tree_greedy", "tree_point"):
            N = P["N"]
            rows = slice(b * N, (b + 1) * N)
            if kind == "tree":
                oracle.verify_tree(A["target"][rows], "bf16", A["draft"][rows], "bf16", P["V"], A["parent"][b:b + 1],
                                   A["token"][b:b + 1], P["T"], A["u"][b:b + 1], with_diag=False)
            elif kind == "tree_greedy":
                oracle.verify_tree_greedy(A["target"][rows], "bf16", P["V"], A["parent"][b:b + 1],
                                          A["token"][b:b + 1])
            else:
                oracle.verify_tree_pointmass(A["target"][rows], "bf16", P["V"], A["parent"][b:b + 1],
                                             A["token"][b:b + 1], P["T"], A["u"][b:b + 1])
        elif kind == "greedy":
            ids, lens, _ = oracle.ngram_draft(A["ctx"][b:b + 1], A["ctx_len"][b:b + 1], P["window"], P["k"])
            oracle.verify_greedy(A["target"], "bf16", P["V"], np.array([b * (P["k"] + 1)]), ids, lens, P["k"])
        elif kind == "tree_build":
            t = oracle.DraftTree()
            frontier = [0]
            for r in range(P["rounds"]):
                rows = A[f"r{r}"][b:b + 1] if r == 0 else A[f"r{r}"][b * P["exp"]:(b + 1) * P["exp"]]
                frontier = t.expand(frontier, [rows[e] for e in range(len(frontier))], "bf16", P["top"], P["exp"])
            t.finalize(P["N"])
        else:
            raise ValueError(kind)
    return out


_POOL = {}


def _pool_init(paths, kind, P):
    """Pool worker start: map the input arrays from their files (no copies)."""
    _POOL["A"] = {name: np.load(p, mmap_mode="r") for name, p in paths.items()}
    _POOL["kind"], _POOL["P"] = kind, P


def _pool_run(reqs):
    oracle_requests(_POOL["kind"], _POOL["A"], _POOL["P"], reqs)
    return len(reqs)


def cpu_baseline(kind, A, P, B, budget_s, unit):
    """The oracle on this workload's requests (ids cycled over input set 0):
    one thread for about budget_s seconds, then the same requests spread over a
    pool of spawned processes, one per available core, each single-threaded.
    Returns (cpu_baseline object, oracle outputs of the one-thread run)."""
    import multiprocessing as mp
    done, t0, outs = 0, time.perf_counter(), {}
    while True:
        outs.update(oracle_requests(kind, A, P, [done % B]))
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    t1 = time.perf_counter() - t0
    ncores = min(len(os.sched_getaffinity(0)), MAX_POOL)
    pool = dict(value=None, unit=unit, cores=ncores)
    try:
        with tempfile.TemporaryDirectory(prefix="svbench_", dir="/tmp") as tmp:
            paths = {}
            for name, arr in A.items():
                paths[name] = os.path.join(tmp, f"{name}.npy")
                np.save(paths[name], np.ascontiguousarray(arr))
            reqs = [i % B for i in range(max(done, ncores))]
            chunks = [reqs[i::ncores] for i in range(ncores)]
            old = os.environ.get("OMP_NUM_THREADS")
            os.environ["OMP_NUM_THREADS"] = "1"
            try:
                ctx = mp.get_context("spawn")  # fresh interpreters that never touch the GPU
                with ctx.Pool(ncores, initializer=_pool_init, initargs=(paths, kind, P)) as p:
                    p.map(_pool_run, [[0]] * ncores, chunksize=1)  # start-up and imports, untimed
                    tp = time.perf_counter()
                    n = sum(p.map(_pool_run, chunks, chunksize=1))
                    pool_s = time.perf_counter() - tp
            finally:
                if old is None:
                    os.environ.pop("OMP_NUM_THREADS", None)
                else:
                    os.environ["OMP_NUM_THREADS"] = old
        pool.update(value=round(n / pool_s, 3),
                    sample=f"{n} requests over {ncores} spawned single-threaded processes in {pool_s:.2f} s")
    except Exception as e:  # the pool figure is an extra; its absence is stated
        pool["error"] = repr(e)
        log(f"oracle pool run failed: {e!r}")
    return dict(value=round(done / t1, 3), unit=unit, cores=1, kind="oracle",
                sample=f"{done} requests of input set 0, one at a time, in {t1:.1f} s (float64 numpy, one thread)",
                pool=pool, cpu_model=cpu_model()), outs


# ---------------------------------------------------------------------------
# workloads: each builds its inputs and returns a description of its step
# ---------------------------------------------------------------------------
def _call_step(calls, graphs=None):
    """A step runs the pre-marshalled library calls of rotation set i % n (or
    replays that set's captured graph).  arm = (call index, arming function)
    arms the measurement hook right before that call (always direct calls)."""
    def step(i, arm=None):
        j = i % len(calls)
        if graphs is not None and arm is None:
            graphs[j].replay()
            return
        for c_idx, c in enumerate(calls[j]):
            if arm is not None and arm[0] == c_idx:
                arm[1]()
            c()
    return step


def _capture(calls, torch):
    """One captured graph per rotation set (after one direct run of it)."""
    graphs = []
    side = torch.cuda.Stream()
    for group in calls:
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in group:
                c()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in group:
                c()
        graphs.append(g)
    return graphs


def w_chain(W, args, torch, sv, synth, dev):
    philox = W == "c3p"
    if W in ("c3", "c3p"):
        sets = [synth.c3_sampled(salt=s) for s in (0, 1, 2)]
        cfg = dict(workload="sampled chain verify (speculative sampling): 64 requests, k=4 drafts, V=248,320, "
                            "bf16 target logits ~N(0,2.5^2)+6 on 5 ids, bf16 draft probabilities, T=0.7"
                            + (", uniforms drawn on the device (Philox4x64-10)" if philox else ""),
                   batch=64, k=4, vocab=248_320, temperature=0.7, inputs="bf16", input_sets=3)
    elif W == "c4":
        sets = [synth.c4_ragged(salt=s) for s in (0, 1, 2)]
        cfg = dict(workload="ragged sampled chain verify: 256 requests, k in 1..8, V=151,936, bf16, T=1",
                   batch=256, vocab=151_936, temperature=1.0, inputs="bf16", input_sets=3)
    else:
        sets = [synth.c1_chain()]
        cfg = dict(workload="fixed-prefix sampled chain: 200,000 rounds sharing 5 target and 4 draft rows, k=4, "
                            "V=2048, fp32, T=1", batch=200_000, k=4, vocab=2048, temperature=1.0, inputs="f32",
                   input_sets=1)
    ci0 = sets[0]
    B, k_max = ci0.B, ci0.k_max
    ds = [dict(tgt=_rows(c.target, c.t_kind, torch, dev), dft=_rows(c.draft, c.q_kind, torch, dev),
               trs=_i32(c.t_row_start, torch, dev), qrs=_i32(c.q_row_start, torch, dev),
               ids=_i32(c.draft_ids[:, :c.k_max], torch, dev), dl=_i32(c.draft_len, torch, dev),
               u=torch.from_numpy(c.uniforms).to(dev)) for c in sets]
    out = (torch.empty((B, k_max + 1), dtype=torch.int32, device=dev), torch.empty((B,), dtype=torch.int32, device=dev),
           torch.empty((B,), dtype=torch.int32, device=dev), None, None)
    ws = sv.Workspace(dev)
    if philox:
        calls = [[sv.prepare(sv.sv_verify_sample_philox, d["tgt"], d["dft"], d["trs"], d["qrs"], d["ids"], d["dl"],
                             ci0.T, 2026, j, workspace=ws, out=out)[0]] for j, d in enumerate(ds)]
    else:
        calls = [[sv.prepare_verify_sample(d["tgt"], d["dft"], d["trs"], d["qrs"], d["ids"], d["dl"], ci0.T, d["u"],
                                           workspace=ws, out=out)[0]] for d in ds]
    esz = lambda kind: 4 if kind == "f32" else 2

    def formula(c):  # target rows read once + draft rows + ids + uniforms
        ks = c.draft_len.astype(np.int64)
        return int(((ks + 1) * c.V * esz(c.t_kind)).sum() + (ks * c.V * esz(c.q_kind)).sum() + 4 * ks.sum()
                   + 4 * (ks + 1).sum())

    def roofline_bytes(accepted):
        """(bytes per launch of the dominant kernel, its name, what they are)."""
        if W in ("c3", "c3p"):
            return (int(np.mean([c.target.shape[0] * c.V * esz(c.t_kind) for c in sets])), "k_row_stats",
                    "every target row of every request, read once (the softmax statistics)")
        # lazy statistics: rows 0 and 1 are decided one by one (k_chain_stats,
        # the timed kernel), so of the rows 0..m a round reads, it streams
        # rows 0..min(m, 1); the later ones go to k_chain_stats_tail
        nb = [int(((np.minimum(acc.astype(np.int64), 1) + 1) * c.V * esz(c.t_kind)).sum())
              for acc, c in zip(accepted, sets)]
        return (int(np.mean(nb)), "k_chain_stats",
                "target rows 0..min(m, 1) of each request (the rows of its round decided one by one)")

    u0 = ci0.uniforms
    if philox:
        import oracle  # the device drew the uniforms; the oracle's own generator gives the same ones
        u0 = oracle.philox_uniforms(2026, 0, B, k_max + 1)
    A = dict(target=ci0.target, draft=ci0.draft, t_rs=ci0.t_row_start, q_rs=ci0.q_row_start,
             ids=ci0.draft_ids[:, :max(k_max, 1)], dlen=ci0.draft_len, u=u0)
    P = dict(t_kind=ci0.t_kind, q_kind=ci0.q_kind, V=ci0.V, k_max=k_max, T=ci0.T)
    graphs = _capture(calls, torch) if args.graph else None
    w = dict(step=_call_step(calls, graphs), arm_call=0, B=B, unit="rounds/s", cfg=cfg,
             dtype="f32", formula=int(np.mean([formula(c) for c in sets])) if W in ("c3", "c3p") else None,
             out=out, nsets=len(sets),
             roofline_bytes=None if W == "c1" else roofline_bytes, cpu=("chain", A, P, B), kind="chain")
    if W == "c1":
        # one request's call alone: the latency a caller waits for at B=1
        d = ds[0]
        one = sv.prepare_verify_sample(d["tgt"], d["dft"], d["trs"][:1], d["qrs"][:1], d["ids"][:1], d["dl"][:1],
                                       ci0.T, d["u"][:1], workspace=ws)[0]
        w["b1"] = one
    return w


def w_tree(W, args, torch, sv, synth, dev):
    ti = synth.c5_tree()
    B, N, V = ti.B, ti.N, ti.V
    tgt, dft = _rows(ti.target, "bf16", torch, dev), _rows(ti.draft, "bf16", torch, dev)
    par, tok = _i32(ti.parent, torch, dev), _i32(ti.token, torch, dev)
    u = torch.from_numpy(ti.uniforms).to(dev)
    ws = sv.Workspace(dev)
    out = (torch.empty((B, N), dtype=torch.int32, device=dev), torch.empty((B,), dtype=torch.int32, device=dev),
           torch.empty((B,), dtype=torch.int32, device=dev), torch.empty((B, N), dtype=torch.int32, device=dev))
    nset = rotation(15 << 20)  # a round reads the visited nodes' rows (~15 MB)
    if W == "c5":
        copies = [(tgt, dft)] + [(tgt.clone(), dft.clone()) for _ in range(nset - 1)]
        calls = [[sv.prepare(sv.sv_verify_tree, t, q, par, tok, ti.T, u, workspace=ws, out=out + (None,))[0]]
                 for t, q in copies]
        name, kind = "tree verify", "tree"
    else:
        tgts = [tgt] + [tgt.clone() for _ in range(nset - 1)]
        if W == "c5g":
            calls = [[sv.prepare(sv.sv_verify_tree_greedy, t, par, tok, workspace=ws, out=out)[0]] for t in tgts]
            name, kind = "greedy tree verify (argmax picks)", "tree_greedy"
        else:
            calls = [[sv.prepare(sv.sv_verify_tree_pointmass, t, par, tok, ti.T, u, workspace=ws, out=out)[0]]
                     for t in tgts]
            name, kind = "point-mass tree verify (each candidate tested as a point mass)", "tree_point"
    cfg = dict(workload=f"{name}: 32 requests, 60-node draft trees (depth <= 6, branching <= 4), V=128,256, "
                        "bf16, T=1", batch=B, nodes=N, vocab=V, temperature=1.0, inputs="bf16", input_sets=nset)
    kids = [[[c for c in range(1, N) if ti.parent[b, c] == v] for v in range(N)] for b in range(B)]

    def walk_bytes(_accepted):
        """The bytes this round must bring from HBM, from the path it took:
        the target row of every visited node (its softmax pair, or its
        argmax) and, in the sampled tree, the draft row of every visited
        node where a child was rejected (the residual passes).  A node's
        further passes over the same rows (one per rejected child, the last
        draw's, the pick's tile) re-read rows the walk has just read."""
        path, acc = out[3].cpu().numpy(), out[2].cpu().numpy()
        total = 0
        for b in range(B):
            visited = [0] + [int(x) for x in path[b, :acc[b]]]
            for j, v in enumerate(visited):
                rej = len(kids[b][v]) if j + 1 == len(visited) else kids[b][v].index(visited[j + 1])
                total += 2 * V
                if W == "c5" and rej:
                    total += 2 * V
        return (total, "k_walk", "the target row of every visited node" +
                ("; the draft row of every visited node with a rejected child" if W == "c5" else ""))

    A = dict(target=ti.target, draft=ti.draft, parent=ti.parent, token=ti.token, u=ti.uniforms)
    return dict(step=_call_step(calls), arm_call=0, B=B, unit="rounds/s", cfg=cfg,
                dtype="bf16 compares" if W == "c5g" else "f32", formula=None,
                out=out, nsets=1, roofline_bytes=walk_bytes, cpu=(kind, A, dict(N=N, V=V, T=ti.T), B), kind=kind)


def w_greedy(W, args, torch, sv, synth, dev):
    g = synth.c2_greedy()
    ctx, cl = _i32(g.ctx, torch, dev), _i32(g.ctx_len, torch, dev)
    tgt = _rows(g.target, "bf16", torch, dev)
    trs = _i32(np.arange(g.B) * (g.k + 1), torch, dev)
    ws = sv.Workspace(dev)
    nset = rotation(g.target.size * 2 + g.ctx.size * 4)
    calls = []
    for j in range(nset):
        c_j, t_j = (ctx, tgt) if j == 0 else (ctx.clone(), tgt.clone())
        draft, (ids, lens) = sv.prepare(sv.sv_ngram_draft, c_j, cl, g.window, g.k)
        verify, outs = sv.prepare(sv.sv_verify_greedy, t_j, trs, ids, lens, workspace=ws)
        calls.append([draft, verify])
        if j == 0:
            out0 = outs
    cfg = dict(workload="prompt-lookup draft + greedy verify: 64 requests, contexts of 4,096 tokens, window 3, "
                        "k=4, V=32,000, bf16", batch=g.B, k=g.k, vocab=g.V, inputs="bf16", input_sets=nset)
    rows_bytes = g.target.size * 2
    A = dict(ctx=g.ctx, ctx_len=g.ctx_len, target=g.target)
    return dict(step=_call_step(calls), arm_call=1, B=g.B, unit="rounds/s", cfg=cfg, dtype="bf16 compares",
                formula=rows_bytes + g.ctx.size * 4, out=out0, nsets=1,
                roofline_bytes=lambda _a: (rows_bytes, "k_row_argmax", "every target row, read once"),
                cpu=("greedy", A, dict(window=g.window, k=g.k, V=g.V), g.B), kind="greedy")


def w_shard(W, args, torch, sv, synth, dev):
    ci = synth.c3_sampled()
    G, V, B, k = 8, ci.V, ci.B, ci.k_max
    bounds = [V * g // G for g in range(G + 1)]
    trs, qrs = _i32(ci.t_row_start, torch, dev), _i32(ci.q_row_start, torch, dev)
    ids, dl = _i32(ci.draft_ids[:, :k], torch, dev), _i32(ci.draft_len, torch, dev)
    u = torch.from_numpy(ci.uniforms).to(dev)
    cols = [(_rows(np.ascontiguousarray(ci.target[:, bounds[g]:bounds[g + 1]]), "bf16", torch, dev),
             _rows(np.ascontiguousarray(ci.draft[:, bounds[g]:bounds[g + 1]]), "bf16", torch, dev)) for g in range(G)]
    # every shard's steps once, so the exchanged arrays (a few KB, stacked as
    # the all-gathers would leave them) hold a real round's values
    wss = [sv.Workspace(dev) for _ in range(G)]
    st1 = [sv.sv_shard_stats(cols[g][0], cols[g][1], bounds, g, trs, qrs, ids, dl, ci.T, workspace=wss[g])
           for g in range(G)]
    all_pairs, all_at = torch.stack([p for p, _ in st1]), torch.stack([a for _, a in st1])
    mass = torch.zeros((G, B, 3), dtype=torch.float64, device=dev)
    for g in range(G):
        sv.sv_shard_residual(cols[g][0], cols[g][1], bounds, g, trs, qrs, ids, dl, ci.T, u, all_pairs, all_at, mass,
                             workspace=wss[g])
    out = (torch.empty((B, k + 1), dtype=torch.int32, device=dev), torch.empty((B,), dtype=torch.int32, device=dev),
           torch.empty((B,), dtype=torch.int32, device=dev), None)
    for g in range(G):
        sv.sv_shard_draw(cols[g][0], cols[g][1], bounds, g, trs, qrs, ids, dl, ci.T, u, all_pairs, mass, out,
                         workspace=wss[g])
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
    cfg = dict(workload="sampled chain verify on one of 8 vocabulary shards: 64 requests, k=4, 31,040 of "
                        "V=248,320 columns per device, bf16, T=0.7 (one device's three shard steps; the all-gathers "
                        "between them not included)", batch=B, k=k, vocab=V, shards=G, inputs="bf16",
               input_sets=nset)
    A = dict(target=ci.target, draft=ci.draft, t_rs=ci.t_row_start, q_rs=ci.q_row_start, ids=ci.draft_ids[:, :k],
             dlen=ci.draft_len, u=ci.uniforms)
    P = dict(t_kind="bf16", q_kind="bf16", V=V, k_max=k, T=ci.T)
    return dict(step=_call_step(calls), arm_call=None, B=B, unit="rounds/s", cfg=cfg, dtype="f32", formula=share,
                out=None, nsets=1, roofline_bytes=None, step_bytes=share,
                step_bytes_are="this shard's columns of every target and draft row, read once",
                cpu=("chain", A, P, B), kind="shard")


def w_tree_build(W, args, torch, sv, synth, dev):
    B, V, top, exp, depth, N = 32, 128_256, 4, 4, 6, 60
    rng = np.random.default_rng(2026)
    host = []
    for r in range(depth):
        n = B * (1 if r == 0 else exp)
        l = rng.standard_normal((n, V)).astype(np.float32) * 1.5
        p = np.exp(l - l.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        host.append(synth.encode(p, "bf16"))
    rounds = [_rows(h, "bf16", torch, dev) for h in host]
    state = sv.DraftTreeState(B, 1 + top + (depth - 1) * exp * top, dev)
    ws = sv.Workspace(dev)
    nexts = [torch.empty((B, exp), dtype=torch.int32, device=dev) for _ in range(depth)]
    outs = [torch.empty((B, N), dtype=torch.int32, device=dev) for _ in range(4)] + \
           [torch.empty((B, N, N), dtype=torch.uint8, device=dev)]
    row_bytes = sum(int(t.numel()) * 2 for t in rounds)
    nset = rotation(row_bytes)
    sets = [rounds] + [[t.clone() for t in rounds] for _ in range(nset - 1)]
    fin = sv.prepare(sv.sv_tree_finalize, state, N, out=outs)[0]
    calls = [[sv.prepare(sv.sv_tree_expand, rs[r], None if r == 0 else nexts[r - 1], top, exp, state,
                         next_exp=nexts[r], workspace=ws)[0] for r in range(depth)] + [fin] for rs in sets]
    cfg = dict(workload="EAGLE-2 draft tree built on the device: 32 requests, V=128,256 bf16 draft rows, top 4 "
                        "children, 4 nodes expanded per round, 6 rounds, 60 nodes kept, ancestor mask", batch=B,
               vocab=V, top_children=top, expand_per_round=exp, rounds=depth, nodes=N, inputs="bf16",
               input_sets=nset)
    A = {f"r{r}": h for r, h in enumerate(host)}
    return dict(step=_call_step(calls), arm_call=None, B=B, unit="trees/s", cfg=cfg, dtype="f32 / f64 sums",
                formula=row_bytes, out=None, nsets=1, roofline_bytes=None, step_bytes=row_bytes,
                step_bytes_are="the expanded nodes' draft rows of the 6 rounds, read once",
                cpu=("tree_build", A, dict(rounds=depth, exp=exp, top=top, N=N), B), kind="tree_build")


# ---------------------------------------------------------------------------
# in-kernel time lines (the timestamped copy of the library)
# ---------------------------------------------------------------------------
TL_TICK_US = 0.01  # the real-time counter runs at 100 MHz


def _tl_read(lib, name, n=16384, slots=64):
    """Records [n, slots] of one time-line array (0: point not reached)."""
    import ctypes
    buf = (ctypes.c_ulonglong * (n * slots))()
    rc = getattr(lib, name + "_read")(buf, ctypes.c_int64(n))
    if rc != 0:
        raise RuntimeError(f"{name}_read failed ({rc})")
    return np.frombuffer(buf, dtype=np.uint64).reshape(n, slots).astype(np.int64)


def _stats(x):
    x = np.asarray([v for v in x if np.isfinite(v)], dtype=np.float64)
    if x.size == 0:
        return None
    return dict(n=int(x.size), mean=round(float(x.mean()), 2), p50=round(float(np.percentile(x, 50)), 2),
                p90=round(float(np.percentile(x, 90)), 2), max=round(float(x.max()), 2))


def timeline_walk(A, B):
    """Phases of the sampled tree walk's exchanges from its records (us)."""
    n = int((A[:, 0] > 0).sum())
    G = n // B
    R = A[:B * G].reshape(B, G, 64).astype(np.float64)
    R[R <= 0] = np.nan
    t0 = np.nanmin(R[:, :, 0])
    R = (R - t0) * TL_TICK_US
    ph = {k: [] for k in ("pass", "fold_waves", "exchange", "barrier", "fold_words", "decide")}
    rounds, ends = [], []
    for b in range(B):
        nx = 0
        while nx < 9 and np.isfinite(R[b, :, 2 + 6 * nx + 5]).all():
            nx += 1
        rounds.append(nx)
        ends.append(np.nanmax(R[b, :, 63]))
        for x in range(nx):
            s = 2 + 6 * x
            ph["pass"].append(np.nanmax(R[b, :, s + 1] - R[b, :, s]))
            ph["fold_waves"].append(np.nanmax(R[b, :, s + 2] - R[b, :, s + 1]))
            ph["exchange"].append(np.nanmax(R[b, :, s + 3]) - np.nanmax(R[b, :, s + 2]))
            ph["barrier"].append(np.nanmax(R[b, :, s + 4] - R[b, :, s + 3]))
            ph["fold_words"].append(np.nanmax(R[b, :, s + 5] - R[b, :, s + 4]))
            if x + 1 < nx:
                ph["decide"].append(np.nanmax(R[b, :, s + 6] - R[b, :, s + 5]))
    slow = int(np.nanargmax(ends))
    path = []
    for x in range(rounds[slow]):
        s = 2 + 6 * x
        path.append(dict(start=round(float(np.nanmin(R[slow, :, s])), 2),
                         pass_us=round(float(np.nanmax(R[slow, :, s + 1] - R[slow, :, s])), 2),
                         words_seen=round(float(np.nanmax(R[slow, :, s + 3])), 2)))
    return dict(requests=B, workgroups_per_request=G, span_us=round(float(np.nanmax(ends)), 2),
                prologue_us=_stats(np.nanmax(R[:, :, 1], axis=1)),
                rounds=dict(mean=round(float(np.mean(rounds)), 2), max=int(max(rounds))),
                phases_us={k: _stats(v) for k, v in ph.items()},
                last_draw_us=dict(after_last_exchange=_stats([np.nanmax(R[b, :, 63]) - np.nanmax(
                    R[b, :, 2 + 6 * (rounds[b] - 1) + 5]) for b in range(B) if rounds[b] > 0]),
                    tile_search=_stats(np.nanmax(R[:, :, 62] - R[:, :, 61], axis=1)),
                    pick_and_write=_stats(np.nanmax(R[:, :, 63] - R[:, :, 62], axis=1))),
                slowest_request=dict(index=slow, end_us=round(float(ends[slow]), 2), exchanges=path))


def _tl_draw(D, t0):
    """The draw's phases from its records (us from t0)."""
    d0 = D[:, 0][D[:, 0] > 0].min()
    D = D.astype(np.float64)
    D[D < d0] = np.nan  # unreached points, and stamps of earlier steps' last blocks
    D = (D - t0) * TL_TICK_US
    last = np.isfinite(D[:, 7])
    return dict(first_start=round(float(np.nanmin(D[:, 0])), 2),
                last_end=round(float(np.nanmax(D[:, 7])), 2),
                break_row_us=_stats(D[:, 1] - D[:, 0]), tiles_us=_stats(D[:, 2] - D[:, 1]),
                count_us=_stats(D[:, 3] - D[:, 2]), tiles_done_at=_stats(D[:, 2]),
                last_block=dict(gather_us=_stats(D[last, 4] - D[last, 3]),
                                find_tile_us=_stats(D[last, 5] - D[last, 4]),
                                pick_us=_stats(D[last, 6] - D[last, 5]),
                                write_us=_stats(D[last, 7] - D[last, 6]),
                                end_at=_stats(D[last, 7])))


def timeline_chain(S, D, n_stats, n_draw):
    """Phases of the headline step (statistics, then the draw) from the
    records of both kernels (us)."""
    S = S[:n_stats].astype(np.float64)
    t0 = S[:, 0][S[:, 0] > 0].min()
    S[S <= 0] = np.nan
    S = (S - t0) * TL_TICK_US
    return dict(stats_blocks=n_stats, draw_blocks=n_draw,
                stats=dict(first_start=round(float(np.nanmin(S[:, 0])), 2),
                           last_start=round(float(np.nanmax(S[:, 0])), 2),
                           last_end=round(float(np.nanmax(S[:, 1])), 2), block_us=_stats(S[:, 1] - S[:, 0])),
                draw=_tl_draw(D[:n_draw], t0))


def timeline_ragged(L, D, rows, per_row, n_draw, n_tail=0):
    """Phases of the ragged step (lazy statistics, then the draw) from the
    records of both kernels (us), row by row of the row-major statistics
    grid, and the items of the later rows taken at once (n_tail records
    after the grid's)."""
    T = L[rows * per_row:rows * per_row + n_tail].astype(np.float64)
    L = L[:rows * per_row].astype(np.float64)
    t0 = L[:, 0][L[:, 0] > 0].min()
    L[L <= 0] = np.nan
    L = (L - t0) * TL_TICK_US
    T[T <= 0] = np.nan
    T = (T - t0) * TL_TICK_US
    tail = None
    if n_tail:
        tail = dict(items=n_tail, start_first=round(float(np.nanmin(T[:, 0])), 2),
                    start_last=round(float(np.nanmax(T[:, 0])), 2), start_at=_stats(T[:, 0]),
                    item_us=_stats(T[:, 2] - T[:, 0]), word_at=_stats(T[:, 2]),
                    last_word=round(float(np.nanmax(T[:, 2])), 2),
                    rows_decided=int(np.isfinite(T[:, 3]).sum()),
                    last_stamp=round(float(np.nanmax(T)), 2))
    out = []
    for i in range(rows):
        r = L[i * per_row:(i + 1) * per_row]
        live = np.isfinite(r[:, 1])
        out.append(dict(row=i, blocks=per_row, loaded=int(live.sum()),
                        start_first=round(float(np.nanmin(r[:, 0])), 2),
                        start_last=round(float(np.nanmax(r[:, 0])), 2),
                        loaded_end_last=round(float(np.nanmax(r[live, 2])), 2) if live.any() else None,
                        decided=int(np.isfinite(r[:, 3]).sum())))
    dead = ~np.isfinite(L[:, 1])
    return dict(stats_blocks=rows * per_row, draw_blocks=n_draw,
                stats=dict(last_start=round(float(np.nanmax(L[:, 0])), 2),
                           last_stamp=round(float(np.nanmax(L)), 2),
                           blocks_not_loading=int(dead.sum()), rows=out),
                tail=tail, draw=_tl_draw(D[:n_draw], t0))


def run_timeline(kind, args, torch, sv, synth, dev):
    """The time line of one step (the last of 20 back-to-back steps after the
    settle phase) of the sampled tree walk (kind "walk", the C5 trees), the
    headline chain ("chain") or the ragged chain ("ragged"), from the
    timestamped library."""
    W = {"walk": "c5", "chain": "c3", "ragged": "c4"}[kind]
    w = WORKLOADS[W](W, args, torch, sv, synth, dev)
    step = w["step"]
    settle(step, args.settle_seconds, torch)
    lib = sv.load()
    names = {"walk": [("sv_timeline_walk", 16384, 64)],
             "chain": [("sv_timeline_stats", 16384, 64), ("sv_timeline_draw", 16384, 64)],
             "ragged": [("sv_timeline_lazy", 65536, 4), ("sv_timeline_draw", 16384, 64)]}[kind]
    for i in range(19):
        step(i)
    torch.cuda.synchronize()
    # records are overwritten in place, and a block that stops early in one
    # step keeps an earlier step's later readings: clear just before the last
    for nm, _, _ in names:
        if getattr(lib, nm + "_clear")() != 0:
            raise RuntimeError(f"{nm}_clear failed")
    step(19)
    torch.cuda.synchronize()
    recs = [_tl_read(lib, nm, n, slots) for nm, n, slots in names]
    if kind == "walk":
        out = timeline_walk(recs[0], w["B"])
    elif kind == "chain":
        n_stats = int((recs[0][:, 0] > 0).sum())
        n_draw = int((recs[1][:, 0] > 0).sum())
        out = timeline_chain(recs[0], recs[1], n_stats, n_draw)
    else:
        per_row = w["B"] * ((w["cfg"]["vocab"] + 8191) // 8192)  # every block stamps its start
        k_max = 8
        rows = min(k_max + 1, 2)  # rows decided one by one; the later ones' items follow
        n_tail = int((recs[0][rows * per_row:, 0] > 0).sum())
        out = timeline_ragged(recs[0], recs[1], rows, per_row, int((recs[1][:, 0] > 0).sum()), n_tail)
    return dict(timeline=kind, workload=W, step="the last of 20 steps after the settle phase (records cleared before it)",
                unit="us from the first block's start", **out)


TIMELINE_TITLES = {
    "walk": "sampled tree walk, C5 trees (B=32, N=60, V=128,256 bf16, T=1)",
    "chain": "headline sampled chain (B=64, k=4, V=248,320 bf16, T=0.7)",
    "ragged": "ragged sampled chain, lazy statistics (B=256, k in 1..8, V=151,936 bf16, T=1)"}


TIMELINE_LEGEND = {
    "walk": [
        "prologue_us: the tree and uniforms loaded, the exchange words zeroed, the ticket stored",
        "rounds: exchanges per request (one per pass over the vocabulary)",
        "phases_us (per request, the slowest of its workgroups, per exchange): pass = the pass over the "
        "workgroup's slice (a node's statistics, or a residual pass from the rows or the LDS copy); "
        "fold_waves = the waves' sums folded and the slice's words built; exchange = from the last "
        "workgroup's store until every workgroup has seen all words; barrier = the exchange's barrier; "
        "fold_words = the request's words folded; decide = the next child's test up to the next pass",
        "last_draw_us: from the last exchange's fold to the outputs; tile_search = the drawing wave's "
        "search for the tile; pick_and_write = the id picked from one re-read tile, and the writes",
        "slowest_request.exchanges: each exchange's start, its pass and the time all words were seen"],
    "chain": [
        "stats: the all-rows statistics kernel; block_us = one block's life",
        "draw.break_row_us: the break row and its pair known (two dependent load rounds, the rows' "
        "combines); tiles_us: the block's tiles summed; count_us: its count returned; tiles_done_at: "
        "when a block's tiles are done",
        "draw.last_block (the request's last block): gather = the tile sums gathered; find_tile; pick = "
        "the id picked from one re-read tile; write = the outputs written; end_at = when they are"],
    "ragged": [
        "stats: the lazy statistics kernel, row-major grid (all requests' row 0 first); blocks_not_loading "
        "= blocks that left without streaming (row past the request's draft length, or its round stopped)",
        "stats.rows: per row of the grid: its blocks, those that streamed their segment, the first and "
        "last block starts, the last streaming block's word stored, and the requests whose row was decided",
        "tail: the kernel that reads rows 2..k_b of the rounds still running at once (items of four "
        "segments of a row): its items' starts, item_us = start to word stored, word_at = when, and the "
        "rows it decided",
        "draw: as for the headline chain's draw (break row, tiles, count; the last block's gather, tile "
        "search, pick and writes)"]}


def timeline_markdown(d):
    """The time line `d` (from run_timeline) as a markdown summary: every
    distribution as median (mean, p90, max) over n, every row list as a
    table."""
    out = [f"# In-kernel time line: {TIMELINE_TITLES[d['timeline']]}", "",
           "Commands (the timestamped copy of the library, then one step's records):", "",
           "    python -m draft_verify_sampling_amd.build --timeline",
           f"    python bench.py --timeline {d['timeline']} --markdown", "",
           f"Step: {d['step']}.  Unit: {d['unit']} (100 MHz real-time counter, 0.01 us).  "
           "Distributions: median (mean, p90, max) over n.", ""]
    out += [f"- {x}" for x in TIMELINE_LEGEND[d["timeline"]]] + [""]

    def dist(v):
        return f"{v['p50']:.2f} (mean {v['mean']:.2f}, p90 {v['p90']:.2f}, max {v['max']:.2f}; n={v['n']})"

    def walk(prefix, obj, rows):
        for k, v in obj.items():
            name = f"{prefix}{k}"
            if isinstance(v, dict) and set(v) == {"n", "mean", "p50", "p90", "max"}:
                rows.append((name, dist(v)))
            elif isinstance(v, dict):
                walk(name + ".", v, rows)
            elif isinstance(v, list):
                tables.append((name, v))
            elif v is None:
                rows.append((name, "-"))
            else:
                rows.append((name, str(v)))

    rows, tables = [], []
    walk("", {k: v for k, v in d.items() if k not in ("timeline", "step", "unit")}, rows)
    out += ["| quantity | value |", "|---|---|"] + [f"| {a} | {b} |" for a, b in rows]
    for name, lst in tables:
        if not lst:
            continue
        keys = list(lst[0])
        out += ["", f"{name}:", "", "| " + " | ".join(keys) + " |", "|" + "---|" * len(keys)]
        out += ["| " + " | ".join("-" if r[k] is None else str(r[k]) for k in keys) + " |" for r in lst]
    return "\n".join(out) + "\n"


WORKLOADS = {"c1": w_chain, "c3": w_chain, "c3p": w_chain, "c4": w_chain, "c5": w_tree, "c5g": w_tree,
             "c5p": w_tree, "c2": w_greedy, "c3s": w_shard, "tb": w_tree_build}


def run_ceiling(args, torch, sv, dev, result):
    """A pure streaming read of 256 MiB per launch over four rotating buffers
    (1 GiB, so no launch finds its bytes in the 256 MB cache), each launch
    timed with HIP events: the practical HBM read ceiling."""
    part = 256 << 20
    bufs = [torch.full((part,), 7, dtype=torch.uint8, device=dev) for _ in range(4)]
    nb = int(sv.load().sv_debug_read_blocks(part))
    outs = [torch.empty((nb,), dtype=torch.int32, device=dev) for _ in bufs]
    def step(i, arm=None):
        if arm is not None:
            arm[1]()
        sv.sv_debug_read_ceiling(bufs[i % 4], out=outs[i % 4])

    settle(step, args.settle_seconds, torch)
    us = kernel_pass(step, 200, sv, torch, 0)
    wall = timed(step, args.steps, args.warmup, torch)
    gbps = part / (us * 1e-6) / 1e9
    result.update(metric="HBM read ceiling (pure streaming read)", value=round(gbps, 1), unit="GB/s",
                  ms_per_step=round(1e3 * wall / args.steps, 5), dtype="u32 words",
                  config=dict(workload="pure streaming read of 256 MiB per launch (16-byte non-temporal loads), four "
                                       "rotating buffers", bytes_per_launch=part),
                  roofline=dict(bound="hbm", kernel="k_read_ceiling", achieved=round(gbps, 1), peak=PEAK_HBM_GBPS,
                                unit="GB/s", frac=round(gbps / PEAK_HBM_GBPS, 4),
                                traffic=traffic("ceiling", "k_read_ceiling"), algorithmic_bytes_per_launch=part,
                                avg_launch_us=round(us, 3),
                                timing="200 launches, each timed by HIP events given to the launch (the kernel's own "
                                       "start and end)"),
                  cpu_baseline=None)


# ---------------------------------------------------------------------------
# counter summaries (rocprofv3 --pmc csv -> profiles/<kernel>_<w>_traffic.json)
# ---------------------------------------------------------------------------
def summarize_counters(workload, kernel, fetch_csv, write_csv):
    """Per-launch HBM traffic of `kernel` from two rocprofv3 --pmc runs (the
    counter_collection.csv of a FETCH_SIZE and of a WRITE_SIZE pass of
    `bench.py --calibrate-copy`, --output-format csv), each
    counter scaled by what it reads for the run's 256 MiB device-to-device
    copies; writes profiles/<kernel>_<workload>_traffic.json."""
    import csv

    def per_kernel(path, counter):
        """{kernel name: [value per dispatch]} from a counter_collection.csv,
        and the values of the run's first 8 copies (the calibration copies
        `--calibrate-copy` runs before anything else)."""
        out, copies = {}, []
        with open(path, newline="") as f:
            rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        for r in rows:
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
            if "copyBuffer" in r["Kernel_Name"] and len(copies) < 8:
                copies.append(float(r["Counter_Value"]))
        return out, copies

    ref_kib = 256 * 1024
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        k, copies = per_kernel(path, counter)
        scale = (sum(copies) / len(copies)) / ref_kib
        vals = [v for name, vs in k.items() if f"{kernel}<" in name or name.startswith(f"{kernel}(")
                or f"::{kernel}(" in name for v in vs]
        res[counter] = dict(raw_kib_per_launch=sum(vals) / len(vals), copy_reading_kib=sum(copies) / len(copies),
                            copy_true_kib=ref_kib, scale=scale, launches=len(vals),
                            bytes_per_launch=sum(vals) / len(vals) / scale * 1024)
        res[counter + "_all_kernels_raw_kib"] = {n[:80]: sum(v) / len(v) for n, v in k.items()}
    res.update(workload=workload, kernel=kernel, kernel_source_sha1=source_hash(kernel),
               bytes_per_launch=int(res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"]))
    with open(traffic_file(kernel, workload), "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps({k: res[k] for k in ("workload", "kernel", "bytes_per_launch", "kernel_source_sha1")}))


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        summarize_counters(*sys.argv[2:6])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOADS) + ["ceiling"])
    ap.add_argument("--settle-seconds", type=float, default=1.0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="chain workloads: replay one captured HIP graph per step instead of launching the step's "
                         "kernels directly")
    ap.add_argument("--timeline", choices=["walk", "chain", "ragged"],
                    help="print the in-kernel time line of one step of the sampled tree walk (C5), the headline "
                         "chain (C3) or the ragged chain (C4) instead of the bench line; needs the timestamped "
                         "library (python -m draft_verify_sampling_amd.build --timeline)")
    ap.add_argument("--markdown", action="store_true",
                    help="with --timeline: print the time line as a markdown summary instead of JSON")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run plain 256 MiB device-to-device copies (the counter calibration reference for "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)
    if args.graph and args.workload not in ("c1", "c3", "c3p", "c4"):
        ap.error("--graph is for the chain workloads (c1, c3, c3p, c4)")

    if args.timeline:
        lib = os.path.join(ROOT, "draft_verify_sampling_amd", "libspecverify_timeline.so")
        if not os.path.exists(lib):
            ap.error("build the timestamped library first: python -m draft_verify_sampling_amd.build --timeline")
        os.environ["SPECVERIFY_LIB"] = lib
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

    result = dict(metric=METRIC, n_gpus=1, steps=args.steps, warmup=args.warmup, higher_is_better=True,
                  scaling="weak", vs_baseline=None, data="synthetic")
    W = args.workload
    if args.timeline:
        tl = run_timeline(args.timeline, args, torch, sv, synth, dev)
        print(timeline_markdown(tl) if args.markdown else json.dumps(tl), end="\n" if not args.markdown else "",
              flush=True)
        return
    if W == "ceiling":
        run_ceiling(args, torch, sv, dev, result)
        print(json.dumps(result), flush=True)
        return
    log(f"generating {W} inputs")
    w = WORKLOADS[W](W, args, torch, sv, synth, dev)
    step = w["step"]
    log("settle, event and kernel passes")
    n_settle = settle(step, args.settle_seconds, torch)
    n_meas = max(20, min(args.steps, 200))
    ev_ms = event_pass(step, n_meas, torch)
    k_us = kernel_pass(step, n_meas, sv, torch, w["arm_call"]) if w["arm_call"] is not None else None
    log(f"{args.warmup} warmup steps, then {args.steps} timed steps")
    wall = timed(step, args.steps, args.warmup, torch)
    ms = 1e3 * wall / args.steps
    # the outputs of each rotation set (the rows a lazy round read, the tokens)
    out, accepted, counts = w["out"], [], None
    if out is not None:
        for j in range(w["nsets"]):
            step(j)
            torch.cuda.synchronize()
            accepted.append(out[2].cpu().numpy().copy())
        step(0)
        torch.cuda.synchronize()
        counts = out[1].cpu().numpy()
    result.update(value=round(w["B"] / (ms * 1e-3), 1), unit=w["unit"], ms_per_step=round(ms, 5), config=w["cfg"],
                  dtype=w["dtype"])
    if counts is not None:
        result.update(tokens_per_s=round(float(counts.sum()) / (ms * 1e-3), 1),
                      mean_tokens_per_round=round(float(counts.mean()), 4))
    fb = w["formula"]
    result.update(event_ms_per_step=dict(mean=round(float(np.mean(ev_ms)), 5),
                                         p10=round(float(np.percentile(ev_ms, 10)), 5),
                                         p50=round(float(np.percentile(ev_ms, 50)), 5),
                                         p90=round(float(np.percentile(ev_ms, 90)), 5)),
                  settle_steps=n_settle)
    if fb is not None:
        # bytes the step's inputs occupy when every row is read once (the
        # lazy and tree workloads read fewer, so they carry only the roofline)
        result.update(formula_bytes_per_step=fb, formula_GBps=round(fb / (ms * 1e-3) / 1e9, 1),
                      formula_frac_of_peak=round(fb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4))
    if W == "c1":
        # cache-resident by construction (every round reads the same 9 rows):
        # one wave per round, bound by its dependent steps; the one-wave
        # round's fp32 work against the vector peak
        B, V = w["B"], w["cfg"]["vocab"]
        flops = B * V * 12.0
        tfl = flops / (k_us * 1e-6) / 1e12
        result["roofline"] = dict(bound="alu", kernel="k_walk_small", achieved=round(tfl, 3), peak=PEAK_FP32_TFLOPS,
                                  unit="TFLOP/s", frac=round(tfl / PEAK_FP32_TFLOPS, 4), traffic=None,
                                  algorithmic_flops_per_launch=flops,
                                  flops_are="12 fp32 operations per element of each round's drawn row: fma, exp2, "
                                            "scale, subtract, clamp and add in the weight pass, the same again in "
                                            "the pick's rescan (exp2 counted as one)",
                                  avg_launch_us=round(k_us, 3), timing=TIMING.format(n=n_meas))
        lat = []
        for _ in range(20):
            w["b1"]()
        torch.cuda.synchronize()
        for _ in range(200):
            t0 = time.perf_counter()
            w["b1"]()
            torch.cuda.synchronize()
            lat.append(time.perf_counter() - t0)
        result["b1_call_latency_us"] = dict(p50=round(1e6 * float(np.percentile(lat, 50)), 2),
                                            p90=round(1e6 * float(np.percentile(lat, 90)), 2),
                                            what="one sv_verify_sample call at B=1 (V=2048 f32, k=4), enqueue to "
                                                 "completion, host wall clock, 200 calls")
    elif w["roofline_bytes"] is not None and k_us is not None:
        nbytes, kname, what = w["roofline_bytes"](accepted)
        gbps = nbytes / (k_us * 1e-6) / 1e9
        result["roofline"] = dict(bound="hbm", kernel=kname, achieved=round(gbps, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                                  frac=round(gbps / PEAK_HBM_GBPS, 4), traffic=traffic(W, kname),
                                  algorithmic_bytes_per_launch=nbytes, bytes_are=what, avg_launch_us=round(k_us, 3),
                                  timing=TIMING.format(n=n_meas))
    else:
        nbytes = w["step_bytes"]
        gbps = nbytes / (ms * 1e-3) / 1e9
        result["roofline"] = dict(bound="hbm", kernel="whole step", achieved=round(gbps, 1), peak=PEAK_HBM_GBPS,
                                  unit="GB/s", frac=round(gbps / PEAK_HBM_GBPS, 4), traffic=None,
                                  algorithmic_bytes_per_launch=nbytes, bytes_are=w["step_bytes_are"],
                                  timing="wall clock per step (several dependent kernels)")
    if not args.no_cpu:
        log("timing the oracle on the host")
        kind, A, P, B = w["cpu"]
        cb, outs = cpu_baseline(kind, A, P, B, args.cpu_seconds, "trees/s" if kind == "tree_build" else "rounds/s")
        result["cpu_baseline"] = cb
        if kind == "chain" and w["kind"] == "chain":
            tok = out[0].cpu().numpy()
            same = near = 0
            for b, (t, c, margin) in outs.items():
                ok = c == counts[b] and np.array_equal(t, tok[b])
                same += ok
                near += (not ok) and margin < 1e-6
            result["parity_sample"] = dict(requests=len(outs), identical=int(same), boundary=int(near),
                                           mismatched=int(len(outs) - same - near))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
