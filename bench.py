"""Throughput of the mixture draft tree path on one MI355X.

A step is one pass of the whole path -- log-softmax + top-k, common cut-off,
tree build, mask + position ids, verification walk -- over one batch of trees
whose inputs already sit in HBM.  Default workload: 64 independent trees with
K=8 modes, L=15 drafted positions, V=151936, B=256, walks alternating T=0 / T=1
(seeded synthetic inputs).

Prints one JSON line: trees/s for the whole step, plus the logits pass's HBM
roofline (algorithmic bytes / measured kernel time) and the fp64 CPU oracle
timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import torch

METRIC = "mixture trees built+verified/sec (K=8,L=15,B=256,V=152K); logits HBM GB/s"
HBM_PEAK_GBS = 8000.0
HERE = os.path.dirname(os.path.abspath(__file__))
# Sources of the logits kernel's code: a traffic figure measured on other code is stale.
LSM_SOURCES = ["mixture_draft_tree_amd/csrc/lsm_topk.hip", "mixture_draft_tree_amd/csrc/mfd_device.hpp"]
TRAFFIC_FILE = "profiles/lsm_topk_kernel_batched_64x8x15x151936_hbm_traffic.txt"
SQ_FILE = "profiles/sq_counters_batched_64x8x15x151936.md"


def lsm_source_sha() -> str:
    h = hashlib.sha256()
    for rel in LSM_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profile_field(rel: str, workload: str, key: str):
    """A figure of the logits kernel from a committed counter summary of the
    batched workload, or None if there is none for this workload or the kernel
    sources changed since the counters were taken."""
    path = os.path.join(HERE, rel)
    if workload != "batched" or not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith((" ", "#", "$", "|")):
                k, val = line.split(":", 1)
                fields[k.strip()] = val.strip()
    if fields.get("kernel_source_sha256") != lsm_source_sha():
        return None
    try:
        return float(fields[key])
    except (KeyError, ValueError):
        return None


def measured_traffic(workload: str):
    """HBM bytes per launch of the logits kernel (FETCH_SIZE + WRITE_SIZE,
    copy-calibrated), or None."""
    return profile_field(TRAFFIC_FILE, workload, "hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="batched",
                    choices=["batched", "single", "stress", "deep", "batched_deep", "subset", "batched_subset",
                             "batched_modes"])
    ap.add_argument("--cpu-baseline-trees", type=int, default=16,
                    help="trees of the workload the fp64 oracle is timed on, at least one per core, one process "
                         "per core (0 = skip)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-gib", type=int, default=0,
                    help="after the run, copy a buffer of this many GiB device to device: a plain copy of "
                         "known size against which hardware byte counters are calibrated (0 = skip)")
    ap.add_argument("--latency-steps", type=int, default=20,
                    help="steps of the single-tree workload timed for per-tree latency (0 = skip)")
    ap.add_argument("--deep-workload", default="batched_deep", choices=["batched_deep", "none"],
                    help="also time the confident-drafter batch (deep trees, pages-like acceptance lengths)")
    ap.add_argument("--subset-workload", default="batched_subset", choices=["batched_subset", "none"],
                    help="also time drafting over a 65536-token subset of the vocabulary (walk over all of it)")
    ap.add_argument("--modes-workload", default="batched_modes", choices=["batched_modes", "none"],
                    help="also time a batch mixing K_n = 8 and K_n = 1 trees (per-request mode counts)")
    ap.add_argument("--lmhead-workload", default="lmhead", choices=["lmhead", "none"],
                    help="also time the fused LM head + log-softmax/top-k call (one tree and 64 trees)")
    return ap.parse_args()


BF16_MFMA_PEAK_TFLOPS = 2500.0


def fused_lmhead(steps: int, stream) -> dict:
    """Time mfd_lmhead_logsoftmax_topk on the drafter's shape (K=8, L=15,
    V=151936, D=2560, k=256) at one tree and at 64 trees, beside the unfused
    route it replaces: the LM-head product into bf16 logits (torch.matmul,
    a library GEMM) followed by mfd_logsoftmax_topk."""
    from mixture_draft_tree_amd import mfdtree as M
    from mixture_draft_tree_amd import synth
    out = {}
    reps = max(3, min(steps, 20))
    for name in ("lmhead_single", "lmhead_batched"):
        b = synth.lmhead_batch(name, device="cuda")
        w = b.workload
        N, K, L, D, V, k = w.N, w.K, w.L, w.D, w.V, min(w.B, w.V)
        H, W = b.hidden, b.weight
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
        lse, ids, raw = e((N, K, L), torch.float64), e((N, K, L, k), torch.int32), e((N, K, L, k), torch.float32)
        st = torch.zeros((N,), dtype=torch.int32, device="cuda")
        ws = M.lmhead_workspace(N, K, L, V, k)

        def timed(fn):
            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        fused_ms = timed(lambda: M.mfd_lmhead_logsoftmax_topk(H, W, k, lse, ids, raw, None, st, ws=ws, stream=stream))
        pk = M.mfd_lmhead_pack_weight(W, stream=stream)
        packed_ms = timed(lambda: M.mfd_lmhead_logsoftmax_topk(H, pk, k, lse, ids, raw, None, st, ws=ws,
                                                               stream=stream))
        del pk
        flops = 2.0 * N * K * L * V * D
        ok = int(st.abs().sum().item()) == 0
        logits = e((N * K * L, V), torch.bfloat16)
        Hf = H.view(N * K * L, D)
        mm_ms = timed(lambda: torch.matmul(Hf, W.t(), out=logits))
        lg = logits.view(N, K, L, V)
        lsm_ms = timed(lambda: M.mfd_logsoftmax_topk(lg, k, lse, ids, raw, None, st, stream=stream))
        # drafting over 65536 of the V tokens (the head's rows of a sorted subset)
        g = torch.Generator(device="cuda")
        g.manual_seed(4242)
        vmap = torch.sort(torch.randperm(V, generator=g, device="cuda")[:65536]).values.to(torch.int32)
        Wsub = W[vmap.long()].contiguous()
        ws_sub = M.lmhead_workspace(N, K, L, 65536, k)
        sub_ms = timed(lambda: M.mfd_lmhead_logsoftmax_topk(H, Wsub, k, lse, ids, raw, None, st, ws=ws_sub,
                                                            stream=stream, vocab_map=vmap, V_full=V))
        ok = ok and int(st.abs().sum().item()) == 0
        del Wsub, ws_sub
        tflops = flops / (fused_ms * 1e-3) / 1e12
        out[name] = {
            "workload": f"{name}: {N} tree(s), K={K}, L={L}, V={V}, D={D}, k={k}, bf16 hidden states and LM head",
            "fused_ms": fused_ms, "status_ok": ok,
            "tflops": tflops, "frac_of_bf16_mfma_peak": tflops / BF16_MFMA_PEAK_TFLOPS,
            "head_read_GBps": V * D * 2 / (fused_ms * 1e-3) / 1e9,
            "unfused_matmul_ms": mm_ms, "unfused_logsoftmax_topk_ms": lsm_ms,
            "unfused_total_ms": mm_ms + lsm_ms, "fused_over_unfused": fused_ms / (mm_ms + lsm_ms),
            "reduced_vocab_fused_ms": sub_ms, "reduced_vocab_tokens": 65536,
            "packed_head_fused_ms": packed_ms,
            "packed_head_read_GBps": V * D * 2 / (packed_ms * 1e-3) / 1e9,
            "packed_head_over_unfused": packed_ms / (mm_ms + lsm_ms),
        }
        del b, H, W, logits, lg, ws
        torch.cuda.empty_cache()
    return out


def _oracle_worker(name, base_seed, trees, barrier, results):
    """One pool worker: draws its trees and their target rows (untimed), waits
    until every worker is ready, then runs the whole oracle path on each tree."""
    try:
        import threadpoolctl
        threadpoolctl.threadpool_limits(1)
    except ImportError:
        pass
    torch.set_num_threads(1)
    import oracle as O
    from mixture_draft_tree_amd import synth

    w = synth.WORKLOADS[name]
    work = []
    for n in trees:
        b = synth.draft_batch(name, base_seed=base_seed, device="cpu", N=1, start=n)
        x = b.logits[0].double().numpy()
        # target rows come from the oracle's own tree, drawn outside the timed part
        tr = O.canonical_tree(O.mixture_select_heap(x, w.B), int(b.anchor[0]), w.B)
        dep = torch.from_numpy(tr["depth"]).to(torch.int32)[None]
        nn = torch.tensor([tr["n_nodes"]], dtype=torch.int32)
        R = synth.target_logits(b, dep, nn, device="cpu", base_seed=base_seed)[0].double().numpy()
        work.append((x, R, int(b.anchor[0]), int(b.pos_base[0]), float(b.temperature[0]),
                     int(b.seed[0]) & ((1 << 64) - 1)))
    barrier.wait(timeout=900)
    t0 = time.perf_counter()
    per_tree = []
    for x, R, anchor, pos, T, seed in work:
        t1 = time.perf_counter()
        sel = O.mixture_select_heap(x, w.B)
        tr = O.canonical_tree(sel, anchor, w.B)
        O.tree_mask(tr["parent"], tr["depth"], tr["n_nodes"], pos, w.B + 1)
        O.verify_walk(tr["node_token"], tr["parent"], tr["depth"], tr["n_nodes"], R, T, seed, w.L)
        per_tree.append(time.perf_counter() - t1)
    t_end = time.perf_counter()
    # untimed: whether each tree's node set is decided by exact comparisons
    # (cut-off band of 1e-4, the score tolerance)
    excluded = 0
    for x, *_ in work:
        excluded += 0 if O.band_is_exact(x, O.mixture_select_heap(x, w.B, band=1e-4), 1e-4) else 1
    results.put((t0, t_end, per_tree, excluded))


def host_cpu_model() -> str:
    """The host's CPU model as lscpu names it (falls back to /proc/cpuinfo)."""
    import subprocess
    try:
        r = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20)
        for ln in r.stdout.splitlines():
            if ln.strip().startswith("Model name:"):
                return ln.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        return ""


def cpu_baseline(name: str, base_seed: int, n_trees: int):
    """Time the fp64 oracle end to end (log-softmax, ranks, heap, layout, mask,
    walk) on trees 0 .. n_trees-1 of the workload, spread over every core this
    process may run on (one single-threaded process per core; n_trees is raised
    to the core count so each core gets at least one tree).  Runs before the
    GPU is touched, so the workers are plain forks."""
    import multiprocessing as mp

    avail = len(os.sched_getaffinity(0))
    n_trees = max(n_trees, avail)
    cores = max(1, min(n_trees, avail))
    ctx = mp.get_context("fork")
    barrier = ctx.Barrier(cores)
    results = ctx.Queue()
    procs = [ctx.Process(target=_oracle_worker, args=(name, base_seed, list(range(c, n_trees, cores)), barrier,
                                                       results))
             for c in range(cores)]
    for pr in procs:
        pr.start()
    out = [results.get(timeout=1800) for _ in procs]
    for pr in procs:
        pr.join(timeout=60)
    assert all(pr.exitcode == 0 for pr in procs), [pr.exitcode for pr in procs]
    wall = max(o[1] for o in out) - min(o[0] for o in out)
    per_tree = sorted(t for o in out for t in o[2])
    excluded = sum(o[3] for o in out)
    return {"value": n_trees / wall, "unit": "trees/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_trees} trees of the {name} workload, full oracle path, {cores} single-threaded "
                      f"processes (one per core this process may use), {wall:.1f} s wall, "
                      f"{sum(per_tree):.1f} s of CPU work",
            "per_tree_s_one_core_median": statistics.median(per_tree), "host_cpu": host_cpu_model(),
            "band_excluded_trees": {"trees": n_trees, "excluded": excluded,
                                    "reason": "node set not decided by exact comparisons: a selected and an "
                                              "unselected prefix within 1e-4 of the cut-off differ in best mode "
                                              "or depth, or have a runner-up mode within 1e-4; such trees are "
                                              "checked for validity, not array for array"}}


def run_steps(P, logits, anchor, pos, R, temps, seeds, steps, warmup, stream):
    """Times `steps` whole steps; returns (total ms, per-stage ms lists)."""
    for _ in range(warmup):
        P.step(logits, anchor, pos, R, temps, seeds)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)] for _ in range(steps)]
    calls = [lambda: P.logsoftmax_topk(logits), lambda: P.mixture_tree(anchor), lambda: P.tree_mask(pos),
             lambda: P.verify_walk(R, temps, seeds)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(steps):
        e = ev[s]
        e[0].record(stream)
        for i, call in enumerate(calls):
            call()
            e[i + 1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    return t_start.elapsed_time(t_end), ev


def separate_tree_calls_ms(P, anchor, reps, stream):
    """The cut-off and the tree as two launches (mfd_mixture_threshold, then
    mfd_tree_build), for comparison with the one-launch mfd_mixture_tree."""
    for _ in range(2):
        P.mixture_threshold()
        P.tree_build(anchor)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    thr, bld = 0.0, 0.0
    for _ in range(reps):
        e[0].record(stream)
        P.mixture_threshold()
        e[1].record(stream)
        P.tree_build(anchor)
        e[2].record(stream)
        torch.cuda.synchronize()
        thr += e[0].elapsed_time(e[1])
        bld += e[1].elapsed_time(e[2])
    return {"mixture_threshold": thr / reps, "tree_build": bld / reps}


def capture_step(P, logits, anchor, pos, R, temps, seeds):
    """The five calls of one step captured in a HIP graph (torch.cuda.CUDAGraph)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        P.step(logits, anchor, pos, R, temps, seeds)   # warm-up on the capturing stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        P.step(logits, anchor, pos, R, temps, seeds)
    torch.cuda.synchronize()
    return g


def graph_steps(g, steps, warmup, stream):
    """Times `steps` replays of a captured step; returns (ms per step, sorted per-step ms)."""
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for s in range(steps):
        g.replay()
        ev[s + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[s].elapsed_time(ev[s + 1]) for s in range(steps))
    return ev[0].elapsed_time(ev[steps]) / steps, per


def setup(name, seed, dev):
    from mixture_draft_tree_amd import synth
    from mixture_draft_tree_amd.pipeline import MixtureTreePath

    w = synth.WORKLOADS[name]
    b = synth.draft_batch(name, base_seed=seed, device=dev)
    N = b.logits.shape[0]
    vmap = None if b.vocab_map is None else b.vocab_map.to(dev)
    modes = None if b.modes is None else b.modes.to(dev)
    P = MixtureTreePath(N, w.K, w.L, b.logits.shape[-1], w.B, vocab_map=vmap, V_full=w.V, modes=modes)
    logits = b.logits.contiguous()
    anchor, pos = b.anchor.to(dev), b.pos_base.to(dev)
    temps, seeds = b.temperature.to(dev), b.seed.to(dev)
    # the target's per-node rows depend on the tree they verify: build once
    P.build(logits, anchor, pos)
    torch.cuda.synchronize()
    R = synth.target_logits(b, P.buf.depth, P.buf.n_nodes, device=dev, base_seed=seed).contiguous()
    torch.cuda.synchronize()
    return w, N, P, logits, anchor, pos, temps, seeds, R


def single_tree_latency(seed, steps, stream, name="single"):
    """One whole step on a one-tree workload (N=1): mean ms per step (eager
    launches, events between the calls), the mean of each stage, and the mean
    of a HIP-graph replay of the step."""
    w, N, P, logits, anchor, pos, temps, seeds, R = setup(name, seed, "cuda")
    total, ev = run_steps(P, logits, anchor, pos, R, temps, seeds, steps, 3, stream)
    status = P.buf.status.cpu()
    assert int(status.abs().sum()) == 0, f"per-tree status flags set ({name}): {status.tolist()}"
    stages = {nm: statistics.mean(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps))
              for i, nm in enumerate(STAGES)}
    stages["median"] = {nm: statistics.median(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps))
                        for i, nm in enumerate(STAGES)}
    stages["separate_threshold_and_build"] = separate_tree_calls_ms(P, anchor, min(steps, 20), stream)
    g = capture_step(P, logits, anchor, pos, R, temps, seeds)
    graph_ms, _ = graph_steps(g, steps, 3, stream)
    del g
    status = P.buf.status.cpu()
    assert int(status.abs().sum()) == 0, f"per-tree status flags set ({name}): {status.tolist()}"
    return {"workload": f"{name}: 1 tree, K={w.K}, L={w.L}, V={w.V}, B={w.B}", "ms": graph_ms,
            "eager_ms": total / steps, "stages_ms": stages, "tau": int(P.buf.tau[0]),
            "n_nodes": int(P.buf.n_nodes[0]),
            "logits_GBps": w.K * w.L * logits.shape[-1] * logits.element_size() / (stages["logsoftmax_topk"] * 1e-3) / 1e9}


def read_ceiling(buf, reps, stream):
    """Rate of mfd_stream_read over `buf` (one read of every byte), GB/s: the
    achievable streaming-read rate, next to the nominal HBM peak."""
    from mixture_draft_tree_amd import mfdtree as M
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        M.mfd_stream_read(buf, sink, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        M.mfd_stream_read(buf, sink, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = buf.numel() * buf.element_size()
    return {"kernel": "stream_read_kernel (mfd_stream_read)", "bytes": nbytes, "avg_launch_ms": ms,
            "GBps": nbytes / (ms * 1e-3) / 1e9, "frac_of_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


STAGES = ["logsoftmax_topk", "mixture_tree", "tree_mask", "verify_walk"]


def covered_mass_stats(P, R, temps, stream, reps=5):
    """Time mfd_covered_mass over the built trees; mean covered mass next to the
    walks' mean accepted count (the two agree in expectation)."""
    from mixture_draft_tree_amd import mfdtree as M
    N = R.shape[0]
    mass = torch.empty(N, dtype=torch.float64, device="cuda")
    ws = M.covered_mass_workspace(N, R.shape[1])
    args = (R, P.buf.node_token, P.buf.parent, P.buf.n_nodes, temps, mass)
    M.mfd_covered_mass(*args, ws=ws, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        M.mfd_covered_mass(*args, ws=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return {"covered_mass_ms": e0.elapsed_time(e1) / reps, "mean_covered_mass": float(mass.mean()),
            "mean_accepted_walk": float((P.buf.tau - 1).float().mean())}


def tree_stats(P) -> dict:
    """Shape of the built trees and walks: tau and depth histograms, per-mode
    keep counts at the cut-off (the per-mode keeps of the common cut-off)."""
    tau = P.buf.tau.cpu()
    nn = P.buf.n_nodes.cpu()
    dep = P.buf.depth.cpu()
    kept = P.buf.per_mode_kept.cpu().to(torch.float64)
    dh = {}
    for n in range(dep.shape[0]):
        for d in dep[n, 1:int(nn[n])].tolist():
            dh[d] = dh.get(d, 0) + 1
    th = {}
    for t in tau.tolist():
        th[t] = th.get(t, 0) + 1
    return {"tau_histogram": {str(k): th[k] for k in sorted(th)},
            "node_depth_histogram": {str(k): dh[k] for k in sorted(dh)},
            "mean_nodes": float(nn.to(torch.float64).mean()),
            "per_mode_kept_mean": [round(float(v), 2) for v in kept.mean(0).tolist()],
            "per_mode_kept_total_mean": float(kept.sum(1).mean()),
            "n_select_mean": float(P.buf.n_select.cpu().to(torch.float64).mean())}


def timed_workload(name, seed, steps, warmup, stream, diagnostics=False):
    """Whole steps on workload `name`: (ms per step, per-stage ms, N, buffers)."""
    w, N, P, logits, anchor, pos, temps, seeds, R = setup(name, seed, "cuda")
    total_ms, ev = run_steps(P, logits, anchor, pos, R, temps, seeds, steps, warmup, stream)
    stage = {nm: statistics.mean(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps))
             for i, nm in enumerate(STAGES)}
    # eager stage times include any host delay in enqueueing the stage's launch;
    # the medians are robust to such single outliers, the means are what the
    # roofline uses (average launch duration)
    stage["median"] = {nm: statistics.median(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps))
                       for i, nm in enumerate(STAGES)}
    per_step = sorted(ev[s][0].elapsed_time(ev[s][len(STAGES)]) for s in range(steps))
    q = lambda f: per_step[min(len(per_step) - 1, int(f * len(per_step)))]
    stage["step_ms_percentiles"] = {"p10": q(0.1), "p50": statistics.median(per_step), "p90": q(0.9)}
    status = P.buf.status.cpu()
    assert int(status.abs().sum()) == 0, f"per-tree status flags set ({name}): {status.tolist()}"
    # the same step captured in a HIP graph: no host launch work between the calls
    g = capture_step(P, logits, anchor, pos, R, temps, seeds)
    graph_ms, gper = graph_steps(g, steps, warmup, stream)
    del g
    stage["eager_ms_per_step"] = total_ms / steps
    stage["eager_step_ms_percentiles"] = stage.pop("step_ms_percentiles")
    q = lambda f: gper[min(len(gper) - 1, int(f * len(gper)))]
    stage["step_ms_percentiles"] = {"p10": q(0.1), "p50": statistics.median(gper), "p90": q(0.9)}
    status = P.buf.status.cpu()
    assert int(status.abs().sum()) == 0, f"per-tree status flags set ({name}): {status.tolist()}"
    stage["separate_threshold_and_build"] = separate_tree_calls_ms(P, anchor, min(steps, 20), stream)
    if diagnostics:
        stage["diagnostics"] = covered_mass_stats(P, R, temps, stream)
    return graph_ms, stage, N, w, P, logits


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); trees are independent, "
              f"so N GPUs would each run this same per-GPU batch.", file=sys.stderr)
        sys.exit(2)
    name = args.workload
    # the CPU oracle runs first, in forked processes, before anything touches the GPU
    cpu = cpu_baseline(name, args.seed, args.cpu_baseline_trees) if args.cpu_baseline_trees > 0 else None
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    stream = torch.cuda.current_stream()
    ms_per_step, stage_ms, N, w, P, logits = timed_workload(name, args.seed, args.steps, args.warmup, stream,
                                                            diagnostics=True)
    diag = stage_ms.pop("diagnostics")
    pcts = stage_ms.pop("step_ms_percentiles")
    eager_ms = stage_ms.pop("eager_ms_per_step")
    eager_pcts = stage_ms.pop("eager_step_ms_percentiles")

    rows = N * w.K * w.L if P.modes is None else int(P.modes.sum()) * w.L   # rows the logits pass reads
    logits_bytes = rows * logits.shape[-1] * logits.element_size()
    lsm_ms = stage_ms["logsoftmax_topk"]
    achieved = logits_bytes / (lsm_ms * 1e-3) / 1e9
    tau = P.buf.tau.cpu().float()
    ceiling = read_ceiling(logits, args.steps, stream)
    out = {
        "metric": METRIC,
        "value": N / (ms_per_step * 1e-3),
        "unit": "trees/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; drafter logits N(0,9) + per-mode futures at +8, target rows N(0,1) + 10 on one future)",
        "config": {"workload": f"{name}: {N} trees, K={w.K}, L={w.L}, V={w.V}, B={w.B}, "
                               f"T pattern {list(w.temperatures)}",
                   "trees": N, "K": w.K, "L": w.L, "V": w.V, "B": w.B},
        "roofline": {"bound": "hbm", "kernel": "lsm_topk_kernel (mfd_logsoftmax_topk)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(name),
                     "algorithmic_bytes_per_launch": logits_bytes, "avg_launch_ms": lsm_ms,
                     "read_ceiling": ceiling, "frac_of_read_ceiling": achieved / ceiling["GBps"],
                     "valu_issue_frac": profile_field(SQ_FILE, name, "lsm_valu_issue_frac")},
        "step_ms_percentiles": pcts,
        "launch": "each step is one replay of a HIP graph holding the path's calls (logits pass, cut-off and tree "
                  "in one launch, mask, walk) and a status clear; stages_ms are timed on eager "
                  "launches with events between the calls",
        "eager_ms_per_step": eager_ms,
        "eager_step_ms_percentiles": eager_pcts,
        "stages_ms": stage_ms,
        "logits_GBps": achieved,
        "per_tree_latency_ms": ms_per_step if N == 1 else None,
        "single_tree_latency_ms": None,
        "tau_mean": float(tau.mean()),
        "diagnostics": diag,
    }
    out["trees"] = tree_stats(P)
    if args.latency_steps > 0 and name == "batched":
        # one tree at a time (batch size 1, the pages' setting): each stage timed
        b1 = {nm: single_tree_latency(args.seed, args.latency_steps, stream, nm) for nm in ("single", "deep", "stress")}
        out["batch1"] = b1
        out["single_tree_latency_ms"] = b1["single"]["ms"]
        out["stress_tree_latency_ms"] = b1["stress"]["ms"]
    if args.deep_workload != "none" and name == "batched":
        del P, logits
        dms, dstage, dN, dw, dP, _ = timed_workload(args.deep_workload, args.seed, args.steps, args.warmup, stream,
                                                    diagnostics=True)
        ddiag = dstage.pop("diagnostics")
        dpcts = dstage.pop("step_ms_percentiles")
        deager = dstage.pop("eager_ms_per_step")
        dstage.pop("eager_step_ms_percentiles")
        out["deep"] = {
            "workload": f"{args.deep_workload}: {dN} trees, K={dw.K}, L={dw.L}, V={dw.V}, B={dw.B}, "
                        f"T pattern {list(dw.temperatures)}",
            "data": "synthetic (seeded; confident drafter: N(0,4) noise, 16 Zipf alternatives, each mode's future "
                    "at 16+N(0,2.25); target rows N(0,1) + 16 on one future up to a random deviation depth)",
            "value": dN / (dms * 1e-3), "unit": "trees/s", "ms_per_step": dms, "step_ms_percentiles": dpcts,
            "eager_ms_per_step": deager,
            "stages_ms": dstage,
            "tau_mean": float(dP.buf.tau.cpu().float().mean()),
            "single_tree_latency_ms": out.get("batch1", {}).get("deep", {}).get("ms"),
            "trees": tree_stats(dP),
            "diagnostics": ddiag,
        }
    if args.subset_workload != "none" and name == "batched":
        sms, sstage, sN, sw, sP, slog = timed_workload(args.subset_workload, args.seed, args.steps, args.warmup,
                                                       stream)
        spcts = sstage.pop("step_ms_percentiles")
        seager = sstage.pop("eager_ms_per_step")
        sstage.pop("eager_step_ms_percentiles")
        sbytes = sN * sw.K * sw.L * slog.shape[-1] * slog.element_size()
        sgbs = sbytes / (sstage["logsoftmax_topk"] * 1e-3) / 1e9
        out["reduced_vocab"] = {
            "workload": f"{args.subset_workload}: {sN} trees, K={sw.K}, L={sw.L}, drafting over {slog.shape[-1]} of "
                        f"V={sw.V} tokens, B={sw.B}, T pattern {list(sw.temperatures)}",
            "value": sN / (sms * 1e-3), "unit": "trees/s", "ms_per_step": sms, "step_ms_percentiles": spcts,
            "eager_ms_per_step": seager,
            "stages_ms": sstage,
            "logits_GBps": sgbs, "logits_frac_of_peak": sgbs / HBM_PEAK_GBS,
            "algorithmic_bytes_per_launch": sbytes, "tau_mean": float(sP.buf.tau.cpu().float().mean()),
        }
        del sP, slog
    if args.modes_workload != "none" and name == "batched":
        mms, mstage, mN, mw, mP, mlog = timed_workload(args.modes_workload, args.seed, args.steps, args.warmup,
                                                       stream)
        mpcts = mstage.pop("step_ms_percentiles")
        meager = mstage.pop("eager_ms_per_step")
        mstage.pop("eager_step_ms_percentiles")
        kn = mP.modes.cpu()
        mbytes = int(kn.sum()) * mw.L * mw.V * mlog.element_size()
        mgbs = mbytes / (mstage["logsoftmax_topk"] * 1e-3) / 1e9
        mtau = mP.buf.tau.cpu().float()
        out["per_request_modes"] = {
            "workload": f"{args.modes_workload}: {mN} trees of the confident-drafter shape, K={mw.K}, L={mw.L}, "
                        f"V={mw.V}, B={mw.B}, K_n cycling {list(mw.modes)}, T pattern {list(mw.temperatures)}",
            "value": mN / (mms * 1e-3), "unit": "trees/s", "ms_per_step": mms, "step_ms_percentiles": mpcts,
            "eager_ms_per_step": meager,
            "stages_ms": mstage,
            "active_rows": int(kn.sum()) * mw.L, "logits_GBps": mgbs, "logits_frac_of_peak": mgbs / HBM_PEAK_GBS,
            "algorithmic_bytes_per_launch": mbytes,
            "tau_mean_by_modes": {str(k): float(mtau[kn == k].mean()) for k in sorted(set(kn.tolist()))},
        }
        del mP, mlog
    if args.lmhead_workload != "none" and name == "batched":
        out["fused_lmhead"] = fused_lmhead(args.steps, stream)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)
    if args.copy_gib > 0:
        src = torch.ones(args.copy_gib << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
