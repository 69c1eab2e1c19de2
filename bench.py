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


def lsm_source_sha() -> str:
    h = hashlib.sha256()
    for rel in LSM_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch of the logits kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None if there is
    none for this workload or the kernel sources changed since it was taken."""
    path = os.path.join(HERE, TRAFFIC_FILE)
    if workload != "batched" or not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith((" ", "#", "$")):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256") != lsm_source_sha():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="batched",
                    choices=["batched", "single", "stress", "deep", "batched_deep", "subset", "batched_subset",
                             "batched_modes"])
    ap.add_argument("--cpu-baseline-trees", type=int, default=2,
                    help="trees of the workload the fp64 oracle is timed on (0 = skip)")
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
    return ap.parse_args()


def cpu_baseline(name: str, base_seed: int, n_trees: int):
    """Time the fp64 oracle end to end (log-softmax, ranks, heap, layout, mask,
    walk) on the first `n_trees` trees of the workload, on this host's cores."""
    import numpy as np
    import oracle as O
    from mixture_draft_tree_amd import synth

    w = synth.WORKLOADS[name]
    b = synth.draft_batch(name, base_seed=base_seed, device="cpu", N=n_trees)
    xs = [b.logits[n].double().numpy() for n in range(n_trees)]
    # target rows come from the oracle's own trees (generated outside the timed part)
    trees = []
    for n in range(n_trees):
        sel = O.mixture_select_heap(xs[n], w.B)
        trees.append(O.canonical_tree(sel, int(b.anchor[n]), w.B))
    dep = torch.stack([torch.from_numpy(t["depth"]).to(torch.int32) for t in trees])
    nn = torch.tensor([t["n_nodes"] for t in trees], dtype=torch.int32)
    R = synth.target_logits(b, dep, nn, device="cpu", base_seed=base_seed)
    Rs = [R[n].double().numpy() for n in range(n_trees)]
    t0 = time.perf_counter()
    for n in range(n_trees):
        sel = O.mixture_select_heap(xs[n], w.B)
        tr = O.canonical_tree(sel, int(b.anchor[n]), w.B)
        O.tree_mask(tr["parent"], tr["depth"], tr["n_nodes"], int(b.pos_base[n]), w.B + 1)
        O.verify_walk(tr["node_token"], tr["parent"], tr["depth"], tr["n_nodes"], Rs[n],
                      float(b.temperature[n]), int(b.seed[n]) & ((1 << 64) - 1), w.L)
    dt = time.perf_counter() - t0
    temps = sorted({float(b.temperature[n]) for n in range(n_trees)})
    return {"value": n_trees / dt, "unit": "trees/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_trees} tree(s) of the {name} workload (T in {temps}), full oracle path, "
                      f"{dt:.1f} s on one host core"}


def run_steps(P, logits, anchor, pos, R, temps, seeds, steps, warmup, stream):
    """Times `steps` whole steps; returns (total ms, per-stage ms lists)."""
    for _ in range(warmup):
        P.step(logits, anchor, pos, R, temps, seeds)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(steps):
        e = ev[s]
        e[0].record(stream)
        P.logsoftmax_topk(logits)
        e[1].record(stream)
        P.mixture_threshold()
        e[2].record(stream)
        P.tree_build(anchor)
        e[3].record(stream)
        P.tree_mask(pos)
        e[4].record(stream)
        P.verify_walk(R, temps, seeds)
        e[5].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    return t_start.elapsed_time(t_end), ev


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
    """Mean time of one whole step on a one-tree workload (N=1), ms."""
    w, N, P, logits, anchor, pos, temps, seeds, R = setup(name, seed, "cuda")
    total, _ = run_steps(P, logits, anchor, pos, R, temps, seeds, steps, 3, stream)
    return total / steps


STAGES = ["logsoftmax_topk", "mixture_threshold", "tree_build", "tree_mask", "verify_walk"]


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


def timed_workload(name, seed, steps, warmup, stream, diagnostics=False):
    """Whole steps on workload `name`: (ms per step, per-stage ms, N, buffers)."""
    w, N, P, logits, anchor, pos, temps, seeds, R = setup(name, seed, "cuda")
    total_ms, ev = run_steps(P, logits, anchor, pos, R, temps, seeds, steps, warmup, stream)
    stage = {nm: statistics.mean(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps))
             for i, nm in enumerate(STAGES)}
    status = P.buf.status.cpu()
    assert int(status.abs().sum()) == 0, f"per-tree status flags set ({name}): {status.tolist()}"
    if diagnostics:
        stage["diagnostics"] = covered_mass_stats(P, R, temps, stream)
    return total_ms / steps, stage, N, w, P, logits


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); trees are independent, "
              f"so N GPUs would each run this same per-GPU batch.", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    name = args.workload
    stream = torch.cuda.current_stream()
    ms_per_step, stage_ms, N, w, P, logits = timed_workload(name, args.seed, args.steps, args.warmup, stream,
                                                            diagnostics=True)
    diag = stage_ms.pop("diagnostics")

    rows = N * w.K * w.L if P.modes is None else int(P.modes.sum()) * w.L   # rows the logits pass reads
    logits_bytes = rows * logits.shape[-1] * logits.element_size()
    lsm_ms = stage_ms["logsoftmax_topk"]
    achieved = logits_bytes / (lsm_ms * 1e-3) / 1e9
    tau = P.buf.tau.cpu().float()
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
                     "algorithmic_bytes_per_launch": logits_bytes, "avg_launch_ms": lsm_ms},
        "stages_ms": stage_ms,
        "logits_GBps": achieved,
        "per_tree_latency_ms": ms_per_step if N == 1 else None,
        "single_tree_latency_ms": None,
        "tau_mean": float(tau.mean()),
        "diagnostics": diag,
    }
    if args.latency_steps > 0 and name != "single":
        out["single_tree_latency_ms"] = single_tree_latency(args.seed, args.latency_steps, stream)
    if args.deep_workload != "none" and name == "batched":
        del P, logits
        dms, dstage, dN, dw, dP, _ = timed_workload(args.deep_workload, args.seed, args.steps, args.warmup, stream,
                                                    diagnostics=True)
        ddiag = dstage.pop("diagnostics")
        out["deep"] = {
            "workload": f"{args.deep_workload}: {dN} trees, K={dw.K}, L={dw.L}, V={dw.V}, B={dw.B}, "
                        f"T pattern {list(dw.temperatures)}",
            "data": "synthetic (seeded; confident drafter: N(0,4) noise, 16 Zipf alternatives, each mode's future "
                    "at 16+N(0,2.25); target rows N(0,1) + 16 on one future up to a random deviation depth)",
            "value": dN / (dms * 1e-3), "unit": "trees/s", "ms_per_step": dms, "stages_ms": dstage,
            "tau_mean": float(dP.buf.tau.cpu().float().mean()),
            "single_tree_latency_ms": (single_tree_latency(args.seed, args.latency_steps, stream, "deep")
                                       if args.latency_steps > 0 else None),
            "diagnostics": ddiag,
        }
    if args.subset_workload != "none" and name == "batched":
        sms, sstage, sN, sw, sP, slog = timed_workload(args.subset_workload, args.seed, args.steps, args.warmup,
                                                       stream)
        sbytes = sN * sw.K * sw.L * slog.shape[-1] * slog.element_size()
        sgbs = sbytes / (sstage["logsoftmax_topk"] * 1e-3) / 1e9
        out["reduced_vocab"] = {
            "workload": f"{args.subset_workload}: {sN} trees, K={sw.K}, L={sw.L}, drafting over {slog.shape[-1]} of "
                        f"V={sw.V} tokens, B={sw.B}, T pattern {list(sw.temperatures)}",
            "value": sN / (sms * 1e-3), "unit": "trees/s", "ms_per_step": sms, "stages_ms": sstage,
            "logits_GBps": sgbs, "logits_frac_of_peak": sgbs / HBM_PEAK_GBS,
            "algorithmic_bytes_per_launch": sbytes, "tau_mean": float(sP.buf.tau.cpu().float().mean()),
        }
        del sP, slog
    if args.modes_workload != "none" and name == "batched":
        mms, mstage, mN, mw, mP, mlog = timed_workload(args.modes_workload, args.seed, args.steps, args.warmup,
                                                       stream)
        kn = mP.modes.cpu()
        mbytes = int(kn.sum()) * mw.L * mw.V * mlog.element_size()
        mgbs = mbytes / (mstage["logsoftmax_topk"] * 1e-3) / 1e9
        mtau = mP.buf.tau.cpu().float()
        out["per_request_modes"] = {
            "workload": f"{args.modes_workload}: {mN} trees of the confident-drafter shape, K={mw.K}, L={mw.L}, "
                        f"V={mw.V}, B={mw.B}, K_n cycling {list(mw.modes)}, T pattern {list(mw.temperatures)}",
            "value": mN / (mms * 1e-3), "unit": "trees/s", "ms_per_step": mms, "stages_ms": mstage,
            "active_rows": int(kn.sum()) * mw.L, "logits_GBps": mgbs, "logits_frac_of_peak": mgbs / HBM_PEAK_GBS,
            "algorithmic_bytes_per_launch": mbytes,
            "tau_mean_by_modes": {str(k): float(mtau[kn == k].mean()) for k in sorted(set(kn.tolist()))},
        }
        del mP, mlog
    if args.cpu_baseline_trees > 0:
        out["cpu_baseline"] = cpu_baseline(name, args.seed, args.cpu_baseline_trees)
    print(json.dumps(out), flush=True)
    if args.copy_gib > 0:
        src = torch.ones(args.copy_gib << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
