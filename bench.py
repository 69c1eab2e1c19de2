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
import json
import os
import statistics
import sys
import time

import torch

METRIC = "mixture trees built+verified/sec (K=8,L=15,B=256,V=152K); logits HBM GB/s"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="batched", choices=["batched", "single", "stress"])
    ap.add_argument("--cpu-baseline-trees", type=int, default=2,
                    help="trees of the workload the fp64 oracle is timed on (0 = skip)")
    ap.add_argument("--seed", type=int, default=0)
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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); trees are independent, "
              f"so N GPUs would each run this same per-GPU batch.", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from mixture_draft_tree_amd import synth
    from mixture_draft_tree_amd.pipeline import MixtureTreePath

    name = args.workload
    w = synth.WORKLOADS[name]
    dev = "cuda"
    b = synth.draft_batch(name, base_seed=args.seed, device=dev)
    N = b.logits.shape[0]
    P = MixtureTreePath(N, w.K, w.L, w.V, w.B)
    logits = b.logits.contiguous()
    anchor, pos = b.anchor.to(dev), b.pos_base.to(dev)
    temps, seeds = b.temperature.to(dev), b.seed.to(dev)
    # the target's per-node rows depend on the tree they verify: build once
    P.build(logits, anchor, pos)
    torch.cuda.synchronize()
    R = synth.target_logits(b, P.buf.depth, P.buf.n_nodes, device=dev, base_seed=args.seed).contiguous()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    names = ["logsoftmax_topk", "mixture_threshold", "tree_build", "tree_mask", "verify_walk"]
    for _ in range(args.warmup):
        P.step(logits, anchor, pos, R, temps, seeds)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
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
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    stage = {nm: [ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)] for i, nm in enumerate(names)}
    stage_ms = {nm: statistics.mean(v) for nm, v in stage.items()}
    status = P.buf.status.cpu()
    assert int(status.abs().sum()) == 0, f"per-tree status flags set: {status.tolist()}"

    logits_bytes = N * w.K * w.L * w.V * logits.element_size()
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
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": logits_bytes, "avg_launch_ms": lsm_ms},
        "stages_ms": stage_ms,
        "logits_GBps": achieved,
        "per_tree_latency_ms": ms_per_step if N == 1 else None,
        "tau_mean": float(tau.mean()),
    }
    if args.cpu_baseline_trees > 0:
        out["cpu_baseline"] = cpu_baseline(name, args.seed, args.cpu_baseline_trees)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
