"""The tree kernel's index arithmetic and capacities, checked on the host.

kernel_model.py replays the kernel's search with bounds-checked arrays of the
kernel's capacities and replays the sorting networks' and the one-wave
level's index arithmetic lane by lane.  These tests drive it with every sort
size and with the level sizes that the 64-tree `batched` and `batched_deep`
inputs and the flat-logit sweep cases produce; any index the kernel would
form outside its arrays fails them.  The model's cut-off is checked against
the oracle, so the sizes it replays are the ones the method produces."""

import numpy as np
import pytest

import oracle as O
from mixture_draft_tree_amd import synth

import kernel_model as KM
from parity_checks import PEAKED, peaked_logits, run_pool


@pytest.mark.parametrize("nt", [1024, 256])
def test_sort_networks_stay_in_bounds(nt):
    """Every LDS index of block_sort_keys<nt> lies in [0, P) for every size it
    serves, and every thread reaches the same number of barriers."""
    kinds = {}
    for lp in range(0, 15):
        P = 1 << lp
        kinds[P] = KM.check_block_sort_keys(P, P, nt)
    assert kinds[64].startswith("static") and kinds[nt].startswith("static")
    assert kinds[2 * nt].startswith("regs") and kinds[4 * nt].startswith("regs")
    assert kinds[8 * nt] == "bitonic" and kinds[32] == "bitonic"


def test_sort_check_catches_a_short_buffer():
    """The replay fails when the buffer is shorter than the keys it sorts."""
    with pytest.raises(IndexError):
        KM.check_block_sort_keys(512, 256)


def test_checked_array_catches_overflow():
    a = KM.CheckedArray("a", 4)
    a[3] = 1
    with pytest.raises(IndexError):
        a[4] = 1
    with pytest.raises(IndexError):
        a[-1]


def _model_vs_oracle(x: np.ndarray, B: int):
    K, L, V = x.shape
    k = min(B, V)
    ids, raw, lse = KM.row_lists(x, k)
    res = KM.TreeModel(ids, raw, lse, B).run()
    sel = O.mixture_select_heap(x, B)
    return res, sel


@pytest.mark.parametrize("seed,K,L,V,B", [
    (1, 2, 4, 16, 8), (2, 3, 5, 40, 30), (3, 1, 6, 20, 50), (4, 4, 3, 30, 60),
    (5, 8, 6, 64, 200), (6, 3, 8, 12, 300), (7, 2, 1, 50, 10), (8, 5, 4, 30, 1),
])
def test_model_cutoff_matches_oracle(seed, K, L, V, B):
    """The model's search finds the oracle's n_select and cut-off, so the level
    sizes it replays are the method's."""
    rng = np.random.default_rng(seed)
    # logits representable in fp32, as the kernel's candidate lists hold them
    x = (rng.normal(size=(K, L, V)) * 2).astype(np.float32).astype(np.float64)
    res, sel = _model_vs_oracle(x, B)
    assert not res.fail
    assert res.n_select == sel.n_select
    if sel.n_select:
        assert abs(res.cutoff - sel.cutoff) <= 1e-9


def test_model_counts_match_a_hand_case():
    """K=1, L=2, V=3, B=3: the search keeps the three best prefixes; worked by
    hand from the log-probabilities."""
    x = np.log(np.array([[[0.5, 0.3, 0.2], [0.6, 0.3, 0.1]]]))
    res, sel = _model_vs_oracle(x, 3)
    # prefixes: (0) .5, (1) .3, (0,0) .3, (1,0) .18, (0,1) .15 ...: the third
    # best is .3 (the model holds the logits in fp32, hence the tolerance)
    assert res.n_select == 3 and sel.n_select == 3
    assert abs(res.cutoff - np.log(0.3)) < 1e-6
    assert abs(sel.cutoff - np.log(0.3)) < 1e-12
    assert res.node_count >= 4  # root plus at least the three selected


def _tree_job(job):
    name, n = job
    w = synth.WORKLOADS[name]
    b = synth.draft_batch(name, start=n, N=1)
    x = b.logits[0].double().numpy()
    ids, raw, lse = KM.row_lists(x, min(w.B, x.shape[-1]))
    res = KM.TreeModel(ids, raw, lse, w.B).run()
    return {
        "fail": res.fail, "n_select": res.n_select, "nodes": res.node_count, "entries": res.ent_count,
        "pooled_P": res.pooled_P, "window": (res.window_hits, res.window_misses),
        "levels": [(r.d, r.path, r.fsize, r.C, r.P, r.sort, r.bisected, r.raised) for r in res.levels],
    }


def _summary(results):
    Ps, small, block, bis, raised = {}, 0, 0, 0, 0
    for r in results:
        for d, path, fsize, C, P, sort, bisected, was_raised in r["levels"]:
            if path == "small":
                small += 1
            elif path == "block":
                block += 1
                Ps[sort] = Ps.get(sort, 0) + 1
            bis += int(bisected)
            raised += int(was_raised)
    return {"trees": len(results), "block_levels": block, "small_levels": small, "bisections": bis,
            "raises": raised, "sorts": dict(sorted(Ps.items())),
            "max_nodes": int(max(r["nodes"] for r in results)),
            "max_entries": int(max(r["entries"] for r in results)),
            "max_C": int(max((lv[3] for r in results for lv in r["levels"]), default=0)),
            "window_hits": sum(r["window"][0] for r in results),
            "window_misses": sum(r["window"][1] for r in results)}


def _oracle_job(job):
    name, n = job
    w = synth.WORKLOADS[name]
    x = synth.draft_batch(name, start=n, N=1).logits[0].double().numpy()
    ids, raw, lse = KM.row_lists(x, min(w.B, x.shape[-1]))
    res = KM.TreeModel(ids, raw, lse, w.B).run()
    sel = O.mixture_select_heap(x, w.B)
    return res.n_select, res.cutoff, sel.n_select, sel.cutoff


@pytest.mark.parametrize("name", ["batched", "batched_deep"])
def test_workload_model_cutoff_matches_oracle(name):
    """On full-size trees (bf16 logits, exact in fp32) the model finds the
    oracle's cut-off (within the fp64 rounding of the two sums)."""
    for ns, cut, ons, ocut in run_pool(_oracle_job, [(name, 0), (name, 1)]):
        assert ns == ons
        assert abs(cut - ocut) <= 1e-9


@pytest.mark.parametrize("name", ["batched", "batched_deep"])
def test_workload_level_sizes_stay_in_bounds(name):
    """All 64 trees of the workload through the model: no index outside the
    kernel's arrays, no capacity failure, B nodes selected."""
    w = synth.WORKLOADS[name]
    results = run_pool(_tree_job, [(name, n) for n in range(w.N)])
    s = _summary(results)
    print(f"[kernel model] {name}: {s}")
    assert not any(r["fail"] for r in results)
    assert all(r["n_select"] == w.B for r in results)
    assert s["block_levels"] > 0 and s["small_levels"] > 0


SWEEP = [
    # K, L, V, B, sigma (0: small integers, many ties): the GPU sweep's cases,
    # whose first levels span the one-key, two-key, four-key and LDS sorts
    (8, 3, 600, 1200, 0.5), (3, 5, 1000, 1000, 0.3), (2, 4, 1000, 1000, 0.3), (6, 4, 300, 700, 1.0),
    (4, 6, 100, 400, 0.0), (2, 10, 64, 150, 2.0), (8, 15, 2000, 256, 3.0),
]


def _sweep_job(job):
    K, L, V, B, sigma, n = job
    import torch
    g = torch.Generator().manual_seed(1000 * K + 10 * L + n)
    if sigma == 0.0:
        x = torch.randint(-2, 3, (1, K, L, V), generator=g).float()
    else:
        x = torch.randn((1, K, L, V), generator=g) * sigma
    x = x[0].double().numpy()
    ids, raw, lse = KM.row_lists(x, min(B, V))
    res = KM.TreeModel(ids, raw, lse, B).run()
    return {"fail": res.fail, "n_select": res.n_select, "nodes": res.node_count, "entries": res.ent_count,
            "pooled_P": res.pooled_P, "window": (res.window_hits, res.window_misses),
            "levels": [(r.d, r.path, r.fsize, r.C, r.P, r.sort, r.bisected, r.raised) for r in res.levels]}


def test_sweep_level_sizes_stay_in_bounds():
    """The flat-logit sweep cases, whose levels span every sort size."""
    jobs = [(*c, n) for c in SWEEP for n in range(4)]
    results = run_pool(_sweep_job, jobs)
    s = _summary(results)
    print(f"[kernel model] sweep: {s}")
    assert not any(r["fail"] for r in results)
    assert any(k.startswith("regs") for k in s["sorts"])


@pytest.mark.parametrize("case", PEAKED, ids=[f"p{c[0]}" for c in PEAKED])
def test_peaked_trees_reach_the_wide_raise(case):
    """On the peaked cases some raise finds its B-th best key beyond the
    one-pass window (key - tau's key >= 255) and takes the radix passes; the
    model's cut-off is still the oracle's."""
    seed, K, L, V, B, gap = case
    x = peaked_logits(seed, K, L, V, gap).astype(np.float64)
    res, sel = _model_vs_oracle(x, B)
    assert not res.fail and res.window_misses > 0
    assert res.n_select == sel.n_select and abs(res.cutoff - sel.cutoff) <= 1e-12
