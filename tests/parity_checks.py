"""Comparisons of GPU outputs (as numpy arrays) against the fp64 oracle.

Numpy and the oracle only (no torch), so that worker processes of a pool can
import it cheaply; tests/gpu_helpers.py re-exports these for the GPU tests.

Bars: ids, node sets, parents, depths, masks, tau and tokens bit-exact; row
log-normalisers within LSE_TOL; prefix scores within SCORE_TOL.  A tree whose
cut-off band is not decided by exact comparisons (oracle.band_is_exact) is
not compared array for array; it must instead be a valid answer: the right
number of prefixes, prefix-closed, in canonical layout, every prefix scoring
clearly above the cut-off present, none clearly below it, and every node's
score equal to the oracle's score of that prefix.
"""

from __future__ import annotations

import os

import numpy as np

import oracle as O

SCORE_TOL = 1e-4      # log-prob scores: absolute tolerance
LSE_TOL = 1e-5        # row log-normalisers: absolute tolerance
BAND = 1e-4           # cut-off band inside which cross-mode order is not decided exactly


def peaked_logits(seed: int, K: int, L: int, V: int, gap: float) -> np.ndarray:
    """Logits [K, L, V] (fp32 values) in which token 5 leads every row by about
    `gap`: the chain of token 5 scores far above every other prefix, so with a
    small B the B best nodes lie many binades above the running threshold."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((K, L, V)).astype(np.float32)
    x[:, :, 5] += np.float32(gap)
    return x


# seed, K, L, V, B, gap: peaked trees whose threshold raise finds the B-th
# best node more than 255 16-bit score keys above the running threshold
PEAKED = [(31, 2, 10, 64, 3, 20.0), (32, 3, 8, 200, 4, 20.0), (33, 1, 12, 100, 5, 20.0),
          (35, 2, 10, 64, 3, 30.0)]


def oracle_rows(x64: np.ndarray, k: int):
    """Oracle lse [..] and ranked ids [.., k] for rows of x64 [..., V]."""
    lse = O.lse_rows(x64)
    flat = x64.reshape(-1, x64.shape[-1])
    ids = np.stack([O.rank_order(r, k) for r in flat]).reshape(x64.shape[:-1] + (k,))
    return lse, ids


def check_lsm_arrays(x32: np.ndarray, g_lse, g_ids, g_raw, k, g_logp=None, o_lse=None, o_ids=None):
    """Compare one logits pass ([..., V] fp32 values of the inputs) against the oracle.
    o_lse / o_ids may be passed when the oracle already ranked these rows."""
    x64 = x32.astype(np.float64)
    if o_lse is None or o_ids is None:
        o_lse, o_ids = oracle_rows(x64, k)
    fin = np.isfinite(o_lse)
    assert np.array_equal(np.isneginf(o_lse), np.isneginf(g_lse))
    err = float(np.max(np.abs(g_lse[fin] - o_lse[fin]))) if fin.any() else 0.0
    assert err < LSE_TOL, f"lse error {err}"
    assert np.array_equal(g_ids, o_ids), "top-k ids differ"
    want_raw = np.take_along_axis(x32, o_ids.astype(np.int64), axis=-1)
    assert np.array_equal(g_raw, want_raw), "top-k values differ"  # float equality: -0.0 == +0.0
    if g_logp is not None:
        lp = np.asarray(g_logp, dtype=np.float64)
        with np.errstate(invalid="ignore"):
            want = want_raw.astype(np.float64) - o_lse[..., None]
        m = np.isfinite(want)
        if m.any():
            assert np.max(np.abs(lp[m] - want[m])) < LSE_TOL
    return err


def per_mode_band(x64: np.ndarray, cutoff: float, k: int, sel=None):
    """Per-mode keep counts just above and just below the cut-off band."""
    lo, _ = O.union_at_cutoff(x64, cutoff + BAND, k, sel=sel)
    hi, _ = O.union_at_cutoff(x64, cutoff - BAND, k, sel=sel)
    return np.array([len(s) for s in lo]), np.array([len(s) for s in hi])


def _runner_up_clear(sc: np.ndarray) -> bool:
    sc = np.sort(sc)[::-1]
    return len(sc) == 1 or sc[0] - sc[1] >= SCORE_TOL


def check_valid_tree(x64: np.ndarray, B: int, anchor: int, g: dict, sel) -> list:
    """The GPU tree is a correct answer for the oracle's selection `sel`, whatever
    the order of prefixes inside the cut-off band.  Returns its prefixes (row order)."""
    K, L, V = x64.shape
    k = min(B, V)
    Bp1 = B + 1
    n = int(g["n_nodes"])
    tok, par, dep = g["node_token"], g["parent"], g["depth"]
    sco, mod = g["score"], g["best_mode"]
    assert n == sel.n_select + 1, (n, sel.n_select)
    assert tok[0] == anchor and par[0] == -1 and dep[0] == 0 and sco[0] == 0.0 and mod[0] == -1, "root row"
    prefixes = [()]
    for i in range(1, n):
        p = int(par[i])
        assert 0 <= p < i, f"row {i}: parent {p} does not precede it"
        assert dep[i] == dep[p] + 1, f"row {i}: depth {dep[i]} under a parent of depth {dep[p]}"
        prefixes.append(prefixes[p] + (int(tok[i]),))
    assert len(set(prefixes)) == n, "a prefix appears twice"
    order = [(len(t), t) for t in prefixes[1:]]
    assert all(a < b for a, b in zip(order, order[1:])), "rows are not in (depth, token sequence) order"
    assert np.all(tok[n:] == -1) and np.all(par[n:] == -1) and np.all(dep[n:] == -1), "tail rows"
    assert np.all(mod[n:] == -1) and np.all(np.isneginf(sco[n:])), "tail rows"
    for i in range(1, n):
        t = prefixes[i]
        sc = O.mode_scores(x64, t, k=k, lse=sel.lse, norm=sel.norm, ranked=sel.topk)
        S = float(sc.max())
        assert np.isfinite(S), f"row {i}: prefix {t} has no finite score among the first {k} ranks"
        assert abs(float(sco[i]) - S) < SCORE_TOL, (i, t, float(sco[i]), S)
        assert S >= sel.cutoff - BAND, f"row {i}: prefix {t} scores {S} below the cut-off {sel.cutoff}"
        if _runner_up_clear(sc):
            assert int(mod[i]) == int(np.argmax(sc)), (i, t, int(mod[i]), sc)
    if sel.n_select > 0:
        _, must = O.union_at_cutoff(x64, sel.cutoff + BAND, k, sel=sel)
        missing = must - set(prefixes[1:])
        assert not missing, f"{len(missing)} prefixes above the cut-off band are missing, e.g. {sorted(missing)[:3]}"
    return prefixes


def compare_tree(x64: np.ndarray, B: int, anchor: int, g: dict, sel=None) -> dict:
    """Compare one GPU tree (dict of numpy rows) against the oracle.  Every tree
    must be valid (check_valid_tree); a tree whose band is decided exactly must
    also equal the oracle's array for array.  Returns {'exact', 'tree', 'sel'}."""
    if sel is None:
        sel = O.mixture_select_heap(x64, B, band=BAND)
    tr = O.canonical_tree(sel, anchor, B)
    assert int(g["n_select"]) == sel.n_select, (int(g["n_select"]), sel.n_select)
    if sel.n_select > 0:
        assert abs(float(g["cutoff"]) - sel.cutoff) < SCORE_TOL
    else:
        assert float(g["cutoff"]) == np.inf
    check_valid_tree(x64, B, anchor, g, sel)
    exact = O.band_is_exact(x64, sel, BAND)
    if exact:
        assert int(g["n_nodes"]) == tr["n_nodes"]
        assert np.array_equal(g["node_token"], tr["node_token"]), "node tokens differ"
        assert np.array_equal(g["parent"], tr["parent"]), "parents differ"
        assert np.array_equal(g["depth"], tr["depth"]), "depths differ"
        n = tr["n_nodes"]
        assert np.max(np.abs(g["score"][:n] - tr["score"][:n])) < SCORE_TOL
        assert np.all(np.isneginf(g["score"][n:]))
        k = min(B, x64.shape[2])
        for i in range(1, n):
            sc = O.mode_scores(x64, tr["prefixes"][i], k=k, lse=sel.lse, norm=sel.norm, ranked=sel.topk)
            if _runner_up_clear(sc):
                assert g["best_mode"][i] == tr["best_mode"][i], (i, tr["prefixes"][i])
    if "per_mode_kept" in g and sel.n_select > 0:
        lo, hi = per_mode_band(x64, sel.cutoff, min(B, x64.shape[2]), sel=sel)
        pk = np.asarray(g["per_mode_kept"])
        assert np.all(lo <= pk) and np.all(pk <= hi), (lo, pk, hi)
    return {"exact": exact, "tree": tr, "sel": sel}


def check_mask(parent, depth, n_nodes, pos_base, Bp1, words, pos_ids, dense=None):
    dm, pos = O.tree_mask(parent, depth, n_nodes, pos_base, Bp1)
    want = O.pack_mask_words(dm).view(np.int64)
    assert np.array_equal(np.asarray(words).view(np.int64), want), "mask words differ"
    assert np.array_equal(pos_ids, pos), "position ids differ"
    if dense is not None:
        assert np.array_equal(dense.astype(bool), dm)


def check_walk(tree: dict, R64: np.ndarray, T: float, seed: int, L: int, tau, toks, path):
    """GPU walk outputs vs the oracle walk on the same tree and target rows.
    A step whose top-two perturbed values are within 1e-12 may legitimately
    differ (fp64 log implementations); such a tree is reported, not failed."""
    o_tau, o_toks, o_path, steps = O.verify_walk(tree["node_token"], tree["parent"], tree["depth"],
                                                 tree["n_nodes"], R64, T, seed, L)
    same = (int(tau) == o_tau and np.array_equal(np.asarray(toks), o_toks)
            and np.array_equal(np.asarray(path), o_path))
    if not same:
        close = T > 0 and any(gap < 1e-12 for (_, _, gap) in steps)
        assert close, f"walk differs: gpu tau={int(tau)} toks={list(toks)} oracle tau={o_tau} toks={list(o_toks)}"
        return False
    return True


# ---------------------------------------------------------------------------
# Pool workers: inputs come through read-only memory maps of the drafter and
# target logits (raw element bits), so only small arrays cross the pipes.

def _rows(path: str, dtype: str, shape: tuple, n: int) -> np.ndarray:
    """Tree n of a memory-mapped [N, ...] array as fp32 values."""
    mm = np.memmap(path, mode="r", dtype=np.uint16 if dtype == "bf16" else np.float32, shape=shape)
    a = np.array(mm[n])
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a


def tree_job(job: dict) -> dict:
    """Logits pass, tree, per-mode keeps and mask of one GPU tree against the oracle.
    Returns {'n', 'ok', 'error', 'exact', and the oracle tree's arrays}."""
    n = job["n"]
    try:
        x32 = _rows(job["path"], job["dtype"], tuple(job["shape"]), n)
        Kn = job.get("Kn", x32.shape[0])
        x32 = x32[:Kn]
        if job.get("vocab_map") is not None:
            vm = job["vocab_map"]
            full = np.full(x32.shape[:-1] + (job["V_full"],), -np.inf, dtype=np.float32)
            full[..., vm] = x32
            x32 = full
        x64 = x32.astype(np.float64)
        B = job["B"]
        sel = O.mixture_select_heap(x64, B, band=BAND)
        k = job["k"]
        assert k == min(B, x64.shape[2])
        o_ids = np.asarray(sel.topk)  # [K, L, k]: the heap ranks every row to k = min(B, V)
        check_lsm_arrays(x32, job["lse"], job["topk_id"], job["topk_raw"], k, job.get("topk_logp"),
                         o_lse=sel.lse, o_ids=o_ids)
        g = job["tree"]
        r = compare_tree(x64, B, job["anchor"], g, sel=sel)
        check_mask(g["parent"], g["depth"], g["n_nodes"], job["pos_base"], B + 1, job["mask_words"],
                   job["position_ids"])
        tr = r["tree"]
        return {"n": n, "ok": True, "error": "", "exact": bool(r["exact"]),
                "node_token": tr["node_token"], "parent": tr["parent"], "depth": tr["depth"],
                "n_nodes": tr["n_nodes"], "prefixes": tr["prefixes"]}
    except AssertionError as e:
        return {"n": n, "ok": False, "error": f"tree {n}: {e!r}", "exact": False}


def walk_job(job: dict) -> dict:
    """One GPU walk against the oracle walk on the same tree and target rows."""
    n = job["n"]
    try:
        R = _rows(job["path"], job["dtype"], tuple(job["shape"]), n).astype(np.float64)
        same = check_walk(job["tree"], R, job["T"], job["seed"], job["L"], job["tau"], job["toks"], job["path_nodes"])
        return {"n": n, "ok": True, "error": "", "same": same}
    except AssertionError as e:
        return {"n": n, "ok": False, "error": f"walk {n}: {e!r}", "same": False}


def run_pool(fn, jobs: list, workers: int | None = None) -> list:
    """Runs fn over jobs in a pool of fresh interpreters (spawned, never forked:
    the parent may hold a GPU context)."""
    import multiprocessing as mp
    if workers is None:
        try:
            avail = len(os.sched_getaffinity(0))
        except AttributeError:
            avail = os.cpu_count() or 1
        workers = max(1, min(16, avail, len(jobs)))
    if workers == 1 or len(jobs) <= 1:
        return [fn(j) for j in jobs]
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers) as pool:
        return pool.map(fn, jobs, chunksize=1)
