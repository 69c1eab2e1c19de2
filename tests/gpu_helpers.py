"""Shared comparison helpers for the GPU parity tests (HIP path vs fp64 oracle)."""

from __future__ import annotations

import numpy as np
import torch

import oracle as O

SCORE_TOL = 1e-4      # log-prob scores: absolute tolerance
LSE_TOL = 1e-5        # row log-normalisers: absolute tolerance
BAND = 1e-4           # cut-off band inside which cross-mode order is not decided exactly


def oracle_rows(x64: np.ndarray, k: int):
    """Oracle lse [..] and ranked ids [.., k] for rows of x64 [..., V]."""
    lse = O.lse_rows(x64)
    flat = x64.reshape(-1, x64.shape[-1])
    ids = np.stack([O.rank_order(r, k) for r in flat]).reshape(x64.shape[:-1] + (k,))
    return lse, ids


def check_lsm(x_cpu: torch.Tensor, lse, topk_id, topk_raw, k, topk_logp=None):
    """Compare one [N, K, L, V] logits pass against the oracle."""
    x64 = x_cpu.double().numpy()
    o_lse, o_ids = oracle_rows(x64, k)
    g_lse = lse.cpu().numpy()
    g_ids = topk_id.cpu().numpy()
    g_raw = topk_raw.cpu().numpy()
    fin = np.isfinite(o_lse)
    assert np.array_equal(np.isneginf(o_lse), np.isneginf(g_lse))
    err = np.max(np.abs(g_lse[fin] - o_lse[fin])) if fin.any() else 0.0
    assert err < LSE_TOL, f"lse error {err}"
    assert np.array_equal(g_ids, o_ids), "top-k ids differ"
    want_raw = np.take_along_axis(x_cpu.float().numpy(), o_ids.astype(np.int64), axis=-1)
    assert np.array_equal(g_raw, want_raw), "top-k values differ"  # float equality: -0.0 == +0.0
    if topk_logp is not None:
        lp = topk_logp.cpu().numpy().astype(np.float64)
        with np.errstate(invalid="ignore"):
            want = want_raw.astype(np.float64) - o_lse[..., None]
        m = np.isfinite(want)
        if m.any():
            assert np.max(np.abs(lp[m] - want[m])) < LSE_TOL
    return err


def per_mode_band(x64: np.ndarray, cutoff: float, k: int):
    """Per-mode keep counts just above and just below the cut-off band."""
    lo, _ = O.union_at_cutoff(x64, cutoff + BAND, k)
    hi, _ = O.union_at_cutoff(x64, cutoff - BAND, k)
    return np.array([len(s) for s in lo]), np.array([len(s) for s in hi])


def compare_tree(x64: np.ndarray, B: int, anchor: int, g: dict, sel=None) -> dict:
    """Compare one GPU tree (dict of numpy rows) against the oracle.  Returns
    {'exact': bool, 'tree': oracle canonical tree, 'sel': selection}."""
    if sel is None:
        sel = O.mixture_select_heap(x64, B, band=BAND)
    tr = O.canonical_tree(sel, anchor, B)
    assert int(g["n_select"]) == sel.n_select, (int(g["n_select"]), sel.n_select)
    if sel.n_select > 0:
        assert abs(float(g["cutoff"]) - sel.cutoff) < SCORE_TOL
    else:
        assert float(g["cutoff"]) == np.inf
    exact = O.band_is_exact(x64, sel, BAND)
    if exact:
        assert int(g["n_nodes"]) == tr["n_nodes"]
        assert np.array_equal(g["node_token"], tr["node_token"]), "node tokens differ"
        assert np.array_equal(g["parent"], tr["parent"]), "parents differ"
        assert np.array_equal(g["depth"], tr["depth"]), "depths differ"
        n = tr["n_nodes"]
        assert np.max(np.abs(g["score"][:n] - tr["score"][:n])) < SCORE_TOL
        assert np.all(np.isneginf(g["score"][n:]))
        # best mode, where the runner-up mode is not within the tolerance
        k = min(B, x64.shape[2])
        for i in range(1, n):
            t = tr["prefixes"][i]
            sc = np.sort(O.mode_scores(x64, t, k=k, lse=sel.lse, norm=sel.norm))[::-1]
            if len(sc) == 1 or sc[0] - sc[1] >= SCORE_TOL:
                assert g["best_mode"][i] == tr["best_mode"][i], (i, t)
        if "per_mode_kept" in g and sel.n_select > 0:
            lo, hi = per_mode_band(x64, sel.cutoff, k)
            pk = np.asarray(g["per_mode_kept"])
            assert np.all(lo <= pk) and np.all(pk <= hi), (lo, pk, hi)
    return {"exact": exact, "tree": tr, "sel": sel}


def check_mask(parent, depth, n_nodes, pos_base, Bp1, words, pos_ids, dense=None):
    dm, pos = O.tree_mask(parent, depth, n_nodes, pos_base, Bp1)
    want = O.pack_mask_words(dm).view(np.int64)
    assert np.array_equal(words, want), "mask words differ"
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


def tree_rows(P, n: int) -> dict:
    b = P.buf
    return {
        "n_select": b.n_select[n].item(), "cutoff": b.cutoff[n].item(), "n_nodes": b.n_nodes[n].item(),
        "node_token": b.node_token[n].cpu().numpy().astype(np.int64),
        "parent": b.parent[n].cpu().numpy().astype(np.int64),
        "depth": b.depth[n].cpu().numpy().astype(np.int64),
        "score": b.score[n].cpu().numpy(),
        "best_mode": b.best_mode[n].cpu().numpy().astype(np.int64),
        "per_mode_kept": b.per_mode_kept[n].cpu().numpy(),
    }


def upload_tree(trees: list, Bp1: int, device="cuda"):
    """Stack oracle trees into device tensors (node_token, parent, depth, n_nodes)."""
    tok = torch.tensor(np.stack([t["node_token"] for t in trees]), dtype=torch.int32, device=device)
    par = torch.tensor(np.stack([t["parent"] for t in trees]), dtype=torch.int32, device=device)
    dep = torch.tensor(np.stack([t["depth"] for t in trees]), dtype=torch.int32, device=device)
    nn = torch.tensor([t["n_nodes"] for t in trees], dtype=torch.int32, device=device)
    return tok, par, dep, nn
