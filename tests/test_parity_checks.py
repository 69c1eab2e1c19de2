"""The GPU parity checks themselves, on the CPU: an oracle tree passes them,
and trees with planted mistakes (a node swapped for one below the cut-off, a
dropped node, a wrong score, a row out of canonical order, a broken parent
link) fail them.  Also the pool runner."""

import copy

import numpy as np
import pytest

import oracle as O
from parity_checks import BAND, check_valid_tree, compare_tree, run_pool, tree_job  # noqa: F401


def _tree_case(seed, K=3, L=4, V=12, B=30):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 2, size=(K, L, V))
    sel = O.mixture_select_heap(x, B, band=BAND)
    tr = O.canonical_tree(sel, 5, B)
    g = {k: np.array(tr[k]) for k in ("node_token", "parent", "depth", "score", "best_mode")}
    g["n_nodes"] = tr["n_nodes"]
    g["n_select"] = sel.n_select
    g["cutoff"] = sel.cutoff
    g["per_mode_kept"] = sel.per_mode_kept.copy()
    return x, sel, tr, g


@pytest.mark.parametrize("seed", range(3))
def test_oracle_tree_is_valid(seed):
    x, sel, tr, g = _tree_case(seed)
    prefixes = check_valid_tree(x, 30, 5, g, sel)
    assert prefixes == tr["prefixes"]
    assert compare_tree(x, 30, 5, g, sel=sel)["exact"] in (True, False)


def _expect_fail(x, sel, g):
    with pytest.raises(AssertionError):
        check_valid_tree(x, 30, 5, g, sel)


def test_planted_mistakes_fail():
    x, sel, tr, g = _tree_case(7)
    n = tr["n_nodes"]
    # a score off by twice the tolerance
    bad = copy.deepcopy(g)
    bad["score"][n - 1] += 2 * 1e-4
    _expect_fail(x, sel, bad)
    # a node dropped (the tree one short)
    bad = copy.deepcopy(g)
    bad["n_nodes"] = n - 1
    for f in ("node_token", "parent", "depth", "best_mode"):
        bad[f][n - 1] = -1
    bad["score"][n - 1] = -np.inf
    _expect_fail(x, sel, bad)
    # two depth-1 siblings swapped (layout out of token order)
    d1 = [i for i in range(1, n) if g["depth"][i] == 1]
    assert len(d1) >= 2
    bad = copy.deepcopy(g)
    i, j = d1[0], d1[1]
    for f in ("node_token", "score", "best_mode"):
        bad[f][i], bad[f][j] = bad[f][j], bad[f][i]
    _expect_fail(x, sel, bad)
    # a parent link pointing at a later row
    bad = copy.deepcopy(g)
    bad["parent"][1] = n - 1
    _expect_fail(x, sel, bad)
    # a wrong best mode where the runner-up is far
    for i in range(1, n):
        sc = O.mode_scores(x, tr["prefixes"][i], k=30, lse=sel.lse, norm=sel.norm, ranked=sel.topk)
        s = np.sort(sc)[::-1]
        if s[0] - s[1] > 1e-3:
            bad = copy.deepcopy(g)
            bad["best_mode"][i] = (bad["best_mode"][i] + 1) % 3
            _expect_fail(x, sel, bad)
            break
    # a selected prefix replaced by an unselected one that scores below the band
    leaf = max(range(1, n), key=lambda r: (tr["depth"][r], r))
    t = tr["prefixes"][leaf]
    V = x.shape[2]
    for tok in range(V):
        cand = t[:-1] + (tok,)
        if cand in sel.S or cand in tr["prefixes"]:
            continue
        sc = O.mode_scores(x, cand, k=30, lse=sel.lse, norm=sel.norm, ranked=sel.topk)
        if np.isfinite(sc.max()) and sc.max() < sel.cutoff - 1e-3:
            bad = copy.deepcopy(g)
            bad["node_token"][leaf] = tok
            bad["score"][leaf] = sc.max()
            _expect_fail(x, sel, bad)
            break
    else:
        pytest.fail("no replacement prefix found")


def _square(v):
    return v * v


def test_run_pool_spawns_workers():
    assert run_pool(_square, list(range(6)), workers=2) == [0, 1, 4, 9, 16, 25]
