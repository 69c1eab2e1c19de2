"""fp64 oracle: what the mixture draft tree path computes, written out plainly.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (the Multi-Future Drafting pages):
  [MC]  model card "MFD drafter for Qwen3.5-4B (1.42M prompts)": summary paragraph
        (B best prefixes by best-mode log-probability; one verification pass;
        lossless standard tree verification), "Model" (block of 16, 15 drafted).
  [PP]  project page "Multi-Future Drafting: Mixture Block Drafters for
        Tree-Verified Speculative Decoding": "In one minute" (common cut-off at
        the B-th best score, per-mode keeps, one deduplicated tree), "Abstract"
        (accepted tokens = covered mass; chimera count for product trees),
        "How it works" step 1 (product of per-position distributions), step 3
        (best-mode scoring, union of per-mode trees, merged best-first heap),
        Figure 2 (one distribution per position per mode; tau counts the bonus).
  [PT]  paper-tracker abstract of arXiv:2611.13017 (chimera count 2^(m-1) - 1).
  [MD]  model card "Qwen3-4B-MDraft-b16", "Evaluation" (acceptance length
        includes the bonus token) and "Model details" (anchor + 15 drafted slots).

Readings where the pages are silent (each listed in the design notes):
  * B counts drafted nodes; the root (anchor) is extra, so a tree has B+1 rows.
  * Scores use natural logs; a prefix's best-mode score is the max over modes,
    unweighted (the gate is unused at inference, [MC] "Model").
  * Total order on prefixes: higher score first, then lower best mode, then
    token ids lexicographically with a proper prefix before its extensions.
    Rank order within a row: higher logit first, then lower token id.
  * Node layout: root first, then nodes by (depth, token sequence).
  * Sampling at T > 0 is Gumbel-max with Philox4x32-10 noise keyed by the
    seed's two 32-bit halves, counter (v div 4, depth, 0, 0), word v mod 4.
  * -inf logits are allowed and never selected.
"""

from __future__ import annotations

import heapq
import itertools
import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "lse_rows", "rank_order", "prefix_norms", "lmhead_logits", "lmhead_abs_bound", "MixtureSelection",
    "mixture_select_heap", "mixture_select_bruteforce", "ddtree_product_select",
    "mode_scores", "union_at_cutoff", "canonical_tree", "tree_mask",
    "pack_mask_words", "philox4x32_10", "gumbel_noise", "verify_walk",
    "covered_mass", "chimera_nodes", "band_is_exact", "build_tree",
    "PHILOX_M0", "PHILOX_M1", "PHILOX_W0", "PHILOX_W1",
]


# ---------------------------------------------------------------------------
# Per-(mode, position) log-softmax and rank order
# ---------------------------------------------------------------------------

def lse_rows(x: np.ndarray) -> np.ndarray:
    """log of the sum of exp over the last axis, in fp64.

    Each of the K block copies gives one distribution per position ([PP]
    Figure 2); a position's log-probabilities are logits minus this value.
    Written as m + log(sum exp(x - m)) with m the row max; a row of only -inf
    gives -inf.
    """
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=-1)
    safe = np.where(np.isfinite(m), m, 0.0)
    s = np.exp(x - safe[..., None]).sum(axis=-1)
    with np.errstate(divide="ignore"):
        out = safe + np.log(s)
    return np.where(np.isneginf(m), -np.inf, out)


def rank_order(row: np.ndarray, k: int) -> np.ndarray:
    """Token ids of one row by logit descending, ties by token id ascending; first k.

    The best-first searches of [PP] step 3 expand each position's candidates
    from most to least probable; ties are broken by the lower id.
    """
    row = np.asarray(row, dtype=np.float64)
    order = np.argsort(-row, kind="stable")  # a stable sort keeps equal logits in id order
    return order[:k]


def prefix_norms(lse: np.ndarray) -> np.ndarray:
    """norm[k, d] = sum_{i<d} lse[k, i], fp64, accumulated from i = 0 upward."""
    K, L = lse.shape
    norm = np.zeros((K, L + 1), dtype=np.float64)
    for k in range(K):
        acc = 0.0
        for i in range(L):
            acc = acc + float(lse[k, i])
            norm[k, i + 1] = acc
    return norm


def lmhead_logits(hidden: np.ndarray, weight: np.ndarray) -> np.ndarray:
    """Drafter logits from final hidden states and the LM head, fp64.

    The drafter has no LM head of its own: it uses its target's at run time
    ([MC] "Model", "Parameters"), and the pages' tree step can take the logits
    fused with that head ([MC] "Usage", fused_logits=True).  A language model's
    logit for token v is the inner product of the hidden state with row v of
    the head:  x[..., v] = sum_d hidden[..., d] * weight[v, d].  hidden has
    shape [..., D], weight [V, D]; the result has shape [..., V].  Its rows then
    go through lse_rows and rank_order like any other logits.
    """
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    if h.shape[-1] != w.shape[1]:
        raise ValueError(f"hidden width {h.shape[-1]} != head width {w.shape[1]}")
    return h @ w.T


def lmhead_abs_bound(hidden: np.ndarray, weight: np.ndarray, unit: float = 2.0 ** -23) -> np.ndarray:
    """Bound on |computed - exact| for the logits of lmhead_logits when the D
    products (exact: bf16 times bf16 fits an fp32 significand) are added in
    binary32 in any order:  gamma_D * sum_d |h_d w_vd|, gamma_n = n u / (1 - n u)
    (Higham, Accuracy and Stability of Numerical Algorithms, 2nd ed., sec. 4.2).
    unit = 2^-23 covers rounding toward zero as well as to nearest.
    """
    h = np.abs(np.asarray(hidden, dtype=np.float64))
    w = np.abs(np.asarray(weight, dtype=np.float64))
    n = h.shape[-1]
    gamma = n * unit / (1.0 - n * unit)
    return gamma * (h @ w.T)


# ---------------------------------------------------------------------------
# Selection of the B best prefixes by best-mode score
# ---------------------------------------------------------------------------

@dataclass
class MixtureSelection:
    """The B best prefixes (in total order) plus what the cut-off implies."""
    order: list                 # unique prefixes (tuples) in total order, at least the first n_select
    S: dict                     # prefix -> best-mode score
    mu: dict                    # prefix -> best mode (lowest index attaining S)
    n_select: int               # min(B, number of prefixes with finite score)
    cutoff: float               # S of the n_select-th prefix (+inf when n_select == 0)
    per_mode_kept: np.ndarray   # [K] number of prefixes with s_k >= cutoff
    pops: int = 0               # heap pops performed (diagnostic)
    lse: np.ndarray = None
    norm: np.ndarray = None
    topk: list = field(default_factory=list)   # [K][L] ranked token ids (first k)

    @property
    def selected(self):
        return self.order[: self.n_select]


def _row_tables(x, k):
    K, L, V = x.shape
    lse = lse_rows(x)
    norm = prefix_norms(lse)
    ids = [[rank_order(x[m, i], k) for i in range(L)] for m in range(K)]
    vals = [[x[m, i][ids[m][i]] for i in range(L)] for m in range(K)]
    return lse, norm, ids, vals


def mixture_select_heap(x: np.ndarray, B: int, band: float = 0.0, k: int | None = None) -> MixtureSelection:
    """Merged K-way best-first search over prefixes, one heap ([PP] step 3).

    x: [K, L, V] fp64 drafter logits of one tree.  A prefix t = (t_1..t_d)
    scores s_k(t) = raw_k(t) - norm_k(d) under mode k, where raw_k sums the
    logits x[k, i, t_i] left to right and norm_k sums the row log-normalisers;
    this is the log of the product of mode k's per-position probabilities
    ([PP] step 1).  Its best-mode score is S(t) = max_k s_k(t) ([PP] "In one
    minute", step 3).

    Each mode runs a best-first search over its own prefixes: the successors of
    a popped prefix are "append the best token of the next position" and
    "replace the last token by the next one in that position's rank order".
    Each mode's pops come out in decreasing s_k; merging the K searches in one
    heap keyed by (-s_k, k, tokens) pops every prefix first under its best
    mode, and unique first pops come out in the total order.  A prefix already
    emitted is skipped but its successors are still pushed.  Only the first
    k = min(B, V) ranks of each row are used: a prefix needs the earlier-ranked
    siblings under its best mode ahead of it, so a token ranked B or worse
    there can never be among the first B.

    The search stops after B unique pops, then keeps popping while the heap
    top scores at least cutoff - band, so that per-mode keep counts (prefixes
    with s_k >= cutoff, the per-mode keeps of "In one minute") and the
    prefixes just below the cut-off are known.
    """
    x = np.asarray(x, dtype=np.float64)
    K, L, V = x.shape
    k = min(B, V) if k is None else k
    lse, norm, ids, vals = _row_tables(x, k)

    heap = []

    def push(m, ranks, raw_parent):
        d = len(ranks)
        r = ranks[-1]
        if r >= k:
            return
        v = vals[m][d - 1][r]
        if v == -np.inf:
            return
        raw = raw_parent + float(v)
        s = raw - norm[m, d]
        toks = tuple(int(ids[m][i][ranks[i]]) for i in range(d))
        heapq.heappush(heap, (-s, m, toks, ranks, raw_parent, raw))

    if k > 0 and L > 0:
        for m in range(K):
            push(m, (0,), 0.0)

    order, S, mu = [], {}, {}
    cutoff = math.inf
    pops = 0
    while heap and B > 0:
        negs, m, toks, ranks, raw_parent, raw = heap[0]
        s = -negs
        if len(order) >= B and s < cutoff - band:
            break
        heapq.heappop(heap)
        pops += 1
        if toks not in S:
            S[toks] = s
            mu[toks] = m
            order.append(toks)
            if len(order) == B:
                cutoff = s
        d = len(ranks)
        if d < L:
            push(m, ranks + (0,), raw)
        push(m, ranks[:-1] + (ranks[-1] + 1,), raw_parent)

    n_select = min(B, len(order))
    cutoff = S[order[n_select - 1]] if n_select > 0 else math.inf
    if n_select > 0:
        kept = _count_kept(ids, vals, norm, K, L, k, cutoff)
    else:
        kept = np.zeros(K, dtype=np.int64)
    return MixtureSelection(order=order, S=S, mu=mu, n_select=n_select, cutoff=cutoff,
                            per_mode_kept=kept, pops=pops, lse=lse, norm=norm, topk=ids)


def _count_kept(ids, vals, norm, K, L, k, cutoff):
    """Per mode, the number of prefixes (within the first k ranks per row) with s_k >= cutoff."""
    kept = np.zeros(K, dtype=np.int64)
    for m in range(K):
        stack = [(0, 0.0)]  # (depth, raw)
        while stack:
            d, raw = stack.pop()
            if d == L:
                continue
            for r in range(k):
                v = vals[m][d][r]
                if v == -np.inf:
                    break
                raw2 = raw + float(v)
                if raw2 - norm[m, d + 1] < cutoff:
                    break  # ranks are in decreasing logit order
                kept[m] += 1
                stack.append((d + 1, raw2))
    return kept


def mixture_select_bruteforce(x: np.ndarray, B: int) -> MixtureSelection:
    """The definition, by enumeration: score every prefix of every length under
    every mode, take the best-mode score, sort by the total order and keep the
    first B ([MC] summary; [PP] "In one minute").  Uses full rows (no top-k
    truncation).  Feasible only for tiny V and L."""
    x = np.asarray(x, dtype=np.float64)
    K, L, V = x.shape
    lse = lse_rows(x)
    norm = prefix_norms(lse)
    keys = []
    allS = {}
    allmu = {}
    per_mode_scores = {}
    for d in range(1, L + 1):
        toks = np.array(list(itertools.product(range(V), repeat=d)), dtype=np.int64)
        sc = np.empty((K, toks.shape[0]))
        for m in range(K):
            raw = np.zeros(toks.shape[0])
            for i in range(d):
                raw = raw + x[m, i, toks[:, i]]
            sc[m] = raw - norm[m, d]
        best = sc.max(axis=0)
        arg = sc.argmax(axis=0)  # first (lowest) mode attaining the max
        for j in range(toks.shape[0]):
            if best[j] == -np.inf:
                continue
            t = tuple(int(a) for a in toks[j])
            allS[t] = float(best[j])
            allmu[t] = int(arg[j])
            per_mode_scores[t] = sc[:, j].copy()
            keys.append((-float(best[j]), int(arg[j]), t))
    keys.sort()
    order = [t for _, _, t in keys]
    n_select = min(B, len(order))
    cutoff = allS[order[n_select - 1]] if n_select > 0 else math.inf
    kept = np.zeros(K, dtype=np.int64)
    if n_select > 0:
        for t, sv in per_mode_scores.items():
            kept += (sv >= cutoff)
    return MixtureSelection(order=order, S=allS, mu=allmu, n_select=n_select, cutoff=cutoff,
                            per_mode_kept=kept, lse=lse, norm=norm)


def ddtree_product_select(x1: np.ndarray, B: int) -> list:
    """The single-mode (product-ranked) tree, by a different route from the heap:
    bisection on a score threshold with depth-first counting, then enumeration
    and a sort ([PP] "How it works" step 1; [PP] "In one minute", drafter (a)).

    x1: [L, V] logits of one mode.  Returns the first B prefixes in the order
    (score desc, tokens lex asc).  Uses full rows.
    """
    x1 = np.asarray(x1, dtype=np.float64)
    L, V = x1.shape
    lse = lse_rows(x1)
    norm = [0.0]
    for i in range(L):
        norm.append(norm[-1] + float(lse[i]))
    srt = [np.lexsort((np.arange(V), -x1[i])) for i in range(L)]
    sv = [x1[i][srt[i]] for i in range(L)]

    def enumerate_at(tau, cap):
        out = []
        stack = [((), 0.0)]
        while stack:
            toks, raw = stack.pop()
            d = len(toks)
            if d == L:
                continue
            for r in range(V):
                v = sv[d][r]
                if v == -np.inf:
                    break
                raw2 = raw + float(v)
                s = raw2 - norm[d + 1]
                if s < tau:
                    break
                t2 = toks + (int(srt[d][r]),)
                out.append((s, t2))
                if len(out) > cap:
                    return None
                stack.append((t2, raw2))
        return out

    if B == 0:
        return []
    cap = 50 * B + 1000
    hi, lo = 0.0, -1.0
    while True:
        got = enumerate_at(lo, cap)
        if got is None or len(got) >= B:
            break
        if lo < -1e6:
            break
        lo *= 2.0
    # bisection: keep lo with count(lo) >= B (or everything, if fewer exist)
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        got = enumerate_at(mid, cap)
        if got is not None and len(got) >= B:
            lo = mid
        else:
            hi = mid
        if hi - lo < 1e-13:
            break
    got = enumerate_at(lo, 10 ** 7)
    got.sort(key=lambda e: (-e[0], e[1]))
    return [t for _, t in got[:B]]


def mode_scores(x: np.ndarray, t: tuple, k: int | None = None, lse=None, norm=None, ranked=None) -> np.ndarray:
    """s_k(t) for every mode k: the log of the product of mode k's per-position
    probabilities of t's tokens ([PP] "How it works" step 1), summed like the
    search sums them (raw logits left to right, minus the normaliser sum).

    With `k`, a mode whose rank order puts any token of t at rank k or worse
    scores -inf (the truncated problem the search uses).  The rank of a token
    is the number of tokens of its row ahead of it in (logit desc, id asc)
    order.  `ranked` ([K][L] arrays of each row's first k ids in that order,
    as MixtureSelection.topk holds them) answers "rank < k" by membership
    instead of counting; the two give the same answer."""
    x = np.asarray(x, dtype=np.float64)
    K, L, V = x.shape
    if lse is None:
        lse = lse_rows(x)
    if norm is None:
        norm = prefix_norms(lse)
    out = np.empty(K)
    for m in range(K):
        raw = 0.0
        ok = True
        for i, tok in enumerate(t):
            raw = raw + float(x[m, i, tok])
            if k is not None:
                if ranked is not None:
                    inside = bool(np.any(np.asarray(ranked[m][i][:k]) == tok))
                else:
                    row = x[m, i]
                    ahead = np.count_nonzero(row > row[tok]) + np.count_nonzero((row == row[tok]) & (np.arange(V) < tok))
                    inside = ahead < k
                if not inside:
                    ok = False
        out[m] = raw - norm[m, len(t)] if ok else -np.inf
    return out


def union_at_cutoff(x: np.ndarray, cutoff: float, k: int, L: int | None = None, sel: MixtureSelection = None) -> tuple:
    """Per mode, the prefixes with s_k >= cutoff (the per-mode keeps), and their union
    ([PP] "In one minute": each mode keeps what reaches the common cut-off and
    the tree is built once from all keeps).  With `sel` (a selection of the
    same x whose rows were ranked to at least k) its normalisers and rank
    lists are reused instead of being computed again."""
    x = np.asarray(x, dtype=np.float64)
    K, Lx, V = x.shape
    if sel is not None and sel.topk and len(sel.topk[0][0]) >= k:
        norm = sel.norm
        ids = [[sel.topk[m][i][:k] for i in range(Lx)] for m in range(K)]
        vals = [[x[m, i][ids[m][i]] for i in range(Lx)] for m in range(K)]
    else:
        lse, norm, ids, vals = _row_tables(x, k)
    per_mode = []
    for m in range(K):
        keep = set()
        stack = [((), 0.0)]
        while stack:
            toks, raw = stack.pop()
            d = len(toks)
            if d == Lx:
                continue
            for r in range(k):
                v = vals[m][d][r]
                if v == -np.inf:
                    break
                raw2 = raw + float(v)
                if raw2 - norm[m, d + 1] < cutoff:
                    break
                t2 = toks + (int(ids[m][d][r]),)
                keep.add(t2)
                stack.append((t2, raw2))
        per_mode.append(keep)
    union = set().union(*per_mode) if per_mode else set()
    return per_mode, union


# ---------------------------------------------------------------------------
# Tree layout, mask and position ids
# ---------------------------------------------------------------------------

def canonical_tree(sel: MixtureSelection, anchor: int, B: int) -> dict:
    """Lay the selected prefixes out as one tree of B+1 rows.

    Row 0 is the root: the committed anchor token ([MD] "Model details": one
    anchor and 15 drafted slots), depth 0, parent -1, score 0, mode -1.  Rows
    1..n are the selected prefixes sorted by (depth, token sequence), so every
    parent precedes its children and siblings sit in token order.  Unused rows
    hold -1 (score -inf).  Shared prefixes appear once ([PP] "In one minute").
    """
    nodes = sorted(sel.selected, key=lambda t: (len(t), t))
    index = {(): 0}
    for i, t in enumerate(nodes):
        index[t] = i + 1
    Bp1 = B + 1
    tok = np.full(Bp1, -1, dtype=np.int64)
    par = np.full(Bp1, -1, dtype=np.int64)
    dep = np.full(Bp1, -1, dtype=np.int64)
    sco = np.full(Bp1, -np.inf, dtype=np.float64)
    mod = np.full(Bp1, -1, dtype=np.int64)
    tok[0], par[0], dep[0], sco[0], mod[0] = anchor, -1, 0, 0.0, -1
    for i, t in enumerate(nodes):
        j = i + 1
        assert t[:-1] in index, "selection is not prefix-closed"
        tok[j] = t[-1]
        par[j] = index[t[:-1]]
        dep[j] = len(t)
        sco[j] = sel.S[t]
        mod[j] = sel.mu[t]
    return {"node_token": tok, "parent": par, "depth": dep, "score": sco, "best_mode": mod,
            "n_nodes": len(nodes) + 1, "prefixes": [()] + nodes}


def tree_mask(parent: np.ndarray, depth: np.ndarray, n_nodes: int, pos_base: int, Bp1: int):
    """Ancestor-or-self mask and position ids for tree verification.

    A node may attend to itself and its ancestors (the root included), as in
    standard tree verification ([MC] summary).  Position id = pos_base + depth.
    Rows and columns at or beyond n_nodes are empty; their position id is -1.
    """
    dense = np.zeros((Bp1, Bp1), dtype=bool)
    for i in range(n_nodes):
        j = i
        while j >= 0:
            dense[i, j] = True
            j = int(parent[j])
    pos = np.full(Bp1, -1, dtype=np.int64)
    pos[:n_nodes] = pos_base + np.asarray(depth[:n_nodes], dtype=np.int64)
    return dense, pos


def pack_mask_words(dense: np.ndarray) -> np.ndarray:
    """Pack a [R, C] boolean mask into uint64 words, column c in word c // 64, bit c % 64."""
    R, C = dense.shape
    W = (C + 63) // 64
    out = np.zeros((R, W), dtype=np.uint64)
    for c in range(C):
        bit = np.uint64(1) << np.uint64(c % 64)
        out[:, c // 64] |= np.where(dense[:, c], bit, np.uint64(0))
    return out


# ---------------------------------------------------------------------------
# Counter-based noise: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11)
# ---------------------------------------------------------------------------

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_M32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds.  ctr: four arrays (or ints) of 32-bit words;
    key: two 32-bit ints.  Returns the four output words as uint64 arrays.

    Each round forms the 64-bit products of counter words 0 and 2 with the two
    round constants; the new words are (hi of the second product ^ word 1 ^
    key 0, its low half, hi of the first product ^ word 3 ^ key 1, its low
    half).  The key is bumped by the two Weyl constants between rounds.
    """
    with np.errstate(over="ignore"):
        x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) & _M32 for c in ctr)
        k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
        for r in range(10):
            p0 = np.uint64(PHILOX_M0) * x0  # < 2^64: exact in uint64
            p1 = np.uint64(PHILOX_M1) * x2
            x0, x1, x2, x3 = ((p1 >> np.uint64(32)) ^ x1 ^ np.uint64(k0), p1 & _M32,
                              (p0 >> np.uint64(32)) ^ x3 ^ np.uint64(k1), p0 & _M32)
            k0 = (k0 + PHILOX_W0) & 0xFFFFFFFF
            k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF
    return x0, x1, x2, x3


def gumbel_noise(seed: int, depth: int, V: int) -> np.ndarray:
    """Standard Gumbel noise g_v for v in [0, V) at one walk depth, fp64.

    w_v = word (v mod 4) of Philox4x32-10(counter = (v div 4, depth, 0, 0),
          key = (seed mod 2^32, seed div 2^32));
    U_v = (w_v + 1/2) * 2^-32, strictly inside (0, 1);  g_v = -log(-log U_v).
    """
    v = np.arange(V, dtype=np.uint64)
    q = v >> np.uint64(2)
    z = np.zeros_like(q)
    seed = int(seed) & ((1 << 64) - 1)
    outs = philox4x32_10((q, np.full_like(q, depth), z, z), (seed & 0xFFFFFFFF, seed >> 32))
    lane = (v & np.uint64(3)).astype(np.int64)
    w = np.choose(lane, outs)
    U = (w.astype(np.float64) + 0.5) * 2.0 ** -32
    return -np.log(-np.log(U))


# ---------------------------------------------------------------------------
# Tree verification walk
# ---------------------------------------------------------------------------

def verify_walk(node_token, parent, depth, n_nodes: int, R: np.ndarray, T: float, seed: int, L: int):
    """Walk the tree with the target's per-node logits R [B+1, V].

    From the root, take the target's token at the current node: the argmax of
    R[u] at T = 0 (ties to the lower id), else a Gumbel-max sample of
    softmax(R[u] / T) with the noise above, keyed by the node's depth.  If the
    node has a child with that token, move there and repeat; otherwise stop.
    The accepted drafted tokens are the path's tokens and the last sampled
    token is the bonus, so tau = depth(last node) + 1 ([PP] Figure 2: 6 drafted
    tokens plus the bonus; [MD] "Evaluation").  The output is the target's own
    choice at every step, so decoding is lossless ([MC] summary).

    Returns (tau, out_tokens[L+1], path_nodes[L+1], steps) with -1 padding;
    `steps` lists (node, chosen token, gap between the top two perturbed values).
    """
    if T < 0 or not np.isfinite(T):
        raise ValueError("temperature must be finite and >= 0")
    children = {}
    for i in range(1, n_nodes):
        children[(int(parent[i]), int(node_token[i]))] = i
    R = np.asarray(R, dtype=np.float64)
    V = R.shape[1]
    u = 0
    path = [0]
    toks = []
    steps = []
    while True:
        d = int(depth[u])
        row = R[u]
        if T == 0:
            y = row
        else:
            y = row / np.float64(T) + gumbel_noise(seed, d, V)
        t = int(np.argmax(y))  # first index among equal maxima
        top2 = np.partition(y, -2)[-2:] if V > 1 else np.array([y[0], -np.inf])
        steps.append((u, t, float(top2[1] - top2[0])))
        toks.append(t)
        c = children.get((u, t))
        if c is None:
            break
        u = c
        path.append(u)
    tau = int(depth[u]) + 1
    out_tokens = np.full(L + 1, -1, dtype=np.int64)
    path_nodes = np.full(L + 1, -1, dtype=np.int64)
    for i, p in enumerate(path):
        path_nodes[i] = p
    for i, p in enumerate(path[1:]):
        out_tokens[i] = int(node_token[p])
    out_tokens[tau - 1] = toks[-1]
    return tau, out_tokens, path_nodes, steps


def covered_mass(node_token, parent, n_nodes: int, R: np.ndarray, T: float) -> float:
    """Sum over drafted nodes of the target probability of reaching them
    ([PP] "Abstract": under tree verification the expected number of accepted
    tokens equals the probability mass the tree covers).  At T = 0 the target's
    token at a node is its argmax (lowest id among equal maxima, as in the
    walk), taken with probability one.  Parents must precede their children."""
    R = np.asarray(R, dtype=np.float64)
    reach = np.zeros(n_nodes)
    reach[0] = 1.0
    total = 0.0
    for i in range(1, n_nodes):
        p = int(parent[i])
        if T == 0:
            prob_t = 1.0 if int(np.argmax(R[p])) == int(node_token[i]) else 0.0
        else:
            z = R[p] / T
            z = z - z.max()
            prob_t = (np.exp(z) / np.exp(z).sum())[int(node_token[i])]
        reach[i] = reach[p] * prob_t
        total += reach[i]
    return total


def chimera_nodes(prefixes, fa, fb) -> list:
    """Prefixes spliced from two futures that are a prefix of neither
    ([PP] TL;DR and "Abstract": chimeras, prefixes stitched from different
    futures that the target never produces)."""
    out = []
    for t in prefixes:
        if len(t) == 0:
            continue
        if all(t[i] in (fa[i], fb[i]) for i in range(len(t))):
            if tuple(t) != tuple(fa[: len(t)]) and tuple(t) != tuple(fb[: len(t)]):
                out.append(t)
    return out


def band_is_exact(x: np.ndarray, sel: MixtureSelection, tol: float = 1e-4) -> bool:
    """Whether the node set is fixed by comparisons that are exact on any
    implementation that sums raw logits in fp64 and differs only in the row
    normalisers by much less than `tol`.

    Every selected prefix p and unselected prefix q with S(p) - S(q) < tol must
    share (best mode, depth), and each must lead its runner-up mode by at least
    `tol`; then their order is decided by raw sums and token ids alone.  Needs
    `sel` computed with band >= tol so that the prefixes just below the cut-off
    are listed.
    """
    if sel.n_select == 0 or len(sel.order) <= sel.n_select:
        return True
    K, L, V = x.shape
    k = min(len(sel.topk[0][0]) if sel.topk else V, V)
    inside = [t for t in sel.selected if sel.S[t] - sel.cutoff < tol]
    outside = [t for t in sel.order[sel.n_select:] if sel.cutoff - sel.S[t] < tol]
    if not outside:
        return True
    group = inside + outside
    keys = {(sel.mu[t], len(t)) for t in group}
    if len(keys) != 1:
        return False
    for t in group:
        sc = mode_scores(x, t, k=k, lse=sel.lse, norm=sel.norm)
        sc = np.sort(sc)[::-1]
        if K > 1 and sc[0] - sc[1] < tol:
            return False
    return True


def build_tree(x: np.ndarray, B: int, anchor: int, band: float = 1e-4) -> tuple:
    """Selection + canonical layout for one tree (convenience for tests)."""
    sel = mixture_select_heap(x, B, band=band)
    return sel, canonical_tree(sel, anchor, B)
