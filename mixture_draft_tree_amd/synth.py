"""Seeded synthetic workloads for the mixture draft tree path.

This module only draws random inputs. It holds none of the method's arithmetic
(no softmax, no scoring, no tree logic), so both the fp64 oracle tests and the
GPU path may use it as a common source of inputs.

The workloads stand in for real drafter logits. The Multi-Future Drafting pages
measure on drafter outputs over public task suites with trained checkpoints;
none of that is used here. What is kept from the pages is the shape of the
problem: a block of 16 slots with 15 drafted positions (MFD-Qwen3.5-4B model
card, "Model"), K = 8 modes and a budget of B = 256 (same card, "Results"), and
modes that each draft one coherent future (project page, "How it works", step 2).
The `single`, `batched` and `stress` workloads follow a fixed recipe: drafter
noise N(0, 3^2) with each mode's future boosted by +8, and target rows N(0,1)
with +10 on the chosen future.  That drafter is nearly flat over 151936
tokens, so its trees are shallow (depth 2 or so, acceptance length about 1.4).
The `deep` and `batched_deep` workloads model a trained, confident drafter
instead: each mode's future token takes most of its row's mass
(log-probability about -0.1 to -1.3), a few alternatives sit far below it, and
the target follows the chosen future for a random number of tokens, so trees
reach the full depth of 15 and acceptance lengths land near the pages'
figures (tau of 6 to 11 at B = 256, project page, Table 1; about 10.7 for MFD
on Qwen3.5-4B at T = 0, model card, "Results").

Named workloads:

  tiny          K=2,  L=4,  V=16,     B=8     fp32, brute-forceable
  product       K=1,  L=15, V=32000,  B=64    bf16, two injected futures at equal mass
  single        K=8,  L=15, V=151936, B=256   bf16, one tree
  batched       64 trees of the `single` shape, T alternating 0 / 1
  stress        K=16, L=15, V=248320, B=1024  bf16, heavy exact ties
  deep          K=8,  L=15, V=151936, B=256   bf16, one tree, confident drafter
  batched_deep  64 trees of the `deep` shape, T alternating 0 / 1
  subset        as `single`, drafting over a 65536-token subset of the V tokens
  batched_subset  64 trees of the `subset` shape
  batched_modes   64 trees of the `deep` shape, K_n alternating 8 / 1 (T 0, 0, 1, 1)

The subset workloads draft over a sorted random subset of 65536 of the 151936
target tokens (the project page's serving setup drafts over the target's 64K
most frequent tokens and verifies over the full vocabulary): drafter logits
cover the subset, futures are drawn from it, target rows cover all V tokens.

The `batched_modes` workload mixes requests drafted with all K modes and
requests drafted with mode 0 only in one batch (the single-mode default path
that the project page's MFD-D configuration switches to in a busy engine, "In
a serving engine").  Logits of the modes a tree does not use are NaN, so any
read of them shows up as a non-finite flag or a wrong tree.  The target follows
one of all K futures either way, as the full drafter's chosen future.

Every draw comes from a torch.Generator seeded from (workload id, tree index,
base seed), on the device the caller names, so a given (device, seed) always
yields the same tensors.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    K: int
    L: int
    V: int
    B: int
    N: int
    dtype: torch.dtype
    sigma: float          # std of the drafter noise
    boost: float          # added to each mode's future tokens
    target_boost: float   # added to the chosen future in the target rows
    temperatures: tuple   # per-tree temperature pattern (cycled)
    jitter: float = 0.0   # std of a per-(mode, position) offset of the future token's boost
    alt_n: int = 0        # per (mode, position) row: alternative tokens given a Zipf bump ...
    alt_height: float = 0.0  # ... of alt_height * r^-1.1, r = 1..alt_n
    dev_lo: int = 0       # target leaves the chosen future at a depth D ~ U{dev_lo..L} (0: never)
    v_draft: int = 0      # drafting vocabulary: a sorted random subset of this many of the V tokens (0: all)
    modes: tuple = ()     # per-tree number of active modes, cycled over the trees (empty: K for every tree)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 4, 16, 8, 1, torch.float32, 2.0, 4.0, 5.0, (0.0,)),
    "product": Workload("product", 2, 1, 15, 32000, 64, 1, torch.bfloat16, 2.0, 0.0, 10.0, (0.0,)),
    "single": Workload("single", 3, 8, 15, 151936, 256, 1, torch.bfloat16, 3.0, 8.0, 10.0, (0.0, 1.0)),
    "batched": Workload("batched", 4, 8, 15, 151936, 256, 64, torch.bfloat16, 3.0, 8.0, 10.0, (0.0, 1.0)),
    "stress": Workload("stress", 5, 16, 15, 248320, 1024, 1, torch.bfloat16, 3.0, 8.0, 10.0, (1.0,)),
    "deep": Workload("deep", 6, 8, 15, 151936, 256, 1, torch.bfloat16, 2.0, 16.0, 16.0, (0.0, 1.0),
                     jitter=1.5, alt_n=16, alt_height=10.0, dev_lo=3),
    "batched_deep": Workload("batched_deep", 7, 8, 15, 151936, 256, 64, torch.bfloat16, 2.0, 16.0, 16.0,
                             (0.0, 1.0), jitter=1.5, alt_n=16, alt_height=10.0, dev_lo=3),
    "subset": Workload("subset", 8, 8, 15, 151936, 256, 1, torch.bfloat16, 3.0, 8.0, 10.0, (0.0, 1.0),
                       v_draft=65536),
    "batched_subset": Workload("batched_subset", 9, 8, 15, 151936, 256, 64, torch.bfloat16, 3.0, 8.0, 10.0,
                               (0.0, 1.0), v_draft=65536),
    "batched_modes": Workload("batched_modes", 10, 8, 15, 151936, 256, 64, torch.bfloat16, 2.0, 16.0, 16.0,
                              (0.0, 0.0, 1.0, 1.0), jitter=1.5, alt_n=16, alt_height=10.0, dev_lo=3,
                              modes=(8, 1)),
}


def tree_seed(wid: int, tree_index: int, base_seed: int) -> int:
    """Mix (workload id, tree index, base seed) into one 63-bit seed (splitmix64 steps)."""
    mask = (1 << 64) - 1
    z = 0
    for part in (wid, tree_index, base_seed):
        z = (z + 0x9E3779B97F4A7C15 + (part & mask)) & mask
        z ^= z >> 30
        z = (z * 0xBF58476D1CE4E5B9) & mask
        z ^= z >> 27
        z = (z * 0x94D049BB133111EB) & mask
        z ^= z >> 31
    return z & ((1 << 63) - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randint(g, high, size, device):
    return torch.randint(0, high, size, generator=g, device=device)


def _distinct_other(g, avoid: int, V: int, device) -> int:
    """A token drawn uniformly from [0, V) \\ {avoid}."""
    t = int(_randint(g, V - 1, (1,), device).item())
    return t + 1 if t >= avoid else t


@dataclasses.dataclass
class DraftBatch:
    """Drafter-side inputs for N trees."""
    workload: Workload
    logits: torch.Tensor        # [N, K, L, V] in workload.dtype
    futures: torch.Tensor       # [N, F, L] int64: the injected futures (F = K, or 2 for `product`)
    chosen_mode: torch.Tensor   # [N] int64: index into F of the future the target follows
    anchor: torch.Tensor        # [N] int32: committed token at the root
    pos_base: torch.Tensor      # [N] int64: position id of the root
    temperature: torch.Tensor   # [N] float32
    seed: torch.Tensor          # [N] uint64 stored as int64 (two's complement)
    tree_seeds: list            # python ints, one per tree
    vocab_map: Optional[torch.Tensor] = None  # [v_draft] int32 full ids (sorted) of the drafting tokens
    modes: Optional[torch.Tensor] = None      # [N] int32: active modes of each tree (None: all K)
    start: int = 0                            # index of the first tree within the workload


def _tiny_tree(w, g, device):
    K, L, V = w.K, w.L, w.V
    x = torch.randn((K, L, V), generator=g, device=device, dtype=torch.float32) * w.sigma
    A = _randint(g, V, (L,), device)
    Bf = A.clone()
    pos = torch.randperm(L, generator=g, device=device)[:2]
    for p in pos.tolist():
        Bf[p] = _distinct_other(g, int(A[p]), V, device)
    fut = torch.stack([A, Bf])  # mode 0 follows A, mode 1 follows B
    ar = torch.arange(L, device=device)
    for k in range(K):
        x[k, ar, fut[k]] += w.boost
    return x, fut


def _zipf_bump(g, L, V, device, n=20, height=6.0, s=1.1):
    """Per position, `n` random tokens get height * r^-s for r = 1..n."""
    bump = torch.zeros((L, V), device=device, dtype=torch.float32)
    r = torch.arange(1, n + 1, device=device, dtype=torch.float32)
    vals = height * r.pow(-s)
    for i in range(L):
        toks = torch.randperm(V, generator=g, device=device)[:n]
        bump[i, toks] = vals
    return bump


# Offsets (in units of 1/2) for the three disagreeing positions of the
# `product` workload: A gets c + d/2, B gets c - d/2.  They sum to zero, so A
# and B carry equal total mass, and no other signed subset sums to zero.
PRODUCT_DELTAS = (1.0, 0.5, -1.5)
PRODUCT_SPLIT_POSITIONS = (1, 2, 3)   # 0-based drafted positions 2..4


def _product_tree(w, g, device):
    L, V = w.L, w.V
    x = torch.randn((1, L, V), generator=g, device=device, dtype=torch.float32) * w.sigma
    x[0] += _zipf_bump(g, L, V, device)
    A = _randint(g, V, (L,), device)
    Bf = A.clone()
    for p in PRODUCT_SPLIT_POSITIONS:
        Bf[p] = _distinct_other(g, int(A[p]), V, device)
    # c: a multiple of 0.25, at least 4 above every row maximum (exact in bf16 below 32).
    rowmax = float(x.max().item())
    c = math.ceil((rowmax + 4.0) * 4.0) / 4.0
    assert c + 1.0 < 32.0
    ar = torch.arange(L, device=device)
    x[0, ar, A] = c
    for p, d in zip(PRODUCT_SPLIT_POSITIONS, PRODUCT_DELTAS):
        x[0, p, A[p]] = c + d / 2.0
        x[0, p, Bf[p]] = c - d / 2.0
    return x, torch.stack([A, Bf])  # futures reported as [2, L] for this workload


def _mode_futures(w, g, device):
    """Each mode's future: a shared prefix of length U{0..7}, then m_k ~ U{1..7}
    positions after it resampled (one coherent future per mode)."""
    K, L, V = w.K, w.L, w.V
    base = _randint(g, V, (L,), device)
    p = int(_randint(g, 8, (1,), device).item())
    fut = base.unsqueeze(0).repeat(K, 1)
    for k in range(K):
        m = int(_randint(g, 7, (1,), device).item()) + 1
        m = min(m, L - p)
        pos = p + torch.randperm(L - p, generator=g, device=device)[:m]
        for q in pos.tolist():
            fut[k, q] = _distinct_other(g, int(base[q]), V, device)
    return fut


def _mixture_tree(w, g, device, ties: bool):
    """A confident drafter: per (mode, position) row, N(0, sigma^2) noise, a
    Zipf bump on `alt_n` alternative tokens, and the mode's future token set
    to boost + N(0, jitter^2), which puts most of the row's mass on it."""
    K, L, V = w.K, w.L, w.V
    x = torch.randn((K, L, V), generator=g, device=device, dtype=torch.float32) * w.sigma
    if w.alt_n > 0:
        r = torch.arange(1, w.alt_n + 1, device=device, dtype=torch.float32)
        bump = w.alt_height * r.pow(-1.1)
        alt = torch.randint(0, V, (K, L, w.alt_n), generator=g, device=device)
        x.scatter_add_(2, alt, bump.expand(K, L, w.alt_n).contiguous())
    fut = _mode_futures(w, g, device)
    ar = torch.arange(L, device=device)
    for k in range(K):
        if w.jitter > 0:
            jit = torch.randn((L,), generator=g, device=device, dtype=torch.float32) * w.jitter
            x[k, ar, fut[k]] = w.boost + jit
        else:
            x[k, ar, fut[k]] += w.boost
    if ties:
        # In 10% of (mode, position) rows a second token gets the bit-identical
        # (after bf16 rounding) value of the boosted future token.
        xb = x.to(torch.bfloat16)
        pick = torch.rand((K, L), generator=g, device=device) < 0.10
        for k, i in pick.nonzero().tolist():
            other = _distinct_other(g, int(fut[k, i]), V, device)
            xb[k, i, other] = xb[k, i, fut[k, i]]
        return xb, fut
    return x, fut


def vocab_subset(w: Workload, base_seed: int = 0, device="cpu") -> Optional[torch.Tensor]:
    """The workload's drafting vocabulary: v_draft sorted distinct ids of [0, V), seeded."""
    if not w.v_draft:
        return None
    g = _gen(device, tree_seed(w.wid + 200, 0, base_seed))
    ids = torch.randperm(w.V, generator=g, device=device)[:w.v_draft]
    return torch.sort(ids).values.to(torch.int32)


def draft_batch(name: str, base_seed: int = 0, device="cpu", N: Optional[int] = None, start: int = 0) -> DraftBatch:
    """Drafter logits and per-tree metadata for trees start .. start+N-1 of workload
    `name` (over the drafting vocabulary when the workload has one; futures are then
    reported as full ids).  Tree n is the same whatever batch it is drawn in."""
    w = WORKLOADS[name]
    N = w.N if N is None else N
    vmap = vocab_subset(w, base_seed, device)
    wd = dataclasses.replace(w, V=w.v_draft) if w.v_draft else w
    logits = torch.empty((N, w.K, w.L, wd.V), dtype=w.dtype, device=device)
    futs, chosen, anchors, seeds = [], [], [], []
    idx = list(range(start, start + N))
    for j, n in enumerate(idx):
        s = tree_seed(w.wid, n, base_seed)
        seeds.append(s)
        g = _gen(device, s)
        if name == "tiny":
            x, fut = _tiny_tree(w, g, device)
        elif name == "product":
            x, fut = _product_tree(w, g, device)
        else:
            x, fut = _mixture_tree(wd, g, device, ties=(name == "stress"))
            if vmap is not None:
                fut = vmap.to(torch.int64)[fut]
        if w.modes:
            x[w.modes[n % len(w.modes)]:] = float("nan")
        logits[j] = x.to(w.dtype)
        futs.append(fut)
        chosen.append(int(_randint(g, fut.shape[0], (1,), device).item()))
        anchors.append(int(_randint(g, w.V, (1,), device).item()))
    temps = torch.tensor([w.temperatures[n % len(w.temperatures)] for n in idx], dtype=torch.float32)
    seed_t = torch.tensor([(s ^ 0x5DEECE66D) & ((1 << 63) - 1) for s in seeds], dtype=torch.int64)
    return DraftBatch(
        workload=w, logits=logits, futures=torch.stack(futs),
        chosen_mode=torch.tensor(chosen, dtype=torch.int64),
        anchor=torch.tensor(anchors, dtype=torch.int32),
        pos_base=torch.tensor([1000 + 17 * n for n in idx], dtype=torch.int64),
        temperature=temps, seed=seed_t, tree_seeds=seeds, vocab_map=vmap,
        modes=(torch.tensor([w.modes[n % len(w.modes)] for n in idx], dtype=torch.int32)
               if w.modes else None), start=start)


def target_logits(batch: DraftBatch, depth: torch.Tensor, n_nodes: torch.Tensor,
                  device="cpu", base_seed: int = 0) -> torch.Tensor:
    """Target per-node logits [N, B+1, V].

    Rows are N(0,1).  The target follows one future F (the chosen mode's): every
    tree node at depth d < L gets `target_boost` on F[d], so from the root the
    target's preferred continuation is F token by token.  With `dev_lo` > 0 the
    target leaves F at a depth D ~ U{dev_lo..L}: from depth D on the boost goes
    to another token G[d] != F[d] instead.  `depth` / `n_nodes` describe the tree
    the rows belong to (node i of tree n has depth depth[n, i]).
    """
    w = batch.workload
    N = batch.logits.shape[0]
    Bp1 = w.B + 1
    out = torch.empty((N, Bp1, w.V), dtype=w.dtype, device=device)
    depth = depth.to("cpu")
    n_nodes = n_nodes.to("cpu")
    for n in range(N):
        g = _gen(device, tree_seed(w.wid + 100, batch.start + n, base_seed))
        r = torch.randn((Bp1, w.V), generator=g, device=device, dtype=torch.float32)
        F = batch.futures[n, int(batch.chosen_mode[n])].to(device).clone()
        if w.dev_lo > 0:
            D = w.dev_lo + int(_randint(g, w.L - w.dev_lo + 1, (1,), device).item())
            for q in range(D, w.L):
                F[q] = _distinct_other(g, int(F[q]), w.V, device)
        nn_ = int(n_nodes[n])
        d = depth[n, :nn_].to(torch.int64)
        rows = torch.nonzero(d < w.L).flatten()
        if rows.numel():
            r[rows.to(device), F[d[rows].to(device)]] += w.target_boost
        out[n] = r.to(w.dtype)
    return out


# ---------------------------------------------------------------------------
# Drafter hidden states and LM head (the fused-logits path)
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class LmHeadWorkload:
    name: str
    wid: int
    K: int
    L: int
    V: int
    D: int        # hidden width (2560 for the MFD drafter of Qwen3.5-4B)
    B: int
    N: int
    grid: bool    # values on a coarse binary grid (every partial sum exact in fp32)


LMHEAD_WORKLOADS = {
    # small shapes: ragged row and vocabulary tiles, whole-row sample
    "lmhead_small": LmHeadWorkload("lmhead_small", 20, 2, 5, 1000, 128, 32, 3, True),
    "lmhead_ragged": LmHeadWorkload("lmhead_ragged", 21, 3, 7, 4133, 192, 64, 5, False),
    # two row tiles (the second ragged) and a sampled threshold
    "lmhead_mid": LmHeadWorkload("lmhead_mid", 22, 8, 15, 40000, 256, 256, 2, True),
    # 360 rows: more than 256, so the 256-column tiles of large batches are used
    "lmhead_wide": LmHeadWorkload("lmhead_wide", 26, 8, 15, 40000, 256, 256, 3, True),
    # 2160 rows over 17 row tiles, the last one ragged
    "lmhead_tall": LmHeadWorkload("lmhead_tall", 27, 8, 15, 10000, 128, 64, 18, True),
    # the MFD drafter's shape: K=8 modes x 15 positions over V=151936 at D=2560
    "lmhead_single": LmHeadWorkload("lmhead_single", 23, 8, 15, 151936, 2560, 256, 1, False),
    "lmhead_single_grid": LmHeadWorkload("lmhead_single_grid", 24, 8, 15, 151936, 2560, 256, 1, True),
    "lmhead_batched": LmHeadWorkload("lmhead_batched", 25, 8, 15, 151936, 2560, 256, 64, False),
}


@dataclasses.dataclass
class LmHeadBatch:
    workload: LmHeadWorkload
    hidden: torch.Tensor     # [N, K, L, D] bf16
    weight: torch.Tensor     # [V, D] bf16
    futures: torch.Tensor    # [N, K, L] int64: each mode's future
    anchor: torch.Tensor     # [N] int32


def lmhead_weight(w: LmHeadWorkload, base_seed: int = 0, device="cpu") -> torch.Tensor:
    """The LM head [V, D] bf16, shared by every tree of the workload.

    Gaussian recipe: N(0, (3 / sqrt(D))^2), so logits of a unit hidden state are
    about N(0, 9) like the drafter noise of the `single` workload.  Grid recipe:
    integers in [-8, 8] times 2^-5."""
    g = _gen(device, tree_seed(w.wid, 1 << 20, base_seed))
    if w.grid:
        x = (torch.randint(-8, 9, (w.V, w.D), generator=g, device=device).to(torch.float32)) * 2.0 ** -5
    else:
        x = torch.randn((w.V, w.D), generator=g, device=device, dtype=torch.float32) * (3.0 / math.sqrt(w.D))
    return x.to(torch.bfloat16)


def lmhead_batch(name: str, base_seed: int = 0, device="cpu", N: Optional[int] = None) -> LmHeadBatch:
    """Hidden states [N, K, L, D] whose logits favour each mode's future.

    Futures are drawn as for the mixture workloads (shared prefix, then a few
    resampled positions per mode).  Gaussian recipe: h = N(0, 1) + (8/9) W[f],
    so the future token's logit gains about 8 (|W[f]|^2 is about 9).  Grid
    recipe: h = integers in [-4, 4] times 2^-2, plus 2^-2 sign(W[f, d]) on a
    random set of min(D, 240) coordinates d.  On the grid every product is a
    multiple of 2^-7 below 0.32 in magnitude, so every partial sum of D <= 2560
    of them is a multiple of 2^-7 below 2^10: exact in fp32 in any order."""
    w = LMHEAD_WORKLOADS[name]
    N = w.N if N is None else N
    W = lmhead_weight(w, base_seed, device)
    Wf = W.to(torch.float32)
    H = torch.empty((N, w.K, w.L, w.D), dtype=torch.bfloat16, device=device)
    futs, anchors = [], []
    for n in range(N):
        g = _gen(device, tree_seed(w.wid, n, base_seed))
        fut = _mode_futures(w, g, device)
        if w.grid:
            h = torch.randint(-4, 5, (w.K, w.L, w.D), generator=g, device=device).to(torch.float32) * 0.25
            nb = min(w.D, 240)
            for k in range(w.K):
                for i in range(w.L):
                    dims = torch.randperm(w.D, generator=g, device=device)[:nb]
                    h[k, i, dims] += 0.25 * torch.sign(Wf[fut[k, i], dims])
        else:
            h = torch.randn((w.K, w.L, w.D), generator=g, device=device, dtype=torch.float32)
            h += (8.0 / 9.0) * Wf[fut]
        H[n] = h.to(torch.bfloat16)
        futs.append(fut)
        anchors.append(int(_randint(g, w.V, (1,), device).item()))
    return LmHeadBatch(workload=w, hidden=H, weight=W, futures=torch.stack(futs),
                       anchor=torch.tensor(anchors, dtype=torch.int32))
