"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars: ids, node sets, parents, depths, masks, tau and tokens bit-exact (trees
whose cut-off band is not decided by exact comparisons are reported and
excluded from node-set exactness); log-normalisers within 1e-5, scores within
1e-4."""

import math
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle as O
from parity_checks import PEAKED, peaked_logits
from mixture_draft_tree_amd import synth
from mixture_draft_tree_amd import mfdtree as M
from mixture_draft_tree_amd.pipeline import MixtureTreePath

from gpu_helpers import (Spill, check_lsm, check_mask, check_walk, compare_tree, run_pool, tree_job,
                         tree_rows, upload_tree, walk_job)

pytestmark = pytest.mark.gpu


def setup_module(_):
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _lsm_run(x_cpu: torch.Tensor, k: int, logp=True, offset_bytes=0):
    N, K, L, V = x_cpu.shape
    if offset_bytes:
        esz = x_cpu.element_size()
        raw = torch.empty(x_cpu.numel() + 16, dtype=x_cpu.dtype, device="cuda")
        x = raw[offset_bytes // esz: offset_bytes // esz + x_cpu.numel()].view(N, K, L, V)
        x.copy_(x_cpu.cuda())
    else:
        x = x_cpu.cuda()
    lse = torch.empty((N, K, L), dtype=torch.float64, device="cuda")
    tid = torch.empty((N, K, L, k), dtype=torch.int32, device="cuda")
    raw_ = torch.empty((N, K, L, k), dtype=torch.float32, device="cuda")
    lp = torch.empty((N, K, L, k), dtype=torch.float32, device="cuda") if logp else None
    st = torch.zeros((N,), dtype=torch.int32, device="cuda")
    M.mfd_logsoftmax_topk(x, k, lse, tid, raw_, lp, st)
    torch.cuda.synchronize()
    return lse, tid, raw_, lp, st


# ------------------------------------------------------------------ logits pass

LSM_CASES = [
    # name, N, K, L, V, k, dtype, maker
    ("f32_tiny", 1, 2, 4, 16, 8, torch.float32, "normal"),
    ("bf16_ragged", 2, 3, 2, 5003, 37, torch.bfloat16, "normal"),
    ("f32_ragged", 1, 2, 3, 1027, 100, torch.float32, "normal"),
    ("bf16_int_ties", 1, 2, 2, 4099, 300, torch.bfloat16, "ints"),
    ("bf16_constant", 1, 1, 2, 3000, 256, torch.bfloat16, "const"),
    ("bf16_neginf", 1, 2, 2, 2000, 256, torch.bfloat16, "neginf"),
    ("bf16_all_neginf", 1, 1, 1, 777, 64, torch.bfloat16, "allneginf"),
    ("bf16_k_eq_V", 1, 2, 2, 300, 300, torch.bfloat16, "normal"),
    ("bf16_ascending", 1, 1, 2, 20000, 256, torch.bfloat16, "ascending"),
    ("bf16_k1024", 1, 2, 1, 248320, 1024, torch.bfloat16, "normal"),
    ("bf16_signed_zero", 1, 1, 1, 1000, 200, torch.bfloat16, "zeros"),
    # full-vocabulary rows: the sampled-threshold path and each of its exits
    ("bf16_vocab", 1, 2, 3, 151936, 256, torch.bfloat16, "normal"),
    ("f32_vocab", 1, 1, 2, 151936, 256, torch.float32, "normal"),
    ("bf16_vocab_clustered", 1, 1, 2, 151936, 256, torch.bfloat16, "clustered"),
    ("bf16_vocab_late_mass", 1, 1, 2, 151936, 256, torch.bfloat16, "late"),
    ("bf16_vocab_early_mass", 1, 1, 2, 151936, 256, torch.bfloat16, "early"),
    ("bf16_vocab_shifted_block", 1, 1, 2, 151936, 256, torch.bfloat16, "shifted"),
    # the row maximum lies far from the sample maximum: the sum is redone
    ("bf16_vocab_spike", 1, 1, 2, 151936, 256, torch.bfloat16, "spike"),
    ("f32_deep_after_neginf", 1, 1, 2, 20000, 64, torch.float32, "deep"),
]


def _make(kind, shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    if kind == "normal":
        x = torch.randn(shape, generator=g) * 3
    elif kind == "ints":
        x = torch.randint(-3, 4, shape, generator=g).float()
    elif kind == "const":
        x = torch.full(shape, 1.5)
    elif kind == "neginf":
        x = torch.randn(shape, generator=g) * 2
        x[torch.rand(shape, generator=g) < 0.95] = -float("inf")
    elif kind == "allneginf":
        x = torch.full(shape, -float("inf"))
    elif kind == "ascending":
        x = torch.linspace(-8, 8, shape[-1]).expand(shape).clone()
    elif kind == "clustered":
        # more elements above the sampled threshold than the candidate list holds
        x = torch.randn(shape, generator=g)
        x[..., 60000:61600] = 10 + 0.5 * torch.randn(shape[:-1] + (1600,), generator=g)
    elif kind == "late":
        # the sample chunk sits far below the rest: staging overflows
        x = torch.randn(shape, generator=g) * 3
        x[..., :20000] -= 30
    elif kind == "early":
        # the sample chunk sits far above the rest: fewer than k reach the threshold
        x = torch.randn(shape, generator=g) * 3
        x[..., :8192] += 30
    elif kind == "shifted":
        # a block after the sample sits higher: staging overflows, and the row
        # is staged again with a threshold taken from what was staged
        x = torch.randn(shape, generator=g) * 3
        x[..., 30000:40000] += 5
    elif kind == "spike":
        x = torch.randn(shape, generator=g)
        x[..., 100000] = 200.0
    elif kind == "deep":
        x = torch.randn(shape, generator=g) - 300
        x[..., :9000] = -float("inf")
    elif kind == "zeros":
        x = torch.zeros(shape)
        x[..., ::3] = -0.0
        x[..., 1::7] = 0.5
    return x.to(dtype)


@pytest.mark.parametrize("case", LSM_CASES, ids=[c[0] for c in LSM_CASES])
def test_logsoftmax_topk_parity(case):
    name, N, K, L, V, k, dt, kind = case
    say(f"[lsm] {name} N={N} K={K} L={L} V={V} k={k}")
    x = _make(kind, (N, K, L, V), dt, seed=zlib.crc32(name.encode()) % 1000)
    lse, tid, raw, lp, st = _lsm_run(x, k)
    err = check_lsm(x, lse, tid, raw, k, lp)
    assert st.cpu().eq(0).all()
    say(f"[lsm] {name} max |lse err| = {err:.2e}")


def test_logsoftmax_topk_unaligned_rows():
    x = _make("normal", (1, 2, 3, 1001), torch.bfloat16, 5)
    for off in (2, 6, 14):
        lse, tid, raw, lp, st = _lsm_run(x, 64, offset_bytes=off)
        check_lsm(x, lse, tid, raw, 64, lp)


def test_logsoftmax_topk_nonfinite_status():
    x = _make("normal", (3, 2, 2, 500), torch.bfloat16, 6)
    x[1, 1, 0, 17] = float("nan")
    x[2, 0, 1, 3] = float("inf")
    _, _, _, _, st = _lsm_run(x, 16)
    assert st.cpu().tolist() == [0, M.MFD_TREE_NONFINITE, M.MFD_TREE_NONFINITE]


# ------------------------------------------------------------------ tree stages on small cases

def _small_tree_case(seed, K, L, V, B, ints=False, neginf=0.0, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    if ints:
        x = torch.randint(-3, 4, (1, K, L, V), generator=g).float()
    else:
        x = torch.randn((1, K, L, V), generator=g) * 2
    if neginf:
        x[torch.rand(x.shape, generator=g) < neginf] = -float("inf")
        x[..., 0] = torch.where(torch.isinf(x[..., 0]), torch.zeros_like(x[..., 0]), x[..., 0])
    return x.to(dtype)


SMALL = [
    # seed, K, L, V, B, ints, neginf
    (1, 2, 4, 16, 8, False, 0.0),
    (2, 3, 5, 40, 30, False, 0.0),
    (3, 1, 6, 20, 50, False, 0.0),
    (4, 4, 3, 9, 60, True, 0.0),
    (5, 2, 3, 6, 20, False, 0.0),     # V < B: k = V
    (6, 3, 4, 12, 25, False, 0.4),
    (7, 2, 1, 50, 10, False, 0.0),    # L = 1
    (8, 5, 4, 30, 1, False, 0.0),     # B = 1
    (9, 2, 4, 10, 0, False, 0.0),     # B = 0
    (10, 8, 6, 64, 200, True, 0.0),
    (11, 3, 8, 7, 300, False, 0.0),   # deep, narrow
]


@pytest.mark.parametrize("case", SMALL, ids=[f"s{c[0]}" for c in SMALL])
def test_tree_small_cases(case):
    seed, K, L, V, B, ints, neginf = case
    say(f"[tree] seed={seed} K={K} L={L} V={V} B={B}")
    x = _small_tree_case(seed, K, L, V, B, ints, neginf)
    P = MixtureTreePath(1, K, L, V, B, with_logp=True, with_dense_mask=True)
    anchor = torch.tensor([7], dtype=torch.int32, device="cuda")
    pos = torch.tensor([100], dtype=torch.int64, device="cuda")
    P.build(x.cuda(), anchor, pos)
    torch.cuda.synchronize()
    assert P.buf.status.item() == 0
    x64 = x[0].double().numpy()
    r = compare_tree(x64, B, 7, tree_rows(P, 0))
    if V ** min(L, 3) < 5000 and B > 0:  # brute force agrees with the oracle heap on small spaces
        bf = O.mixture_select_bruteforce(x64, B)
        assert bf.selected == r["sel"].selected
    g = tree_rows(P, 0)
    check_mask(g["parent"], g["depth"], g["n_nodes"], 100, B + 1,
               P.buf.mask_words[0].cpu().numpy(), P.buf.position_ids[0].cpu().numpy(),
               P.buf.dense_mask[0].cpu().numpy())
    say(f"[tree] seed={seed} exact={r['exact']} n_nodes={g['n_nodes']}")


# Modes that share their tokens: the cut-off's starting bound pools each
# mode's first depth-1 candidates and merges equal tokens, so runs of one
# token across modes, exact ties across modes (a constant shift leaves the
# log-probabilities unchanged) and pools with fewer than B distinct tokens all
# have to give the oracle's tree.
SHARED = [
    # seed, K, L, V, B, per-mode noise (0: identical modes), per-mode shift
    (21, 4, 3, 200, 100, 0.0, 0.0),
    (22, 8, 4, 300, 120, 0.3, 0.0),
    (23, 6, 3, 500, 150, 0.0, 0.75),
    (24, 8, 3, 1000, 256, 1.0, 0.0),
    (25, 32, 3, 2000, 300, 0.5, 0.0),   # K = 32: 2048 pooled candidates
    (26, 32, 2, 500, 40, 0.2, 0.0),     # K = 32 with k = B = 40 < 64
]


@pytest.mark.parametrize("case", SHARED, ids=[f"m{c[0]}" for c in SHARED])
def test_tree_shared_modes(case):
    seed, K, L, V, B, noise, shift = case
    say(f"[tree shared modes] seed={seed} K={K} L={L} V={V} B={B}")
    g = torch.Generator().manual_seed(seed)
    base = torch.randn((1, 1, L, V), generator=g) * 2
    x = base.expand(1, K, L, V) + noise * torch.randn((1, K, L, V), generator=g)
    x = x + shift * torch.arange(K, dtype=torch.float32).view(1, K, 1, 1)
    x = x.contiguous()
    P = MixtureTreePath(1, K, L, V, B, with_logp=True)
    anchor = torch.tensor([3], dtype=torch.int32, device="cuda")
    pos = torch.tensor([0], dtype=torch.int64, device="cuda")
    P.build(x.cuda(), anchor, pos)
    torch.cuda.synchronize()
    assert P.buf.status.item() == 0
    r = compare_tree(x[0].double().numpy(), B, 3, tree_rows(P, 0))
    say(f"[tree shared modes] seed={seed} exact={r['exact']} n_nodes={tree_rows(P, 0)['n_nodes']}")


@pytest.mark.parametrize("case", PEAKED, ids=[f"p{c[0]}" for c in PEAKED])
def test_tree_peaked_rows(case):
    """One token leads every row by a wide gap: the B best prefixes score many
    binades above the running threshold, so the threshold's raise takes its
    radix passes rather than the one-pass window."""
    seed, K, L, V, B, gap = case
    say(f"[tree peaked] seed={seed} K={K} L={L} V={V} B={B} gap={gap}")
    x = torch.from_numpy(peaked_logits(seed, K, L, V, gap))[None]
    P = MixtureTreePath(1, K, L, V, B, with_logp=True)
    anchor = torch.tensor([2], dtype=torch.int32, device="cuda")
    pos = torch.tensor([0], dtype=torch.int64, device="cuda")
    P.build(x.cuda(), anchor, pos)
    torch.cuda.synchronize()
    assert P.buf.status.item() == 0
    # the normaliser of a row never falls below its top logit
    assert bool((P.buf.lse.cpu() >= P.buf.topk_raw[..., 0].double().cpu()).all())
    r = compare_tree(x[0].double().numpy(), B, 2, tree_rows(P, 0))
    say(f"[tree peaked] seed={seed} exact={r['exact']} n_nodes={tree_rows(P, 0)['n_nodes']}")


def test_modes_small_batch():
    """Per-tree mode counts in one launch: each tree equals the oracle over its first
    K_n modes, a tree with K_n = K equals the plain calls bit for bit, and counts
    outside [1, K] are clamped and flagged."""
    K, L, V, B = 4, 5, 40, 30
    modes_h = [4, 1, 2, 3, 0, 7]
    kn = [min(max(m, 1), K) for m in modes_h]
    N = len(modes_h)
    x = torch.cat([_small_tree_case(40 + n, K, L, V, B, ints=(n % 2 == 1)) for n in range(N)])
    anchor = torch.arange(N, dtype=torch.int32, device="cuda") + 3
    pos = torch.full((N,), 50, dtype=torch.int64, device="cuda")
    modes = torch.tensor(modes_h, dtype=torch.int32, device="cuda")
    P = MixtureTreePath(N, K, L, V, B, with_logp=True, modes=modes)
    Q = MixtureTreePath(N, K, L, V, B, with_logp=True)
    P.build(x.cuda(), anchor, pos)
    Q.build(x.cuda(), anchor, pos)
    torch.cuda.synchronize()
    want_status = [M.MFD_TREE_BAD_MODES if m != c else 0 for m, c in zip(modes_h, kn)]
    assert P.buf.status.cpu().tolist() == want_status
    assert Q.buf.status.eq(0).all()
    for n in range(N):
        say(f"[modes] tree {n}: K_n={modes_h[n]} -> {kn[n]}")
        x64 = x[n, :kn[n]].double().numpy()
        check_lsm(x[n:n + 1, :kn[n]], P.buf.lse[n:n + 1, :kn[n]], P.buf.topk_id[n:n + 1, :kn[n]],
                  P.buf.topk_raw[n:n + 1, :kn[n]], P.k, P.buf.topk_logp[n:n + 1, :kn[n]])
        g = tree_rows(P, n)
        assert np.all(g["per_mode_kept"][kn[n]:] == 0)
        g["per_mode_kept"] = g["per_mode_kept"][:kn[n]]
        compare_tree(x64, B, n + 3, g)
        if kn[n] == K:
            for f in ("lse", "topk_id", "topk_raw", "cutoff", "n_select", "per_mode_kept", "node_token", "parent",
                      "depth", "score", "best_mode", "n_nodes", "mask_words", "position_ids"):
                assert torch.equal(getattr(P.buf, f)[n], getattr(Q.buf, f)[n]), f


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_tree_build_from_lower_cutoff(seed):
    """The build call alone, fed a cut-off well below the true one (so it
    materialises extra prefixes and must pick the first n_select by the total
    order), gives the oracle's tree."""
    x = _small_tree_case(seed, 3, 5, 30, 40, ints=(seed % 2 == 1))
    x64 = x[0].double().numpy()
    sel = O.mixture_select_heap(x64, 40, band=1e-4)
    P = MixtureTreePath(1, 3, 5, 30, 40)
    P.logsoftmax_topk(x.cuda())
    P.buf.cutoff.fill_(sel.cutoff - 0.75)
    P.buf.n_select.fill_(sel.n_select)
    P.tree_build(torch.tensor([3], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert P.buf.status.item() == 0
    g = tree_rows(P, 0)
    g["cutoff"] = sel.cutoff
    g.pop("per_mode_kept")
    r = compare_tree(x64, 40, 3, g, sel=sel)
    say(f"[build-only] seed={seed} exact={r['exact']}")


def test_walk_parity_small():
    """Walk kernel vs oracle walk on oracle trees, T = 0 and T > 0, fp32 and bf16 rows."""
    rng = np.random.default_rng(3)
    for dt in (torch.float32, torch.bfloat16):
        trees, Rs = [], []
        K, L, V, B = 2, 5, 33, 24
        for t in range(6):
            x = rng.normal(0, 2, size=(K, L, V))
            sel = O.mixture_select_heap(x, B)
            tr = O.canonical_tree(sel, 1, B)
            trees.append(tr)
            R = rng.normal(0, 1, size=(B + 1, V))
            # follow the first drafted path for a while so walks go deep
            for i in range(tr["n_nodes"]):
                kids = [j for j in range(1, tr["n_nodes"]) if tr["parent"][j] == i]
                if kids:
                    R[i, tr["node_token"][kids[0]]] += 6.0
            Rs.append(R)
        Rt = torch.tensor(np.stack(Rs)).to(dt)
        R64 = Rt.double().numpy()
        tok, par, dep, nn = upload_tree(trees, B + 1)
        N = len(trees)
        temps = torch.tensor([0.0, 1.0, 0.5, 2.0, 0.0, 1.0], dtype=torch.float32, device="cuda")
        seeds = torch.tensor([11, 12, 13, 2 ** 62 + 5, 15, -7], dtype=torch.int64, device="cuda")
        for ws in (M.walk_workspace(N), M.walk_workspace(N, Bp1=B + 1, V=V)):  # row by row, then speculative
            tau = torch.empty(N, dtype=torch.int32, device="cuda")
            ot = torch.empty((N, L + 1), dtype=torch.int32, device="cuda")
            pn = torch.empty((N, L + 1), dtype=torch.int32, device="cuda")
            st = torch.zeros(N, dtype=torch.int32, device="cuda")
            M.mfd_verify_walk(Rt.cuda(), L, tok, par, dep, nn, temps, seeds, tau, ot, pn, st, ws=ws)
            torch.cuda.synchronize()
            assert st.eq(0).all()
            for n in range(N):
                seed_u64 = int(seeds[n].item()) & ((1 << 64) - 1)
                check_walk(trees[n], R64[n], float(temps[n].item()), seed_u64, L, tau[n].item(),
                           ot[n].cpu().numpy(), pn[n].cpu().numpy())


def test_walk_near_tie_exact():
    """Two tokens whose perturbed values differ by 3e-5 (built from the oracle's
    own noise): too close for the fp32 noise estimate, so the kernel must take
    the exact fp64 round, and must agree with the oracle on the winner."""
    V, Bp1, L = 20000, 8, 3
    temps = [1.0, 1.0, 0.5, 2.0]
    seeds = [101, 2 ** 63 + 3, 77, 5]
    deltas = [3e-5, -3e-5, 3e-5, -3e-5]
    trees, Rs = [], []
    for T, sd, dl in zip(temps, seeds, deltas):
        g = O.gumbel_noise(sd, 0, V)
        R = np.full((Bp1, V), -1000.0)
        a, b = 100, V - 50
        R[0, a] = T * (20.0 - g[a])
        R[0, b] = T * (20.0 - g[b] + dl)
        Rs.append(R)
        tr = {"node_token": np.full(Bp1, -1, dtype=np.int64), "parent": np.full(Bp1, -1, dtype=np.int64),
              "depth": np.full(Bp1, -1, dtype=np.int64), "n_nodes": 1}
        tr["node_token"][0] = 7
        tr["depth"][0] = 0
        trees.append(tr)
    Rt = torch.tensor(np.stack(Rs), dtype=torch.float32)
    R64 = Rt.double().numpy()
    tok, par, dep, nn = upload_tree(trees, Bp1)
    N = len(trees)
    tt = torch.tensor(temps, dtype=torch.float32, device="cuda")
    sd_t = torch.tensor([s if s < 2 ** 63 else s - 2 ** 64 for s in seeds], dtype=torch.int64, device="cuda")
    for ws in (M.walk_workspace(N), M.walk_workspace(N, Bp1=Bp1, V=V)):  # row by row, then speculative
        tau = torch.empty(N, dtype=torch.int32, device="cuda")
        ot = torch.empty((N, L + 1), dtype=torch.int32, device="cuda")
        pn = torch.empty((N, L + 1), dtype=torch.int32, device="cuda")
        st = torch.zeros(N, dtype=torch.int32, device="cuda")
        M.mfd_verify_walk(Rt.cuda(), L, tok, par, dep, nn, tt, sd_t, tau, ot, pn, st, ws=ws)
        torch.cuda.synchronize()
        assert st.eq(0).all()
        for n in range(N):
            assert check_walk(trees[n], R64[n], temps[n], seeds[n], L, tau[n].item(), ot[n].cpu().numpy(),
                              pn[n].cpu().numpy())
            assert int(ot[n, 0].item()) == (V - 50 if deltas[n] > 0 else 100)


def test_walk_bad_temperature():
    x = _small_tree_case(31, 2, 3, 16, 8)
    P = MixtureTreePath(2, 2, 3, 16, 8)
    xx = torch.cat([x, x]).cuda()
    P.build(xx, torch.tensor([1, 2], dtype=torch.int32, device="cuda"), torch.zeros(2, dtype=torch.int64, device="cuda"))
    R = torch.randn((2, 9, 16), device="cuda")
    P.verify_walk(R, torch.tensor([-1.0, float("nan")], device="cuda"), torch.tensor([1, 2], device="cuda"))
    torch.cuda.synchronize()
    assert P.buf.status.cpu().tolist() == [M.MFD_TREE_BAD_TEMPERATURE] * 2
    assert P.buf.tau.cpu().tolist() == [0, 0]
    assert (P.buf.out_tokens == -1).all()


# ------------------------------------------------------------------ the workloads end to end

def _run_workload(name, N=None, device_gen="cpu"):
    """Every tree of a workload: logits pass, tree, keeps, mask and walk against
    the oracle, the per-tree oracle work spread over a pool of processes."""
    w = synth.WORKLOADS[name]
    b = synth.draft_batch(name, device=device_gen, N=N)
    N = b.logits.shape[0]
    logits = b.logits.cuda()
    vmap = None if b.vocab_map is None else b.vocab_map.cuda()
    modes = None if b.modes is None else b.modes.cuda()
    P = MixtureTreePath(N, w.K, w.L, logits.shape[-1], w.B, with_logp=True, vocab_map=vmap, V_full=w.V,
                        modes=modes)
    if modes is not None:
        # rows of inactive modes must come back untouched
        for t, v in ((P.buf.lse, -123.5), (P.buf.topk_id, -7), (P.buf.topk_raw, -5.25), (P.buf.topk_logp, -9.5)):
            t.fill_(v)
    anchor, pos = b.anchor.cuda(), b.pos_base.cuda()
    say(f"[{name}] build N={N}")
    P.build(logits, anchor, pos)
    torch.cuda.synchronize()
    assert P.buf.status.eq(0).all(), P.buf.status
    Bp1 = w.B + 1
    kn = [w.K if b.modes is None else int(b.modes[n]) for n in range(N)]
    for n in range(N):
        if kn[n] < w.K:
            assert torch.all(P.buf.lse[n, kn[n]:] == -123.5) and torch.all(P.buf.topk_id[n, kn[n]:] == -7)
            assert torch.all(P.buf.topk_raw[n, kn[n]:] == -5.25) and torch.all(P.buf.topk_logp[n, kn[n]:] == -9.5)
            assert torch.all(P.buf.per_mode_kept[n, kn[n]:] == 0)
    need = logits.numel() * logits.element_size() + N * Bp1 * w.V * 4
    with Spill(need) as sp:
        lpath, ltag, lshape = sp.dump("logits", b.logits)
        host = {f: getattr(P.buf, f).cpu().numpy() for f in (
            "lse", "topk_id", "topk_raw", "topk_logp", "n_select", "cutoff", "n_nodes", "node_token", "parent",
            "depth", "score", "best_mode", "per_mode_kept", "mask_words", "position_ids")}
        vm = None if b.vocab_map is None else b.vocab_map.cpu().numpy().astype(np.int64)
        jobs = []
        for n in range(N):
            K_ = kn[n]
            g = {"n_select": int(host["n_select"][n]), "cutoff": float(host["cutoff"][n]),
                 "n_nodes": int(host["n_nodes"][n]),
                 "per_mode_kept": host["per_mode_kept"][n][:K_]}
            for f in ("node_token", "parent", "depth", "best_mode"):
                g[f] = host[f][n].astype(np.int64)
            g["score"] = host["score"][n]
            jobs.append({"n": n, "path": lpath, "dtype": ltag, "shape": lshape, "Kn": K_, "B": w.B, "k": P.k,
                         "vocab_map": vm, "V_full": w.V, "anchor": int(b.anchor[n]),
                         "pos_base": int(b.pos_base[n]), "lse": host["lse"][n][:K_],
                         "topk_id": host["topk_id"][n][:K_], "topk_raw": host["topk_raw"][n][:K_],
                         "topk_logp": host["topk_logp"][n][:K_], "tree": g,
                         "mask_words": host["mask_words"][n], "position_ids": host["position_ids"][n]})
        res = sorted(run_pool(tree_job, jobs), key=lambda r: r["n"])
        bad = [r["error"] for r in res if not r["ok"]]
        assert not bad, bad[:3]
        excluded = [r["n"] for r in res if not r["exact"]]
        say(f"[{name}] {N} trees valid; {N - len(excluded)} exact, {len(excluded)} outside exactness "
            f"(cut-off band not decided by exact comparisons): {excluded}")
        trees = {r["n"]: r for r in res}
        # target rows from the oracle trees' depths; the walk kernel on the
        # oracle trees (all N) and on the built trees
        dep = torch.tensor(np.stack([trees[n]["depth"] for n in range(N)]), dtype=torch.int32)
        nn = torch.tensor([trees[n]["n_nodes"] for n in range(N)], dtype=torch.int32)
        R = synth.target_logits(b, dep, nn, device=device_gen)
        temps = b.temperature.cuda()
        seeds = b.seed.cuda()
        Rg = R.cuda()
        P.verify_walk(Rg, temps, seeds)
        tok, par, dp, nnn = upload_tree([trees[n] for n in range(N)], Bp1)
        tau = torch.empty(N, dtype=torch.int32, device="cuda")
        ot = torch.empty((N, w.L + 1), dtype=torch.int32, device="cuda")
        pn = torch.empty_like(ot)
        M.mfd_verify_walk(Rg, w.L, tok, par, dp, nnn, temps, seeds, tau, ot, pn,
                          ws=M.walk_workspace(N, Bp1=Bp1, V=w.V))  # with the speculative pass's arrays
        torch.cuda.synchronize()
        del Rg
        rpath, rtag, rshape = sp.dump("target", R)
        del R
        tau_h, ot_h, pn_h = tau.cpu().numpy(), ot.cpu().numpy(), pn.cpu().numpy()
        wjobs = [{"n": n, "path": rpath, "dtype": rtag, "shape": rshape, "T": float(b.temperature[n]),
                  "seed": int(b.seed[n]) & ((1 << 64) - 1), "L": w.L,
                  "tree": {f: trees[n][f] for f in ("node_token", "parent", "depth", "n_nodes")},
                  "tau": int(tau_h[n]), "toks": ot_h[n], "path_nodes": pn_h[n]} for n in range(N)]
        wres = sorted(run_pool(walk_job, wjobs), key=lambda r: r["n"])
        bad = [r["error"] for r in wres if not r["ok"]]
        assert not bad, bad[:3]
        near = [r["n"] for r in wres if not r["same"]]
        p_tau, p_ot = P.buf.tau.cpu().numpy(), P.buf.out_tokens.cpu().numpy()
        for n in range(N):
            if trees[n]["exact"]:
                assert p_tau[n] == tau_h[n] and np.array_equal(p_ot[n], ot_h[n]), n
        say(f"[{name}] {N} walks equal the oracle's (ulp-level near ties reported: {near}); "
            f"mean tau {float(tau_h.mean()):.2f}")
    return b, P, trees


def test_workload_tiny():
    b, P, trees = _run_workload("tiny")
    # brute force over all 2 * 16^4 full-length prefixes (and shorter ones)
    x64 = b.logits[0].double().numpy()
    assert set(O.mixture_select_bruteforce(x64, 8).selected) == set(trees[0]["prefixes"][1:])


def test_workload_product_chimeras():
    b, P, trees = _run_workload("product")
    A, Bf = b.futures[0, 0].tolist(), b.futures[0, 1].tolist()
    chims = O.chimera_nodes(trees[0]["prefixes"], A, Bf)
    assert len([c for c in chims if len(c) == max(synth.PRODUCT_SPLIT_POSITIONS) + 1]) >= 3


def test_workload_single():
    _run_workload("single")


@pytest.mark.timeout(600)
def test_workload_batched():
    """All 64 trees of the benchmarked batch."""
    _run_workload("batched", device_gen="cuda")


def test_workload_stress():
    _run_workload("stress")


def test_workload_deep():
    """Confident drafter: trees of full depth, walks of pages-like length."""
    b, P, trees = _run_workload("deep")
    assert max(int(trees[0]["depth"].max()), 0) == b.workload.L


@pytest.mark.timeout(600)
def test_workload_batched_deep():
    _run_workload("batched_deep", device_gen="cuda")


def test_workload_subset():
    """Drafting over a 65536-token subset, tree in full ids, walk over the full vocabulary."""
    _run_workload("subset")


@pytest.mark.timeout(600)
def test_workload_batched_subset():
    _run_workload("batched_subset", device_gen="cuda")


@pytest.mark.timeout(600)
def test_workload_batched_modes():
    """K_n = 8 and K_n = 1 trees in one launch; each against the oracle over its own
    first K_n modes (the K_n = 1 trees are single-future product trees)."""
    b, P, trees = _run_workload("batched_modes", device_gen="cuda")
    # a single-mode tree takes best_mode 0 everywhere
    for n in range(b.logits.shape[0]):
        if int(b.modes[n]) == 1:
            nn_ = int(P.buf.n_nodes[n])
            assert torch.all(P.buf.best_mode[n, 1:nn_] == 0)


def test_determinism_and_batch_order():
    """Same trees in another batch order give identical outputs."""
    b = synth.draft_batch("single", base_seed=5, N=3)
    w = b.workload
    outs = []
    for perm in ([0, 1, 2], [2, 0, 1]):
        P = MixtureTreePath(3, w.K, w.L, w.V, w.B)
        P.build(b.logits[perm].cuda(), b.anchor[perm].cuda(), b.pos_base[perm].cuda())
        torch.cuda.synchronize()
        inv = np.argsort(perm)
        outs.append([getattr(P.buf, f).cpu()[inv] for f in ("node_token", "parent", "depth", "score", "best_mode",
                                                               "cutoff", "n_select", "per_mode_kept", "mask_words")])
    for a, c in zip(*outs):
        assert torch.equal(a, c)


# ------------------------------------------------------------------ diagnostics (next row f3)

def _oracle_trees(name, N, seed):
    """Oracle trees, target rows and futures for N trees of workload `name`."""
    w = synth.WORKLOADS[name]
    b = synth.draft_batch(name, base_seed=seed, N=N)
    trees = [O.canonical_tree(O.mixture_select_heap(b.logits[n].double().numpy(), w.B), int(b.anchor[n]), w.B)
             for n in range(N)]
    dep = torch.stack([torch.from_numpy(t["depth"]).to(torch.int32) for t in trees])
    nn = torch.tensor([t["n_nodes"] for t in trees], dtype=torch.int32)
    R = synth.target_logits(b, dep, nn, base_seed=seed)
    return w, b, trees, R


@pytest.mark.parametrize("name,T,dtype", [("tiny", 0.0, torch.float32), ("tiny", 0.7, torch.float32),
                                          ("product", 1.0, torch.bfloat16), ("deep", 0.0, torch.bfloat16),
                                          ("deep", 1.0, torch.bfloat16), ("single", 1.0, torch.bfloat16)])
def test_covered_mass_parity(name, T, dtype):
    """Expected accepted tokens (covered target mass) against the oracle, per tree."""
    N = 2
    w, b, trees, R = _oracle_trees(name, N, seed=3)
    say(f"[mass] {name} T={T}")
    tok, par, dep, nn = upload_tree(trees, w.B + 1)
    Rg = R.to(dtype).cuda().contiguous()
    temps = torch.full((N,), T, dtype=torch.float32, device="cuda")
    mass = torch.empty(N, dtype=torch.float64, device="cuda")
    M.mfd_covered_mass(Rg, tok, par, nn, temps, mass)
    torch.cuda.synchronize()
    for n in range(N):
        want = O.covered_mass(trees[n]["node_token"], trees[n]["parent"], trees[n]["n_nodes"],
                              R[n].to(dtype).double().numpy(), T)
        got = mass[n].item()
        assert abs(got - want) <= 1e-6 * max(1.0, abs(want)), (n, got, want)
        if T == 0.0:
            tau, *_ = O.verify_walk(trees[n]["node_token"], trees[n]["parent"], trees[n]["depth"],
                                    trees[n]["n_nodes"], R[n].to(dtype).double().numpy(), 0.0, 0, w.L)
            assert got == tau - 1


def test_covered_mass_bad_temperature_and_nan_tree():
    w, b, trees, R = _oracle_trees("tiny", 2, seed=4)
    tok, par, dep, nn = upload_tree(trees, w.B + 1)
    par[1, 1] = w.B + 5  # a parent outside the tree
    temps = torch.tensor([-1.0, 1.0], dtype=torch.float32, device="cuda")
    mass = torch.empty(2, dtype=torch.float64, device="cuda")
    status = torch.zeros(2, dtype=torch.int32, device="cuda")
    M.mfd_covered_mass(R.cuda().contiguous(), tok, par, nn, temps, mass, status)
    torch.cuda.synchronize()
    assert math.isnan(mass[0].item()) and status[0].item() == M.MFD_TREE_BAD_TEMPERATURE
    assert math.isnan(mass[1].item()) and status[1].item() == 0


@pytest.mark.parametrize("name", ["product", "single", "tiny"])
def test_chimera_count_parity(name):
    """Chimeras relative to two futures against the oracle's list."""
    N = 2 if name != "product" else 1
    w, b, trees, R = _oracle_trees(name, N, seed=5)
    tok, par, dep, nn = upload_tree(trees, w.B + 1)
    fa = b.futures[:, 0].to(torch.int32).cuda().contiguous()
    fb = b.futures[:, 1].to(torch.int32).cuda().contiguous()
    count = torch.empty(N, dtype=torch.int32, device="cuda")
    M.mfd_chimera_count(tok, par, dep, nn, w.L, fa, fb, count)
    torch.cuda.synchronize()
    for n in range(N):
        want = len(O.chimera_nodes(trees[n]["prefixes"], b.futures[n, 0].tolist(), b.futures[n, 1].tolist()))
        assert count[n].item() == want, (n, count[n].item(), want)
    if name == "product":
        assert count[0].item() >= 3  # the 2^(m-1)-1 = 3 spliced prefixes at full split depth, at least


SWEEP = [
    # K, L, V, B, sigma (0: small integers, many ties); first-level children K * min(B, V)
    (8, 3, 600, 1200, 0.5),    # ~4800 children: past the register sorts (LDS network)
    (3, 5, 1000, 1000, 0.3),   # ~3000: register sort of 4096 keys (four per lane)
    (2, 4, 1000, 1000, 0.3),   # ~2000: register sort of 2048 keys (two per lane)
    (6, 4, 300, 700, 1.0),     # ~1800
    (4, 6, 100, 400, 0.0),     # ~400 with ties: one key per lane
    (2, 10, 64, 150, 2.0),     # deeper, small levels
    (8, 15, 2000, 256, 3.0),   # the specified mixture shape at a small vocabulary
]


@pytest.mark.parametrize("case", SWEEP, ids=[f"K{c[0]}L{c[1]}V{c[2]}B{c[3]}" for c in SWEEP])
def test_tree_sweep_level_sizes(case):
    """Batches of flat-logit trees whose search levels span every level-sort
    size (one key per lane up to past 4096 keys): each tree, mask and the
    per-mode keep counts against the oracle."""
    K, L, V, B, sigma = case
    N = 4
    say(f"[sweep] K={K} L={L} V={V} B={B} sigma={sigma}")
    xs = []
    for n in range(N):
        g = torch.Generator().manual_seed(1000 * K + 10 * L + n)
        if sigma == 0.0:
            xs.append(torch.randint(-2, 3, (1, K, L, V), generator=g).float())
        else:
            xs.append(torch.randn((1, K, L, V), generator=g) * sigma)
    x = torch.cat(xs)
    P = MixtureTreePath(N, K, L, V, B)
    anchor = torch.arange(N, dtype=torch.int32, device="cuda") + 11
    pos = torch.arange(N, dtype=torch.int64, device="cuda") * 64
    P.build(x.cuda(), anchor, pos)
    torch.cuda.synchronize()
    assert P.buf.status.eq(0).all()
    n_exact = 0
    for n in range(N):
        r = compare_tree(x[n].double().numpy(), B, n + 11, tree_rows(P, n))
        n_exact += int(r["exact"])
        g = tree_rows(P, n)
        check_mask(g["parent"], g["depth"], g["n_nodes"], n * 64, B + 1,
                   P.buf.mask_words[n].cpu().numpy(), P.buf.position_ids[n].cpu().numpy())
    # every tree was checked for validity; the exact ones also array for array
    say(f"[sweep] exact trees {n_exact}/{N}, the rest valid answers inside the cut-off band")


# ------------------------------------------------------------------ capacity paths

def _two_level_case(seed, K, distinct_parents, flat_second_row):
    """K modes, L = 2, V = 1000, B = 256 (fp32).  Row 1 of each mode: 64 tokens
    near 0, the rest near -20; row 2: N(0, 0.5^2), or all 0.0.  After level 1
    the running cut-off is the 256th depth-1 score (about -24), so every one of
    the 64 strong parents passes every one of its 256 second-row candidates:
    64 * 256 * K children, past the 2048-key level capacity."""
    g = torch.Generator().manual_seed(seed)
    V = 1000
    x = torch.full((1, K, 2, V), -20.0) + torch.randn((1, K, 2, V), generator=g)
    for m in range(K):
        hot = torch.randperm(V, generator=g)[:64]
        x[0, m, 0, hot] = 0.05 * torch.randn(64, generator=g) if distinct_parents else 0.0
        x[0, m, 1] = 0.0 if flat_second_row else 0.5 * torch.randn(V, generator=g)
    return x


@pytest.mark.parametrize("K", [1, 2])
def test_threshold_bisection_rescues_an_overflowing_level(K):
    """The threshold call raises its cut-off by bisection when a level would not
    fit, and still finds the oracle's tree."""
    x = _two_level_case(50 + K, K, distinct_parents=True, flat_second_row=False)
    say(f"[bisection] K={K}")
    P = MixtureTreePath(1, K, 2, 1000, 256, with_logp=True)
    caps = 2 * K * 256
    assert 64 * 256 * K > max(caps, 2048)
    anchor = torch.tensor([9], dtype=torch.int32, device="cuda")
    pos = torch.tensor([0], dtype=torch.int64, device="cuda")
    P.build(x.cuda(), anchor, pos)
    torch.cuda.synchronize()
    assert P.buf.status.item() == 0
    g = tree_rows(P, 0)
    r = compare_tree(x[0].double().numpy(), 256, 9, g)
    assert max(g["depth"]) == 2
    say(f"[bisection] K={K} exact={r['exact']} n_nodes={g['n_nodes']}")


def test_threshold_capacity_flag_gives_root_only_tree():
    """A level that cannot be cut below the capacity (16384 children tied at the
    cut-off) sets MFD_TREE_CAPACITY; the tree is the root alone, its mask the
    root's bit, and the walk still runs on it."""
    x = _two_level_case(60, 1, distinct_parents=False, flat_second_row=True)
    P = MixtureTreePath(1, 1, 2, 1000, 256)
    anchor = torch.tensor([4], dtype=torch.int32, device="cuda")
    pos = torch.tensor([10], dtype=torch.int64, device="cuda")
    P.build(x.cuda(), anchor, pos)
    torch.cuda.synchronize()
    assert P.buf.status.item() & M.MFD_TREE_CAPACITY
    assert P.buf.n_select.item() == 0 and math.isnan(P.buf.cutoff.item())
    assert P.buf.per_mode_kept.eq(0).all()
    Q = MixtureTreePath(1, 1, 2, 1000, 256)
    Q.build(x.cuda(), anchor, pos, fused=False)
    torch.cuda.synchronize()
    assert Q.buf.status.item() & M.MFD_TREE_CAPACITY
    assert torch.equal(Q.buf.node_token, P.buf.node_token) and torch.equal(Q.buf.n_nodes, P.buf.n_nodes)
    g = tree_rows(P, 0)
    assert g["n_nodes"] == 1 and g["node_token"][0] == 4 and g["parent"][0] == -1 and g["depth"][0] == 0
    assert np.all(g["node_token"][1:] == -1) and np.all(g["parent"][1:] == -1) and np.all(np.isneginf(g["score"][1:]))
    check_mask(g["parent"], g["depth"], 1, 10, 257, P.buf.mask_words[0].cpu().numpy(),
               P.buf.position_ids[0].cpu().numpy())
    R = torch.randn((1, 257, 1000), device="cuda")
    P.verify_walk(R, torch.tensor([0.0], device="cuda"), torch.tensor([3], device="cuda"))
    torch.cuda.synchronize()
    assert P.buf.tau.item() == 1
    assert P.buf.out_tokens[0, 0].item() == int(torch.argmax(R[0, 0]).item())


def test_walk_more_trees_than_one_launch():
    """2700 one- and two-node trees over rows of 65536 bf16 logits.  A launch
    takes at most two trees per resident workgroup (2048 or 2560 on this
    device), so the walk needs two launches, and in the first one every
    group of one workgroup serves two trees: one in five sampled at T = 1,
    the rest greedy, which exercises the sampled-first pairing of trees to
    groups.  Every tree against the oracle walk."""
    N, V, L, Bp1 = 2700, 65536, 1, 2
    say(f"[walk launches] N={N} V={V}")
    g = torch.Generator().manual_seed(77)
    child = torch.randint(0, V, (N,), generator=g)
    has_child = torch.rand(N, generator=g) < 0.8
    tok = torch.full((N, Bp1), -1, dtype=torch.int32)
    par = torch.full((N, Bp1), -1, dtype=torch.int32)
    dep = torch.full((N, Bp1), -1, dtype=torch.int32)
    tok[:, 0], dep[:, 0] = 5, 0
    tok[has_child, 1] = child[has_child].to(torch.int32)
    par[has_child, 1] = 0
    dep[has_child, 1] = 1
    nn = torch.where(has_child, 2, 1).to(torch.int32)
    gd = torch.Generator(device="cuda").manual_seed(78)
    R = torch.randn((N, Bp1, V), generator=gd, device="cuda")
    boost = (torch.rand(N, generator=g) < 0.7).cuda()
    idx = torch.arange(N, device="cuda")
    R[idx[boost], 0, child.cuda()[boost]] += 6.0
    R = R.to(torch.bfloat16)
    temps = torch.where(torch.arange(N) % 5 == 2, 1.0, 0.0).to(torch.float32).cuda()
    seeds = (torch.arange(N, dtype=torch.int64) * 7919 + 1).cuda()
    tau = torch.empty(N, dtype=torch.int32, device="cuda")
    ot = torch.empty((N, L + 1), dtype=torch.int32, device="cuda")
    pn = torch.empty_like(ot)
    st = torch.zeros(N, dtype=torch.int32, device="cuda")
    M.mfd_verify_walk(R, L, tok.cuda(), par.cuda(), dep.cuda(), nn.cuda(), temps, seeds, tau, ot, pn, st,
                      ws=M.walk_workspace(N))
    torch.cuda.synchronize()
    assert st.eq(0).all()
    tau_h, ot_h, pn_h = tau.cpu().numpy(), ot.cpu().numpy(), pn.cpu().numpy()
    Rc = R.cpu()
    deep = 0
    for n in range(N):
        tr = {"node_token": tok[n].numpy(), "parent": par[n].numpy(), "depth": dep[n].numpy(),
              "n_nodes": int(nn[n])}
        check_walk(tr, Rc[n].double().numpy(), float(temps[n]), int(seeds[n]), L, tau_h[n], ot_h[n], pn_h[n])
        deep += int(tau_h[n] == 2)
    say(f"[walk launches] {N} walks equal the oracle's, {deep} accepted the drafted token")
    assert deep > N // 3


# ------------------------------------------------------------------ one search for the cut-off and the tree

TREE_FIELDS = ("cutoff", "n_select", "per_mode_kept", "node_token", "parent", "depth", "score", "best_mode", "n_nodes",
               "mask_words", "position_ids", "status")


@pytest.mark.parametrize("name,N", [("batched", 64), ("batched_deep", 64), ("stress", 1), ("batched_modes", 64),
                                    ("batched_subset", 16), ("tiny", 1), ("product", 1)])
def test_fused_tree_equals_separate_calls(name, N):
    """mfd_mixture_tree (one launch) gives the outputs of mfd_mixture_threshold
    followed by mfd_tree_build, bit for bit."""
    say(f"[fused tree] {name} N={N}")
    w = synth.WORKLOADS[name]
    b = synth.draft_batch(name, device="cuda", N=N, base_seed=11)
    vmap = None if b.vocab_map is None else b.vocab_map.cuda()
    modes = None if b.modes is None else b.modes.cuda()
    out = []
    for fused in (True, False):
        P = MixtureTreePath(N, w.K, w.L, b.logits.shape[-1], w.B, vocab_map=vmap, V_full=w.V, modes=modes)
        P.build(b.logits.cuda(), b.anchor.cuda(), b.pos_base.cuda(), fused=fused)
        torch.cuda.synchronize()
        out.append({f: getattr(P.buf, f).clone() for f in TREE_FIELDS})
    for f in TREE_FIELDS:
        assert torch.equal(out[0][f], out[1][f]), f
    assert out[0]["status"].eq(0).all()


@pytest.mark.parametrize("case", SMALL + [(12, 3, 4, 12, 25, True, 0.4)], ids=[f"s{c[0]}" for c in SMALL] + ["s12"])
def test_fused_tree_equals_separate_calls_small(case):
    seed, K, L, V, B, ints, neginf = case
    x = _small_tree_case(seed, K, L, V, B, ints, neginf).cuda()
    anchor = torch.tensor([7], dtype=torch.int32, device="cuda")
    pos = torch.tensor([100], dtype=torch.int64, device="cuda")
    out = []
    for fused in (True, False):
        P = MixtureTreePath(1, K, L, V, B)
        P.build(x, anchor, pos, fused=fused)
        torch.cuda.synchronize()
        out.append({f: getattr(P.buf, f).clone() for f in TREE_FIELDS})
    for f in TREE_FIELDS:
        assert torch.equal(out[0][f], out[1][f]), (f, out[0][f], out[1][f])


# ------------------------------------------------------------------ the walk's speculative pass

SPEC_CASES = [("tiny", 1), ("product", 1), ("single", 1), ("deep", 1), ("subset", 1), ("stress", 1),
              ("batched_deep", 2), ("batched_deep", 4), ("batched", 64), ("batched_deep", 64)]


@pytest.mark.parametrize("name,N", SPEC_CASES, ids=[f"{c[0]}-{c[1]}" for c in SPEC_CASES])
def test_walk_speculation_equals_row_by_row(name, N):
    """The walk with the speculative pass's workspace gives the row-by-row
    walk's outputs bit for bit (the pass may or may not run: its choice is a
    cost estimate; every route must give the same tokens)."""
    w = synth.WORKLOADS[name]
    b = synth.draft_batch(name, device="cuda", N=N, base_seed=21)
    vmap = None if b.vocab_map is None else b.vocab_map.cuda()
    modes = None if b.modes is None else b.modes.cuda()
    P = MixtureTreePath(N, w.K, w.L, b.logits.shape[-1], w.B, vocab_map=vmap, V_full=w.V, modes=modes)
    P.build(b.logits.cuda(), b.anchor.cuda(), b.pos_base.cuda())
    torch.cuda.synchronize()
    R = synth.target_logits(b, P.buf.depth, P.buf.n_nodes, device="cuda", base_seed=21).contiguous()
    outs = []
    for ws in (M.walk_workspace(N), M.walk_workspace(N, Bp1=w.B + 1, V=w.V)):
        tau = torch.full((N,), -9, dtype=torch.int32, device="cuda")
        ot = torch.full((N, w.L + 1), -9, dtype=torch.int32, device="cuda")
        pn = torch.full((N, w.L + 1), -9, dtype=torch.int32, device="cuda")
        st = torch.zeros(N, dtype=torch.int32, device="cuda")
        M.mfd_verify_walk(R, w.L, P.buf.node_token, P.buf.parent, P.buf.depth, P.buf.n_nodes, b.temperature.cuda(),
                          b.seed.cuda(), tau, ot, pn, st, ws=ws)
        torch.cuda.synchronize()
        assert st.eq(0).all()
        outs.append((tau.cpu(), ot.cpu(), pn.cpu()))
    for a_, b_ in zip(*outs):
        assert torch.equal(a_, b_)
    say(f"[walk speculation] {name} N={N}: equal, mean tau {outs[0][0].float().mean().item():.2f}")


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_walk_speculation_on_a_chain_tree(T):
    """A root with 1000 leaf children and one chain of depth 15 (N = 1, V =
    151936): the walk's rows are the chain's, so the speculative pass reduces
    the 15 rows of nodes that have a child and the walk ends at the leaf.
    Against the oracle walk and the row-by-row walk, with the target following
    the chain to its end, and leaving it half way."""
    V, L, Bp1 = 151936, 15, 1016
    g = torch.Generator().manual_seed(99)
    toks = torch.randperm(V, generator=g)[:Bp1 + L].tolist()
    tok = np.full(Bp1, -1, dtype=np.int64)
    par = np.full(Bp1, -1, dtype=np.int64)
    dep = np.full(Bp1, -1, dtype=np.int64)
    tok[0], dep[0] = 5, 0
    # rows 1..15: the chain (root -> c1 -> ... -> c15), rows 16..1015: leaves under the root
    for i in range(1, L + 1):
        tok[i], par[i], dep[i] = toks[i], i - 1, i
    for i in range(L + 1, Bp1):
        tok[i], par[i], dep[i] = toks[i], 0, 1
    tree = {"node_token": tok, "parent": par, "depth": dep, "n_nodes": Bp1}
    for leave_at in (L, 7):
        R = torch.randn((1, Bp1, V), generator=g)
        for i in range(0, L):
            if i < leave_at:
                R[0, i, tok[i + 1]] += 12.0
        Rb = R.to(torch.bfloat16)
        R64 = Rb[0].double().numpy()
        tt, pp, dd, nn = upload_tree([tree], Bp1)
        outs = []
        for ws in (M.walk_workspace(1), M.walk_workspace(1, Bp1=Bp1, V=V)):
            tau = torch.empty(1, dtype=torch.int32, device="cuda")
            ot = torch.empty((1, L + 1), dtype=torch.int32, device="cuda")
            pn = torch.empty_like(ot)
            st = torch.zeros(1, dtype=torch.int32, device="cuda")
            M.mfd_verify_walk(Rb.cuda(), L, tt, pp, dd, nn, torch.tensor([T], device="cuda"),
                              torch.tensor([31], dtype=torch.int64, device="cuda"), tau, ot, pn, st, ws=ws)
            torch.cuda.synchronize()
            assert st.item() == 0
            check_walk(tree, R64, T, 31, L, tau.item(), ot[0].cpu().numpy(), pn[0].cpu().numpy())
            outs.append((tau.cpu(), ot.cpu(), pn.cpu()))
        for a_, b_ in zip(*outs):
            assert torch.equal(a_, b_)
        say(f"[walk speculation chain] T={T} leave_at={leave_at}: tau {outs[0][0].item()}")
