"""GPU parity of the fused LM head + log-softmax/top-k call against the fp64 oracle.

Grid workloads have every fp32 partial sum exact, so the fused logits equal the
oracle's and ids, values and trees must match bit for bit.  Gaussian workloads
are compared through the rigorous fp32 summation bound of oracle.lmhead_abs_bound:
an id may differ from the oracle's only where the two logits lie within twice
the bound of each other."""

import sys

import numpy as np
import pytest
import torch

import oracle as O
from mixture_draft_tree_amd import synth
from tests.gpu_helpers import LSE_TOL, compare_tree, oracle_rows, tree_rows

pytestmark = pytest.mark.gpu

M = pytest.importorskip("mixture_draft_tree_amd.mfdtree", reason="libmfdtree.so not built")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(hidden, weight, k):
    N, K, L, D = hidden.shape
    d = "cuda"
    H = hidden.to(d).contiguous()
    W = weight if isinstance(weight, M.PackedHead) else weight.to(d).contiguous()
    lse = torch.empty((N, K, L), dtype=torch.float64, device=d)
    ids = torch.empty((N, K, L, k), dtype=torch.int32, device=d)
    raw = torch.empty((N, K, L, k), dtype=torch.float32, device=d)
    lp = torch.empty((N, K, L, k), dtype=torch.float32, device=d)
    st = torch.zeros((N,), dtype=torch.int32, device=d)
    M.mfd_lmhead_logsoftmax_topk(H, W, k, lse, ids, raw, lp, st)
    torch.cuda.synchronize()
    return lse.cpu().numpy(), ids.cpu().numpy(), raw.cpu().numpy(), lp.cpu().numpy(), st.cpu().numpy()


def _check_exact(x64, k, lse, ids, raw, lp):
    o_lse, o_ids = oracle_rows(x64, k)
    assert np.max(np.abs(lse - o_lse)) < LSE_TOL
    assert np.array_equal(ids, o_ids), "top-k ids differ"
    want = np.take_along_axis(x64, o_ids.astype(np.int64), axis=-1)
    assert np.array_equal(raw.astype(np.float64), want), "top-k logits differ"
    assert np.max(np.abs(lp.astype(np.float64) - (want - o_lse[..., None]))) < LSE_TOL


def _check_bounded(x64, eps, k, lse, ids, raw):
    """Rows of x64 [R, V] (exact logits), eps [R, V] (summation bound)."""
    for r in range(x64.shape[0]):
        x, e = x64[r], eps[r]
        g = ids[r].astype(np.int64)
        em = float(e.max())
        assert len(set(g.tolist())) == k and g.min() >= 0 and g.max() < x.shape[0]
        assert np.all(np.abs(raw[r].astype(np.float64) - x[g]) <= e[g]), "logit outside the fp32 bound"
        order = O.rank_order(x, k)
        xk = x[order[-1]]
        must = np.nonzero(x > xk + 2 * em)[0]
        assert np.all(np.isin(must, g)), "a clear top-k token is missing"
        assert np.all(x[g] >= xk - 2 * em), "a clearly outside token was listed"
        assert np.all(x[g[:-1]] >= x[g[1:]] - 2 * em), "listed out of order beyond the bound"
        same = np.abs(x[g] - x[order]) <= 2 * em
        assert np.all(same | (g == order))
        assert abs(lse[r] - O.lse_rows(x)) < LSE_TOL + em


@pytest.mark.parametrize("name", ["lmhead_small", "lmhead_mid", "lmhead_wide", "lmhead_tall"])
def test_lmhead_grid_bit_exact(name):
    _say(f"lmhead grid parity {name}")
    b = synth.lmhead_batch(name)
    w = b.workload
    k = min(w.B, w.V)
    lse, ids, raw, lp, st = _run(b.hidden, b.weight, k)
    assert np.all(st == 0)
    x64 = O.lmhead_logits(b.hidden.float().numpy(), b.weight.float().numpy())
    _check_exact(x64, k, lse, ids, raw, lp)


def test_lmhead_gaussian_within_bound():
    _say("lmhead gaussian parity lmhead_ragged")
    b = synth.lmhead_batch("lmhead_ragged")
    w = b.workload
    k = min(w.B, w.V)
    lse, ids, raw, lp, st = _run(b.hidden, b.weight, k)
    assert np.all(st == 0)
    h, W = b.hidden.float().numpy(), b.weight.float().numpy()
    x64 = O.lmhead_logits(h, W).reshape(-1, w.V)
    eps = O.lmhead_abs_bound(h, W).reshape(-1, w.V)
    _check_bounded(x64, eps, k, lse.reshape(-1), ids.reshape(-1, k), raw.reshape(-1, k))


@pytest.mark.parametrize("k", [1, 7, 100])
def test_lmhead_grid_other_k(k):
    _say(f"lmhead grid parity lmhead_small k={k}")
    b = synth.lmhead_batch("lmhead_small")
    lse, ids, raw, lp, st = _run(b.hidden, b.weight, k)
    assert np.all(st == 0)
    x64 = O.lmhead_logits(b.hidden.float().numpy(), b.weight.float().numpy())
    _check_exact(x64, k, lse, ids, raw, lp)


@pytest.mark.parametrize("name", ["lmhead_small", "lmhead_mid", "lmhead_wide"])
def test_lmhead_tree_equals_oracle_tree(name):
    # The tree built from the fused outputs equals the oracle's tree over the
    # exact logits (grid inputs).
    from mixture_draft_tree_amd.pipeline import MixtureTreePath
    _say(f"lmhead tree parity {name}")
    b = synth.lmhead_batch(name)
    w = b.workload
    P = MixtureTreePath(w.N, w.K, w.L, w.V, w.B)
    anchor = b.anchor.cuda()
    pos = torch.arange(w.N, dtype=torch.int64, device="cuda") * 100
    P.build_from_hidden(b.hidden.cuda(), b.weight.cuda(), anchor, pos)
    torch.cuda.synchronize()
    assert int(P.buf.status.abs().sum().item()) == 0
    x64 = O.lmhead_logits(b.hidden.float().numpy(), b.weight.float().numpy())
    # every tree is checked for validity, the exact ones also array for array
    n_exact = 0
    for n in range(w.N):
        res = compare_tree(x64[n], w.B, int(b.anchor[n]), tree_rows(P, n))
        n_exact += int(res["exact"])
    _say(f"lmhead tree parity {name}: {n_exact}/{w.N} exact, the rest valid inside the cut-off band")


def test_lmhead_full_size_sampled_rows():
    # The drafter's shape (K=8, L=15, V=151936, D=2560, k=256): one tree with
    # grid inputs bit-exact on sampled rows, one tree and the 64-tree batch
    # (256-column tiles) with Gaussian inputs within the bound.
    for name in ("lmhead_single_grid", "lmhead_single", "lmhead_batched"):
        _say(f"lmhead full-size sampled rows {name}")
        b = synth.lmhead_batch(name)
        w = b.workload
        k = min(w.B, w.V)
        lse, ids, raw, lp, st = _run(b.hidden, b.weight, k)
        assert np.all(st == 0)
        h = b.hidden.float().numpy().reshape(-1, w.D)
        W = b.weight.float().numpy()
        rows = [0, 1, 14, 15, 59, 60, 100, 119] if w.N == 1 else [0, 127, 128, 3001, 7679]
        x64 = O.lmhead_logits(h[rows], W)
        if w.grid:
            _check_exact(x64, k, lse.reshape(-1)[rows], ids.reshape(-1, k)[rows], raw.reshape(-1, k)[rows],
                         lp.reshape(-1, k)[rows])
        else:
            eps = O.lmhead_abs_bound(h[rows], W)
            _check_bounded(x64, eps, k, lse.reshape(-1)[rows], ids.reshape(-1, k)[rows], raw.reshape(-1, k)[rows])


def test_lmhead_capacity_and_nonfinite_flags():
    _say("lmhead flags lmhead_mid")
    b = synth.lmhead_batch("lmhead_mid")
    w = b.workload
    k = min(w.B, w.V)
    # tree 0: every logit 0 (all tie) -> more candidates than the workspace holds
    # tree 1: a NaN hidden value -> non-finite logits
    H = b.hidden.clone()
    H[0] = 0
    H[1, 3, 2, 5] = float("nan")
    lse, ids, raw, lp, st = _run(H, b.weight, k)
    assert st[0] == M.MFD_TREE_CAPACITY
    assert st[1] & M.MFD_TREE_NONFINITE
    assert np.all(ids[0] == -1) and np.all(np.isneginf(raw[0]))
    assert np.max(np.abs(lse[0] - np.log(w.V))) < LSE_TOL


def test_lmhead_flags_few_rows():
    """The same flags on the path for at most 128 rows (one workgroup per CU,
    head streamed through LDS rings): tree 0 all-equal logits overflow the
    candidate list, tree 1 holds NaN logits, tree 2 stays exact."""
    _say("lmhead flags few rows")
    N, K, L, D, V, k = 3, 3, 5, 64, 20000, 32
    h, w = _grid_inputs(N, K, L, D, V, seed=11)
    h[0] = 0
    h[1, 2, 3, 7] = float("nan")
    lse, ids, raw, lp, st = _run(h, w, k)
    assert st[0] == M.MFD_TREE_CAPACITY
    assert st[1] & M.MFD_TREE_NONFINITE
    assert st[2] == 0
    assert np.all(ids[0] == -1) and np.all(np.isneginf(raw[0]))
    assert np.max(np.abs(lse[0] - np.log(V))) < LSE_TOL
    x64 = O.lmhead_logits(h[2:3].float().numpy(), w.float().numpy())
    _check_exact(x64, k, lse[2:3], ids[2:3], raw[2:3], lp[2:3])


def _grid_inputs(N, K, L, D, V, seed):
    g = torch.Generator().manual_seed(seed)
    h = torch.randint(-4, 5, (N, K, L, D), generator=g).to(torch.float32) * 0.25
    w = torch.randint(-8, 9, (V, D), generator=g).to(torch.float32) * 2.0 ** -5
    return h.to(torch.bfloat16), w.to(torch.bfloat16)


@pytest.mark.parametrize("N,K,L,D,V,k", [
    (1, 1, 1, 64, 16, 16),      # one row in a 128-row tile, one partial vocabulary tile, k = V
    (2, 3, 2, 64, 300, 256),    # fewer sample groups than k: every column is a candidate
    (1, 2, 3, 128, 1000, 1000), # k = V: the whole row, ranked
    (5, 1, 30, 64, 2049, 5),    # 150 rows over two row tiles, V one past a tile multiple
    (1, 4, 4, 2560, 8192, 2048),  # the largest k, full drafter width
])
def test_lmhead_grid_edge_shapes(N, K, L, D, V, k):
    _say(f"lmhead grid edge N={N} K={K} L={L} D={D} V={V} k={k}")
    h, w = _grid_inputs(N, K, L, D, V, seed=N * 1000 + V)
    lse, ids, raw, lp, st = _run(h, w, k)
    assert np.all(st == 0)
    x64 = O.lmhead_logits(h.float().numpy(), w.float().numpy())
    _check_exact(x64, k, lse, ids, raw, lp)


def test_lmhead_repeat_calls_and_workspace_reuse():
    # The same workspace serves calls of different sizes in a row; results
    # do not depend on what an earlier call left in it.
    _say("lmhead workspace reuse")
    big_h, big_w = _grid_inputs(2, 2, 3, 128, 5000, seed=5)
    small_h, small_w = _grid_inputs(1, 2, 2, 64, 700, seed=6)
    k = 64
    ws = M.lmhead_workspace(2, 2, 3, 5000, k)
    outs = []
    for h, w in ((big_h, big_w), (small_h, small_w), (big_h, big_w)):
        N, K, L, D = h.shape
        H, W = h.cuda(), w.cuda()
        lse = torch.empty((N, K, L), dtype=torch.float64, device="cuda")
        ids = torch.empty((N, K, L, k), dtype=torch.int32, device="cuda")
        raw = torch.empty((N, K, L, k), dtype=torch.float32, device="cuda")
        st = torch.zeros((N,), dtype=torch.int32, device="cuda")
        M.mfd_lmhead_logsoftmax_topk(H, W, k, lse, ids, raw, None, st, ws=ws)
        torch.cuda.synchronize()
        assert int(st.abs().sum()) == 0
        x64 = O.lmhead_logits(h.float().numpy(), w.float().numpy())
        o_lse, o_ids = oracle_rows(x64, k)
        assert np.array_equal(ids.cpu().numpy(), o_ids)
        assert np.max(np.abs(lse.cpu().numpy() - o_lse)) < LSE_TOL
        outs.append(ids.cpu().numpy())
    assert np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("V_full,V_draft,k", [(40000, 9000, 256), (5000, 300, 32)])
def test_lmhead_mapped_subset_bit_exact(V_full, V_draft, k):
    # Drafting over a sorted subset of the vocabulary: the head's rows of the
    # subset, ids reported through the map; equal to the oracle's ranking of
    # the subset logits, relabelled (grid inputs, exact).
    _say(f"lmhead mapped subset V_full={V_full} V_draft={V_draft} k={k}")
    h, w_full = _grid_inputs(2, 8, 15, 128, V_full, seed=V_full + V_draft)
    g = torch.Generator().manual_seed(77)
    vmap = torch.sort(torch.randperm(V_full, generator=g)[:V_draft]).values.to(torch.int32)
    w = w_full[vmap.long()].contiguous()
    N, K, L, D = h.shape
    H, W, VM = h.cuda(), w.cuda(), vmap.cuda()
    lse = torch.empty((N, K, L), dtype=torch.float64, device="cuda")
    ids = torch.empty((N, K, L, k), dtype=torch.int32, device="cuda")
    raw = torch.empty((N, K, L, k), dtype=torch.float32, device="cuda")
    st = torch.zeros((N,), dtype=torch.int32, device="cuda")
    M.mfd_lmhead_logsoftmax_topk(H, W, k, lse, ids, raw, None, st, vocab_map=VM, V_full=V_full)
    torch.cuda.synchronize()
    assert int(st.abs().sum()) == 0
    x64 = O.lmhead_logits(h.float().numpy(), w.float().numpy())
    o_lse, o_ids = oracle_rows(x64, k)
    assert np.array_equal(ids.cpu().numpy(), vmap.numpy()[o_ids])
    assert np.array_equal(raw.cpu().numpy().astype(np.float64), np.take_along_axis(x64, o_ids.astype(np.int64), -1))
    assert np.max(np.abs(lse.cpu().numpy() - o_lse)) < LSE_TOL


def test_lmhead_pack_weight_layout():
    # The packer is a pure re-layout: unpacking on the CPU gives the head back,
    # padded rows are zero.
    _say("lmhead pack layout")
    _, w = _grid_inputs(1, 1, 1, 192, 1000, seed=3)
    pk = M.mfd_lmhead_pack_weight(w.cuda())
    torch.cuda.synchronize()
    V, D = w.shape
    Vp, nS = (V + 255) // 256 * 256, D // 32
    p = pk.buf.cpu().view(Vp // 64, nS, 64, 32)                 # [row block, k block, row, k]
    un = p.permute(0, 2, 1, 3).reshape(Vp, D)
    assert torch.equal(un[:V], w) and torch.all(un[V:] == 0)


@pytest.mark.parametrize("name", ["lmhead_small", "lmhead_ragged", "lmhead_wide", "lmhead_tall", "lmhead_single"])
def test_lmhead_packed_equals_rows(name):
    # Same operands in the same k order: the packed head gives bit-identical outputs.
    _say(f"lmhead packed vs rows {name}")
    b = synth.lmhead_batch(name)
    w = b.workload
    k = min(w.B, w.V)
    ref = _run(b.hidden, b.weight, k)
    pk = M.mfd_lmhead_pack_weight(b.weight.cuda())
    got = _run(b.hidden, pk, k)
    for r, g in zip(ref, got):
        assert np.array_equal(r, g)
