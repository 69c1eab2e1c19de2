"""mfd_verify_walk_noalloc (the walk on the library's built-in workspace)
against mfd_verify_walk (the walk on a caller's workspace): two calls in a
row on one GPU, the second with fewer trees and other seeds, each equal to
the workspace call bit for bit."""

import sys

import pytest
import torch

from mixture_draft_tree_amd import mfdtree as M
from mixture_draft_tree_amd import synth
from mixture_draft_tree_amd.pipeline import MixtureTreePath

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _trees(name, N, seed):
    w = synth.WORKLOADS[name]
    b = synth.draft_batch(name, base_seed=seed, device="cuda", N=N)
    P = MixtureTreePath(N, w.K, w.L, w.V, w.B)
    P.build(b.logits, b.anchor.cuda(), b.pos_base.cuda())
    torch.cuda.synchronize()
    assert P.buf.status.eq(0).all()
    R = synth.target_logits(b, P.buf.depth, P.buf.n_nodes, device="cuda", base_seed=seed).contiguous()
    temps = b.temperature.cuda()
    seeds = b.seed.cuda()
    return w, P, R, temps, seeds


def _walk_both(w, P, R, temps, seeds):
    N = R.shape[0]
    outs = []
    for noalloc in (False, True):
        tau = torch.full((N,), -9, dtype=torch.int32, device="cuda")
        ot = torch.full((N, w.L + 1), -9, dtype=torch.int32, device="cuda")
        pn = torch.full((N, w.L + 1), -9, dtype=torch.int32, device="cuda")
        st = torch.zeros(N, dtype=torch.int32, device="cuda")
        args = (R, w.L, P.buf.node_token, P.buf.parent, P.buf.depth, P.buf.n_nodes, temps, seeds, tau, ot, pn, st)
        if noalloc:
            M.mfd_verify_walk_noalloc(*args)
        else:
            M.mfd_verify_walk(*args, ws=M.walk_workspace(N))
        torch.cuda.synchronize()
        outs.append((tau.cpu(), ot.cpu(), pn.cpu(), st.cpu()))
    return outs


@pytest.mark.parametrize("first,second", [(("batched_deep", 24, 3), ("deep", 1, 4)),
                                          (("batched", 64, 5), ("batched_deep", 7, 6))])
def test_walk_noalloc_equals_workspace_walk(first, second):
    for name, N, seed in (first, second):
        _say(f"[noalloc walk] {name} N={N} seed={seed}")
        w, P, R, temps, seeds = _trees(name, N, seed)
        (t0, o0, p0, s0), (t1, o1, p1, s1) = _walk_both(w, P, R, temps, seeds)
        assert s0.eq(0).all() and s1.eq(0).all()
        assert torch.equal(t0, t1) and torch.equal(o0, o1) and torch.equal(p0, p1)
        assert t0.min().item() >= 1
        _say(f"[noalloc walk] {name} N={N}: equal, mean tau {t0.float().mean().item():.2f}")
        del P, R
        torch.cuda.empty_cache()


def test_walk_noalloc_rejects_more_trees_than_it_holds():
    N = M.walk_noalloc_max_trees(1) + 1
    R = torch.zeros((N, 2, 8), dtype=torch.float32, device="cuda")
    z = lambda *s: torch.zeros(s, dtype=torch.int32, device="cuda")
    with pytest.raises(M.MfdError) as e:
        M.mfd_verify_walk_noalloc(R, 1, z(N, 2), z(N, 2), z(N, 2), z(N), torch.zeros(N, device="cuda"),
                                  torch.zeros(N, dtype=torch.int64, device="cuda"), z(N), z(N, 2), z(N, 2))
    assert e.value.code == M.MFD_ERR_WORKSPACE
