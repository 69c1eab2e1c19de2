"""The five calls of one step captured in a HIP graph: every replay gives the
eager results, with eager work and synchronisation between the replays."""

import sys

import pytest
import torch

pytestmark = pytest.mark.gpu


def test_step_graph_replays_equal_eager():
    import bench
    print("graph replay batched", flush=True)
    sys.stdout.flush()
    w, N, P, logits, anchor, pos, temps, seeds, R = bench.setup("batched", 0, "cuda")
    P.step(logits, anchor, pos, R, temps, seeds)
    torch.cuda.synchronize()
    keys = ("lse", "topk_id", "topk_raw", "cutoff", "n_select", "per_mode_kept", "node_token", "parent", "depth",
            "score", "best_mode", "n_nodes", "mask_words", "position_ids", "tau", "out_tokens", "path_nodes",
            "status")
    ref = {k: getattr(P.buf, k).clone() for k in keys}
    g = bench.capture_step(P, logits, anchor, pos, R, temps, seeds)
    for rep in range(4):
        for k in keys:
            getattr(P.buf, k).zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in keys:
            assert torch.equal(getattr(P.buf, k), ref[k]), (rep, k)
        # eager work on the same device between replays
        torch.randn(4096, device="cuda").sum().item()
        P.tree_mask(pos)
        torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["lmhead_small", "lmhead_wide"])
def test_fused_lmhead_graph_replays_equal_eager(name):
    # the fused call's four launches captured once; its per-row counters live
    # in the workspace and are reset by its own kernels on every replay
    from mixture_draft_tree_amd import mfdtree as M
    from mixture_draft_tree_amd import synth
    print(f"graph replay fused lm head {name}", flush=True)
    sys.stdout.flush()
    b = synth.lmhead_batch(name, device="cuda")
    w = b.workload
    N, K, L, V = w.N, w.K, w.L, w.V
    k = min(w.B, V)
    H, W = b.hidden.contiguous(), b.weight.contiguous()
    ws = M.lmhead_workspace(N, K, L, V, k)
    out = {
        "lse": torch.empty((N, K, L), dtype=torch.float64, device="cuda"),
        "ids": torch.empty((N, K, L, k), dtype=torch.int32, device="cuda"),
        "raw": torch.empty((N, K, L, k), dtype=torch.float32, device="cuda"),
        "logp": torch.empty((N, K, L, k), dtype=torch.float32, device="cuda"),
        "status": torch.zeros((N,), dtype=torch.int32, device="cuda"),
    }

    def call():
        M.mfd_lmhead_logsoftmax_topk(H, W, k, out["lse"], out["ids"], out["raw"], out["logp"], out["status"],
                                     ws=ws)

    call()
    torch.cuda.synchronize()
    assert int(out["status"].abs().sum()) == 0
    ref = {key: t.clone() for key, t in out.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up on the capturing stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in out.values():
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in out:
            assert torch.equal(out[key], ref[key]), (rep, key)
        # eager work on the same device between replays, the fused call included
        torch.randn(4096, device="cuda").sum().item()
        call()
        torch.cuda.synchronize()
