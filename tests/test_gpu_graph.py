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
