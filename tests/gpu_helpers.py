"""Shared helpers for the GPU parity tests (HIP path vs fp64 oracle): the
numpy comparisons of parity_checks plus torch-side readers and uploaders."""

from __future__ import annotations

import os
import shutil
import tempfile

import numpy as np
import torch

import oracle as O  # noqa: F401  (re-exported for the tests)
from parity_checks import (BAND, LSE_TOL, SCORE_TOL, check_lsm_arrays, check_mask, check_valid_tree,  # noqa: F401
                           check_walk, compare_tree, oracle_rows, per_mode_band, run_pool, tree_job, walk_job)


def check_lsm(x_cpu: torch.Tensor, lse, topk_id, topk_raw, k, topk_logp=None):
    """Compare one [N, K, L, V] logits pass against the oracle."""
    return check_lsm_arrays(x_cpu.float().numpy(), lse.cpu().numpy(), topk_id.cpu().numpy(),
                            topk_raw.cpu().numpy(), k, None if topk_logp is None else topk_logp.cpu().numpy())


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


class Spill:
    """A scratch directory for memory maps that pool workers read (RAM-backed
    when /dev/shm has room), removed on exit."""

    def __init__(self, need_bytes: int):
        base = None
        try:
            st = os.statvfs("/dev/shm")
            if st.f_bavail * st.f_frsize > 2 * need_bytes:
                base = "/dev/shm"
        except OSError:
            pass
        self.dir = tempfile.mkdtemp(prefix="mfd_parity_", dir=base)

    def dump(self, name: str, t: torch.Tensor):
        """Writes a tensor's raw element bits (bf16 as uint16) and returns (path, dtype tag, shape)."""
        path = os.path.join(self.dir, name)
        if t.dtype == torch.bfloat16:
            tag, npdt = "bf16", np.uint16
        elif t.dtype == torch.float32:
            tag, npdt = "f32", np.float32
        else:
            raise TypeError(t.dtype)
        mm = np.memmap(path, mode="w+", dtype=npdt, shape=tuple(t.shape))
        rows = t.shape[0]
        step = max(1, rows // 16)
        for r0 in range(0, rows, step):
            c = t[r0:r0 + step].detach().cpu().contiguous()
            mm[r0:r0 + c.shape[0]] = (c.view(torch.int16).numpy().view(np.uint16) if tag == "bf16" else c.numpy())
        mm.flush()
        del mm
        return path, tag, tuple(t.shape)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        shutil.rmtree(self.dir, ignore_errors=True)
