"""The five libmfdtree calls in decoding-round order, with their buffers.

Allocation (torch device memory) and call order only; all compute is in the
library's kernels.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import mfdtree as M


@dataclasses.dataclass
class TreeBatch:
    """Output buffers of one batch of N trees."""
    lse: torch.Tensor
    topk_id: torch.Tensor
    topk_raw: torch.Tensor
    topk_logp: Optional[torch.Tensor]
    cutoff: torch.Tensor
    n_select: torch.Tensor
    per_mode_kept: torch.Tensor
    node_token: torch.Tensor
    parent: torch.Tensor
    depth: torch.Tensor
    score: torch.Tensor
    best_mode: torch.Tensor
    n_nodes: torch.Tensor
    mask_words: torch.Tensor
    position_ids: torch.Tensor
    dense_mask: Optional[torch.Tensor]
    tau: torch.Tensor
    out_tokens: torch.Tensor
    path_nodes: torch.Tensor
    status: torch.Tensor
    ws: torch.Tensor


class MixtureTreePath:
    """Buffers for N trees of shape (K, L, V, B) and the calls that fill them."""

    def __init__(self, N: int, K: int, L: int, V: int, B: int, device="cuda", k: Optional[int] = None,
                 with_logp: bool = False, with_dense_mask: bool = False,
                 vocab_map: Optional[torch.Tensor] = None, V_full: Optional[int] = None,
                 modes: Optional[torch.Tensor] = None):
        """V is the drafting vocabulary; with `vocab_map` ([V] int32, increasing ids in a
        vocabulary of V_full tokens) the tree is built in full-vocabulary ids.  With
        `modes` ([N] int32 on the GPU, values in [1, K]) tree n uses its first modes[n]
        futures; its contents may change between steps, its storage may not."""
        if modes is not None and vocab_map is not None:
            raise ValueError("per-tree mode counts and a drafting vocabulary map are separate calls")
        self.N, self.K, self.L, self.V, self.B = N, K, L, V, B
        self.vocab_map = vocab_map
        self.modes = modes
        self.V_full = V if V_full is None else V_full
        self.k = min(B, V) if k is None else k
        if self.k < 1:
            self.k = 1
        d = device
        k_ = self.k
        Bp1 = B + 1
        W = (Bp1 + 63) // 64
        ws_bytes = max(M.workspace_size(M.MFD_OP_MIXTURE_THRESHOLD, N, K, L, V, B),
                       M.workspace_size(M.MFD_OP_TREE_BUILD, N, K, L, V, B),
                       M.workspace_size(M.MFD_OP_VERIFY_WALK, N, K, L, self.V_full, B))  # the walk reads full rows
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=d)
        self.buf = TreeBatch(
            lse=e((N, K, L), torch.float64),
            topk_id=e((N, K, L, k_), torch.int32),
            topk_raw=e((N, K, L, k_), torch.float32),
            topk_logp=e((N, K, L, k_), torch.float32) if with_logp else None,
            cutoff=e((N,), torch.float64),
            n_select=e((N,), torch.int32),
            per_mode_kept=e((N, K), torch.int32),
            node_token=e((N, Bp1), torch.int32),
            parent=e((N, Bp1), torch.int32),
            depth=e((N, Bp1), torch.int32),
            score=e((N, Bp1), torch.float64),
            best_mode=e((N, Bp1), torch.int32),
            n_nodes=e((N,), torch.int32),
            mask_words=e((N, Bp1, W), torch.int64),
            position_ids=e((N, Bp1), torch.int64),
            dense_mask=e((N, Bp1, Bp1), torch.uint8) if with_dense_mask else None,
            tau=e((N,), torch.int32),
            out_tokens=e((N, L + 1), torch.int32),
            path_nodes=e((N, L + 1), torch.int32),
            status=torch.zeros((N,), dtype=torch.int32, device=d),
            ws=torch.empty(((max(ws_bytes, 8) + 7) // 8,), dtype=torch.int64, device=d),
        )

    def logsoftmax_topk(self, logits, stream=None):
        b = self.buf
        if self.vocab_map is not None:
            M.mfd_logsoftmax_topk_mapped(logits, self.vocab_map, self.V_full, self.k, b.lse, b.topk_id, b.topk_raw,
                                         b.topk_logp, b.status, stream=stream)
        elif self.modes is not None:
            M.mfd_logsoftmax_topk_modes(logits, self.modes, self.k, b.lse, b.topk_id, b.topk_raw, b.topk_logp,
                                        b.status, stream=stream)
        else:
            M.mfd_logsoftmax_topk(logits, self.k, b.lse, b.topk_id, b.topk_raw, b.topk_logp, b.status,
                                  stream=stream)

    def lmhead_logsoftmax_topk(self, hidden, weight, stream=None):
        """Call 1 fused with the LM head: hidden [N, K, L, D] bf16, weight [V, D] bf16 (the
        drafting tokens' rows when the path has a vocabulary map)."""
        b = self.buf
        if self.modes is not None:
            raise ValueError("the fused LM-head call covers trees of all K modes")
        if getattr(self, "_lmh_ws", None) is None:
            self._lmh_ws = M.lmhead_workspace(self.N, self.K, self.L, self.V, self.k, hidden.device)
        M.mfd_lmhead_logsoftmax_topk(hidden, weight, self.k, b.lse, b.topk_id, b.topk_raw, b.topk_logp, b.status,
                                     ws=self._lmh_ws, stream=stream, vocab_map=self.vocab_map, V_full=self.V_full)

    def build_from_hidden(self, hidden, weight, anchor, pos_base, stream=None):
        """Calls 1-4 with the fused LM head: hidden states -> tree, mask, position ids."""
        self.clear_status(stream)
        self.lmhead_logsoftmax_topk(hidden, weight, stream)
        self.mixture_tree(anchor, stream)
        self.tree_mask(pos_base, stream)

    def mixture_threshold(self, stream=None):
        b = self.buf
        M.mfd_mixture_threshold_modes(b.topk_id, b.topk_raw, b.lse, self.B, self.modes, b.cutoff, b.n_select,
                                      b.per_mode_kept, b.status, b.ws, stream=stream)

    def tree_build(self, anchor, stream=None):
        b = self.buf
        M.mfd_tree_build_modes(b.topk_id, b.topk_raw, b.lse, b.cutoff, b.n_select, anchor, self.B, self.modes,
                               b.node_token, b.parent, b.depth, b.score, b.best_mode, b.n_nodes, b.status, b.ws,
                               stream=stream)

    def mixture_tree(self, anchor, stream=None):
        """The cut-off and the tree from one search (calls 2 and 3 in one launch)."""
        b = self.buf
        M.mfd_mixture_tree(b.topk_id, b.topk_raw, b.lse, anchor, self.B, b.cutoff, b.n_select, b.per_mode_kept,
                           b.node_token, b.parent, b.depth, b.score, b.best_mode, b.n_nodes, b.status, b.ws,
                           stream=stream, modes=self.modes)

    def tree_mask(self, pos_base, stream=None):
        b = self.buf
        M.mfd_tree_mask(b.parent, b.depth, b.n_nodes, pos_base, b.mask_words, b.position_ids, b.dense_mask,
                        stream=stream)

    def verify_walk(self, target, temperature, seed, stream=None):
        b = self.buf
        M.mfd_verify_walk(target, self.L, b.node_token, b.parent, b.depth, b.n_nodes, temperature, seed, b.tau,
                          b.out_tokens, b.path_nodes, b.status, ws=b.ws, stream=stream)

    def clear_status(self, stream=None):
        """Zero the per-tree status flags (the kernels only OR flags in).  A fill
        kernel, not a memset, so that a captured step clears them on every replay."""
        if stream is None:
            self.buf.status.zero_()
        else:
            with torch.cuda.stream(stream):
                self.buf.status.zero_()

    def build(self, logits, anchor, pos_base, stream=None, fused=True):
        """Calls 1-4: logits -> tree, mask, position ids (status flags cleared
        first).  The cut-off and the tree come from one launch (mfd_mixture_tree),
        or with fused=False from the separate threshold and build calls."""
        self.clear_status(stream)
        self.logsoftmax_topk(logits, stream)
        if fused:
            self.mixture_tree(anchor, stream)
        else:
            self.mixture_threshold(stream)
            self.tree_build(anchor, stream)
        self.tree_mask(pos_base, stream)

    def step(self, logits, anchor, pos_base, target, temperature, seed, stream=None):
        """One whole pass of the path: logits pass, cut-off and tree, mask, walk."""
        self.build(logits, anchor, pos_base, stream)
        self.verify_walk(target, temperature, seed, stream)
