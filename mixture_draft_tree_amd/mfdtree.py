"""ctypes binding of libmfdtree (include/mfdtree.h).

Argument marshalling only: each function checks tensor dtypes, shapes and
devices, passes raw device pointers and the stream to the library, and raises
MfdError when the library rejects the call.  Every step of the path runs in the
library's HIP kernels; importing this module fails if the library is missing.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmfdtree.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing; build it with `python -m mixture_draft_tree_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

MFD_OK, MFD_ERR_INVALID_ARG, MFD_ERR_DTYPE, MFD_ERR_WORKSPACE, MFD_ERR_DEVICE = 0, 1, 2, 3, 4
MFD_BF16, MFD_F32 = 0, 1
(MFD_OP_LOGSOFTMAX_TOPK, MFD_OP_MIXTURE_THRESHOLD, MFD_OP_TREE_BUILD,
 MFD_OP_TREE_MASK, MFD_OP_VERIFY_WALK, MFD_OP_COVERED_MASS, MFD_OP_LMHEAD_TOPK, MFD_OP_MIXTURE_TREE) = range(8)
MFD_TREE_NONFINITE, MFD_TREE_CAPACITY, MFD_TREE_BAD_TEMPERATURE, MFD_TREE_BAD_MODES = 1, 2, 4, 8
MFD_HEAD_ROWS, MFD_HEAD_PACKED = 0, 1

EXPORTED = ["mfd_last_error", "mfd_version", "mfd_workspace_size", "mfd_logsoftmax_topk",
            "mfd_logsoftmax_topk_mapped", "mfd_mixture_threshold", "mfd_tree_build", "mfd_tree_mask",
            "mfd_verify_walk", "mfd_covered_mass", "mfd_chimera_count", "mfd_logsoftmax_topk_modes",
            "mfd_mixture_threshold_modes", "mfd_tree_build_modes", "mfd_stream_read",
            "mfd_lmhead_logsoftmax_topk", "mfd_lmhead_logsoftmax_topk_mapped",
            "mfd_lmhead_packed_size", "mfd_lmhead_pack_weight", "mfd_verify_walk_noalloc",
            "mfd_mixture_tree", "mfd_mixture_tree_modes"]

_p = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

_lib.mfd_last_error.restype = ctypes.c_char_p
_lib.mfd_last_error.argtypes = []
_lib.mfd_version.restype = ctypes.c_char_p
_lib.mfd_version.argtypes = []
_lib.mfd_workspace_size.restype = _i
_lib.mfd_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i, ctypes.POINTER(_sz)]
_lib.mfd_logsoftmax_topk.restype = _i
_lib.mfd_logsoftmax_topk.argtypes = [_p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _sz, _p]
_lib.mfd_logsoftmax_topk_mapped.restype = _i
_lib.mfd_logsoftmax_topk_mapped.argtypes = [_p, _i, _i, _i, _i, _i, _p, _i, _i, _p, _p, _p, _p, _p, _p]
_lib.mfd_mixture_threshold.restype = _i
_lib.mfd_mixture_threshold.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _sz, _p]
_lib.mfd_tree_build.restype = _i
_lib.mfd_tree_build.argtypes = [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i,
                                _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]
_lib.mfd_mixture_tree.restype = _i
_lib.mfd_mixture_tree.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                  _p, _sz, _p]
_lib.mfd_mixture_tree_modes.restype = _i
_lib.mfd_mixture_tree_modes.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                        _p, _p, _p, _sz, _p]
_lib.mfd_logsoftmax_topk_modes.restype = _i
_lib.mfd_logsoftmax_topk_modes.argtypes = [_p, _i, _i, _i, _i, _i, _p, _i, _p, _p, _p, _p, _p, _p]
_lib.mfd_mixture_threshold_modes.restype = _i
_lib.mfd_mixture_threshold_modes.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _sz, _p]
_lib.mfd_tree_build_modes.restype = _i
_lib.mfd_tree_build_modes.argtypes = [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p,
                                      _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]
_lib.mfd_lmhead_logsoftmax_topk.restype = _i
_lib.mfd_lmhead_logsoftmax_topk.argtypes = [_p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _sz, _p]
_lib.mfd_lmhead_packed_size.restype = _i
_lib.mfd_lmhead_packed_size.argtypes = [_i, _i, ctypes.POINTER(_sz)]
_lib.mfd_lmhead_pack_weight.restype = _i
_lib.mfd_lmhead_pack_weight.argtypes = [_p, _i, _i, _p, _sz, _p]
_lib.mfd_lmhead_logsoftmax_topk_mapped.restype = _i
_lib.mfd_lmhead_logsoftmax_topk_mapped.argtypes = [_p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p,
                                                   _p, _sz, _p]
_lib.mfd_stream_read.restype = _i
_lib.mfd_stream_read.argtypes = [_p, _sz, _p, _p]
_lib.mfd_tree_mask.restype = _i
_lib.mfd_tree_mask.argtypes = [_p, _p, _p, _p, _i, _i, _p, _p, _p, _p]
_lib.mfd_covered_mass.restype = _i
_lib.mfd_covered_mass.argtypes = [_p, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _sz, _p]
_lib.mfd_chimera_count.restype = _i
_lib.mfd_chimera_count.argtypes = [_p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p]
_lib.mfd_verify_walk.restype = _i
_lib.mfd_verify_walk.argtypes = [_p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]
_lib.mfd_verify_walk_noalloc.restype = _i
_lib.mfd_verify_walk_noalloc.argtypes = [_p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]


class MfdError(RuntimeError):
    def __init__(self, code: int, call: str):
        self.code = code
        msg = _lib.mfd_last_error().decode(errors="replace")
        super().__init__(f"{call} failed with status {code}: {msg}")


def _check(code: int, call: str) -> None:
    if code != MFD_OK:
        raise MfdError(code, call)


def version() -> str:
    return _lib.mfd_version().decode()


def last_error() -> str:
    return _lib.mfd_last_error().decode(errors="replace")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _want(t: Optional[torch.Tensor], name: str, dtype, shape, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MFD_BF16
    if t.dtype == torch.float32:
        return MFD_F32
    raise ValueError(f"unsupported logits dtype {t.dtype}")


def walk_workspace(N: int, device="cuda", Bp1: Optional[int] = None, V: Optional[int] = None,
                   L: int = 32) -> torch.Tensor:
    """A device workspace for mfd_verify_walk on N trees of draft length up to L.
    With the trees' row count Bp1 and the vocabulary V it also holds the
    speculative pass's arrays (without them the walk runs row after row; the
    results are the same)."""
    if Bp1 is None or V is None:
        n = workspace_size(MFD_OP_VERIFY_WALK, N, 1, L, 1, -1)
    else:
        n = workspace_size(MFD_OP_VERIFY_WALK, N, 1, L, V, Bp1 - 1)
    return torch.empty((max(n, 8) + 7) // 8, dtype=torch.int64, device=device)


def workspace_size(op: int, N: int, K: int, L: int, V: int, B: int) -> int:
    out = _sz(0)
    _check(_lib.mfd_workspace_size(op, N, K, L, V, B, ctypes.byref(out)), "mfd_workspace_size")
    return int(out.value)


def mfd_logsoftmax_topk(logits, k, lse, topk_id, topk_raw, topk_logp=None, status=None, stream=None):
    """logits [N, K, L, V] bf16/fp32 -> lse [N, K, L] fp64, topk_* [N, K, L, k]."""
    if logits.dim() != 4 or not logits.is_contiguous() or logits.device.type != "cuda":
        raise ValueError("logits must be a contiguous [N, K, L, V] GPU tensor")
    N, K, L, V = logits.shape
    _want(lse, "lse", torch.float64, (N, K, L))
    _want(topk_id, "topk_id", torch.int32, (N, K, L, k))
    _want(topk_raw, "topk_raw", torch.float32, (N, K, L, k))
    _want(topk_logp, "topk_logp", torch.float32, (N, K, L, k), optional=True)
    _want(status, "status", torch.int32, (N,), optional=True)
    _check(_lib.mfd_logsoftmax_topk(_ptr(logits), _dtype_code(logits), N, K, L, V, k, _ptr(lse), _ptr(topk_id),
                                    _ptr(topk_raw), _ptr(topk_logp), _ptr(status), None, 0,
                                    _stream_handle(stream)), "mfd_logsoftmax_topk")


def mfd_logsoftmax_topk_mapped(logits, vocab_map, V_full, k, lse, topk_id, topk_raw, topk_logp=None, status=None,
                               stream=None):
    """logits [N, K, L, V] over a drafting vocabulary; vocab_map [V] int32 (increasing
    full-vocabulary ids) -> lse [N, K, L] fp64, topk_* [N, K, L, k] with full ids."""
    if logits.dim() != 4 or not logits.is_contiguous() or logits.device.type != "cuda":
        raise ValueError("logits must be a contiguous [N, K, L, V] GPU tensor")
    N, K, L, V = logits.shape
    _want(vocab_map, "vocab_map", torch.int32, (V,))
    _want(lse, "lse", torch.float64, (N, K, L))
    _want(topk_id, "topk_id", torch.int32, (N, K, L, k))
    _want(topk_raw, "topk_raw", torch.float32, (N, K, L, k))
    _want(topk_logp, "topk_logp", torch.float32, (N, K, L, k), optional=True)
    _want(status, "status", torch.int32, (N,), optional=True)
    _check(_lib.mfd_logsoftmax_topk_mapped(_ptr(logits), _dtype_code(logits), N, K, L, V, _ptr(vocab_map), V_full, k,
                                           _ptr(lse), _ptr(topk_id), _ptr(topk_raw), _ptr(topk_logp), _ptr(status),
                                           _stream_handle(stream)), "mfd_logsoftmax_topk_mapped")


def mfd_logsoftmax_topk_modes(logits, modes, k, lse, topk_id, topk_raw, topk_logp=None, status=None, stream=None):
    """As mfd_logsoftmax_topk for the rows of modes m < modes[n] (modes: [N] int32 on
    the GPU); the other rows are neither read nor written."""
    if logits.dim() != 4 or not logits.is_contiguous() or logits.device.type != "cuda":
        raise ValueError("logits must be a contiguous [N, K, L, V] GPU tensor")
    N, K, L, V = logits.shape
    _want(modes, "modes", torch.int32, (N,))
    _want(lse, "lse", torch.float64, (N, K, L))
    _want(topk_id, "topk_id", torch.int32, (N, K, L, k))
    _want(topk_raw, "topk_raw", torch.float32, (N, K, L, k))
    _want(topk_logp, "topk_logp", torch.float32, (N, K, L, k), optional=True)
    _want(status, "status", torch.int32, (N,), optional=True)
    _check(_lib.mfd_logsoftmax_topk_modes(_ptr(logits), _dtype_code(logits), N, K, L, V, _ptr(modes), k, _ptr(lse),
                                          _ptr(topk_id), _ptr(topk_raw), _ptr(topk_logp), _ptr(status),
                                          _stream_handle(stream)), "mfd_logsoftmax_topk_modes")


def lmhead_workspace(N: int, K: int, L: int, V: int, k: int, device="cuda") -> torch.Tensor:
    """A device workspace (256-byte aligned) for mfd_lmhead_logsoftmax_topk."""
    n = workspace_size(MFD_OP_LMHEAD_TOPK, N, K, L, V, k)
    return torch.empty((max(n, 256) + 255) // 8, dtype=torch.int64, device=device)


class PackedHead:
    """An LM head re-laid out by mfd_lmhead_pack_weight (device buffer + its shape)."""

    def __init__(self, buf: torch.Tensor, V: int, D: int):
        self.buf, self.V, self.D = buf, V, D
        self.device = buf.device


def lmhead_packed_size(V: int, D: int) -> int:
    out = _sz(0)
    _check(_lib.mfd_lmhead_packed_size(V, D, ctypes.byref(out)), "mfd_lmhead_packed_size")
    return int(out.value)


def mfd_lmhead_pack_weight(weight, stream=None) -> PackedHead:
    """weight [V, D] bf16 on the GPU -> the packed head (allocated here, with torch)."""
    if weight.dim() != 2 or weight.dtype != torch.bfloat16 or not weight.is_contiguous() or weight.device.type != "cuda":
        raise ValueError("weight must be a contiguous [V, D] bf16 GPU tensor")
    V, D = weight.shape
    n = lmhead_packed_size(V, D)
    buf = torch.empty((n // 2,), dtype=torch.bfloat16, device=weight.device)
    _check(_lib.mfd_lmhead_pack_weight(_ptr(weight), V, D, _ptr(buf), n, _stream_handle(stream)),
           "mfd_lmhead_pack_weight")
    return PackedHead(buf, V, D)


def mfd_lmhead_logsoftmax_topk(hidden, weight, k, lse, topk_id, topk_raw, topk_logp=None, status=None, ws=None,
                               stream=None, vocab_map=None, V_full=None):
    """hidden [N, K, L, D] bf16, weight [V, D] bf16 -> lse [N, K, L] fp64, topk_* [N, K, L, k]
    over the logits hidden . weight^T (never stored).  With vocab_map ([V] int32,
    increasing ids in a vocabulary of V_full tokens; weight holds those tokens'
    rows) topk_id holds full-vocabulary ids."""
    if hidden.dim() != 4 or not hidden.is_contiguous() or hidden.device.type != "cuda":
        raise ValueError("hidden must be a contiguous [N, K, L, D] GPU tensor")
    if hidden.dtype != torch.bfloat16:
        raise ValueError(f"hidden must be bf16, got {hidden.dtype}")
    N, K, L, D = hidden.shape
    if isinstance(weight, PackedHead):
        if weight.D != D:
            raise ValueError(f"packed head has D = {weight.D}, hidden has {D}")
        V, layout, wptr = weight.V, MFD_HEAD_PACKED, _ptr(weight.buf)
    else:
        if weight.dim() != 2 or weight.shape[1] != D:
            raise ValueError(f"weight must be [V, {D}], got {tuple(weight.shape)}")
        V = weight.shape[0]
        _want(weight, "weight", torch.bfloat16, (V, D))
        layout, wptr = MFD_HEAD_ROWS, _ptr(weight)
    _want(lse, "lse", torch.float64, (N, K, L))
    _want(topk_id, "topk_id", torch.int32, (N, K, L, k))
    _want(topk_raw, "topk_raw", torch.float32, (N, K, L, k))
    _want(topk_logp, "topk_logp", torch.float32, (N, K, L, k), optional=True)
    _want(status, "status", torch.int32, (N,), optional=True)
    if ws is None:
        ws = lmhead_workspace(N, K, L, V, k, hidden.device)
    ptr = ws.data_ptr()
    off = (-ptr) % 256
    nbytes = ws.numel() * ws.element_size() - off
    if vocab_map is not None:
        _want(vocab_map, "vocab_map", torch.int32, (V,))
        _check(_lib.mfd_lmhead_logsoftmax_topk_mapped(
            _ptr(hidden), wptr, layout, _ptr(vocab_map), V if V_full is None else V_full, N, K, L, D, V, k,
            _ptr(lse), _ptr(topk_id), _ptr(topk_raw), _ptr(topk_logp), _ptr(status), ctypes.c_void_p(ptr + off),
            max(nbytes, 0), _stream_handle(stream)), "mfd_lmhead_logsoftmax_topk_mapped")
        return
    _check(_lib.mfd_lmhead_logsoftmax_topk(_ptr(hidden), wptr, layout, N, K, L, D, V, k, _ptr(lse), _ptr(topk_id),
                                           _ptr(topk_raw), _ptr(topk_logp), _ptr(status),
                                           ctypes.c_void_p(ptr + off), max(nbytes, 0), _stream_handle(stream)),
           "mfd_lmhead_logsoftmax_topk")


def mfd_mixture_threshold(topk_id, topk_raw, lse, B, cutoff, n_select, per_mode_kept=None, status=None,
                          ws=None, stream=None):
    mfd_mixture_threshold_modes(topk_id, topk_raw, lse, B, None, cutoff, n_select, per_mode_kept, status, ws, stream)


def mfd_mixture_threshold_modes(topk_id, topk_raw, lse, B, modes, cutoff, n_select, per_mode_kept=None, status=None,
                                ws=None, stream=None):
    """The common cut-off; with modes ([N] int32 on the GPU) tree n uses its first
    modes[n] futures (modes=None: the plain mfd_mixture_threshold call)."""
    N, K, L, k = topk_id.shape
    _want(topk_id, "topk_id", torch.int32, (N, K, L, k))
    _want(topk_raw, "topk_raw", torch.float32, (N, K, L, k))
    _want(lse, "lse", torch.float64, (N, K, L))
    _want(cutoff, "cutoff", torch.float64, (N,))
    _want(n_select, "n_select", torch.int32, (N,))
    _want(per_mode_kept, "per_mode_kept", torch.int32, (N, K), optional=True)
    _want(status, "status", torch.int32, (N,), optional=True)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    if modes is None:
        _check(_lib.mfd_mixture_threshold(_ptr(topk_id), _ptr(topk_raw), _ptr(lse), N, K, L, k, B, _ptr(cutoff),
                                          _ptr(n_select), _ptr(per_mode_kept), _ptr(status), _ptr(ws), ws_bytes,
                                          _stream_handle(stream)), "mfd_mixture_threshold")
        return
    _want(modes, "modes", torch.int32, (N,))
    _check(_lib.mfd_mixture_threshold_modes(_ptr(topk_id), _ptr(topk_raw), _ptr(lse), N, K, L, k, B, _ptr(modes),
                                            _ptr(cutoff), _ptr(n_select), _ptr(per_mode_kept), _ptr(status),
                                            _ptr(ws), ws_bytes, _stream_handle(stream)), "mfd_mixture_threshold_modes")


def mfd_tree_build(topk_id, topk_raw, lse, cutoff, n_select, anchor_token, B, node_token, parent, depth, score,
                   best_mode, n_nodes, status=None, ws=None, stream=None):
    mfd_tree_build_modes(topk_id, topk_raw, lse, cutoff, n_select, anchor_token, B, None, node_token, parent, depth,
                         score, best_mode, n_nodes, status, ws, stream)


def mfd_tree_build_modes(topk_id, topk_raw, lse, cutoff, n_select, anchor_token, B, modes, node_token, parent, depth,
                         score, best_mode, n_nodes, status=None, ws=None, stream=None):
    """The tree; with modes ([N] int32 on the GPU) tree n is built from its first
    modes[n] futures (modes=None: the plain mfd_tree_build call)."""
    N, K, L, k = topk_id.shape
    Bp1 = B + 1
    _want(topk_id, "topk_id", torch.int32, (N, K, L, k))
    _want(topk_raw, "topk_raw", torch.float32, (N, K, L, k))
    _want(lse, "lse", torch.float64, (N, K, L))
    _want(cutoff, "cutoff", torch.float64, (N,))
    _want(n_select, "n_select", torch.int32, (N,))
    _want(anchor_token, "anchor_token", torch.int32, (N,))
    for name, t, dt in (("node_token", node_token, torch.int32), ("parent", parent, torch.int32),
                        ("depth", depth, torch.int32), ("score", score, torch.float64),
                        ("best_mode", best_mode, torch.int32)):
        _want(t, name, dt, (N, Bp1))
    _want(n_nodes, "n_nodes", torch.int32, (N,))
    _want(status, "status", torch.int32, (N,), optional=True)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    if modes is None:
        _check(_lib.mfd_tree_build(_ptr(topk_id), _ptr(topk_raw), _ptr(lse), _ptr(cutoff), _ptr(n_select),
                                   _ptr(anchor_token), N, K, L, k, B, _ptr(node_token), _ptr(parent), _ptr(depth),
                                   _ptr(score), _ptr(best_mode), _ptr(n_nodes), _ptr(status), _ptr(ws), ws_bytes,
                                   _stream_handle(stream)), "mfd_tree_build")
        return
    _want(modes, "modes", torch.int32, (N,))
    _check(_lib.mfd_tree_build_modes(_ptr(topk_id), _ptr(topk_raw), _ptr(lse), _ptr(cutoff), _ptr(n_select),
                                     _ptr(anchor_token), N, K, L, k, B, _ptr(modes), _ptr(node_token), _ptr(parent),
                                     _ptr(depth), _ptr(score), _ptr(best_mode), _ptr(n_nodes), _ptr(status),
                                     _ptr(ws), ws_bytes, _stream_handle(stream)), "mfd_tree_build_modes")


def mfd_mixture_tree(topk_id, topk_raw, lse, anchor_token, B, cutoff, n_select, per_mode_kept, node_token, parent,
                     depth, score, best_mode, n_nodes, status=None, ws=None, stream=None, modes=None):
    """The cut-off and the tree from one search (mfd_mixture_threshold and
    mfd_tree_build in one launch); with modes ([N] int32 on the GPU) tree n uses
    its first modes[n] futures."""
    N, K, L, k = topk_id.shape
    Bp1 = B + 1
    _want(topk_id, "topk_id", torch.int32, (N, K, L, k))
    _want(topk_raw, "topk_raw", torch.float32, (N, K, L, k))
    _want(lse, "lse", torch.float64, (N, K, L))
    _want(anchor_token, "anchor_token", torch.int32, (N,))
    _want(cutoff, "cutoff", torch.float64, (N,))
    _want(n_select, "n_select", torch.int32, (N,))
    _want(per_mode_kept, "per_mode_kept", torch.int32, (N, K), optional=True)
    for name, t, dt in (("node_token", node_token, torch.int32), ("parent", parent, torch.int32),
                        ("depth", depth, torch.int32), ("score", score, torch.float64),
                        ("best_mode", best_mode, torch.int32)):
        _want(t, name, dt, (N, Bp1))
    _want(n_nodes, "n_nodes", torch.int32, (N,))
    _want(status, "status", torch.int32, (N,), optional=True)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    common = (_ptr(topk_id), _ptr(topk_raw), _ptr(lse), _ptr(anchor_token), N, K, L, k, B)
    outs = (_ptr(cutoff), _ptr(n_select), _ptr(per_mode_kept), _ptr(node_token), _ptr(parent), _ptr(depth),
            _ptr(score), _ptr(best_mode), _ptr(n_nodes), _ptr(status), _ptr(ws), ws_bytes, _stream_handle(stream))
    if modes is None:
        _check(_lib.mfd_mixture_tree(*common, *outs), "mfd_mixture_tree")
        return
    _want(modes, "modes", torch.int32, (N,))
    _check(_lib.mfd_mixture_tree_modes(*common, _ptr(modes), *outs), "mfd_mixture_tree_modes")


def mfd_tree_mask(parent, depth, n_nodes, pos_base, mask_words, position_ids, dense_mask=None, stream=None):
    N, Bp1 = parent.shape
    W = (Bp1 + 63) // 64
    _want(parent, "parent", torch.int32, (N, Bp1))
    _want(depth, "depth", torch.int32, (N, Bp1))
    _want(n_nodes, "n_nodes", torch.int32, (N,))
    _want(pos_base, "pos_base", torch.int64, (N,))
    _want(mask_words, "mask_words", torch.int64, (N, Bp1, W))
    _want(position_ids, "position_ids", torch.int64, (N, Bp1))
    _want(dense_mask, "dense_mask", torch.uint8, (N, Bp1, Bp1), optional=True)
    _check(_lib.mfd_tree_mask(_ptr(parent), _ptr(depth), _ptr(n_nodes), _ptr(pos_base), N, Bp1, _ptr(mask_words),
                              _ptr(position_ids), _ptr(dense_mask), _stream_handle(stream)), "mfd_tree_mask")


def mfd_verify_walk(target_logits, L, node_token, parent, depth, n_nodes, temperature, seed, tau, out_tokens,
                    path_nodes, status=None, ws=None, stream=None):
    """target_logits [N, B+1, V] bf16/fp32; seed [N] int64 holding the uint64 bits."""
    if target_logits.dim() != 3 or not target_logits.is_contiguous() or target_logits.device.type != "cuda":
        raise ValueError("target_logits must be a contiguous [N, B+1, V] GPU tensor")
    N, Bp1, V = target_logits.shape
    for name, t in (("node_token", node_token), ("parent", parent), ("depth", depth)):
        _want(t, name, torch.int32, (N, Bp1))
    _want(n_nodes, "n_nodes", torch.int32, (N,))
    _want(temperature, "temperature", torch.float32, (N,))
    _want(seed, "seed", torch.int64, (N,))
    _want(tau, "tau", torch.int32, (N,))
    _want(out_tokens, "out_tokens", torch.int32, (N, L + 1))
    _want(path_nodes, "path_nodes", torch.int32, (N, L + 1))
    _want(status, "status", torch.int32, (N,), optional=True)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.mfd_verify_walk(_ptr(target_logits), _dtype_code(target_logits), N, Bp1, V, L, _ptr(node_token),
                                _ptr(parent), _ptr(depth), _ptr(n_nodes), _ptr(temperature), _ptr(seed), _ptr(tau),
                                _ptr(out_tokens), _ptr(path_nodes), _ptr(status), _ptr(ws), ws_bytes,
                                _stream_handle(stream)), "mfd_verify_walk")


WALK_NOALLOC_BYTES = 16 << 20  # the library's built-in walk workspace


def walk_noalloc_max_trees(L: int) -> int:
    """The most trees mfd_verify_walk_noalloc takes at draft length L: those
    whose walk workspace fits the built-in WALK_NOALLOC_BYTES."""
    lo, hi = 0, 1 << 20
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if workspace_size(MFD_OP_VERIFY_WALK, mid, 1, L, 1, -1) <= WALK_NOALLOC_BYTES:
            lo = mid
        else:
            hi = mid - 1
    return lo


def mfd_verify_walk_noalloc(target_logits, L, node_token, parent, depth, n_nodes, temperature, seed, tau,
                            out_tokens, path_nodes, status=None, stream=None):
    """mfd_verify_walk on the library's built-in workspace (no workspace argument,
    no allocation); at most walk_noalloc_max_trees(L) trees, calls on one GPU must not overlap."""
    if target_logits.dim() != 3 or not target_logits.is_contiguous() or target_logits.device.type != "cuda":
        raise ValueError("target_logits must be a contiguous [N, B+1, V] GPU tensor")
    N, Bp1, V = target_logits.shape
    for name, t in (("node_token", node_token), ("parent", parent), ("depth", depth)):
        _want(t, name, torch.int32, (N, Bp1))
    _want(n_nodes, "n_nodes", torch.int32, (N,))
    _want(temperature, "temperature", torch.float32, (N,))
    _want(seed, "seed", torch.int64, (N,))
    _want(tau, "tau", torch.int32, (N,))
    _want(out_tokens, "out_tokens", torch.int32, (N, L + 1))
    _want(path_nodes, "path_nodes", torch.int32, (N, L + 1))
    _want(status, "status", torch.int32, (N,), optional=True)
    _check(_lib.mfd_verify_walk_noalloc(_ptr(target_logits), _dtype_code(target_logits), N, Bp1, V, L,
                                        _ptr(node_token), _ptr(parent), _ptr(depth), _ptr(n_nodes),
                                        _ptr(temperature), _ptr(seed), _ptr(tau), _ptr(out_tokens), _ptr(path_nodes),
                                        _ptr(status), _stream_handle(stream)), "mfd_verify_walk_noalloc")


def covered_mass_workspace(N: int, Bp1: int, device="cuda") -> torch.Tensor:
    """A device workspace for mfd_covered_mass on N trees of Bp1 rows."""
    n = workspace_size(MFD_OP_COVERED_MASS, N, 0, 0, 0, Bp1 - 1)
    return torch.empty((max(n, 8) + 7) // 8, dtype=torch.int64, device=device)


def mfd_covered_mass(target_logits, node_token, parent, n_nodes, temperature, mass, status=None, ws=None,
                     stream=None):
    """Expected accepted drafted tokens per tree: target_logits [N, B+1, V] -> mass [N] fp64."""
    if target_logits.dim() != 3 or not target_logits.is_contiguous() or target_logits.device.type != "cuda":
        raise ValueError("target_logits must be a contiguous [N, B+1, V] GPU tensor")
    N, Bp1, V = target_logits.shape
    for name, t in (("node_token", node_token), ("parent", parent)):
        _want(t, name, torch.int32, (N, Bp1))
    _want(n_nodes, "n_nodes", torch.int32, (N,))
    _want(temperature, "temperature", torch.float32, (N,))
    _want(mass, "mass", torch.float64, (N,))
    _want(status, "status", torch.int32, (N,), optional=True)
    if ws is None:
        ws = covered_mass_workspace(N, Bp1, target_logits.device)
    ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.mfd_covered_mass(_ptr(target_logits), _dtype_code(target_logits), N, Bp1, V, _ptr(node_token),
                                 _ptr(parent), _ptr(n_nodes), _ptr(temperature), _ptr(mass), _ptr(status), _ptr(ws),
                                 ws_bytes, _stream_handle(stream)), "mfd_covered_mass")


def mfd_chimera_count(node_token, parent, depth, n_nodes, L, future_a, future_b, count, stream=None):
    """Chimeras per tree relative to two futures [N, L] -> count [N] int32."""
    N, Bp1 = node_token.shape
    for name, t in (("node_token", node_token), ("parent", parent), ("depth", depth)):
        _want(t, name, torch.int32, (N, Bp1))
    _want(n_nodes, "n_nodes", torch.int32, (N,))
    _want(future_a, "future_a", torch.int32, (N, L))
    _want(future_b, "future_b", torch.int32, (N, L))
    _want(count, "count", torch.int32, (N,))
    _check(_lib.mfd_chimera_count(_ptr(node_token), _ptr(parent), _ptr(depth), _ptr(n_nodes), N, Bp1, L,
                                  _ptr(future_a), _ptr(future_b), _ptr(count), _stream_handle(stream)),
           "mfd_chimera_count")


def mfd_stream_read(buf, sink, stream=None):
    """Reads every byte of the contiguous GPU tensor `buf` once (the device's
    streaming-read reference rate); sink: [1] int32 on the GPU, XOR-ed with the
    XOR of all 32-bit words of buf."""
    if not buf.is_contiguous() or buf.device.type != "cuda":
        raise ValueError("buf must be a contiguous GPU tensor")
    _want(sink, "sink", torch.int32, (1,))
    nbytes = buf.numel() * buf.element_size()
    _check(_lib.mfd_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream_handle(stream)), "mfd_stream_read")
