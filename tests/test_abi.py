"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, sizes workspaces, and rejects bad arguments before launching anything.
No call here reaches a kernel, so these run without a GPU."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mfdtree.h")

M = pytest.importorskip("mixture_draft_tree_amd.mfdtree", reason="libmfdtree.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mfd_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(M.EXPORTED)
    lib = ctypes.CDLL(M.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_clean_error():
    assert "gfx950" in M.version()
    assert M.last_error() == ""


def test_workspace_sizes():
    for op in (M.MFD_OP_LOGSOFTMAX_TOPK, M.MFD_OP_TREE_MASK):
        assert M.workspace_size(op, 64, 8, 15, 151936, 256) == 0
    assert M.workspace_size(M.MFD_OP_VERIFY_WALK, 64, 8, 15, 151936, 256) > 0
    assert M.workspace_size(M.MFD_OP_VERIFY_WALK, 0, 8, 15, 151936, 256) == 0
    one = M.workspace_size(M.MFD_OP_MIXTURE_THRESHOLD, 1, 8, 15, 151936, 256)
    many = M.workspace_size(M.MFD_OP_MIXTURE_THRESHOLD, 64, 8, 15, 151936, 256)
    assert one > 0 and many == 64 * one
    assert M.workspace_size(M.MFD_OP_TREE_BUILD, 1, 16, 15, 248320, 1024) > one
    assert M.workspace_size(M.MFD_OP_TREE_BUILD, 0, 8, 15, 151936, 256) == 0
    with pytest.raises(M.MfdError) as e:
        M.workspace_size(M.MFD_OP_TREE_BUILD, 1, 33, 15, 100, 8)
    assert e.value.code == M.MFD_ERR_INVALID_ARG and "K must be" in str(e.value)
    with pytest.raises(M.MfdError):
        M.workspace_size(M.MFD_OP_TREE_BUILD, 1, 8, 15, 1 << 20, 8)
    with pytest.raises(M.MfdError):
        M.workspace_size(99, 1, 8, 15, 100, 8)


FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails its checks first


def _lsm(**kw):
    a = dict(logits=FAKE, dt=M.MFD_BF16, N=1, K=8, L=15, V=1000, k=256, lse=FAKE, tid=FAKE, raw=FAKE)
    a.update(kw)
    return M._lib.mfd_logsoftmax_topk(a["logits"], a["dt"], a["N"], a["K"], a["L"], a["V"], a["k"], a["lse"],
                                      a["tid"], a["raw"], None, None, None, 0, None)


@pytest.mark.parametrize("kw,code", [
    (dict(K=0), M.MFD_ERR_INVALID_ARG), (dict(K=33), M.MFD_ERR_INVALID_ARG), (dict(L=0), M.MFD_ERR_INVALID_ARG),
    (dict(L=33), M.MFD_ERR_INVALID_ARG), (dict(V=0), M.MFD_ERR_INVALID_ARG), (dict(N=-1), M.MFD_ERR_INVALID_ARG),
    (dict(k=0), M.MFD_ERR_INVALID_ARG), (dict(k=1001), M.MFD_ERR_INVALID_ARG), (dict(k=4096, V=10000), M.MFD_ERR_INVALID_ARG),
    (dict(dt=7), M.MFD_ERR_DTYPE), (dict(logits=None), M.MFD_ERR_INVALID_ARG), (dict(lse=None), M.MFD_ERR_INVALID_ARG),
    (dict(logits=ctypes.c_void_p(0x100001)), M.MFD_ERR_INVALID_ARG),
])
def test_logsoftmax_topk_rejects(kw, code):
    assert _lsm(**kw) == code
    assert M.last_error() != ""


def _lsm_mapped(N=1, K=2, L=3, V=1000, vmap=FAKE, V_full=5000, k=10, dt=M.MFD_BF16):
    return M._lib.mfd_logsoftmax_topk_mapped(FAKE, dt, N, K, L, V, vmap, V_full, k, FAKE, FAKE, FAKE, None, None,
                                             None)


@pytest.mark.parametrize("kw,code", [
    (dict(V_full=999), M.MFD_ERR_INVALID_ARG), (dict(V_full=1 << 20), M.MFD_ERR_INVALID_ARG),
    (dict(vmap=None), M.MFD_ERR_INVALID_ARG), (dict(k=1001), M.MFD_ERR_INVALID_ARG),
    (dict(dt=7), M.MFD_ERR_DTYPE),
])
def test_logsoftmax_topk_mapped_rejects(kw, code):
    assert _lsm_mapped(**kw) == code
    assert M.last_error() != ""


def test_logsoftmax_topk_mapped_zero_trees():
    assert _lsm_mapped(N=0, vmap=None) == M.MFD_OK


def _mass(N=2, Bp1=9, V=16, dt=M.MFD_BF16, ws=FAKE, ws_bytes=1 << 20, mass=FAKE):
    return M._lib.mfd_covered_mass(FAKE, dt, N, Bp1, V, FAKE, FAKE, FAKE, FAKE, mass, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(N=70000), M.MFD_ERR_INVALID_ARG), (dict(Bp1=0), M.MFD_ERR_INVALID_ARG), (dict(V=0), M.MFD_ERR_INVALID_ARG),
    (dict(dt=9), M.MFD_ERR_DTYPE), (dict(ws=None), M.MFD_ERR_WORKSPACE), (dict(ws_bytes=8), M.MFD_ERR_WORKSPACE),
    (dict(mass=None), M.MFD_ERR_INVALID_ARG),
])
def test_covered_mass_rejects(kw, code):
    assert _mass(**kw) == code
    assert M.last_error() != ""


def test_chimera_count_rejects_and_zero_trees():
    f = M._lib.mfd_chimera_count
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 9, 0, FAKE, FAKE, FAKE, None) == M.MFD_ERR_INVALID_ARG  # L = 0
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 0, 4, FAKE, FAKE, FAKE, None) == M.MFD_ERR_INVALID_ARG  # Bp1 = 0
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 9, 4, None, FAKE, FAKE, None) == M.MFD_ERR_INVALID_ARG
    assert f(None, None, None, None, 0, 9, 4, None, None, None, None) == M.MFD_OK
    assert _mass(N=0, ws=None, mass=None) == M.MFD_OK
    n = M.workspace_size(M.MFD_OP_COVERED_MASS, 3, 0, 0, 0, 8)
    assert n >= 3 * 9 * 12


def test_zero_trees_is_a_no_op():
    assert _lsm(N=0, logits=None, lse=None, tid=None, raw=None) == M.MFD_OK


def _thr(ws=None, ws_bytes=0, **kw):
    a = dict(N=2, K=8, L=15, k=256, B=256)
    a.update(kw)
    return M._lib.mfd_mixture_threshold(FAKE, FAKE, FAKE, a["N"], a["K"], a["L"], a["k"], a["B"], FAKE, FAKE, None,
                                        None, ws, ws_bytes, None)


def test_tree_calls_check_workspace_and_limits():
    need = M.workspace_size(M.MFD_OP_MIXTURE_THRESHOLD, 2, 8, 15, 151936, 256)
    assert _thr() == M.MFD_ERR_WORKSPACE
    assert "workspace needs" in M.last_error()
    assert _thr(ws=FAKE, ws_bytes=need - 1) == M.MFD_ERR_WORKSPACE
    assert _thr(K=17, k=1024, B=1024) == M.MFD_ERR_INVALID_ARG  # K*k > 16384
    assert _thr(B=-1) == M.MFD_ERR_INVALID_ARG
    assert _thr(B=16384) == M.MFD_ERR_INVALID_ARG
    rc = M._lib.mfd_tree_build(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 15, 256, 256, FAKE, FAKE, FAKE, FAKE, FAKE,
                               None, None, FAKE, 1 << 30, None)
    assert rc == M.MFD_ERR_INVALID_ARG and "n_nodes" in M.last_error()


def test_mask_and_walk_reject():
    assert M._lib.mfd_tree_mask(FAKE, FAKE, FAKE, FAKE, 1, 0, FAKE, FAKE, None, None) == M.MFD_ERR_INVALID_ARG
    assert M._lib.mfd_tree_mask(FAKE, FAKE, FAKE, None, 1, 9, FAKE, FAKE, None, None) == M.MFD_ERR_INVALID_ARG
    args = [FAKE, M.MFD_F32, 1, 9, 16, 4] + [FAKE] * 9 + [None, None, 0, None]
    bad = list(args)
    bad[1] = 5
    assert M._lib.mfd_verify_walk(*bad) == M.MFD_ERR_DTYPE
    bad = list(args)
    bad[5] = 0
    assert M._lib.mfd_verify_walk(*bad) == M.MFD_ERR_INVALID_ARG
    bad = list(args)
    bad[6] = None
    assert M._lib.mfd_verify_walk(*bad) == M.MFD_ERR_INVALID_ARG
    assert M._lib.mfd_verify_walk(*args) == M.MFD_ERR_WORKSPACE  # no workspace


def test_walk_noalloc_limit_and_rejects():
    """The built-in walk workspace holds 16 MiB: the trees whose workspace fits
    are accepted, one more is refused before anything touches a device, and
    fewer trees fit at a longer draft length (a tree keeps slots per round)."""
    cap = M.walk_noalloc_max_trees(4)
    assert M.workspace_size(M.MFD_OP_VERIFY_WALK, cap, 1, 4, 1, -1) <= 16 << 20
    assert M.workspace_size(M.MFD_OP_VERIFY_WALK, cap + 1, 1, 4, 1, -1) > 16 << 20
    assert M.walk_noalloc_max_trees(32) < M.walk_noalloc_max_trees(15) < cap
    assert M.walk_noalloc_max_trees(15) >= 64  # a batch of 64 trees of 15 tokens fits
    # the speculative pass's arrays come on top when the trees' B and V are given
    assert (M.workspace_size(M.MFD_OP_VERIFY_WALK, 64, 8, 15, 151936, 256) >
            M.workspace_size(M.MFD_OP_VERIFY_WALK, 64, 8, 15, 151936, -1))
    args = [FAKE, M.MFD_F32, cap + 1, 9, 16, 4] + [FAKE] * 9 + [None, None]
    assert M._lib.mfd_verify_walk_noalloc(*args) == M.MFD_ERR_WORKSPACE
    assert f"N <= {cap}" in M.last_error()
    bad = list(args)
    bad[1] = 5
    assert M._lib.mfd_verify_walk_noalloc(*bad) == M.MFD_ERR_DTYPE
    bad = list(args)
    bad[6] = None
    assert M._lib.mfd_verify_walk_noalloc(*bad) == M.MFD_ERR_INVALID_ARG
    zero = [None, M.MFD_F32, 0, 9, 16, 4] + [None] * 9 + [None, None]
    assert M._lib.mfd_verify_walk_noalloc(*zero) == M.MFD_OK


def test_binding_checks_shapes_on_cpu_tensors():
    import torch
    x = torch.zeros((1, 2, 3, 16), dtype=torch.float32)
    with pytest.raises(ValueError):
        M.mfd_logsoftmax_topk(x, 4, None, None, None)


def test_modes_calls_reject_before_launch():
    """The per-tree mode-count calls: a missing modes array and the checks of the
    calls they extend are reported before anything launches."""
    lsm = M._lib.mfd_logsoftmax_topk_modes
    assert lsm(FAKE, M.MFD_BF16, 1, 8, 15, 1000, None, 256, FAKE, FAKE, FAKE, None, None, None) == M.MFD_ERR_INVALID_ARG
    assert "modes" in M.last_error()
    assert lsm(FAKE, M.MFD_BF16, 1, 8, 15, 1000, FAKE, 1001, FAKE, FAKE, FAKE, None, None, None) == M.MFD_ERR_INVALID_ARG
    assert lsm(FAKE, 7, 1, 8, 15, 1000, FAKE, 256, FAKE, FAKE, FAKE, None, None, None) == M.MFD_ERR_DTYPE
    assert lsm(None, M.MFD_BF16, 0, 8, 15, 1000, None, 256, None, None, None, None, None, None) == M.MFD_OK
    thr = M._lib.mfd_mixture_threshold_modes
    need = M.workspace_size(M.MFD_OP_MIXTURE_THRESHOLD, 2, 8, 15, 151936, 256)
    assert thr(FAKE, FAKE, FAKE, 2, 8, 15, 256, 256, None, FAKE, FAKE, None, None, FAKE, need,
               None) == M.MFD_ERR_INVALID_ARG
    assert thr(FAKE, FAKE, FAKE, 2, 8, 15, 256, 256, FAKE, FAKE, FAKE, None, None, FAKE, need - 1,
               None) == M.MFD_ERR_WORKSPACE
    assert thr(FAKE, FAKE, FAKE, 2, 33, 15, 256, 256, FAKE, FAKE, FAKE, None, None, FAKE, need,
               None) == M.MFD_ERR_INVALID_ARG
    bld = M._lib.mfd_tree_build_modes
    nb = M.workspace_size(M.MFD_OP_TREE_BUILD, 1, 8, 15, 151936, 256)
    args = [FAKE] * 6 + [1, 8, 15, 256, 256]
    outs = [FAKE] * 6
    assert bld(*args, None, *outs, None, FAKE, nb, None) == M.MFD_ERR_INVALID_ARG
    assert bld(*args, FAKE, *outs, None, None, 0, None) == M.MFD_ERR_WORKSPACE
    assert bld(*[None] * 6, 0, 8, 15, 256, 256, None, *[None] * 6, None, None, 0, None) == M.MFD_OK


def test_stream_read_rejects():
    f = M._lib.mfd_stream_read
    assert f(FAKE, 17, FAKE, None) == M.MFD_ERR_INVALID_ARG
    assert "multiple of 16" in M.last_error()
    assert f(ctypes.c_void_p(0x100008), 32, FAKE, None) == M.MFD_ERR_INVALID_ARG
    assert f(FAKE, 32, None, None) == M.MFD_ERR_INVALID_ARG
    assert f(None, 0, None, None) == M.MFD_OK


def _lmh(**kw):
    a = dict(h=FAKE, w=FAKE, N=1, K=8, L=15, D=2560, V=151936, k=256, lse=FAKE, tid=FAKE, raw=FAKE,
             ws=ctypes.c_void_p(0x100000), ws_bytes=1 << 40)
    a.update(kw)
    return M._lib.mfd_lmhead_logsoftmax_topk(a["h"], a["w"], a.get("layout", M.MFD_HEAD_ROWS), a["N"], a["K"], a["L"],
                                             a["D"], a["V"], a["k"], a["lse"], a["tid"], a["raw"], None, None, a["ws"],
                                             a["ws_bytes"], None)


def test_lmhead_call_rejects_before_launch():
    assert _lmh(D=100) == M.MFD_ERR_INVALID_ARG and "multiple of 64" in M.last_error()
    assert _lmh(D=96) == M.MFD_ERR_INVALID_ARG
    assert _lmh(D=16384) == M.MFD_ERR_INVALID_ARG and "V*D" in M.last_error()
    assert _lmh(N=20000, D=16384, V=1000) == M.MFD_ERR_INVALID_ARG and "N*K*L*D" in M.last_error()
    assert _lmh(D=0) == M.MFD_ERR_INVALID_ARG
    assert _lmh(D=16416) == M.MFD_ERR_INVALID_ARG
    assert _lmh(k=0) == M.MFD_ERR_INVALID_ARG
    assert _lmh(V=100, k=101) == M.MFD_ERR_INVALID_ARG
    assert _lmh(k=2049) == M.MFD_ERR_INVALID_ARG
    assert _lmh(K=33) == M.MFD_ERR_INVALID_ARG
    assert _lmh(h=None) == M.MFD_ERR_INVALID_ARG
    assert _lmh(h=ctypes.c_void_p(0x100008)) == M.MFD_ERR_INVALID_ARG and "aligned" in M.last_error()
    assert _lmh(ws=None) == M.MFD_ERR_WORKSPACE
    assert _lmh(ws_bytes=1000) == M.MFD_ERR_WORKSPACE and "workspace needs" in M.last_error()
    assert _lmh(ws=ctypes.c_void_p(0x100010)) == M.MFD_ERR_WORKSPACE
    assert _lmh(N=0, h=None, w=None) == M.MFD_OK
    assert _lmh(layout=2) == M.MFD_ERR_INVALID_ARG and "layout" in M.last_error()


def test_lmhead_workspace_size():
    one = M.workspace_size(M.MFD_OP_LMHEAD_TOPK, 1, 8, 15, 151936, 256)
    many = M.workspace_size(M.MFD_OP_LMHEAD_TOPK, 64, 8, 15, 151936, 256)
    assert 0 < one < many and many <= 70 * one   # one tree takes the few-row path, 64 trees 256-column tiles
    three = M.workspace_size(M.MFD_OP_LMHEAD_TOPK, 3, 8, 15, 151936, 256)
    six = M.workspace_size(M.MFD_OP_LMHEAD_TOPK, 6, 8, 15, 151936, 256)
    assert abs(six - 2 * three) <= 5 * 256        # same tile shape: linear in the rows
    assert M.workspace_size(M.MFD_OP_LMHEAD_TOPK, 0, 8, 15, 151936, 256) == 0
    assert M.workspace_size(M.MFD_OP_LMHEAD_TOPK, 1, 8, 15, 151936, 1024) > one
    with pytest.raises(M.MfdError):
        M.workspace_size(M.MFD_OP_LMHEAD_TOPK, 1, 8, 15, 151936, 4096)


def test_lmhead_mapped_rejects_before_launch():
    f = M._lib.mfd_lmhead_logsoftmax_topk_mapped
    args = lambda vm=FAKE, V_full=200000, V=65536, N=1: (FAKE, FAKE, M.MFD_HEAD_ROWS, vm, V_full, N, 8, 15, 2560, V,
                                                       256, FAKE, FAKE, FAKE, None, None, ctypes.c_void_p(0x100000),
                                                       1000, None)
    assert f(*args(V_full=1000)) == M.MFD_ERR_INVALID_ARG and "V_full" in M.last_error()
    assert f(*args(V_full=1 << 20)) == M.MFD_ERR_INVALID_ARG
    assert f(*args(vm=None)) == M.MFD_ERR_INVALID_ARG and "vocab_map" in M.last_error()
    assert f(*args()) == M.MFD_ERR_WORKSPACE          # 1000 bytes of workspace: rejected, nothing launched
    assert f(*args(vm=None, N=0)) == M.MFD_OK


def test_lmhead_pack_checks():
    assert M.lmhead_packed_size(151936, 2560) == 152064 * 2560 * 2
    assert M.lmhead_packed_size(1, 64) == 256 * 64 * 2
    with pytest.raises(M.MfdError):
        M.lmhead_packed_size(1000, 100)
    f = M._lib.mfd_lmhead_pack_weight
    assert f(FAKE, 1000, 128, FAKE, 1000, None) == M.MFD_ERR_INVALID_ARG and "packed needs" in M.last_error()
    assert f(None, 1000, 128, FAKE, 1 << 30, None) == M.MFD_ERR_INVALID_ARG
    assert f(FAKE, 1000, 128, ctypes.c_void_p(0x100008), 1 << 30, None) == M.MFD_ERR_INVALID_ARG
