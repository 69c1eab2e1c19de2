"""The C ABI called from a plain C program (tests/c/abi_smoke.c, built by
build()): no Python binding, no torch on the calling side."""

import os
import struct
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle as O
from mixture_draft_tree_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c", "abi_smoke")

needs_bin = pytest.mark.skipif(not os.path.exists(BIN), reason="tests/c/abi_smoke not built (run build())")


@needs_bin
def test_c_caller_cpu_checks():
    r = subprocess.run([BIN, "cpu"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_smoke cpu: ok" in r.stdout


SAN_BIN = os.path.join(ROOT, "tests", "c", "hostsan", "abi_smoke")


@pytest.mark.skipif(not os.path.exists(SAN_BIN), reason="tests/c/hostsan not built (run build())")
def test_c_caller_cpu_checks_under_sanitizers():
    """The host layer (argument checks, workspace sizes, error text) driven from
    C with AddressSanitizer and UndefinedBehaviorSanitizer on the library's host
    code and on the caller: any finding aborts the run."""
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([SAN_BIN, "cpu"], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_smoke cpu: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


@needs_bin
@pytest.mark.gpu
@pytest.mark.own_process_gpu
def test_c_caller_gpu_round(tmp_path):
    # two trees of the tiny workload; the second is walked at T = 1
    print("C caller: tiny workload, 2 trees", flush=True)
    sys.stdout.flush()
    b = synth.draft_batch("tiny", base_seed=5, N=2)
    w = b.workload
    N, K, L, V, B = 2, w.K, w.L, w.V, w.B
    temps = np.array([0.0, 1.0], dtype=np.float32)
    seeds = b.seed.numpy().astype(np.int64).view(np.uint64)
    trees = []
    for n in range(N):
        sel = O.mixture_select_heap(b.logits[n].double().numpy(), B)
        trees.append(O.canonical_tree(sel, int(b.anchor[n]), B))
    dep = torch.tensor(np.stack([t["depth"] for t in trees]), dtype=torch.int32)
    nn = torch.tensor([t["n_nodes"] for t in trees], dtype=torch.int32)
    R = synth.target_logits(b, dep, nn).float()
    src = tmp_path / "in.bin"
    with open(src, "wb") as f:
        f.write(struct.pack("<5i", N, K, L, V, B))
        f.write(b.logits.float().numpy().tobytes())
        f.write(b.anchor.numpy().astype(np.int32).tobytes())
        f.write(b.pos_base.numpy().astype(np.int64).tobytes())
        f.write(R.numpy().tobytes())
        f.write(temps.tobytes())
        f.write(seeds.tobytes())
    out = tmp_path / "out.bin"
    r = subprocess.run([BIN, "gpu", str(src), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    raw = out.read_bytes()
    Bp1, W = B + 1, (B + 64) // 64
    off = 0

    def take(dtype, count):
        nonlocal off
        a = np.frombuffer(raw, dtype=dtype, count=count, offset=off)
        off += a.nbytes
        return a

    n_nodes = take(np.int32, N)
    tok = take(np.int32, N * Bp1).reshape(N, Bp1)
    par = take(np.int32, N * Bp1).reshape(N, Bp1)
    depth = take(np.int32, N * Bp1).reshape(N, Bp1)
    mask = take(np.uint64, N * Bp1 * W).reshape(N, Bp1, W)
    pos = take(np.int64, N * Bp1).reshape(N, Bp1)
    tau = take(np.int32, N)
    toks = take(np.int32, N * (L + 1)).reshape(N, L + 1)
    status = take(np.int32, N)
    assert off == len(raw)
    assert np.all(status == 0)
    for n in range(N):
        t = trees[n]
        assert n_nodes[n] == t["n_nodes"]
        assert np.array_equal(tok[n], t["node_token"]) and np.array_equal(par[n], t["parent"])
        assert np.array_equal(depth[n], t["depth"])
        dm, want_pos = O.tree_mask(t["parent"], t["depth"], t["n_nodes"], int(b.pos_base[n]), Bp1)
        assert np.array_equal(mask[n].view(np.int64), O.pack_mask_words(dm).view(np.int64))
        assert np.array_equal(pos[n], want_pos)
        o_tau, o_toks, _, _ = O.verify_walk(t["node_token"], t["parent"], t["depth"], t["n_nodes"],
                                            R[n].double().numpy(), float(temps[n]), int(seeds[n]), L)
        assert tau[n] == o_tau and np.array_equal(toks[n], o_toks), (n, tau[n], o_tau, toks[n], o_toks)
