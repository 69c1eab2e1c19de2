"""Build libmfdtree.so (HIP kernels for gfx950 + the C ABI) in place.

    python -m mixture_draft_tree_amd.build [--jobs N]

Compiles every source under csrc/ with hipcc for gfx950 and links them into
mixture_draft_tree_amd/libmfdtree.so.  Always rebuilds.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmfdtree.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
# Packed fp32 VALU forms are kept out of the generated code.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]
SOURCES = ["lsm_topk.hip", "lmhead_topk.hip", "tree_build.hip", "tree_mask.hip", "verify_walk.hip", "diagnostics.hip", "stream_read.hip",
           "mfd_api.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), "-O3", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-Wall",
               "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    noise = [ln for ln in res.stderr.splitlines() if "not a recognized feature" not in ln]
    if any(ln.strip() for ln in noise):
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    build_c_smoke()
    build_hostsan(jobs)
    build_wave_check()
    return LIB


C_SMOKE_SRC = os.path.join(ROOT, "tests", "c", "abi_smoke.c")
C_SMOKE_BIN = os.path.join(ROOT, "tests", "c", "abi_smoke")


def build_c_smoke() -> None:
    """The plain-C caller of the C ABI used by the tests (host code only, gcc)."""
    if not os.path.exists(C_SMOKE_SRC) or shutil.which("gcc") is None:
        return
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = ["gcc", "-std=c11", "-Wall", "-Werror", "-O2", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(rocm, "include"), C_SMOKE_SRC, "-L", HERE, "-lmfdtree", "-L", os.path.join(rocm, "lib"),
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../mixture_draft_tree_amd", "-Wl,-rpath," + os.path.join(rocm, "lib"),
           "-o", C_SMOKE_BIN]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"C smoke build failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")


WAVE_CHECK_SRC = os.path.join(ROOT, "tests", "c", "wave_primitives.hip")
WAVE_CHECK_BIN = os.path.join(ROOT, "tests", "c", "wave_primitives")


def build_wave_check() -> None:
    """The standalone GPU check of the kernels' wave-level primitives (built
    with the library's device flags)."""
    if not os.path.exists(WAVE_CHECK_SRC):
        return
    flags = [f for f in COMMON if f != "-fPIC"] + ["-I", CSRC]
    cmd = [hipcc()] + flags + [WAVE_CHECK_SRC, "-o", WAVE_CHECK_BIN]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"wave primitive check build failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")


HOSTSAN_DIR = os.path.join(ROOT, "tests", "c", "hostsan")
# Host code only: each sanitizer flag goes to the host compilation (device
# code is built as in the library proper).
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile_hostsan(src: str) -> str:
    obj = os.path.join(HOSTSAN_DIR, os.path.basename(src) + ".o")
    flags = [f for f in COMMON if f != "-O3"] + ["-O1", "-g"] + HOST_SANITIZE
    if src.endswith(".cpp"):
        flags = ["-O1", "-g", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-Wall"] + HOST_SANITIZE
    cmd = [hipcc()] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build_hostsan(jobs: int = 8) -> None:
    """The library with AddressSanitizer and UndefinedBehaviorSanitizer on its
    host code, and the plain-C caller built with both, under tests/c/hostsan/.
    Test infrastructure: the CPU tests run the caller's argument and workspace
    checks through it."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        return
    os.makedirs(HOSTSAN_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile_hostsan, SOURCES))
    lib = os.path.join(HOSTSAN_DIR, "libmfdtree.so")
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}"] + HOST_SANITIZE + ["-o", lib] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = [clang, "-std=c11", "-O1", "-g", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"), C_SMOKE_SRC,
           "-L", HOSTSAN_DIR, "-lmfdtree", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(rocm, "lib"),
           "-o", os.path.join(HOSTSAN_DIR, "abi_smoke")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized C caller build failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    args = ap.parse_args()
    print(build(args.jobs))


if __name__ == "__main__":
    main()
