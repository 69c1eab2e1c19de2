"""The kernels' wave-level primitives on the GPU: lane exchanges (DPP and
permlane moves), wave and block scans, and the sorting networks, each against
a host computation (tests/c/wave_primitives.hip, built by the package build)."""

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(__file__), "c", "wave_primitives")


def test_wave_primitives_match_host():
    assert os.path.exists(BIN), f"{BIN} is missing: run `python -m mixture_draft_tree_amd.build`"
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=60)
    print(res.stdout, flush=True)
    assert res.returncode == 0 and "ALL OK" in res.stdout, res.stdout + res.stderr
