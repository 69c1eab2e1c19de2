import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libmfdtree.so")
    config.addinivalue_line("markers", "own_process_gpu: runs the GPU in a child process; collected first")


def pytest_collection_modifyitems(config, items):
    # The plain-C caller's GPU round runs in a child process; it is collected
    # first so that it meets a GPU this process has not touched yet.
    first = [it for it in items if it.get_closest_marker("own_process_gpu")]
    if first:
        rest = [it for it in items if not it.get_closest_marker("own_process_gpu")]
        items[:] = first + rest
