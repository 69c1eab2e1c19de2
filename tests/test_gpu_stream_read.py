"""GPU check of the streaming-read reference kernel (mfd_stream_read): every
32-bit word of the buffer is read exactly once, whatever its size relative to
the grid."""

import numpy as np
import pytest
import torch

from mixture_draft_tree_amd import mfdtree as M

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nwords", [4, 60, 4096 * 4 + 12, 3 * (1 << 20) + 36, 256 * 8 * 256 * 4 * 3 + 4])
def test_stream_read_xor(nwords):
    print(f"[stream_read] words={nwords}", flush=True)
    rng = np.random.default_rng(nwords)
    h = rng.integers(-(1 << 31), 1 << 31, size=nwords, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(h).cuda()
    sink = torch.tensor([0x5A5A], dtype=torch.int32, device="cuda")
    M.mfd_stream_read(buf, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(h.view(np.uint32)) ^ np.uint32(0x5A5A)
    assert np.uint32(sink.cpu().numpy().view(np.uint32)[0]) == want
