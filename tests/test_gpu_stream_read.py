"""The streaming-read reference kernel (attnres_stream_read): every 32-bit
word of the source is read exactly once, so the XOR of the sink words equals
the XOR of the source words, which numpy computes on the host (exact: the
kernel's only arithmetic is XOR). Covers an empty read, sizes below one word
per thread, a ragged tail of the grid-stride loop and a multi-MiB buffer."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_tools import DEV, lib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [0, 16, 4096 + 48, (1 << 22) + 16 * 777, 3 << 23])
def test_stream_read_xor(nbytes):
    sga = lib()
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    sink = torch.full((sga.STREAM_READ_SINK_WORDS,), -1, dtype=torch.int32, device=DEV)
    sga.attnres_stream_read(src, sink)
    torch.cuda.synchronize()
    words = sink.cpu().numpy().view(np.uint32)
    expect = np.bitwise_xor.reduce(host) if host.size else np.uint32(0)
    assert np.bitwise_xor.reduce(words) == expect
    if nbytes == 0:
        assert np.all(words == 0), "every sink word is written"
