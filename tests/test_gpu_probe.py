"""The streaming-read probe (a measurement aid of the benchmark) reads every
byte it is given: the XOR of its per-workgroup words equals the XOR of all
32-bit words of the buffer, for sizes that fill several rounds of the grid,
one partial round and a single 16-byte vector."""

import numpy as np
import pytest
import torch

from gpu_common import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nwords", [4, 4 * 1000 + 4, 64 * 1024 * 1024 + 12])
def test_stream_read_checksum(gpu, nwords):
    rng = np.random.default_rng(nwords)
    host = rng.integers(-2 ** 31, 2 ** 31, size=nwords, dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(host).cuda()
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    say("stream read %d bytes" % (4 * nwords))
    gpu.stream_read(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy())
    assert got == np.bitwise_xor.reduce(host)


def test_stream_read_rejects_bad_sizes(gpu):
    src = torch.zeros(6, dtype=torch.int32, device="cuda")  # 24 bytes: not a multiple of 16
    sink = torch.zeros(8, dtype=torch.int32, device="cuda")
    with pytest.raises(gpu.GlassError) as ei:
        gpu.stream_read(src, sink)
    assert ei.value.code == -1
