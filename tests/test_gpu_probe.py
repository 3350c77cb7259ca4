"""The streaming-read probe (a measurement aid of the benchmark) reads every
byte it is given: the XOR of its per-workgroup words equals the XOR of all
32-bit words of the buffer, for sizes that fill several rounds of the grid,
one partial round and a single 16-byte vector.  The LDS read probe's
per-workgroup XOR equals the one computed here from its documented fill and
read pattern."""

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


def lds_probe_expected(rounds):
    """XOR of the words a 256-thread workgroup of the LDS probe reads: word i
    of the buffer is i * 0x9E3779B1 (mod 2^32); thread t reads 16-byte vector
    (t + 256 u + 8 r) mod 2048 for u < 8, r < rounds."""
    words = (np.arange(4 * 2048, dtype=np.uint64) * 0x9E3779B1) & 0xFFFFFFFF
    vec = np.bitwise_xor.reduce(words.reshape(2048, 4), axis=1)
    t = np.arange(256)[:, None, None]
    u = np.arange(8)[None, :, None]
    r = np.arange(rounds)[None, None, :]
    idx = (t + 256 * u + 8 * r) % 2048
    return int(np.bitwise_xor.reduce(vec[idx].ravel()))


@pytest.mark.parametrize("rounds,sink_words,width", [(1, 4096, 16), (3, 5, 16), (257, 4096, 16),
                                                    (3, 5, 8), (257, 4096, 8), (3, 5, 4),
                                                    (257, 4096, 4)])
def test_lds_read_checksum(gpu, rounds, sink_words, width):
    sink = torch.zeros(sink_words, dtype=torch.int32, device="cuda")
    say("lds read rounds=%d sink=%d width=%d" % (rounds, sink_words, width))
    wg = gpu.lds_read(sink, rounds, width)
    torch.cuda.synchronize()
    assert 1 <= wg <= sink_words
    got = sink.cpu().numpy().view(np.uint32)
    assert np.all(got[:wg] == np.uint32(lds_probe_expected(rounds)))
    assert np.all(got[wg:] == 0)


def test_lds_read_rejects_bad_arguments(gpu):
    sink = torch.zeros(8, dtype=torch.int32, device="cuda")
    for rounds, width in ((0, 16), (4, 12)):
        with pytest.raises(gpu.GlassError) as ei:
            gpu.lds_read(sink, rounds, width)
        assert ei.value.code == -1


def test_stream_read_rejects_bad_sizes(gpu):
    src = torch.zeros(6, dtype=torch.int32, device="cuda")  # 24 bytes: not a multiple of 16
    sink = torch.zeros(8, dtype=torch.int32, device="cuda")
    with pytest.raises(gpu.GlassError) as ei:
        gpu.stream_read(src, sink)
    assert ei.value.code == -1
